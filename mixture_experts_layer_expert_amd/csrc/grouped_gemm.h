// Interface of the grouped GEMM over experts (grouped_gemm.hip,
// grouped_gemm_f32.hip), included at the end of moe_internal.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Grouped GEMM over experts:  C[r, n] = act(sum_k A[row(r), k] * B[e, n, k] + bias[e, n])
// for r in [offsets[e], offsets[e+1]).  row(r) = perm[r] / topk when perm is
// non-null (gather of x), else r.  For SwiGLU, B = w1 and B2 = w3 and
// C[r, n] = silu(A.w1[e,n]) * (A.w3[e,n]).
struct GroupedGemm {
  const void* A;
  const int32_t* perm;
  int topk;
  const int32_t* offsets;
  int n_experts;
  int64_t a_rows;  // rows addressable in A (for clamping of tail loads)
  const void* B;
  const void* B2;
  const void* bias;
  void* C;
  int K;
  int n_out;
  int act;      // GemmAct
  float* part;  // bf16 path: workspace for split-K partial tiles, or nullptr
};

// Picks the bf16 MFMA tile configuration from the expected rows per expert
// and the most rows any expert can have (max_rows_per_expert).  With g.part,
// a partial last round of tiles is split along K into that workspace and
// finished by a second launch.
hipError_t launch_grouped_gemm_bf16(const GroupedGemm& g, int64_t expected_rows_per_expert,
                                    int64_t max_rows_per_expert, hipStream_t st);
// Bytes of g.part the bf16 grouped GEMM may use (both projections).
size_t grouped_gemm_bf16_part_bytes(int64_t expected_rows_per_expert, int64_t max_rows_per_expert);
// fp32 (VALU) grouped GEMM; the expected rows per expert pick the tile height.
hipError_t launch_grouped_gemm_f32(const GroupedGemm& g, int64_t expected_rows_per_expert, hipStream_t st);

}  // namespace moe
