// Internal declarations shared by the HIP translation units of libmoe_mi355x.
// Nothing here is part of the C ABI (include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 8;
// A token whose fp32 top-(k+1) logits are closer than this is re-ranked from
// fp64 logits.  fp32 accumulation error at the supported D is ~1e-6.
constexpr float kRefineMargin = 1e-4f;

enum GemmAct { kActNone = 0, kActGelu = 1, kActRelu = 2, kActSwiGLU = 3 };

// Number of compute units of the current device (cached per device).
int device_cu_count();

// ---- launchers (stream-ordered, no synchronisation, return hipError_t) ----
hipError_t launch_route(const moe_shape& s, const void* x, const void* wr, const float* br,
                        int32_t* idx, float* gate, float* logits, float* prob_part, int R, int32_t* fb_idx,
                        float* fb_gate, hipStream_t st);

// Router of few-token bf16 batches in two launches over many waves (partial
// logit tiles per 128-wide k chunk, then sum and rank); part is device
// scratch of route_split_bytes(s) bytes.  Same selection as launch_route.
bool use_split_route(const moe_shape& s);
size_t route_split_bytes(const moe_shape& s);
hipError_t launch_route_split(const moe_shape& s, const void* x, const void* wr, const float* br, int32_t* idx,
                              float* gate, float* logits, float* part, hipStream_t st);

// Router blocks of a launch (tokens per block depend on the shape and the
// device's CU count); prob_part holds N * route_blocks(s) floats.
int route_rows_per_block(const moe_shape& s);
int64_t route_blocks(const moe_shape& s);
unsigned long long* stats_ticket(const moe_shape& s, const float* prob_part);
hipError_t launch_router_stats(const moe_shape& s, const float* prob_part, const int32_t* counts,
                               const int32_t* n_dropped, double* prob_mean, double* frac, double* summary,
                               hipStream_t st);

hipError_t launch_dispatch(const moe_shape& s, const int32_t* idx, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* slot, int32_t* n_dropped,
                           hipStream_t st);
// The same dispatch over many workgroups (two launches): bc is device
// scratch of dispatch_ws_bytes(s) bytes for the per-segment counts.
size_t dispatch_ws_bytes(const moe_shape& s);
hipError_t launch_dispatch_multi(const moe_shape& s, const int32_t* idx, int32_t* counts, int32_t* offsets,
                                 int32_t* perm, int32_t* slot, int32_t* n_dropped, int32_t* bc, hipStream_t st);
// Dispatch with R levels of overflow rerouting (compact layout); rewrites
// idx and gate of the rerouted assignments.
hipError_t launch_dispatch_reroute(const moe_shape& s, int R, const int32_t* fb_idx, const float* fb_gate,
                                   int32_t* idx, float* gate, int32_t* counts, int32_t* offsets, int32_t* perm,
                                   int32_t* slot, int32_t* n_dropped, hipStream_t st);

hipError_t launch_combine(const moe_shape& s, const void* y_perm, const int32_t* slot,
                          const float* gate, const void* x_res, void* out, hipStream_t st);

// Decode path: fused per-(expert, F-shard) weight-streaming MLP writing fp32
// shard partials part[NS][T*k][D]; used when rows per expert are few.
int decode_shards(const moe_shape& s);
bool decode_applicable(const moe_shape& s, int64_t expected_rows_per_expert);
size_t decode_part_bytes(const moe_shape& s);
hipError_t launch_decode_ffn(const moe_shape& s, const void* x, const int32_t* perm,
                             const int32_t* offsets, const void* w1, const void* b1, const void* w3,
                             const void* w2, const void* b2, float* part, hipStream_t st);
// y_perm = sum of the shard partials (bf16), for the stage API.
hipError_t launch_reduce_shards(const moe_shape& s, const float* part, const int32_t* offsets,
                                void* y_perm, hipStream_t st);
// Combine reading the fp32 shard partials directly (whole-layer path).
hipError_t launch_combine_shards(const moe_shape& s, const float* part, int n_shards,
                                 const int32_t* slot, const float* gate, const void* x_res, void* out,
                                 hipStream_t st);

}  // namespace moe

#include "grouped_gemm.h"
