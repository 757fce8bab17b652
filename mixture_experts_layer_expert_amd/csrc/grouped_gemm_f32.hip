// Grouped GEMM of the expert MLPs in fp32, for fp32 layers such as the
// notebook's own 1024-token example ("Dispatch and gather" section of
// "Mixture-of-experts and expert parallelism").  Same contract and work list
// as the bf16 kernel: (expert, row tile, 64-column tile) items for all
// experts in one persistent launch; rows of x gathered through perm for fc1;
// bias + GELU/ReLU or SwiGLU fused into the store.
//
// Tile: TBM x 64 outputs (TBM = 64, 32 or 16 rows: the tallest whose
// expected tile count still fills half the grid), 4 waves.  Wave w owns
// output columns 16w .. 16w+15 and computes them for every row of the tile
// with v_mfma_f32_16x16x4f32 (fp32 products, fp32 accumulation): lane l
// feeds row (l % 16) of the 16-row block and column (l % 16) of the wave's
// columns at k offset l / 16, and holds outputs (rows 4*(l/16) + v, column
// l % 16).  Operands are staged k-major in LDS, 16 k per step, and the next
// step's operands are loaded into registers while the current one is
// computed.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int TBN = 64, TBK = 16;

struct ParamsF {
  const float* A;
  const int32_t* perm;
  int topk;
  const int32_t* offsets;
  int n_experts;
  const float* B;
  const float* B2;
  const float* bias;
  float* C;
  int K;
  int n_out;
  int act;
};

__device__ inline float gelu_erf(float z) { return 0.5f * z * (1.f + erff(z * 0.70710678118654752f)); }
__device__ inline float silu(float z) { return z / (1.f + expf(-z)); }

template <bool SWIGLU, int TBM>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(ParamsF p) {
  constexpr int MT = TBM / 16;  // 16-row MFMA blocks per wave
  static_assert(MT == 1 || MT == 2 || MT == 4, "16, 32 or 64 rows");
  // row stride of the k-major tiles: the four 16-lane groups of an operand
  // read (one k each) start 80 floats apart, on different banks
  constexpr int LDW = 80;
  __shared__ float sA[TBK][LDW];
  __shared__ float sB[TBK][LDW];
  __shared__ float sB2[SWIGLU ? TBK : 1][LDW];
  __shared__ int s_tile_start[kMaxExperts + 1];
  __shared__ int s_scan[kMaxExperts];
  const int tid = threadIdx.x;
  const int N = p.n_experts;
  const int ntiles = (p.n_out + TBN - 1) / TBN;

  int my_tiles = 0;
  if (tid < N) {
    int rows = p.offsets[tid + 1] - p.offsets[tid];
    my_tiles = ((rows + TBM - 1) / TBM) * ntiles;
    s_scan[tid] = my_tiles;
  }
  __syncthreads();
  for (int d = 1; d < kMaxExperts; d <<= 1) {
    int v = 0;
    if (tid < N && tid >= d) v = s_scan[tid - d];
    __syncthreads();
    if (tid < N && tid >= d) s_scan[tid] += v;
    __syncthreads();
  }
  if (tid < N) s_tile_start[tid] = s_scan[tid] - my_tiles;
  if (tid == 0) s_tile_start[N] = (N > 0) ? s_scan[N - 1] : 0;
  __syncthreads();
  const int total = s_tile_start[N];

  const int wave = tid / 64, lane = tid % 64;
  const int lr = lane % 16, lk = lane / 16;  // MFMA operand row/column, k offset
  // loader mapping: 64 rows x 16 k = 1024 floats = 256 float4s for B; the
  // first TBM * 4 threads load the TBM rows of A the same way
  const int ld_row = tid / 4, ld_k4 = (tid % 4) * 4;
  const bool ld_a = ld_row < TBM;

  for (int L = blockIdx.x; L < total; L += gridDim.x) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (s_tile_start[mid] <= L) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int row_begin = p.offsets[e];
    const int rows_e = p.offsets[e + 1] - row_begin;
    const int mtiles = (rows_e + TBM - 1) / TBM;
    const int local = L - s_tile_start[e];
    const int mt = local % mtiles, nt = local / mtiles;
    const int row0 = row_begin + mt * TBM, row_end = row_begin + rows_e;
    const int n0 = nt * TBN;

    int r = row0 + (ld_a ? ld_row : 0);
    if (r > row_end - 1) r = row_end - 1;
    const int src = p.perm ? p.perm[r] / p.topk : r;
    const float* a_src = p.A + (size_t)src * p.K + ld_k4;
    int fb = n0 + ld_row;
    if (fb > p.n_out - 1) fb = p.n_out - 1;
    const float* b_src = p.B + ((size_t)e * p.n_out + fb) * p.K + ld_k4;
    const float* b2_src = SWIGLU ? p.B2 + ((size_t)e * p.n_out + fb) * p.K + ld_k4 : nullptr;

    f32x4 acc[MT], acc3[SWIGLU ? MT : 1];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < (SWIGLU ? MT : 1); ++i) acc3[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the operands of k step k0 + TBK are loaded into registers while step
    // k0 is computed from LDS, so each step's global latency is hidden
    float4 av = ld_a ? *(const float4*)a_src : float4{};
    float4 bv = *(const float4*)b_src;
    float4 b3 = SWIGLU ? *(const float4*)b2_src : float4{};
    for (int k0 = 0; k0 < p.K; k0 += TBK) {
      if (ld_a) {
        sA[ld_k4 + 0][ld_row] = av.x;
        sA[ld_k4 + 1][ld_row] = av.y;
        sA[ld_k4 + 2][ld_row] = av.z;
        sA[ld_k4 + 3][ld_row] = av.w;
      }
      sB[ld_k4 + 0][ld_row] = bv.x;
      sB[ld_k4 + 1][ld_row] = bv.y;
      sB[ld_k4 + 2][ld_row] = bv.z;
      sB[ld_k4 + 3][ld_row] = bv.w;
      if constexpr (SWIGLU) {
        sB2[ld_k4 + 0][ld_row] = b3.x;
        sB2[ld_k4 + 1][ld_row] = b3.y;
        sB2[ld_k4 + 2][ld_row] = b3.z;
        sB2[ld_k4 + 3][ld_row] = b3.w;
      }
      __syncthreads();
      if (k0 + TBK < p.K) {
        if (ld_a) av = *(const float4*)(a_src + k0 + TBK);
        bv = *(const float4*)(b_src + k0 + TBK);
        if constexpr (SWIGLU) b3 = *(const float4*)(b2_src + k0 + TBK);
      }
#pragma unroll
      for (int ks = 0; ks < TBK / 4; ++ks) {
        const float bv_ = sB[4 * ks + lk][16 * wave + lr];
        float b3_ = 0.f;
        if constexpr (SWIGLU) b3_ = sB2[4 * ks + lk][16 * wave + lr];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const float av_ = sA[4 * ks + lk][16 * i + lr];
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(av_, bv_, acc[i], 0, 0, 0);
          if constexpr (SWIGLU) acc3[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(av_, b3_, acc3[i], 0, 0, 0);
        }
      }
      __syncthreads();
    }
    const int f = n0 + 16 * wave + lr;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int ro = row0 + 16 * i + 4 * lk + v;
        if (ro >= row_end || f >= p.n_out) continue;
        float z = acc[i][v];
        if constexpr (SWIGLU) {
          z = silu(z) * acc3[i][v];
        } else {
          if (p.bias) z += p.bias[(size_t)e * p.n_out + f];
          if (p.act == kActGelu) z = gelu_erf(z);
          else if (p.act == kActRelu) z = fmaxf(z, 0.f);
        }
        p.C[(size_t)ro * p.n_out + f] = z;
      }
    }
  }
}

}  // namespace

hipError_t launch_grouped_gemm_f32(const GroupedGemm& g, int64_t expected_rows, hipStream_t st) {
  ParamsF p;
  p.A = (const float*)g.A;
  p.perm = g.perm;
  p.topk = g.topk;
  p.offsets = g.offsets;
  p.n_experts = g.n_experts;
  p.B = (const float*)g.B;
  p.B2 = (const float*)g.B2;
  p.bias = (const float*)g.bias;
  p.C = (float*)g.C;
  p.K = g.K;
  p.n_out = g.n_out;
  p.act = g.act;
  const int grid = device_cu_count() * 4;
  // tile height: the tallest whose expected tile count fills half the grid
  // (two blocks per CU), else 16 rows.  Shorter tiles give each wave fewer
  // MFMA blocks per B operand read, so they pay only where the launch would
  // otherwise leave most CUs idle (measured on the 1024-token layer, 64 / 32
  // / 16 rows: the up projection, 512 tiles at 64 rows, 30.6 / 29.8 / 32.8
  // us; the down projection, 128 tiles at 64 rows, 43.1 / 37.5 / 35.6 us).
  const int64_t ncol = (g.n_out + TBN - 1) / TBN;
  const int64_t er = expected_rows > 0 ? expected_rows : 1;
  auto tiles = [&](int tbm) { return (int64_t)g.n_experts * ((er + tbm - 1) / tbm) * ncol; };
  const int tbm = 2 * tiles(64) >= grid ? 64 : 2 * tiles(32) >= grid ? 32 : 16;
#define MOE_F32(SW, TBM) hipLaunchKernelGGL((grouped_gemm_f32_kernel<SW, TBM>), dim3(grid), dim3(256), 0, st, p)
  if (g.act == kActSwiGLU) {
    if (tbm == 64) MOE_F32(true, 64); else if (tbm == 32) MOE_F32(true, 32); else MOE_F32(true, 16);
  } else {
    if (tbm == 64) MOE_F32(false, 64); else if (tbm == 32) MOE_F32(false, 32); else MOE_F32(false, 16);
  }
#undef MOE_F32
  return hipGetLastError();
}

}  // namespace moe
