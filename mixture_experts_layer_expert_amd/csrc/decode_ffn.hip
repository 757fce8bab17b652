// Fused weight-streaming expert MLP for few rows per expert (decode).
//
// Work item = (expert e, F-shard s, token group g): the shard is the column
// block [s*Fs, (s+1)*Fs) of W1/W3 (rows of the nn.Linear weights) and the
// matching row block of W2^T (a column block of w2[e]) -- the row/column
// decomposition of expert matrices of "Accelerating MoE Model Inference with
// Expert Sharding" (abstract), applied on one GPU to the CUs instead of to
// GPUs.  Every item of an expert streams the same number of weight bytes,
// so with NS shards per expert the list is balanced whatever the routing
// skew, and the fc1 and fc2 pieces of a shard run in one launch (the fusion
// of decomposed expert computations, same abstract).
//
//  phase 1  H[g rows, Fs] = act(X_e[g rows] . W1_s^T (+b1))   (SwiGLU: with W3_s)
//           weight rows go straight from global memory into MFMA operand
//           registers (each byte is used once); H goes to LDS as bf16.
//  phase 2  P[s][row, D] = H . W2[:, s]^T (+b2 on shard 0), fp32 partials.
// The shard partials are summed (in fixed shard order) by the combine.
//
// MFMA v_mfma_f32_16x16x32_bf16 with the weight as the first operand (16
// weight rows x 32 k) and the activations as the second (32 k x 16 tokens):
// a lane then holds 4 consecutive output columns of one token.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int TG = 32;  // tokens per work item (two 16-token MFMA tiles)
constexpr int U1 = 8;   // k sub-steps loaded together in phase 1
constexpr int U2 = 4;   // ... in phase 2

struct DecodeParams {
  const bf16* x;
  const int32_t* perm;
  int topk;
  const int32_t* offsets;
  int n_experts;
  const bf16* w1;
  const bf16* w3;
  const bf16* w2;
  const bf16* b1;
  const bf16* b2;
  float* part;       // [NS][rows_cap][D]
  int64_t rows_cap;  // rows per shard slab (T*k)
  int D, F, NS, Fs;
  int act;
};

__device__ inline float gelu_erf(float z) { return 0.5f * z * (1.f + erff(z * 0.70710678118654752f)); }
__device__ inline float fast_silu(float z) { return z * __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

template <int ACT>
__global__ __launch_bounds__(kThreads, 1) void decode_ffn_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16* Hs = (bf16*)smem_raw;  // [TG][HS], HS = Fs + 8 (conflict-free row stride)
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_scan[kMaxExperts];
  constexpr bool kSwiGLU = ACT == kActSwiGLU;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int l16 = lane & 15, lq = lane >> 4;
  const int N = p.n_experts, D = p.D, F = p.F, NS = p.NS, Fs = p.Fs;
  const int HS = Fs + 8;

  // ---- work list: NS * ceil(rows/TG) items per expert with rows
  int mine = 0;
  if (tid < N) {
    const int rows = p.offsets[tid + 1] - p.offsets[tid];
    mine = ((rows + TG - 1) / TG) * NS;
    s_scan[tid] = mine;
  }
  __syncthreads();
  for (int d = 1; d < kMaxExperts; d <<= 1) {
    int v = 0;
    if (tid < N && tid >= d) v = s_scan[tid - d];
    __syncthreads();
    if (tid < N && tid >= d) s_scan[tid] += v;
    __syncthreads();
  }
  if (tid < N) s_start[tid] = s_scan[tid] - mine;
  if (tid == 0) s_start[N] = N > 0 ? s_scan[N - 1] : 0;
  __syncthreads();
  const int total = s_start[N];

  const int KS1 = D / 32, KS2 = Fs / 32;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_start[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int local = item - s_start[e];
    const int s = local % NS, g = local / NS;
    const int row0 = p.offsets[e] + g * TG;
    const int nrows = min(TG, p.offsets[e + 1] - row0);
    const int ntt = nrows > 16 ? 2 : 1;  // token tiles in use (uniform)

    // activation rows of this lane (B operand: token l16 of each tile)
    const bf16* xrow[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      int r = row0 + tt * 16 + l16;
      if (r > row0 + nrows - 1) r = row0 + nrows - 1;  // padding tokens reuse a valid row
      xrow[tt] = p.x + (int64_t)(p.perm[r] / p.topk) * D + lq * 8;
    }

    // ---- phase 1: hidden tile for this shard's Fs columns
    const int FT = Fs / 16;
    for (int ft = wave; ft < FT; ft += kWaves) {
      const int f = s * Fs + ft * 16 + l16;  // weight row of this lane
      const bf16* wa = p.w1 + ((int64_t)e * F + f) * D + lq * 8;
      const bf16* wb = kSwiGLU ? p.w3 + ((int64_t)e * F + f) * D + lq * 8 : wa;
      f32x4 ag[2] = {}, au[2] = {};
      for (int kb = 0; kb < KS1; kb += U1) {
        bf16x8 va[U1], vb[U1], vx[U1][2];
#pragma unroll
        for (int u = 0; u < U1; ++u) {
          const bool in = kb + u < KS1;  // uniform
          const int ko = in ? (kb + u) * 32 : 0;  // always an in-bounds address
          const bf16x8 z{};
          const bf16x8 la = *(const bf16x8*)(wa + ko);
          va[u] = in ? la : z;
          if constexpr (kSwiGLU) {
            const bf16x8 lb = *(const bf16x8*)(wb + ko);
            vb[u] = in ? lb : z;
          }
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const bf16x8 lx = *(const bf16x8*)(xrow[tt] + ko);
            vx[u][tt] = (in && tt < ntt) ? lx : z;
          }
        }
#pragma unroll
        for (int u = 0; u < U1; ++u)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            ag[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[u], vx[u][tt], ag[tt], 0, 0, 0);
            if constexpr (kSwiGLU)
              au[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb[u], vx[u][tt], au[tt], 0, 0, 0);
          }
      }
      // lane holds features ft*16 + 4*lq + r of token tt*16 + l16
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        bf16x4 h;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float z = ag[tt][r];
          if constexpr (kSwiGLU) {
            z = fast_silu(z) * au[tt][r];
          } else {
            if (p.b1) z += (float)p.b1[(int64_t)e * F + s * Fs + ft * 16 + 4 * lq + r];
            if constexpr (ACT == kActGelu) z = gelu_erf(z);
            if constexpr (ACT == kActRelu) z = fmaxf(z, 0.f);
          }
          h[r] = (bf16)z;
        }
        *(bf16x4*)(Hs + (tt * 16 + l16) * HS + ft * 16 + 4 * lq) = h;
      }
    }
    __syncthreads();

    // ---- phase 2: fp32 partial rows of y for this shard
    const int DT = D / 16;
    float* pout = p.part + (int64_t)s * p.rows_cap * D;
    for (int dt = wave; dt < DT; dt += kWaves) {
      const int d = dt * 16 + l16;  // weight row (output column) of this lane
      const bf16* w2p = p.w2 + ((int64_t)e * D + d) * F + s * Fs + lq * 8;
      f32x4 acc[2] = {};
      for (int kb = 0; kb < KS2; kb += U2) {
        bf16x8 va[U2], vh[U2][2];
#pragma unroll
        for (int u = 0; u < U2; ++u) {
          const bool in = kb + u < KS2;  // uniform
          const int ko = in ? (kb + u) * 32 : 0;  // always an in-bounds address
          const bf16x8 z{};
          const bf16x8 la = *(const bf16x8*)(w2p + ko);
          va[u] = in ? la : z;
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const bf16x8 lh = *(const bf16x8*)(Hs + (tt * 16 + l16) * HS + ko + lq * 8);
            vh[u][tt] = (in && tt < ntt) ? lh : z;
          }
        }
#pragma unroll
        for (int u = 0; u < U2; ++u)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
            acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[u], vh[u][tt], acc[tt], 0, 0, 0);
      }
      // lane holds output columns dt*16 + 4*lq + r of token tt*16 + l16
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int i = tt * 16 + l16;
        if (i < nrows) {
          f32x4 v = acc[tt];
          if (p.b2 && s == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] += (float)p.b2[(int64_t)e * D + dt * 16 + 4 * lq + r];
          }
          *(f32x4*)(pout + (int64_t)(row0 + i) * D + dt * 16 + 4 * lq) = v;
        }
      }
    }
    __syncthreads();  // H is rewritten by the next item
  }
}

// y_perm[r] = sum over shards of P[s][r] (stage API output), cast to bf16.
__global__ __launch_bounds__(256) void reduce_shards_kernel(const float* __restrict__ part, int NS,
                                                            int64_t rows_cap, const int32_t* offsets,
                                                            int N, int D, bf16* __restrict__ y) {
  const int64_t rows = offsets[N];
  const int chunks = D / 4;
  const int64_t items = rows * chunks;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < items;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / chunks;
    const int c = (int)(i - r * chunks);
    f32x4 acc = *(const f32x4*)(part + r * D + c * 4);
    for (int s = 1; s < NS; ++s) acc += *(const f32x4*)(part + ((int64_t)s * rows_cap + r) * D + c * 4);
    bf16x4 o;
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = (bf16)acc[u];
    *(bf16x4*)(y + r * D + c * 4) = o;
  }
}

template <int ACT>
hipError_t launch_act(const DecodeParams& p, size_t lds, hipStream_t st) {
  auto kern = decode_ffn_kernel<ACT>;
  static const hipError_t attr_err = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 64 * 1024);
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL(kern, dim3(device_cu_count()), dim3(kThreads), lds, st, p);
  return hipGetLastError();
}

}  // namespace

// Shards per expert: about one work item per CU of a 256-CU device, each
// shard a multiple of 32 columns whose hidden tile fits the 64 KiB of LDS
// the kernel asks for.  0 = no such split.
int decode_shards(const moe_shape& s) {
  auto fits = [&](int n) {
    return s.F % n == 0 && (s.F / n) % 32 == 0 && (size_t)TG * (s.F / n + 8) * 2 <= 64 * 1024;
  };
  int want = kMaxExperts / s.N;
  if (want < 1) want = 1;
  if (want > 16) want = 16;
  for (int n = want; n <= 64; ++n)
    if (fits(n)) return n;
  for (int n = want - 1; n >= 1; --n)
    if (fits(n)) return n;
  return 0;
}

bool decode_applicable(const moe_shape& s, int64_t expected_rows) {
  if (s.dtype != MOE_DTYPE_BF16 || expected_rows > 16 || s.D % 32) return false;
  return decode_shards(s) > 0;
}

size_t decode_part_bytes(const moe_shape& s) {
  return (size_t)decode_shards(s) * (size_t)s.T * s.k * s.D * sizeof(float);
}

hipError_t launch_decode_ffn(const moe_shape& s, const void* x, const int32_t* perm,
                             const int32_t* offsets, const void* w1, const void* b1, const void* w3,
                             const void* w2, const void* b2, float* part, hipStream_t st) {
  DecodeParams p;
  p.x = (const bf16*)x;
  p.perm = perm;
  p.topk = s.k;
  p.offsets = offsets;
  p.n_experts = s.N;
  p.w1 = (const bf16*)w1;
  p.w3 = (const bf16*)w3;
  p.w2 = (const bf16*)w2;
  const bool bias = (s.flags & MOE_HAS_BIAS) != 0;
  p.b1 = bias ? (const bf16*)b1 : nullptr;
  p.b2 = bias ? (const bf16*)b2 : nullptr;
  p.part = part;
  p.rows_cap = s.T * (int64_t)s.k;
  p.D = s.D;
  p.F = s.F;
  p.NS = decode_shards(s);
  p.Fs = s.F / p.NS;
  p.act = s.act;
  const size_t lds = (size_t)TG * (p.Fs + 8) * 2;
  switch (s.act) {
    case MOE_ACT_SWIGLU: return launch_act<kActSwiGLU>(p, lds, st);
    case MOE_ACT_RELU: return launch_act<kActRelu>(p, lds, st);
    default: return launch_act<kActGelu>(p, lds, st);
  }
}

hipError_t launch_reduce_shards(const moe_shape& s, const float* part, const int32_t* offsets,
                                void* y_perm, hipStream_t st) {
  const int64_t items = s.T * (int64_t)s.k * (s.D / 4);
  const int64_t cap = (int64_t)device_cu_count() * 8;
  const int64_t blocks = (items + 255) / 256 < cap ? (items + 255) / 256 : cap;
  hipLaunchKernelGGL(reduce_shards_kernel, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0, st,
                     part, decode_shards(s), s.T * (int64_t)s.k, offsets, s.N, s.D, (bf16*)y_perm);
  return hipGetLastError();
}

}  // namespace moe
