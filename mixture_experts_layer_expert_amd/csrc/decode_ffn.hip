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
//           the item's x rows sit in LDS; weight rows go straight from
//           global memory into MFMA operand registers (each byte is used
//           once); H goes to LDS as bf16.
//  phase 2  P[s][row, D] = H . W2[:, s]^T (+b2 on shard 0), fp32 partials.
// The shard partials are summed (in fixed shard order) by the combine.
//
// A direct-to-register operand load gives each lane 16 bytes of one weight
// row, so one load instruction covers 16 rows x 64 bytes (half cache lines);
// the grouped GEMM's DMA ring moves 256-byte row pieces.  Per byte this
// kernel makes twice the memory requests, which is why it streams more
// slowly than the two grouped-GEMM launches it replaces.
//
// MFMA v_mfma_f32_16x16x32_bf16 with the weight as the first operand (16
// weight rows x 32 k) and the activations as the second (32 k x 16 tokens):
// a lane then holds 4 consecutive output columns of one token.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int TG = 32;       // tokens per work item (two 16-token MFMA tiles)
constexpr int U1 = 4;        // phase-1 k sub-steps (of 32) per job
constexpr int NB1 = 2;       // phase-1 jobs per wave in flight (register buffers)
constexpr int kGather = 16;  // x chunks per thread loaded together
constexpr int NB2 = 2;       // phase-2 jobs per wave in flight
// Most dynamic LDS of one item (x rows, hidden tile, bias slices); the
// static arrays of the work list take about 2 KiB more.
constexpr size_t kDecodeLds = 152 * 1024;

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

// Block barrier that completes only the waves' LDS traffic: the weight loads
// that are meant to stay in flight across it are not waited for (a
// __syncthreads would drain every outstanding vector memory operation).
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Software pipeline over a wave's jobs 0 .. n-1 with NB register buffers:
// job j + NB is loaded into buffer j % NB right after job j has used it, so
// NB - 1 to NB jobs are in flight while one is multiplied.  The steady loop
// has no load under a branch, so the compiler's waits count exactly the
// loads of the older jobs; only the prologue and the tail branch.  The
// first `preloaded` jobs' loads were issued by the caller.
template <int NB, typename Load, typename Comp>
__device__ __attribute__((always_inline)) inline void pipeline(int n, int preloaded, Load&& load, Comp&& comp) {
#pragma unroll
  for (int k = 0; k < NB; ++k)
    if (k >= preloaded && k < n) load(k, k);
  int j = 0;
  for (; j + 2 * NB - 1 < n; j += NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      comp(j + k, k);
      load(j + k + NB, k);
    }
  }
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    if (j + k < n) {
      comp(j + k, k);
      if (j + k + NB < n) load(j + k + NB, k);
    }
  }
#pragma unroll
  for (int k = 0; k < NB; ++k)
    if (j + NB + k < n) comp(j + NB + k, k);
}

// Per item, once: the item's x rows (gathered through perm) go to LDS, so
// that the weight loads are the only global loads of the streaming phases.
// Weight rows go straight into MFMA operand registers, job by job
// (phase 1: U1 k sub-steps of one 16-row tile of W1 (and W3); phase 2: the
// KS2 k sub-steps of one 16-row tile of W2), through the pipeline above.
// D is a multiple of 32 * U1 and KS2 = Fs / 32 is a compile-time constant,
// so no load depends on a condition.
template <int ACT, bool BIAS, int KS2>
__global__ __launch_bounds__(kThreads, 1) void decode_ffn_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_scan[kMaxExperts];
  __shared__ int s_tok[TG];
  constexpr bool kSwiGLU = ACT == kActSwiGLU;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int l16 = lane & 15, lq = lane >> 4;
  const int N = p.n_experts, D = p.D, F = p.F, NS = p.NS, Fs = p.Fs;
  const int XS = D + 8, HS = Fs + 8;  // row strides (elements): 16 bytes of padding per row
  bf16* Xs = (bf16*)smem_raw;         // [TG][XS]  x rows of the item
  bf16* Hs = Xs + TG * XS;            // [TG][HS]  hidden tile of the shard
  bf16* B1s = Hs + TG * HS;           // [Fs]      b1 slice of the shard (BIAS)
  bf16* B2s = B1s + Fs;               // [D]       b2 of the expert (BIAS)

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

  const int KS1 = D / 32;
  const int nb1 = KS1 / U1;
  const int FT = Fs / 16, DT = D / 16;
  // this wave's 16-row weight tiles: ft = wave + i * kWaves (phase 1, nb1
  // jobs each) and dt = wave + i * kWaves (phase 2, one job each)
  const int nj1 = (FT > wave ? (FT - wave + kWaves - 1) / kWaves : 0) * nb1;
  const int nj2 = DT > wave ? (DT - wave + kWaves - 1) / kWaves : 0;
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
    const bf16* w1e = p.w1 + ((int64_t)e * F + (int64_t)s * Fs) * D;
    const bf16* w3e = kSwiGLU ? p.w3 + ((int64_t)e * F + (int64_t)s * Fs) * D : w1e;
    const bf16* w2e = p.w2 + (int64_t)e * D * F + (int64_t)s * Fs;
    float* pout = p.part + (int64_t)s * p.rows_cap * D;

    // NTT: 16-token MFMA tiles per item
    auto run = [&](auto ntt_tag) __attribute__((always_inline)) {
      constexpr int NTT = decltype(ntt_tag)::value;

      // ---- phase 1: lane (l16, lq) loads 16 bytes of weight row
      // ft*16 + l16 of the shard at k = ks*32 + lq*8
      bf16x8 wa[NB1][U1], wb[NB1][U1];
      auto load1 = [&](int j, int k) __attribute__((always_inline)) {
        const int i = j / nb1, b = j - i * nb1;
        const int64_t roff = (int64_t)((wave + i * kWaves) * 16 + l16) * D + lq * 8;
#pragma unroll
        for (int kk = 0; kk < NB1; ++kk) {
          if (kk != k) continue;  // k is a compile-time position after unrolling
#pragma unroll
          for (int u = 0; u < U1; ++u) {
            const int ks = b * U1 + u;
            wa[kk][u] = *(const bf16x8*)(w1e + roff + ks * 32);
            if constexpr (kSwiGLU) wb[kk][u] = *(const bf16x8*)(w3e + roff + ks * 32);
          }
        }
      };
      f32x4 ag[NTT], au[NTT];
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) ag[tt] = au[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      auto comp1 = [&](int j, int k) __attribute__((always_inline)) {
        const int i = j / nb1, b = j - i * nb1;
        const int ft = wave + i * kWaves;
#pragma unroll
        for (int kk = 0; kk < NB1; ++kk) {
          if (kk != k) continue;
#pragma unroll
          for (int u = 0; u < U1; ++u) {
            const int ks = b * U1 + u;
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
              const bf16x8 vx = *(const bf16x8*)(Xs + (tt * 16 + l16) * XS + ks * 32 + lq * 8);
              ag[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[kk][u], vx, ag[tt], 0, 0, 0);
              if constexpr (kSwiGLU)
                au[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[kk][u], vx, au[tt], 0, 0, 0);
            }
          }
        }
        if (b == nb1 - 1) {
          // lane holds features ft*16 + 4*lq + r of token tt*16 + l16
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt) {
            bf16x4 h;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float z = ag[tt][r];
              if constexpr (kSwiGLU) {
                z = fast_silu(z) * au[tt][r];
              } else {
                if constexpr (BIAS) z += (float)B1s[ft * 16 + 4 * lq + r];
                if constexpr (ACT == kActGelu) z = gelu_erf(z);
                if constexpr (ACT == kActRelu) z = fmaxf(z, 0.f);
              }
              h[r] = (bf16)z;
            }
            *(bf16x4*)(Hs + (tt * 16 + l16) * HS + ft * 16 + 4 * lq) = h;
            ag[tt] = au[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
      };

      // Every wave has phase-1 and phase-2 jobs (Fs >= 128 and D >= 128 give
      // at least kWaves tiles of 16 rows in each phase), so the first loads
      // need no condition; a second job that does not exist reloads the
      // first (its buffer is then never used).
      load1(0, 0);
      // the item's tokens and the bias slices.  Rows past nrows are not
      // loaded: an MFMA output column depends only on its own token's
      // operand column, so whatever those LDS rows hold reaches only
      // discarded columns.
      if (tid < nrows) s_tok[tid] = p.perm[row0 + tid] / p.topk;
      if constexpr (BIAS) {
        for (int i = tid; i < Fs; i += kThreads) B1s[i] = p.b1[(int64_t)e * F + (int64_t)s * Fs + i];
        for (int i = tid; i < D; i += kThreads) B2s[i] = p.b2[(int64_t)e * D + i];
      }
      __syncthreads();
      // x rows -> LDS through registers, kGather 16-byte chunks per thread
      // in flight together (plain loads: the compiler then counts exactly
      // which loads a later wait needs, which it cannot do for LDS DMA).
      // The second weight job is issued after the first pass of chunks, so
      // waiting for those leaves it in flight.
      const int cpr = D / 8;
      const int nchunk = nrows * cpr;
      auto gather = [&](int c0, bool second) __attribute__((always_inline)) {
        bf16x8 v[kGather];
#pragma unroll
        for (int q = 0; q < kGather; ++q) {
          const int c = min(c0 + q * kThreads + tid, nchunk - 1);
          const int r = c / cpr;
          v[q] = *(const bf16x8*)(p.x + (int64_t)s_tok[r] * D + (c - r * cpr) * 8);
        }
        if (second) load1(min(1, nj1 - 1), 1);
#pragma unroll
        for (int q = 0; q < kGather; ++q) {
          const int c = c0 + q * kThreads + tid;
          if (c < nchunk) {
            const int r = c / cpr;
            *(bf16x8*)(Xs + r * XS + (c - r * cpr) * 8) = v[q];
          }
        }
      };
      gather(0, true);
      for (int c0 = kGather * kThreads; c0 < nchunk; c0 += kGather * kThreads) gather(c0, false);
      lds_barrier();

      // ---- phase 1: H[tokens, Fs] = act(X . W1_s^T (+b1)) (SwiGLU: with W3_s)
      pipeline<NB1>(nj1, NB1, load1, comp1);

      // ---- phase 2: lane loads 16 bytes of W2 row d = dt*16 + l16 at shard
      // column ks*32 + lq*8; job i is tile dt = wave + i*kWaves.  The hidden
      // tile's MFMA operands do not depend on dt: they are read from LDS
      // once, into registers, for all of the wave's tiles.
      bf16x8 wv[NB2][KS2];
      auto load2 = [&](int i, int k) __attribute__((always_inline)) {
        const bf16* row = w2e + (int64_t)((wave + i * kWaves) * 16 + l16) * F + lq * 8;
#pragma unroll
        for (int kk = 0; kk < NB2; ++kk) {
          if (kk != k) continue;
#pragma unroll
          for (int u = 0; u < KS2; ++u) wv[kk][u] = *(const bf16x8*)(row + u * 32);
        }
      };
      bf16x8 hf[KS2][NTT];
      auto comp2 = [&](int i, int k) __attribute__((always_inline)) {
        const int dt = wave + i * kWaves;
        f32x4 acc[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NB2; ++kk) {
          if (kk != k) continue;
#pragma unroll
          for (int u = 0; u < KS2; ++u)
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
              acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[kk][u], hf[u][tt], acc[tt], 0, 0, 0);
        }
        // lane holds output columns dt*16 + 4*lq + r of token tt*16 + l16
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          f32x4 v = acc[tt];
          if constexpr (BIAS) {
            if (s == 0) {
#pragma unroll
              for (int r = 0; r < 4; ++r) v[r] += (float)B2s[dt * 16 + 4 * lq + r];
            }
          }
          const int r0 = tt * 16 + l16;
          if (r0 < nrows) *(f32x4*)(pout + (int64_t)(row0 + r0) * D + dt * 16 + 4 * lq) = v;
        }
      };
      static_assert(NB2 == 2, "two phase-2 jobs preloaded");
      load2(0, 0);
      load2(min(1, nj2 - 1), 1);
      lds_barrier();  // the whole hidden tile is in LDS
#pragma unroll
      for (int u = 0; u < KS2; ++u)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) hf[u][tt] = *(const bf16x8*)(Hs + (tt * 16 + l16) * HS + u * 32 + lq * 8);

      // ---- phase 2: P[s][rows, D] = H . W2[:, shard]^T (+b2 on shard 0)
      pipeline<NB2>(nj2, NB2, load2, comp2);
    };
    // Both 16-token tiles always run (an item of at most 16 rows computes
    // discarded columns): with two instantiations of the streaming loops in
    // one kernel the registers no longer fit.  The MFMA work is small next to
    // the weight stream.
    run(std::integral_constant<int, 2>{});
    __syncthreads();  // Xs, Hs, s_tok and the bias slices are rewritten by the next item
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

template <int ACT, bool BIAS, int KS2>
hipError_t launch_ks(const DecodeParams& p, size_t lds, hipStream_t st) {
  auto kern = decode_ffn_kernel<ACT, BIAS, KS2>;
  static const hipError_t attr_err =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDecodeLds);
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL(kern, dim3(device_cu_count()), dim3(kThreads), lds, st, p);
  return hipGetLastError();
}

// Shard widths the kernel is compiled for (Fs / 32 k sub-steps per phase-2
// tile): 128, 256, 352 and 384 columns.
constexpr int kShardKS[] = {4, 8, 11, 12};

template <int ACT, bool BIAS>
hipError_t launch_act(const DecodeParams& p, size_t lds, hipStream_t st) {
  switch (p.Fs / 32) {
    case 4: return launch_ks<ACT, BIAS, 4>(p, lds, st);
    case 8: return launch_ks<ACT, BIAS, 8>(p, lds, st);
    case 11: return launch_ks<ACT, BIAS, 11>(p, lds, st);
    default: return launch_ks<ACT, BIAS, 12>(p, lds, st);
  }
}

bool shard_compiled(int fs) {
  for (int ks : kShardKS)
    if (fs == 32 * ks) return true;
  return false;
}

// Dynamic LDS of one item: x rows, hidden tile and (with biases) the b1
// slice and b2, all bf16.
size_t item_lds(const moe_shape& s, int n_shards) {
  const size_t fs = (size_t)(s.F / n_shards);
  const bool bias = (s.flags & MOE_HAS_BIAS) != 0;
  return ((size_t)TG * (s.D + 8) + (size_t)TG * (fs + 8) + (bias ? fs + (size_t)s.D : 0)) * 2;
}

}  // namespace

// Shards per expert: about one work item per CU of a 256-CU device, each
// shard one of the compiled widths, with the item's x rows, hidden tile and
// bias slices within the kernel's LDS.  0 = no such split.
int decode_shards(const moe_shape& s) {
  auto fits = [&](int n) {
    return s.F % n == 0 && shard_compiled(s.F / n) && item_lds(s, n) <= kDecodeLds;
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
  // D a multiple of 128: whole phase-1 jobs of U1 k sub-steps
  if (s.dtype != MOE_DTYPE_BF16 || expected_rows > 16 || s.D % (32 * U1)) return false;
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
  const size_t lds = item_lds(s, p.NS);
  if (p.b1) {
    switch (s.act) {
      case MOE_ACT_SWIGLU: return launch_act<kActSwiGLU, true>(p, lds, st);
      case MOE_ACT_RELU: return launch_act<kActRelu, true>(p, lds, st);
      default: return launch_act<kActGelu, true>(p, lds, st);
    }
  }
  switch (s.act) {
    case MOE_ACT_SWIGLU: return launch_act<kActSwiGLU, false>(p, lds, st);
    case MOE_ACT_RELU: return launch_act<kActRelu, false>(p, lds, st);
    default: return launch_act<kActGelu, false>(p, lds, st);
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
