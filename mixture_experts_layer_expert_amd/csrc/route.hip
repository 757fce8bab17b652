// Router: logits, softmax and top-k of every token ("Top-k router" section of
// the notebook "Mixture-of-experts and expert parallelism").
//
// One block = 4 waves = 64 tokens, 16 tokens per wave.
//  1. bf16: each wave computes its 16x(16*NT) logit tile with
//     v_mfma_f32_16x16x32_bf16, operands read straight from global memory
//     (x rows are used once; the router matrix is L2-resident).  fp32: VALU
//     dot products.  The tile goes to LDS.
//  2. A 16-lane group ranks one token: every lane owns experts l, l+16, ...;
//     k+1 rounds of (value, index) arg-max over the group with xor shuffles.
//     Larger value wins, equal values go to the lower expert index.
//  3. If two of the top-(k+1) fp32 logits are closer than kRefineMargin, the
//     wave recomputes that token's logits in fp64 from exact products
//     (bf16*bf16 and fp32*fp32 are exact in fp64) and ranks those instead.
//  4. Gates are softmax probabilities of the chosen experts, optionally
//     renormalised over the k choices.
#include <float.h>
#include <limits.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTokPerWave = 16;
constexpr int kWaves = 4;
constexpr int kTokPerBlock = kTokPerWave * kWaves;

struct RouteArgs {
  const void* x;
  const void* wr;
  const float* br;
  int64_t T;
  int D, N, k;
  int renorm, has_bias;
  int32_t* idx;
  float* gate;
  float* logits;
};

template <typename V>
__device__ inline bool better(V va, int ia, V vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <typename V>
__device__ inline V neg_inf();
template <>
__device__ inline float neg_inf<float>() { return -FLT_MAX; }
template <>
__device__ inline double neg_inf<double>() { return -DBL_MAX; }

__device__ inline float vexp(float v) { return expf(v); }
__device__ inline double vexp(double v) { return exp(v); }

// Ranks one token within a 16-lane group.  vals: LDS row of N logits.
// Returns true when the top-(k+1) are separated by at least `margin`
// (always true for fp64 ranking, margin = -1).  On success (or when
// `force`), lane 0 of the group writes idx/gate for token t.
template <typename V, int NV>
__device__ bool group_rank(const V* vals, const RouteArgs& a, int64_t t, int l16, V margin,
                           bool force) {
  const int N = a.N, k = a.k;
  V v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int e = l16 + 16 * i;
    v[i] = (e < N) ? vals[e] : neg_inf<V>();
  }
  const int nsel = (k + 1 <= N) ? k + 1 : N;
  V tv[kMaxTopK + 1];
  int ti[kMaxTopK + 1];
  uint32_t taken = 0;
#pragma unroll
  for (int r = 0; r < kMaxTopK + 1; ++r) {
    if (r < nsel) {
    V bv = neg_inf<V>();
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int e = l16 + 16 * i;
      if (e < N && !((taken >> i) & 1u) && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
      V ov = __shfl_xor(bv, off, 16);
      int oi = __shfl_xor(bi, off, 16);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    tv[r] = bv;
    ti[r] = bi;
    if ((bi & 15) == l16) taken |= 1u << (bi >> 4);
    }
  }
  bool ok = true;
  const int ngap = (k < N - 1) ? k : N - 1;
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r)
    if (r < ngap) ok = ok && (tv[r] - tv[r + 1] >= margin);
  if (!ok && !force) return false;
  // softmax denominator over all N experts
  const V vmax = tv[0];
  V s = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int e = l16 + 16 * i;
    if (e < N) s += vexp(v[i] - vmax);
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off, 16);
  if (l16 == 0 && t < a.T) {
    V p[kMaxTopK];
    V ps = 0;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      p[j] = (j < k) ? vexp(tv[j] - vmax) / s : V(0);
      ps += p[j];
    }
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        a.idx[t * k + j] = ti[j];
        a.gate[t * k + j] = (float)(a.renorm ? p[j] / ps : p[j]);
      }
    }
  }
  return true;
}

template <typename T>
__device__ inline double to_f64(T v) { return (double)(float)v; }
template <>
__device__ inline double to_f64<float>(float v) { return (double)v; }

// fp64 logits of token t for all N experts, written to dl[0..N).  The wave
// splits D over its 64 lanes and reduces with xor shuffles.
template <typename T>
__device__ void refine_logits(const RouteArgs& a, int64_t t, int lane, double* dl) {
  const T* x = (const T*)a.x + t * (int64_t)a.D;
  const T* w = (const T*)a.wr;
  for (int e = 0; e < a.N; ++e) {
    const T* we = w + (int64_t)e * a.D;
    double s = 0.0;
    for (int d = lane; d < a.D; d += kWave) s = fma(to_f64(x[d]), to_f64(we[d]), s);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) dl[e] = s + (a.has_bias ? (double)a.br[e] : 0.0);
  }
}

// fp32 logits of the wave's 16 tokens with bf16 MFMA, into lds[16][ldl].
template <int NT>
__device__ void logits_bf16(const RouteArgs& a, int64_t t0, int lane, float* lds, int ldl) {
  const bf16* x = (const bf16*)a.x;
  const bf16* wr = (const bf16*)a.wr;
  const int D = a.D;
  int64_t row = t0 + (lane & 15);
  if (row > a.T - 1) row = a.T - 1;
  const bf16* xa = x + row * D + (lane >> 4) * 8;
  const bf16* wb[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int e = nt * 16 + (lane & 15);
    if (e > a.N - 1) e = a.N - 1;
    wb[nt] = wr + (int64_t)e * D + (lane >> 4) * 8;
  }
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kk = 0; kk < D; kk += 32) {
    bf16x8 av = *(const bf16x8*)(xa + kk);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bf16x8 bv = *(const bf16x8*)(wb[nt] + kk);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[nt], 0, 0, 0);
    }
  }
  const float* br = a.br;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int e = nt * 16 + (lane & 15);
    float b = (a.has_bias && e < a.N) ? br[e] : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) lds[(4 * (lane >> 4) + r) * ldl + e] = acc[nt][r] + b;
  }
}

// fp32 logits with VALU fma: lane = token (lane & 15), experts lane>>4, +4, ...
__device__ void logits_f32(const RouteArgs& a, int64_t t0, int lane, float* lds, int ldl) {
  const float* x = (const float*)a.x;
  const float* wr = (const float*)a.wr;
  const int D = a.D;
  int64_t row = t0 + (lane & 15);
  if (row > a.T - 1) row = a.T - 1;
  const float4* xr = (const float4*)(x + row * D);
  for (int e = lane >> 4; e < a.N; e += 4) {
    const float4* we = (const float4*)(wr + (int64_t)e * D);
    float s = 0.f;
    for (int d = 0; d < D / 4; ++d) {
      float4 xv = xr[d], wv = we[d];
      s = fmaf(xv.x, wv.x, s);
      s = fmaf(xv.y, wv.y, s);
      s = fmaf(xv.z, wv.z, s);
      s = fmaf(xv.w, wv.w, s);
    }
    lds[(lane & 15) * ldl + e] = s + (a.has_bias ? a.br[e] : 0.f);
  }
}

template <typename T, int NT>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  constexpr int ldl = 16 * NT + 1;
  __shared__ float lds_all[kTokPerBlock * ldl];
  __shared__ double dl_all[kWaves][16 * NT];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t t0 = (int64_t)blockIdx.x * kTokPerBlock + wave * kTokPerWave;
  float* lds = lds_all + wave * kTokPerWave * ldl;
  double* dl = dl_all[wave];

  if constexpr (sizeof(T) == 2) {
    logits_bf16<NT>(a, t0, lane, lds, ldl);
  } else {
    logits_f32(a, t0, lane, lds, ldl);
  }
  __syncthreads();

  const int grp = lane >> 4, l16 = lane & 15;
  uint32_t need = 0;  // tokens of this wave (bit = token within wave) to refine
  for (int it = 0; it < 4; ++it) {
    const int tk = it * 4 + grp;
    const int64_t t = t0 + tk;
    bool ok = group_rank<float, NT>(lds + tk * ldl, a, t, l16, kRefineMargin, false);
    if (a.logits && t < a.T)
      for (int e = l16; e < a.N; e += 16) a.logits[t * a.N + e] = lds[tk * ldl + e];
    uint64_t bad = __ballot(!ok && l16 == 0 && t < a.T);
    for (int g = 0; g < 4; ++g)
      if ((bad >> (16 * g)) & 1ull) need |= 1u << (it * 4 + g);
  }
  while (need) {
    const int tk = __builtin_ctz(need);
    need &= need - 1;
    const int64_t t = t0 + tk;
    refine_logits<T>(a, t, lane, dl);
    // dl is private to this wave: order its LDS traffic at wavefront scope
    // (waves refine different numbers of tokens, so no block barrier here).
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (grp == 0) {
      group_rank<double, NT>(dl, a, t, l16, -1.0, true);
      if (a.logits)
        for (int e = l16; e < a.N; e += 16) a.logits[t * a.N + e] = (float)dl[e];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
}

template <typename T, int NT>
hipError_t launch_nt(const RouteArgs& a, hipStream_t st) {
  const int64_t blocks = (a.T + kTokPerBlock - 1) / kTokPerBlock;
  hipLaunchKernelGGL((route_kernel<T, NT>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const RouteArgs& a, hipStream_t st) {
  if (a.N <= 16) return launch_nt<T, 1>(a, st);
  if (a.N <= 32) return launch_nt<T, 2>(a, st);
  if (a.N <= 64) return launch_nt<T, 4>(a, st);
  if (a.N <= 128) return launch_nt<T, 8>(a, st);
  return launch_nt<T, 16>(a, st);
}

}  // namespace

hipError_t launch_route(const moe_shape& s, const void* x, const void* wr, const float* br,
                        int32_t* idx, float* gate, float* logits, hipStream_t st) {
  RouteArgs a;
  a.x = x;
  a.wr = wr;
  a.br = br;
  a.T = s.T;
  a.D = s.D;
  a.N = s.N;
  a.k = s.k;
  a.renorm = (s.flags & MOE_RENORM) ? 1 : 0;
  a.has_bias = (s.flags & MOE_ROUTER_BIAS) ? 1 : 0;
  a.idx = idx;
  a.gate = gate;
  a.logits = logits;
  if (s.dtype == MOE_DTYPE_BF16) return launch_t<bf16>(a, st);
  return launch_t<float>(a, st);
}

}  // namespace moe
