// Router: logits, softmax and top-k of every token ("Top-k router" section of
// the notebook "Mixture-of-experts and expert parallelism").
//
// One block = 4 waves.  bf16 with D a multiple of 128: route_ring_kernel,
// TB = 16/32/64 tokens per block, x rows and the router matrix streamed
// through an LDS ring by DMA.  Otherwise route_kernel, 32 tokens per block.
//  1. bf16: the block's token x (16*NT) logit tile is computed with
//     v_mfma_f32_16x16x32_bf16 (D split over the waves when a wave has no
//     tile of its own; partial tiles summed in LDS).  fp32: VALU dot
//     products.
//  2. A 16-lane group ranks one token: every lane owns experts l, l+16, ...;
//     k+1 rounds of (value, index) arg-max over the group, exchanged with DPP
//     moves inside the 16 lanes.  Larger value wins, equal values go to the
//     lower expert index.
//  3. If two of the top-(k+1) fp32 logits are closer than kRefineMargin, the
//     token is ranked again by its wave from exact logits: only the experts
//     whose fp32 logit lies within the margin of the (k+1)-th value can change
//     places (the fp32 error is far below half the margin), and only those
//     are recomputed, in fp64 from exact products (bf16*bf16 and fp32*fp32
//     are exact in fp64).  Near-ties are rare: a handful of tokens per batch.
//  4. Gates are softmax probabilities of the chosen experts, optionally
//     renormalised over the k choices.
// With R fallback ranks the same steps select the top k + R (the near-tie
// test then covers the top k + R + 1): ranks k .. k+R-1 go to fb_idx and
// fb_gate, their gates scaled like the k gates.
#include <float.h>
#include <limits.h>

#include "moe_internal.h"

namespace moe {
namespace {

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
  int R;            // fallback ranks after the k choices (0 = none)
  int32_t* fb_idx;  // [T, R]: experts of ranks k .. k+R-1
  float* fb_gate;   // [T, R]: their gates, scaled like the k gates
  float* prob_part;  // optional: [N][blocks] per-block probability sums
  unsigned long long* stats_ticket;  // with prob_part: cleared by block 0
};

template <typename V>
__device__ inline bool better(V va, int ia, V vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <typename V>
__device__ inline V neg_inf();
template <>
__device__ inline float neg_inf<float>() { return -FLT_MAX; }

// exp of a non-positive argument (logit minus the row maximum) with the
// hardware exponential: a few ulp, far below the gate tolerance
__device__ inline float vexp(float v) { return __expf(v); }

// Exchanges within a 16-lane group through DPP (no LDS round trip): after
// xor 1, xor 2, the mirror within 8 lanes and the mirror within 16 lanes,
// every lane of the group has combined all 16 values.  All lanes of the wave
// take part.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int CTRL>
__device__ inline int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
template <int CTRL>
__device__ inline void argmax_step(float& bv, int& bi) {
  const float ov = dpp_f<CTRL>(bv);
  const int oi = dpp_i<CTRL>(bi);
  const bool take = (ov > bv) | ((ov == bv) & (oi < bi));  // better(), branch-free
  bv = take ? ov : bv;
  bi = take ? oi : bi;
}
// (value, lower index) arg-max of the group, in every lane; a total order,
// so the result does not depend on the exchange pattern
__device__ inline void group16_argmax(float& bv, int& bi) {
  argmax_step<kDppXor1>(bv, bi);
  argmax_step<kDppXor2>(bv, bi);
  argmax_step<kDppHalfMirror>(bv, bi);
  argmax_step<kDppMirror>(bv, bi);
}
// sum of the group in every lane (fixed pairing, so deterministic)
__device__ inline float group16_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return v;
}

// Ranks one token within a 16-lane group.  vals: LDS row of N logits.
// Returns true when the top-(k+1) are separated by at least `margin`
// (always true for fp64 ranking, margin = -1).  On success (or when
// `force`), lane 0 of the group writes idx/gate for token t.  With `stats`
// (load statistics), every valid token's softmax probabilities of the lane's
// experts l16 + 16 i are added to pacc[i], near-tie tokens included.
template <typename V, int NV>
__device__ __forceinline__ bool group_rank(const V* vals, const RouteArgs& a, int64_t t, int l16, V margin,
                                           bool force, bool stats, V (&pacc)[NV]) {
  const int N = a.N, k = a.k, KS = a.k + a.R;  // ranks to select
  V v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int e = l16 + 16 * i;
    v[i] = (e < N) ? vals[e] : neg_inf<V>();
  }
  const int nsel = (KS + 1 <= N) ? KS + 1 : N;
  V tv[kMaxTopK + 1];
  int ti[kMaxTopK + 1];
  // experts of this lane still to rank (bit i: expert l16 + 16 i); the
  // selection is written with bitwise conditions and selects so that it
  // compiles without branches
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) avail |= (l16 + 16 * i < N) ? (1u << i) : 0u;
#pragma unroll
  for (int r = 0; r < kMaxTopK + 1; ++r) {
    if (r < nsel) {  // wave-uniform
      V bv = neg_inf<V>();
      int bi = INT_MAX;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = l16 + 16 * i;
        const bool take = ((avail >> i) & 1u) & ((v[i] > bv) | ((v[i] == bv) & (e < bi)));
        bv = take ? v[i] : bv;
        bi = take ? e : bi;
      }
      group16_argmax(bv, bi);
      tv[r] = bv;
      ti[r] = bi;
      const bool mine = (bi < N) & ((bi & 15) == l16);
      avail &= mine ? ~(1u << ((bi >> 4) & 31)) : ~0u;
    }
  }
  bool ok = true;
  const int ngap = (KS < N - 1) ? KS : N - 1;
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r)
    if (r < ngap) ok = ok && (tv[r] - tv[r + 1] >= margin);
  if (!ok && !force && !stats) return false;
  // softmax denominator over all N experts
  const V vmax = tv[0];
  V s = 0;
  V ex[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int e = l16 + 16 * i;
    ex[i] = (e < N) ? vexp(v[i] - vmax) : V(0);
    s += ex[i];
  }
  s = group16_sum(s);
  if (stats && t < a.T) {
    const V inv = V(1) / s;
#pragma unroll
    for (int i = 0; i < NV; ++i) pacc[i] += ex[i] * inv;
  }
  if (!ok && !force) return false;
  // lane j of the group finishes rank j (j < KS): one exponential and one
  // division per lane instead of KS of each in one lane
  V myv = tv[0];
  int myi = ti[0];
#pragma unroll
  for (int r = 1; r < kMaxTopK; ++r)
    if (l16 == r && r < nsel) {
      myv = tv[r];
      myi = ti[r];
    }
  const V p = (l16 < KS) ? vexp(myv - vmax) / s : V(0);
  const V ps = group16_sum(l16 < k ? p : V(0));
  if (t < a.T) {
    const float g = (float)(a.renorm ? p / ps : p);
    if (l16 < k) {
      a.idx[t * k + l16] = myi;
      a.gate[t * k + l16] = g;
    } else if (l16 < KS) {
      a.fb_idx[t * a.R + (l16 - k)] = myi;
      a.fb_gate[t * a.R + (l16 - k)] = g;
    }
  }
  return true;
}

// Chunk of 16 bytes of the input dtype.
template <typename T>
struct Chunk;
template <>
struct Chunk<bf16> {
  static constexpr int W = 8;
  typedef bf16x8 type;
};
template <>
struct Chunk<float> {
  static constexpr int W = 4;
  typedef f32x4 type;
};

// fp32 partial logits of the block's 32 tokens with bf16 MFMA.  Wave w takes
// the 32-wide k steps w, w+4, w+8, ... (4-way split of D); each lane loads its
// 16-byte fragments straight from global memory, U steps at a time so that
// several loads are in flight.  Result: lg[token][expert].  Contains block
// barriers: every thread of the block must call it.
template <int NT, int U>
__device__ void logits_bf16(const RouteArgs& a, int64_t t0, int wave, int lane, float* lg,
                            int ldl) {
  const bf16* x = (const bf16*)a.x;
  const bf16* wr = (const bf16*)a.wr;
  const int D = a.D;
  const bf16* xa[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    int64_t row = t0 + m * 16 + (lane & 15);
    if (row > a.T - 1) row = a.T - 1;
    xa[m] = x + row * D + (lane >> 4) * 8;
  }
  const bf16* wb[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int e = nt * 16 + (lane & 15);
    if (e > a.N - 1) e = a.N - 1;
    wb[nt] = wr + (int64_t)e * D + (lane >> 4) * 8;
  }
  f32x4 acc[2][NT];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int steps = D / 32;
  for (int s0 = wave; s0 < steps; s0 += 4 * U) {
    bf16x8 av[U][2], bv[U][NT];
    // MFMAs run whatever the EXEC mask is, so an out-of-range step gets zero
    // operands (adding exactly 0) instead of being skipped by a branch.
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + 4 * u;
      const bool in = s < steps;
#pragma unroll
      for (int m = 0; m < 2; ++m) av[u][m] = in ? *(const bf16x8*)(xa[m] + s * 32) : bf16x8{};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bv[u][nt] = in ? *(const bf16x8*)(wb[nt] + s * 32) : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[m][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u][m], bv[u][nt], acc[m][nt], 0, 0, 0);
  }
  // Sum the four partial tiles into lg in fixed wave order (deterministic);
  // wave 0 adds the router bias.
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int e = nt * 16 + (lane & 15);
        const float b = (w == 0 && a.has_bias && e < a.N) ? a.br[e] : 0.f;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float* dst = &lg[(m * 16 + 4 * (lane >> 4) + r) * ldl + e];
            *dst = (w == 0 ? b : *dst) + acc[m][nt][r];
          }
      }
    }
    __syncthreads();
  }
}

// fp32 logits with VALU fma (fp32 layers): thread = (token, expert subset).
__device__ void logits_f32(const RouteArgs& a, int64_t t0, int tid, float* lg, int ldl) {
  const float* x = (const float*)a.x;
  const float* wr = (const float*)a.wr;
  const int D = a.D;
  const int r = tid / 8;  // 32 tokens x 8 threads
  int64_t row = t0 + r;
  if (row > a.T - 1) row = a.T - 1;
  const f32x4* xr = (const f32x4*)(x + row * D);
  for (int e = tid % 8; e < a.N; e += 8) {
    const f32x4* we = (const f32x4*)(wr + (int64_t)e * D);
    // four partial sums (lane c of every chunk) instead of one chain, and
    // four chunks' loads issued together: the loop is latency-bound
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll 4
    for (int d = 0; d < D / 4; ++d) {
      const f32x4 xv = xr[d], wv = we[d];
      s0 = fmaf(xv[0], wv[0], s0);
      s1 = fmaf(xv[1], wv[1], s1);
      s2 = fmaf(xv[2], wv[2], s2);
      s3 = fmaf(xv[3], wv[3], s3);
    }
    lg[r * ldl + e] = ((s0 + s1) + (s2 + s3)) + (a.has_bias ? a.br[e] : 0.f);
  }
}

// Product of two stored input values, exact: a bf16*bf16 product has at most
// 16 significant bits and is exact in fp32; fp32*fp32 is exact in fp64.
__device__ inline double exact_product(float x, bf16 w) { return (double)(x * (float)w); }
__device__ inline double exact_product(float x, float w) { return (double)x * (double)w; }

// Exact ranking of one near-tie token by one whole wave.  The token's fp32
// logits (row lgrow, N values) locate the candidates: the experts whose fp32
// logit is at least the (k+1)-th largest minus kRefineMargin.  Any other
// expert lies, in exact arithmetic, below k+1 of the candidates, because the
// fp32 logits differ from the exact ones by far less than half the margin.
// Each candidate's logit is recomputed in fp64 from exact products (the wave
// splits D into 16-byte chunks; butterfly sum, so identical router rows give
// identical values) and the top k candidates by exact logit, ties to the
// lower index, are the selection.  Gates: softmax over all N experts with the
// exact values for the candidates and the fp32 values for the rest.
// NJ = experts held per lane (expert e = lane + 64 j).
template <typename T, int NJ>
__device__ void exact_rank_wave(const RouteArgs& a, const float* lgrow, int64_t t, int lane) {
  constexpr int W = Chunk<T>::W;
  typedef typename Chunk<T>::type V;
  const int N = a.N, k = a.k, D = a.D, KS = a.k + a.R;
  float v[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    v[j] = (e < N) ? lgrow[e] : -FLT_MAX;
  }
  // the (KS+1)-th largest fp32 logit (or the N-th when KS = N)
  const int nsel = (KS + 1 <= N) ? KS + 1 : N;
  uint32_t taken = 0;
  float vk = 0.f;
#pragma unroll
  for (int r = 0; r < kMaxTopK + 1; ++r) {
    if (r < nsel) {
      float bv = -FLT_MAX;
      int bi = INT_MAX;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int e = lane + 64 * j;
        if (e < N && !((taken >> j) & 1u) && better(v[j], e, bv, bi)) {
          bv = v[j];
          bi = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      vk = bv;
    }
  }
  const float th = (nsel == N) ? -FLT_MAX : vk - kRefineMargin;
  uint32_t cand = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    if (e < N && v[j] >= th) cand |= 1u << j;
  }
  // exact logits of the candidates, one candidate at a time
  const V* xv = (const V*)((const T*)a.x + t * (int64_t)D);
  const int chunks = D / W;
  double ex[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) ex[j] = -DBL_MAX;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    uint64_t m = __ballot((cand >> j) & 1u);
    while (m) {
      const int l = __builtin_ctzll(m);
      m &= m - 1;
      const int e = l + 64 * j;
      const V* wv = (const V*)((const T*)a.wr + (int64_t)e * D);
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
      for (int c0 = lane; c0 < chunks; c0 += 64 * 4) {
        V xs[4], ws[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = c0 + 64 * u;
          if (c < chunks) {
            xs[u] = xv[c];
            ws[u] = wv[c];
          }
        }
        // keep the loads together: otherwise each is sunk to its use
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (c0 + 64 * u < chunks) {
#pragma unroll
            for (int q = 0; q < W; ++q) acc[q & 3] += exact_product((float)xs[u][q], ws[u][q]);
          }
        }
      }
      double sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
      if (a.has_bias) sum += (double)a.br[e];
      if (lane == l) ex[j] = sum;
    }
  }
  // top KS of the candidates by exact logit; lane r keeps round r's choice
  int my_i = 0;
  double my_v = 0.0;
  uint32_t used = 0;
  for (int r = 0; r < KS; ++r) {
    double bv = -DBL_MAX;
    int bi = INT_MAX;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      if (((cand >> j) & 1u) && !((used >> j) & 1u) && better(ex[j], e, bv, bi)) {
        bv = ex[j];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) used |= 1u << (bi >> 6);
    if (lane == r) {
      my_i = bi;
      my_v = bv;
    }
  }
  const double vmax = __shfl(my_v, 0);
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    if (e < N) s += exp((((cand >> j) & 1u) ? ex[j] : (double)v[j]) - vmax);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  const double p = (lane < KS) ? exp(my_v - vmax) / s : 0.0;
  double ps = (lane < k) ? p : 0.0;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off);
  const float g = (float)(a.renorm ? p / ps : p);
  if (lane < k) {
    a.idx[t * k + lane] = my_i;
    a.gate[t * k + lane] = g;
  } else if (lane < KS) {
    a.fb_idx[t * a.R + (lane - k)] = my_i;
    a.fb_gate[t * a.R + (lane - k)] = g;
  }
  if (a.logits) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      if ((cand >> j) & 1u) a.logits[t * N + e] = (float)ex[j];
    }
  }
}

// Load statistics (notebook section "Switch Transformer auxiliary loss"):
// the sum over the block's valid tokens of every expert's softmax
// probability, stored as prob_part[e * gridDim.x + blockIdx.x].  The
// ranking already forms exp(l - max) and the denominator of every token, so
// each lane has added its experts' probabilities over the tokens its group
// ranked (pacc[i]: expert l16 + 16 i).  Here the four groups of a wave are
// summed with two xor shuffles, then the four waves in LDS, in a fixed
// order.  Block 0 also clears the ticket of the second pass.
// red: 4 * 16 * NT floats of LDS, not otherwise in use.
template <int NT>
__device__ void block_prob_sums(const RouteArgs& a, float (&pacc)[NT], int wave, int lane, int tid, float* red) {
  constexpr int NP = 16 * NT;
  if (blockIdx.x == 0 && tid == 0) *a.stats_ticket = 0ull;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    float x = pacc[i];
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    if (lane < 16) red[wave * NP + lane + 16 * i] = x;
  }
  __syncthreads();
  for (int e = tid; e < a.N; e += 256)
    a.prob_part[(int64_t)e * gridDim.x + blockIdx.x] =
        ((red[e] + red[NP + e]) + red[2 * NP + e]) + red[3 * NP + e];
}

// Ranks the rows r = it*16 + wave*4 + group of the block's logits (16-lane
// groups, fp32); the tokens whose top-(k+1) fp32 logits are too close are
// then ranked again, one after the other, by the whole wave.
template <typename T, int NT, int ITERS>
__device__ void rank_rows(const RouteArgs& a, const float* lg, int ldl, int64_t t0, int wave,
                          int lane, float* red) {
  constexpr int NJ = (16 * NT + 63) / 64;
  const int grp = lane >> 4, l16 = lane & 15;
  float pacc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) pacc[i] = 0.f;
  const bool stats = a.prob_part != nullptr;
  uint32_t marked = 0;
#pragma unroll 1
  for (int it = 0; it < ITERS; ++it) {
    const int r = it * 16 + wave * 4 + grp;
    const int64_t t = t0 + r;
    const bool ok = group_rank<float, NT>(lg + r * ldl, a, t, l16, kRefineMargin, false, stats, pacc);
    if (a.logits && t < a.T)
      for (int e = l16; e < a.N; e += 16) a.logits[t * a.N + e] = lg[r * ldl + e];
    const uint64_t bad = __ballot(!ok && t < a.T);
#pragma unroll
    for (int g = 0; g < 4; ++g)
      if ((bad >> (16 * g)) & 1ull) marked |= 1u << (it * 4 + g);
  }
  if (stats) block_prob_sums<NT>(a, pacc, wave, lane, threadIdx.x, red);
  marked = __builtin_amdgcn_readfirstlane(marked);
  while (marked) {
    const int m = __builtin_ctz(marked);
    marked &= marked - 1;
    const int r = (m / 4) * 16 + wave * 4 + (m % 4);
    exact_rank_wave<T, NJ>(a, lg + r * ldl, t0 + r, lane);
  }
}

// Block = 4 waves = 32 tokens.
template <typename T, int NT>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  constexpr int ldl = 16 * NT + 1;
  // k steps whose operands are loaded together (loads in flight per wave)
  constexpr int U = NT >= 16 ? 2 : (NT >= 8 ? 3 : (NT >= 4 ? 6 : 8));
  __shared__ float lg[32 * ldl];  // logits of the block's 32 tokens
  __shared__ float red[4 * 16 * NT];  // statistics: per-wave probability sums
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int64_t t0 = (int64_t)blockIdx.x * 32;

  if constexpr (sizeof(T) == 2) {
    logits_bf16<NT, U>(a, t0, wave, lane, lg, ldl);
  } else {
    logits_f32(a, t0, tid, lg, ldl);
    __syncthreads();
  }

  rank_rows<T, NT, 2>(a, lg, ldl, t0, wave, lane, red);
}

// ---------------------------------------------------------------------------
// bf16 router for D a multiple of 128: x rows and router rows are streamed
// global -> LDS with global_load_lds_dwordx4 through an S-stage ring, K taken
// 128 at a time (256-byte rows, 4 rows per 1 KiB dma instruction, so x and
// the router matrix both split evenly over the 4 waves).  TB tokens per
// block (64, 32 or 16): wave w computes m-tile w % (TB/16) over the k
// sub-steps congruent to w / (TB/16); partial tiles are summed in LDS in
// fixed wave order.  Selection and near-tie marking as above.
// TWO: the ring is sized so that two blocks share a CU (80 KiB each),
// so that one block's ranking overlaps the other's loads; otherwise it takes
// up to 140 KiB.
template <int NT, int TB, bool TWO>
struct RouteRing {
  static constexpr int NP = 16 * NT;          // expert rows held (padded)
  static constexpr int MT = TB / 16;          // 16-token m-tiles per block
  static constexpr int KSPLIT = 4 / MT;       // waves sharing an m-tile
  static constexpr int IA = TB / 4;           // dma instructions for x per stage
  static constexpr int IB = NP / 4;           // ... for the router matrix
  static constexpr int NJ = (IA + IB) / 4;    // per wave per stage
  static constexpr int kStageElems = (TB + NP) * 128;
  static constexpr int kStageBytes = kStageElems * 2;
  static constexpr int S0 = ((TWO ? 80 : 140) * 1024) / kStageBytes;
  static constexpr int S = S0 > 8 ? 8 : S0;
  static constexpr int kLogitFloats = KSPLIT * TB * (NP + 1);
  static constexpr int kRedFloats = 4 * NP;  // statistics, after the logits
  static constexpr int kBytes = (S * kStageBytes > (kLogitFloats + kRedFloats) * 4)
                                    ? S * kStageBytes
                                    : (kLogitFloats + kRedFloats) * 4;
  static_assert(S >= 2, "ring needs two stages");
  static_assert(!TWO || kBytes <= 80 * 1024, "two blocks per CU");
  static_assert((IA + IB) % 4 == 0, "even dma split");
  static_assert(NJ * (S - 1) <= 63, "vmcnt range");
};

template <int NJ, int K>
__device__ inline void wait_vm_k(int younger) {
  if constexpr (K >= 0) {
    if (younger == K) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K * NJ) : "memory");
      return;
    }
    wait_vm_k<NJ, K - 1>(younger);
  }
}

__device__ inline void ring_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ inline void dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)l, 16, 0, 0);
}

template <int NT, int TB, bool TWO>
__global__ __launch_bounds__(256) void route_ring_kernel(RouteArgs a) {
  using R = RouteRing<NT, TB, TWO>;
  constexpr int ldl = R::NP + 1;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16* ring = (bf16*)smem_raw;
  float* lg = (float*)smem_raw;  // logits tiles, after the ring is drained

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int64_t t0 = (int64_t)blockIdx.x * TB;
  const int D = a.D;
  const int KT = D / 128;

  // dma sources: wave's instruction q covers 4 rows of A (x) or B (router)
  uint32_t src[R::NJ];
  bool is_a[R::NJ];
#pragma unroll
  for (int q = 0; q < R::NJ; ++q) {
    const int g = wave * R::NJ + q;
    const int lrow = lane / 16, pc = lane % 16;
    if (g < R::IA) {
      const int row = g * 4 + lrow;
      int64_t t = t0 + row;
      if (t > a.T - 1) t = a.T - 1;
      src[q] = (uint32_t)(t * D + ((pc ^ (row & 15)) * 8)) * 2u;
      is_a[q] = true;
    } else {
      const int row = (g - R::IA) * 4 + lrow;
      const int e = row < a.N ? row : a.N - 1;
      src[q] = (uint32_t)(e * D + ((pc ^ (row & 15)) * 8)) * 2u;
      is_a[q] = false;
    }
  }
  const char* xb = (const char*)a.x;
  const char* wb = (const char*)a.wr;
  int issued = 0;
  auto issue = [&]() {
    if (issued >= KT) return;
    bf16* dst = ring + (issued % R::S) * R::kStageElems;
    const uint32_t kb = (uint32_t)issued * 256u;
#pragma unroll
    for (int q = 0; q < R::NJ; ++q) {
      const int g = wave * R::NJ + q;
      const char* base = (g < R::IA ? xb : wb) + kb;
      dma16(base + src[q], dst + g * 512);
    }
    ++issued;
  };
#pragma unroll
  for (int s = 0; s < R::S - 1; ++s) issue();

  const int mt = wave % R::MT, kp = wave / R::MT;
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kt = 0; kt < KT; ++kt) {
    wait_vm_k<R::NJ, R::S - 1>(issued - kt - 1);
    ring_sync();
    issue();  // refills the stage read in the previous step
    const bf16* st = ring + (kt % R::S) * R::kStageElems;
    const bf16* sa = st;
    const bf16* sb = st + TB * 128;
    // this wave's k sub-steps: kp, kp + KSPLIT, ... (no per-wave branch
    // around the MFMAs)
#pragma unroll
    for (int j = 0; j < 4 / R::KSPLIT; ++j) {
      const int ss = j * R::KSPLIT + kp;
      const int c = ss * 4 + (lane >> 4);
      const int ra = mt * 16 + (lane & 15);
      const bf16x8 av = *(const bf16x8*)(sa + ra * 128 + ((c ^ (ra & 15)) * 8));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int rb = nt * 16 + (lane & 15);
        const bf16x8 bv = *(const bf16x8*)(sb + rb * 128 + ((c ^ (rb & 15)) * 8));
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[nt], 0, 0, 0);
      }
    }
  }
  ring_sync();  // every wave is done with the ring: reuse it for the logits
  // partial tile of this wave -> lg[kp][token][expert]
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      lg[(kp * TB + mt * 16 + 4 * (lane >> 4) + r) * ldl + nt * 16 + (lane & 15)] = acc[nt][r];
  __syncthreads();
  // sum the KSPLIT partial tiles in fixed order, add the router bias (with a
  // single partial tile and no bias the tile is already final)
  if (R::KSPLIT > 1 || a.has_bias) {
    for (int i = tid; i < TB * R::NP; i += 256) {
      const int r = i / R::NP, e = i % R::NP;
      float v = (a.has_bias && e < a.N) ? a.br[e] : 0.f;
#pragma unroll
      for (int p = 0; p < R::KSPLIT; ++p) v += lg[(p * TB + r) * ldl + e];
      lg[r * ldl + e] = v;  // p = 0 tile is overwritten by its own final value only
    }
    __syncthreads();
  }

  rank_rows<bf16, NT, TB / 16>(a, lg, ldl, t0, wave, lane, lg + R::kLogitFloats);
}

// Split router for batches of few tokens (bf16, D a multiple of 128).  With
// few tokens the ring kernel has few blocks, and each streams the whole
// router matrix through one CU.  Here the work is spread over
// (16-token tile, 64-expert group, 128-wide k chunk) waves:
//  route_partial_kernel: one wave computes the 16 x 64 partial logit tile of
//    its k chunk with v_mfma_f32_16x16x32_bf16, operands loaded straight into
//    registers (lane group q of a row reads 64 contiguous bytes; A and B take
//    the same k positions in each lane group, so every product pairs matching
//    k), and stores it to part[chunk][token][expert];
//  route_rank_kernel: one wave per 4 tokens sums the chunks of each logit in
//    increasing chunk order (fixed order, so the result does not depend on
//    timing), adds the router bias and ranks the tokens as the other kernels
//    do (group_rank, exact re-ranking of near-ties).
constexpr int kSplitChunk = 128;  // k per partial tile
constexpr int kRankRows = 4;      // tokens per ranking wave

template <int NE>  // expert tiles of 16 per wave (1..4)
__global__ __launch_bounds__(64) void route_partial_kernel(RouteArgs a, float* part, int np) {
  const int lane = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  const int e0 = blockIdx.y * 16 * NE;
  const int kc = blockIdx.z;
  const int D = a.D;
  const int q = lane >> 4, r16 = lane & 15;
  int64_t row = t0 + r16;
  if (row > a.T - 1) row = a.T - 1;
  const int koff = kc * kSplitChunk + q * (kSplitChunk / 4);
  const bf16x8* xa = (const bf16x8*)((const bf16*)a.x + row * D + koff);
  bf16x8 av[4], bv[NE][4];
#pragma unroll
  for (int u = 0; u < 4; ++u) av[u] = xa[u];
#pragma unroll
  for (int n = 0; n < NE; ++n) {
    int e = e0 + n * 16 + r16;
    if (e > a.N - 1) e = a.N - 1;
    const bf16x8* wb = (const bf16x8*)((const bf16*)a.wr + (int64_t)e * D + koff);
#pragma unroll
    for (int u = 0; u < 4; ++u) bv[n][u] = wb[u];
  }
  f32x4 acc[NE];
#pragma unroll
  for (int n = 0; n < NE; ++n) {
    acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bv[n][u], acc[n], 0, 0, 0);
  }
  // C layout: lane holds tokens 4q .. 4q+3 of column r16
  float* dst = part + ((int64_t)kc * a.T) * np;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = t0 + 4 * q + i;
    if (t < a.T) {
#pragma unroll
      for (int n = 0; n < NE; ++n) {
        const int e = e0 + n * 16 + r16;
        if (e < np) dst[t * np + e] = acc[n][i];
      }
    }
  }
}

template <int NT>
__global__ __launch_bounds__(64) void route_rank_kernel(RouteArgs a, const float* part, int np, int nchunks) {
  constexpr int NP = 16 * NT;
  constexpr int ldl = NP + 1;
  __shared__ float lg[kRankRows * ldl];
  const int lane = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * kRankRows;
  // value i of the lane is entry f = 64 i + lane of the block's 4 x NP logit
  // tile: token f / NP, expert f % NP
  constexpr int PER = (kRankRows * NP + 63) / 64;
  constexpr int kBatch = 16;  // partial loads in flight per value (one batch for D <= 2048)
  float acc[PER];
  int64_t base[PER];
  bool valid[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int f = i * 64 + lane;
    const int r = f / NP, e = f % NP;
    int64_t t = t0 + r;
    valid[i] = (r < kRankRows) && (e < a.N) && (t < a.T);
    if (t > a.T - 1) t = a.T - 1;
    base[i] = t * np + (e < np ? e : np - 1);
    acc[i] = (valid[i] && a.has_bias) ? a.br[e] : 0.f;
  }
  const int64_t cstride = (int64_t)a.T * np;
  for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
    float v[kBatch][PER];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int c = (c0 + b < nchunks) ? c0 + b : nchunks - 1;
#pragma unroll
      for (int i = 0; i < PER; ++i) v[b][i] = part[c * cstride + base[i]];
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      if (c0 + b < nchunks) {
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] += v[b][i];
      }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int f = i * 64 + lane;
    const int r = f / NP, e = f % NP;
    if (r < kRankRows) lg[r * ldl + e] = valid[i] ? acc[i] : 0.f;
  }
  __syncthreads();
  rank_rows<bf16, NT, 1>(a, lg, ldl, t0, 0, lane, nullptr);  // never with statistics
}

template <int NT, int TB, bool TWO>
hipError_t launch_ring(const RouteArgs& a, hipStream_t st) {
  using R = RouteRing<NT, TB, TWO>;
  auto kern = route_ring_kernel<NT, TB, TWO>;
  static const hipError_t attr_err =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, R::kBytes);
  if (attr_err != hipSuccess) return attr_err;
  const int64_t blocks = (a.T + TB - 1) / TB;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), R::kBytes, st, a);
  return hipGetLastError();
}

// rows < 0: -rows tokens per block, two blocks per CU
template <int NT>
hipError_t launch_ring_nt(const RouteArgs& a, int rows, hipStream_t st) {
  if constexpr (NT < 16) {
    if (rows == 64) return launch_ring<NT, 64, false>(a, st);
    if (rows == 32) return launch_ring<NT, 32, false>(a, st);
  }
  if constexpr (NT == 8) {
    if (rows == -32) return launch_ring<NT, 32, true>(a, st);
  }
  return launch_ring<NT, 16, false>(a, st);
}

template <typename T, int NT>
hipError_t launch_nt(const RouteArgs& a, hipStream_t st) {
  const int64_t blocks = (a.T + 31) / 32;
  hipLaunchKernelGGL((route_kernel<T, NT>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const RouteArgs& a, int rows, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (a.D % 128 == 0) {
      if (a.N <= 16) return launch_ring_nt<1>(a, rows, st);
      if (a.N <= 32) return launch_ring_nt<2>(a, rows, st);
      if (a.N <= 64) return launch_ring_nt<4>(a, rows, st);
      if (a.N <= 128) return launch_ring_nt<8>(a, rows, st);
      return launch_ring_nt<16>(a, rows, st);
    }
  }
  if (a.N <= 16) return launch_nt<T, 1>(a, st);
  if (a.N <= 32) return launch_nt<T, 2>(a, st);
  if (a.N <= 64) return launch_nt<T, 4>(a, st);
  if (a.N <= 128) return launch_nt<T, 8>(a, st);
  return launch_nt<T, 16>(a, st);
}

template <int NE>
hipError_t launch_partial(const RouteArgs& a, float* part, int np, hipStream_t st) {
  const dim3 grid((unsigned)((a.T + 15) / 16), (unsigned)((a.N + 16 * NE - 1) / (16 * NE)),
                  (unsigned)(a.D / kSplitChunk));
  hipLaunchKernelGGL(route_partial_kernel<NE>, grid, dim3(64), 0, st, a, part, np);
  return hipGetLastError();
}

template <int NT>
hipError_t launch_rank(const RouteArgs& a, const float* part, int np, hipStream_t st) {
  const int64_t blocks = (a.T + kRankRows - 1) / kRankRows;
  hipLaunchKernelGGL(route_rank_kernel<NT>, dim3((unsigned)blocks), dim3(64), 0, st, a, part, np,
                     a.D / kSplitChunk);
  return hipGetLastError();
}

hipError_t launch_split(const RouteArgs& a, float* part, hipStream_t st) {
  const int np = (a.N + 15) / 16 * 16;
  hipError_t e = (a.N <= 16)   ? launch_partial<1>(a, part, np, st)
                 : (a.N <= 32) ? launch_partial<2>(a, part, np, st)
                               : launch_partial<4>(a, part, np, st);
  if (e != hipSuccess) return e;
  if (a.N <= 16) return launch_rank<1>(a, part, np, st);
  if (a.N <= 32) return launch_rank<2>(a, part, np, st);
  if (a.N <= 64) return launch_rank<4>(a, part, np, st);
  if (a.N <= 128) return launch_rank<8>(a, part, np, st);
  return launch_rank<16>(a, part, np, st);
}

// Statistics, second pass, one wave per expert e (grid N): lane l adds the
// block partials b = l, l + 64, ... in increasing b in fp64 (loads issued 8
// at a time), then a butterfly; P_e = sum / T and f_e = counts[e] / T.  The
// order is fixed, so the result does not depend on timing.  Each wave then
// takes a ticket; the wave that draws the last one of this call (N tickets
// per call, the count cleared by the router) reads every P_e back and forms
// the Switch auxiliary loss N * sum_e f_e * P_e, the imbalance
// max_e count_e / (T*k/N) and the drop rate n_dropped / (T*k).
__global__ __launch_bounds__(64) void router_stats_kernel(const float* part, int nblk, int N, int64_t T, int k,
                                                          const int32_t* counts, const int32_t* n_dropped,
                                                          double* prob_mean, double* frac, double* summary,
                                                          unsigned long long* ticket) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const float* row = part + (int64_t)e * nblk;
  double sum = 0.0;
  for (int b0 = 0; b0 < nblk; b0 += 8 * kWave) {
    // clamped, unconditional loads: all 8 are in flight before the first add
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int b = b0 + i * kWave + lane;
      v[i] = row[b < nblk ? b : nblk - 1];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (b0 + i * kWave + lane < nblk) sum += (double)v[i];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  int last = 0;
  if (lane == 0) {
    prob_mean[e] = sum / (double)T;
    if (frac) frac[e] = (double)counts[e] / (double)T;
    __threadfence();  // publish prob_mean[e] before the ticket
    const unsigned long long old = atomicAdd(ticket, 1ull);
    last = (old % (unsigned long long)N) == (unsigned long long)(N - 1);
  }
  last = __shfl(last, 0);
  if (!last) return;
  __threadfence();  // every other wave's prob_mean is visible past its ticket
  // at most 4 experts per lane, loads clamped and all in flight
  static_assert(kMaxExperts <= 4 * kWave, "experts per lane");
  int c[4];
  double p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = lane + j * kWave < N ? lane + j * kWave : N - 1;
    c[j] = counts[i];
    p[j] = prob_mean[i];
  }
  double acc = 0.0;
  int mx = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (lane + j * kWave < N) {
      acc += ((double)c[j] / (double)T) * p[j];
      mx = c[j] > mx ? c[j] : mx;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    acc += __shfl_xor(acc, off);
    const int o = __shfl_xor(mx, off);
    mx = o > mx ? o : mx;
  }
  if (lane == 0) {
    const double A = (double)T * (double)k;
    summary[0] = (double)N * acc;
    summary[1] = (double)mx / (A / (double)N);
    summary[2] = (double)*n_dropped / A;
  }
}

}  // namespace

// Tokens per router block, negated when the ring is sized for two blocks
// per CU.  bf16 with D a multiple of 128 uses the DMA ring kernel: as many
// tokens as keep >= ~2 blocks per CU busy, 16 for the widest expert counts
// (their ring stages are large) and for at most 16 experts (8 KiB stages: an
// 8-deep ring and two blocks per CU beat fewer, larger blocks); with 65-128
// experts and at least 64 tokens per CU, 32-token blocks two to a CU, so
// that one block ranks while the other loads; otherwise 32.
static int route_block_mode(const moe_shape& s) {
  if (s.dtype == MOE_DTYPE_BF16 && s.D % 128 == 0) {
    if (s.N > 128 || s.N <= 16) return 16;
    const int64_t cus = device_cu_count();
    if (s.T >= 64 * cus) return s.N > 64 ? -32 : 64;
    if (s.T >= 32 * cus) return 32;
    return 16;
  }
  return 32;
}

int route_rows_per_block(const moe_shape& s) {
  const int m = route_block_mode(s);
  return m < 0 ? -m : m;
}

int64_t route_blocks(const moe_shape& s) {
  const int rows = route_rows_per_block(s);
  return (s.T + rows - 1) / rows;
}

// The second pass's ticket sits after the partials, 256-byte aligned.
unsigned long long* stats_ticket(const moe_shape& s, const float* part) {
  const size_t off = ((size_t)route_blocks(s) * (size_t)s.N * sizeof(float) + 255) & ~(size_t)255;
  return (unsigned long long*)((const unsigned char*)part + off);
}

hipError_t launch_router_stats(const moe_shape& s, const float* part, const int32_t* counts,
                               const int32_t* n_dropped, double* prob_mean, double* frac, double* summary,
                               hipStream_t st) {
  hipLaunchKernelGGL(router_stats_kernel, dim3(s.N), dim3(kWave), 0, st, part, (int)route_blocks(s), s.N, s.T,
                     s.k, counts, n_dropped, prob_mean, frac, summary, stats_ticket(s, part));
  return hipGetLastError();
}

// The split router takes bf16 batches of at most kSplitRouteMaxT tokens with
// D a multiple of 128; its partial tiles need route_split_bytes(s) of scratch.
constexpr int64_t kSplitRouteMaxT = 1024;

bool use_split_route(const moe_shape& s) {
  return s.dtype == MOE_DTYPE_BF16 && s.D % kSplitChunk == 0 && s.T > 0 && s.T <= kSplitRouteMaxT;
}

size_t route_split_bytes(const moe_shape& s) {
  const size_t np = (size_t)(s.N + 15) / 16 * 16;
  return (size_t)(s.D / kSplitChunk) * (size_t)s.T * np * sizeof(float);
}

hipError_t launch_route_split(const moe_shape& s, const void* x, const void* wr, const float* br, int32_t* idx,
                              float* gate, float* logits, float* part, hipStream_t st) {
  RouteArgs a{};
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
  return launch_split(a, part, st);
}

hipError_t launch_route(const moe_shape& s, const void* x, const void* wr, const float* br,
                        int32_t* idx, float* gate, float* logits, float* prob_part, int R, int32_t* fb_idx,
                        float* fb_gate, hipStream_t st) {
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
  a.R = R;
  a.fb_idx = fb_idx;
  a.fb_gate = fb_gate;
  a.prob_part = prob_part;
  a.stats_ticket = prob_part ? stats_ticket(s, prob_part) : nullptr;
  const int rows = route_block_mode(s);
  if (s.dtype == MOE_DTYPE_BF16) return launch_t<bf16>(a, rows, st);
  return launch_t<float>(a, rows, st);
}

}  // namespace moe
