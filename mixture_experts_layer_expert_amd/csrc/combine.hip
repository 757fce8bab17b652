// Combine: gate-weighted sum of each token's kept expert outputs, back in
// token order ("Dispatch and gather" section of the notebook
// "Mixture-of-experts and expert parallelism": the output starts at zero and
// receives every chosen expert's output scaled by its gate).  With a
// residual the start value is x instead (dropped tokens pass through).  The
// rows s*T + t of S shared (always-on) experts are added with gate 1.
//
// Memory-bound: each token reads k rows of y_perm (+ x) and writes one row.
// Every thread handles one 16-byte chunk of one token at a time.
// The sum runs in fp32 in increasing choice order, so it is deterministic.
#include "moe_internal.h"

namespace moe {
namespace {

template <typename T>
struct Vec;
template <>
struct Vec<bf16> {
  static constexpr int W = 8;
  typedef bf16x8 type;
};
template <>
struct Vec<float> {
  static constexpr int W = 4;
  typedef f32x4 type;
};

// NI items per thread per pass (a pass covers NI * the grid's threads): the
// slot and gate loads of all NI items go out together, then their row loads,
// so a wave has NI times the rows in flight per round trip.  KM >= k bounds
// the choices held in registers (2 for top-1 and top-2 layers, else 8).
template <typename T, int NI, int KM>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y, const int32_t* __restrict__ slot,
                                                      const float* __restrict__ gate,
                                                      const T* __restrict__ x, T* __restrict__ out,
                                                      int64_t T_, int D, int k, int S) {
  constexpr int W = Vec<T>::W;
  typedef typename Vec<T>::type V;
  const int chunks = D / W;
  const int64_t items = T_ * chunks;  // one 16-byte chunk of one token each
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i0 < items; i0 += NI * nthreads) {
    int64_t t[NI];
    int c[NI];
    bool in[NI];
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int64_t i = i0 + n * nthreads;
      in[n] = i < items;
      const int64_t ii = in[n] ? i : i0;  // a valid item: its loads stay in bounds
      t[n] = ii / chunks;
      c[n] = (int)(ii - t[n] * chunks);
    }
    float acc[NI][W];
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      if (x) {
        V xv = *(const V*)(x + t[n] * D + c[n] * W);
#pragma unroll
        for (int u = 0; u < W; ++u) acc[n][u] = (float)xv[u];
      } else {
#pragma unroll
        for (int u = 0; u < W; ++u) acc[n][u] = 0.f;
      }
      for (int sh = 0; sh < S; ++sh) {
        V yv = *(const V*)(y + ((int64_t)sh * T_ + t[n]) * D + c[n] * W);
#pragma unroll
        for (int u = 0; u < W; ++u) acc[n][u] += (float)yv[u];
      }
    }
    // every slot and gate first, then every kept row, then the sums: the
    // loads of all k choices (of all NI items) are in flight together
    int sl[NI][KM];
    float gv[NI][KM];
#pragma unroll
    for (int n = 0; n < NI; ++n)
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        sl[n][j] = (j < k) ? slot[t[n] * k + j] : -1;
        gv[n][j] = (j < k) ? gate[t[n] * k + j] : 0.f;
      }
    V yv[NI][KM];
#pragma unroll
    for (int n = 0; n < NI; ++n)
#pragma unroll
      for (int j = 0; j < KM; ++j)
        if (sl[n][j] >= 0) yv[n][j] = *(const V*)(y + (int64_t)sl[n][j] * D + c[n] * W);
#pragma unroll
    for (int n = 0; n < NI; ++n) {
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (sl[n][j] >= 0) {
#pragma unroll
          for (int u = 0; u < W; ++u) acc[n][u] = fmaf(gv[n][j], (float)yv[n][j][u], acc[n][u]);
        }
      }
      if (in[n]) {
        V o;
#pragma unroll
        for (int u = 0; u < W; ++u) o[u] = (T)acc[n][u];
        *(V*)(out + t[n] * D + c[n] * W) = o;
      }
    }
  }
}

// Same combine, reading fp32 partial rows of NS shards (summed in shard
// order) instead of one y_perm row.  A thread takes 4 columns of one token:
// it loads the token's slots and gates, then the partial pieces of every
// choice for up to kShardBatch shards at once (a dropped choice reads row 0,
// in range, and is selected away), so that its loads are in flight
// together rather than one dependent load after another.  Per choice the
// shards are summed in increasing order and the choices are added in
// increasing order, so the result does not depend on the batching.
constexpr int kShardBatch = 4;

template <typename T, int KM>
__global__ __launch_bounds__(256) void combine_shards_kernel(const float* __restrict__ part, int NS,
                                                             int64_t rows_cap,
                                                             const int32_t* __restrict__ slot,
                                                             const float* __restrict__ gate,
                                                             const T* __restrict__ x, T* __restrict__ out,
                                                             int64_t T_, int D, int k) {
  const int chunks = D / 4;
  const int64_t items = T_ * chunks;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < items;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / chunks;
    const int c = (int)(i - t * chunks);
    int sl[KM];
    float g[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      sl[j] = j < k ? slot[t * k + j] : -1;
      g[j] = j < k ? gate[t * k + j] : 0.f;
    }
    float acc[4];
    if (x) {
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] = (float)x[t * D + c * 4 + u];
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] = 0.f;
    }
    f32x4 y[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) y[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < NS; s0 += kShardBatch) {
      f32x4 v[KM][kShardBatch];
#pragma unroll
      for (int j = 0; j < KM; ++j)
#pragma unroll
        for (int b = 0; b < kShardBatch; ++b) {
          const int sh = s0 + b < NS ? s0 + b : NS - 1;
          const int64_t row = sl[j] >= 0 ? sl[j] : 0;
          v[j][b] = *(const f32x4*)(part + ((int64_t)sh * rows_cap + row) * D + c * 4);
        }
#pragma unroll
      for (int j = 0; j < KM; ++j)
#pragma unroll
        for (int b = 0; b < kShardBatch; ++b)
          if (s0 + b < NS) y[j] += v[j][b];
    }
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const bool kept = sl[j] >= 0;  // also false for j >= k
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] = kept ? fmaf(g[j], y[j][u], acc[u]) : acc[u];
    }
    if constexpr (sizeof(T) == 2) {
      bf16x4 o;
#pragma unroll
      for (int u = 0; u < 4; ++u) o[u] = (bf16)acc[u];
      *(bf16x4*)(out + t * D + c * 4) = o;
    } else {
      *(f32x4*)(out + t * D + c * 4) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    }
  }
}

}  // namespace

hipError_t launch_combine(const moe_shape& s, const void* y_perm, const int32_t* slot,
                          const float* gate, const void* x_res, void* out, hipStream_t st) {
  const int W = s.dtype == MOE_DTYPE_BF16 ? 8 : 4;
  const int64_t items = s.T * (s.D / W);
  const int64_t cap = (int64_t)device_cu_count() * 8;  // blocks of 256: 32 waves per CU
  // two items per thread once a full grid would still loop over the items
  // (top-1 and top-2 layers: with up to 8 choices in registers the kernel's
  // occupancy would halve)
  const bool two = items >= 2 * cap * 256 && s.k <= 2 && s.dtype == MOE_DTYPE_BF16;
  const int64_t per = two ? 512 : 256;
  const int64_t blocks = (items + per - 1) / per;
  const dim3 grid((unsigned)(blocks < cap ? blocks : cap));
  const void* xr = (s.flags & MOE_RESIDUAL) ? x_res : nullptr;
  const bool k2 = s.k <= 2;
#define MOE_COMBINE(TY, NI, KM)                                                                          \
  hipLaunchKernelGGL((combine_kernel<TY, NI, KM>), grid, dim3(256), 0, st, (const TY*)y_perm, slot, gate, \
                     (const TY*)xr, (TY*)out, s.T, s.D, s.k, s.n_shared)
  if (s.dtype == MOE_DTYPE_BF16) {
    if (two) MOE_COMBINE(bf16, 2, 2);
    else if (k2) MOE_COMBINE(bf16, 1, 2);
    else MOE_COMBINE(bf16, 1, kMaxTopK);
  } else {
    if (k2) MOE_COMBINE(float, 1, 2);
    else MOE_COMBINE(float, 1, kMaxTopK);
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe

namespace moe {
hipError_t launch_combine_shards(const moe_shape& s, const float* part, int n_shards,
                                 const int32_t* slot, const float* gate, const void* x_res, void* out,
                                 hipStream_t st) {
  const int64_t items = s.T * (s.D / 4);
  const int64_t cap = (int64_t)device_cu_count() * 8;
  const int64_t blocks = (items + 255) / 256;
  const dim3 grid((unsigned)(blocks < cap ? blocks : cap));
  const void* xr = (s.flags & MOE_RESIDUAL) ? x_res : nullptr;
  const int64_t rows_cap = s.T * (int64_t)s.k;
#define MOE_COMBINE_SHARDS(TY, KM)                                                                        \
  hipLaunchKernelGGL((combine_shards_kernel<TY, KM>), grid, dim3(256), 0, st, part, n_shards, rows_cap, slot, \
                     gate, (const TY*)xr, (TY*)out, s.T, s.D, s.k)
  if (s.dtype == MOE_DTYPE_BF16) {
    if (s.k <= 2) MOE_COMBINE_SHARDS(bf16, 2);
    else MOE_COMBINE_SHARDS(bf16, kMaxTopK);
  } else {
    if (s.k <= 2) MOE_COMBINE_SHARDS(float, 2);
    else MOE_COMBINE_SHARDS(float, kMaxTopK);
  }
#undef MOE_COMBINE_SHARDS
  return hipGetLastError();
}
}  // namespace moe
