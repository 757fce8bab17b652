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

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y, const int32_t* __restrict__ slot,
                                                      const float* __restrict__ gate,
                                                      const T* __restrict__ x, T* __restrict__ out,
                                                      int64_t T_, int D, int k, int S) {
  constexpr int W = Vec<T>::W;
  typedef typename Vec<T>::type V;
  const int chunks = D / W;
  const int64_t items = T_ * chunks;  // one 16-byte chunk of one token each
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < items;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / chunks;
    const int c = (int)(i - t * chunks);
    float acc[W];
    if (x) {
      V xv = *(const V*)(x + t * D + c * W);
#pragma unroll
      for (int u = 0; u < W; ++u) acc[u] = (float)xv[u];
    } else {
#pragma unroll
      for (int u = 0; u < W; ++u) acc[u] = 0.f;
    }
    for (int sh = 0; sh < S; ++sh) {
      V yv = *(const V*)(y + ((int64_t)sh * T_ + t) * D + c * W);
#pragma unroll
      for (int u = 0; u < W; ++u) acc[u] += (float)yv[u];
    }
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        const int s = slot[t * k + j];
        if (s >= 0) {
          const float g = gate[t * k + j];
          V yv = *(const V*)(y + (int64_t)s * D + c * W);
#pragma unroll
          for (int u = 0; u < W; ++u) acc[u] = fmaf(g, (float)yv[u], acc[u]);
        }
      }
    }
    V o;
#pragma unroll
    for (int u = 0; u < W; ++u) o[u] = (T)acc[u];
    *(V*)(out + t * D + c * W) = o;
  }
}

// Same combine, reading fp32 partial rows of NS shards (summed in shard
// order) instead of one y_perm row.
template <typename T>
__global__ __launch_bounds__(256) void combine_shards_kernel(const float* __restrict__ part, int NS,
                                                             int64_t rows_cap,
                                                             const int32_t* __restrict__ slot,
                                                             const float* __restrict__ gate,
                                                             const T* __restrict__ x, T* __restrict__ out,
                                                             int64_t T_, int D, int k) {
  constexpr int W = Vec<T>::W;
  typedef typename Vec<T>::type V;
  const int chunks = D / W;
  const int64_t items = T_ * chunks;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < items;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / chunks;
    const int c = (int)(i - t * chunks);
    float acc[W];
    if (x) {
      V xv = *(const V*)(x + t * D + c * W);
#pragma unroll
      for (int u = 0; u < W; ++u) acc[u] = (float)xv[u];
    } else {
#pragma unroll
      for (int u = 0; u < W; ++u) acc[u] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        const int sl = slot[t * k + j];
        if (sl >= 0) {
          const float g = gate[t * k + j];
          float y[W];
#pragma unroll
          for (int u = 0; u < W; ++u) y[u] = 0.f;
          for (int s = 0; s < NS; ++s) {
            const float* src = part + ((int64_t)s * rows_cap + sl) * D + c * W;
#pragma unroll
            for (int u = 0; u < W; u += 4) {
              const f32x4 v = *(const f32x4*)(src + u);
              y[u] += v[0];
              y[u + 1] += v[1];
              y[u + 2] += v[2];
              y[u + 3] += v[3];
            }
          }
#pragma unroll
          for (int u = 0; u < W; ++u) acc[u] = fmaf(g, y[u], acc[u]);
        }
      }
    }
    V o;
#pragma unroll
    for (int u = 0; u < W; ++u) o[u] = (T)acc[u];
    *(V*)(out + t * D + c * W) = o;
  }
}

}  // namespace

hipError_t launch_combine(const moe_shape& s, const void* y_perm, const int32_t* slot,
                          const float* gate, const void* x_res, void* out, hipStream_t st) {
  const int W = s.dtype == MOE_DTYPE_BF16 ? 8 : 4;
  const int64_t items = s.T * (s.D / W);
  const int64_t cap = (int64_t)device_cu_count() * 8;
  const int64_t blocks = (items + 255) / 256;
  const dim3 grid((unsigned)(blocks < cap ? blocks : cap));
  const void* xr = (s.flags & MOE_RESIDUAL) ? x_res : nullptr;
  if (s.dtype == MOE_DTYPE_BF16)
    hipLaunchKernelGGL(combine_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)y_perm, slot, gate,
                       (const bf16*)xr, (bf16*)out, s.T, s.D, s.k, s.n_shared);
  else
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, st, (const float*)y_perm, slot, gate,
                       (const float*)xr, (float*)out, s.T, s.D, s.k, s.n_shared);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {
hipError_t launch_combine_shards(const moe_shape& s, const float* part, int n_shards,
                                 const int32_t* slot, const float* gate, const void* x_res, void* out,
                                 hipStream_t st) {
  const int W = s.dtype == MOE_DTYPE_BF16 ? 8 : 4;
  const int64_t items = s.T * (s.D / W);
  const int64_t cap = (int64_t)device_cu_count() * 8;
  const int64_t blocks = (items + 255) / 256;
  const dim3 grid((unsigned)(blocks < cap ? blocks : cap));
  const void* xr = (s.flags & MOE_RESIDUAL) ? x_res : nullptr;
  const int64_t rows_cap = s.T * (int64_t)s.k;
  if (s.dtype == MOE_DTYPE_BF16)
    hipLaunchKernelGGL(combine_shards_kernel<bf16>, grid, dim3(256), 0, st, part, n_shards, rows_cap, slot,
                       gate, (const bf16*)xr, (bf16*)out, s.T, s.D, s.k);
  else
    hipLaunchKernelGGL(combine_shards_kernel<float>, grid, dim3(256), 0, st, part, n_shards, rows_cap, slot,
                       gate, (const float*)xr, (float*)out, s.T, s.D, s.k);
  return hipGetLastError();
}
}  // namespace moe
