// Dispatch: group assignments by expert with a per-expert slot budget
// ("Dispatch and gather" and "Capacity factor" sections of the notebook
// "Mixture-of-experts and expert parallelism"; grouping inputs by assigned
// expert is trick 2 of "MoE Parallelism for Inference: Tricks and PyTorch
// Deep Dive").
//
// One workgroup of 1024 threads (16 waves), two passes over the T*k
// assignments:
//  1. histogram of expert ids with LDS atomics (order-free, so exact), then
//     an exclusive scan of min(count, capacity) -> offsets.
//  2. stable ranking in chunks of 1024 assignments, chunk after chunk:
//     inside a wave the lanes holding the same expert are found with one
//     ballot per bit of the expert id; a lane's rank is the number of such
//     lanes below it, plus the counts of the same expert in lower waves of
//     the chunk, plus the running count of earlier chunks.  The rank is the
//     position in increasing flat index, so the result is the stable order.
// The assignment volume is small (T*k <= a few 10^4 on the workloads), so a
// single workgroup finishes in a few microseconds without global atomics.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kBatch = 8192;  // assignments staged in LDS at a time

__global__ __launch_bounds__(kThreads) void dispatch_kernel(const int32_t* __restrict__ idx,
                                                            int64_t A, int N, int C,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ slot,
                                                            int32_t* __restrict__ n_dropped) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];
  __shared__ int base[kMaxExperts];
  __shared__ int wcnt[kWavesPerBlock][kMaxExperts];
  __shared__ int scan_tmp[kMaxExperts];
  __shared__ int ids[kBatch];
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;

  for (int i = tid; i < kMaxExperts; i += kThreads) {
    cnt[i] = 0;
    base[i] = 0;
  }
  for (int i = tid; i < kWavesPerBlock * kMaxExperts; i += kThreads) (&wcnt[0][0])[i] = 0;
  __syncthreads();

  // pass 1: histogram (batches staged in LDS with coalesced loads)
  for (int64_t b0 = 0; b0 < A; b0 += kBatch) {
    const int nb = (int)(A - b0 < kBatch ? A - b0 : kBatch);
    for (int i = tid; i < nb; i += kThreads) ids[i] = idx[b0 + i];
    __syncthreads();
    for (int i = tid; i < nb; i += kThreads) {
      const int e = ids[i];
      if (e >= 0 && e < N) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
  }

  // exclusive scan of kept counts (N <= 256: Hillis-Steele in LDS)
  int kept = 0;
  if (tid < N) {
    kept = cnt[tid];
    if (C >= 0 && kept > C) kept = C;
    scan_tmp[tid] = kept;
    counts[tid] = cnt[tid];
  }
  __syncthreads();
  for (int d = 1; d < kMaxExperts; d <<= 1) {
    int v = 0;
    if (tid < N && tid >= d) v = scan_tmp[tid - d];
    __syncthreads();
    if (tid < N && tid >= d) scan_tmp[tid] += v;
    __syncthreads();
  }
  if (tid < N) {
    off[tid] = scan_tmp[tid] - kept;  // exclusive
    offsets[tid] = scan_tmp[tid] - kept;
  }
  if (tid == 0) {
    int total = N > 0 ? scan_tmp[N - 1] : 0;
    off[N] = total;
    offsets[N] = total;
    *n_dropped = (int32_t)(A - total);
  }
  __syncthreads();

  // bits needed to tell the expert ids apart
  int bits = 0;
  while ((1 << bits) < N) ++bits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // pass 2: stable ranks, chunk by chunk (chunks of a batch read from LDS)
  for (int64_t c0 = 0; c0 < A; c0 += kThreads) {
    if (c0 % kBatch == 0) {
      const int nb = (int)(A - c0 < kBatch ? A - c0 : kBatch);
      __syncthreads();
      for (int i = tid; i < nb; i += kThreads) ids[i] = idx[c0 + i];
      __syncthreads();
    }
    const int64_t a = c0 + tid;
    int e = (a < A) ? ids[(int)(a % kBatch)] : -1;
    const bool valid = (e >= 0 && e < N);
    uint64_t same = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t bb = __ballot(bit);
      same &= bit ? bb : ~bb;
    }
    if (!valid) same = 0;
    const int below = __popcll(same & lt_mask);
    const bool leader = valid && below == 0;
    if (leader) wcnt[wave][e] = __popcll(same);
    __syncthreads();
    int rank = 0;
    if (valid) {
      rank = base[e] + below;
      for (int w = 0; w < wave; ++w) rank += wcnt[w][e];
    }
    __syncthreads();
    if (valid) {
      atomicAdd(&base[e], 1);
      if (C < 0 || rank < C) {
        const int s = off[e] + rank;
        slot[a] = s;
        perm[s] = (int32_t)a;
      } else {
        slot[a] = -1;
      }
    } else if (a < A) {
      slot[a] = -1;
    }
    if (leader) wcnt[wave][e] = 0;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_dispatch(const moe_shape& s, const int32_t* idx, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* slot, int32_t* n_dropped,
                           hipStream_t st) {
  const int64_t A = s.T * (int64_t)s.k;
  hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(kThreads), 0, st, idx, A, s.N, s.capacity,
                     counts, offsets, perm, slot, n_dropped);
  return hipGetLastError();
}

}  // namespace moe
