// Dispatch: group assignments by expert with a per-expert slot budget
// ("Dispatch and gather" and "Capacity factor" sections of the notebook
// "Mixture-of-experts and expert parallelism"; grouping inputs by assigned
// expert is trick 2 of "MoE Parallelism for Inference: Tricks and PyTorch
// Deep Dive").
//
// One workgroup of 1024 threads (16 waves).  The T*k assignments, taken in
// priority order i (i = a = t*k + j by token, or i = j*T + t by choice, the
// GShard order), are split into 16 contiguous segments, one per wave, so
// that the result is the stable order (segments, 64-wide chunks inside a
// segment and lanes inside a chunk all follow increasing i):
//  A. each wave walks its segment chunk by chunk; the lanes holding the same
//     expert are found with one ballot per bit of the expert id, a lane's
//     rank inside its wave is the wave's running count of that expert plus
//     the same-expert lanes below it; the lowest such lane advances the
//     running count (wave-private LDS counters, no atomics, no barriers).
//     The in-wave rank is parked in slot[a].
//  B. per expert, an exclusive scan of the 16 wave counts gives each wave's
//     base and the expert's total; a scan of min(total, capacity) over the
//     experts gives offsets.
//  C. each wave re-walks its segment: rank = wave base + in-wave rank; a
//     rank below the capacity gets slot[a] = offsets[e] + rank and
//     perm[slot] = a, the rest slot[a] = -1.
// With S shared (always-on) experts their S*T rows come first: offsets[s] =
// s*T for s <= S, perm[s*T + t] = t*k, and every routed offset and slot is
// shifted by S*T.  In the padded layout expert e's rows start at S*T + e*C
// and its C - kept padding rows get perm = 0 (a valid gather row whose
// output nobody reads).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kPrefetch = 8;  // chunks whose ids are loaded ahead

// Flat index a = t*k + j of the i-th assignment in priority order.
__device__ inline int64_t flat_of(int64_t i, int64_t T, int k, bool by_choice) {
  if (!by_choice) return i;
  const int64_t j = i / T;
  return (i - j * T) * k + j;
}

__global__ __launch_bounds__(kThreads) void dispatch_kernel(const int32_t* __restrict__ idx,
                                                            int64_t A, int64_t T, int k, int by_choice,
                                                            int N, int C, int S, int pad,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ slot,
                                                            int32_t* __restrict__ n_dropped) {
  __shared__ int wcnt[kWaves][kMaxExperts];  // A: running counts; then wave bases
  __shared__ int scan[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  for (int i = tid; i < kWaves * kMaxExperts; i += kThreads) (&wcnt[0][0])[i] = 0;
  __syncthreads();

  int bits = 0;
  while ((1 << bits) < N) ++bits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // segment of this wave, in whole 64-wide chunks
  const int64_t chunks = (A + kWave - 1) / kWave;
  const int64_t per = (chunks + kWaves - 1) / kWaves;
  const int64_t a_begin = (int64_t)wave * per * kWave;
  const int64_t a_end = (a_begin + per * kWave < A) ? a_begin + per * kWave : A;

  // ---- A: in-wave ranks
  for (int64_t b0 = a_begin; b0 < a_end; b0 += kPrefetch * kWave) {
    int ev[kPrefetch];
#pragma unroll
    for (int c = 0; c < kPrefetch; ++c) {
      const int64_t i = b0 + c * kWave + lane;
      ev[c] = (i < a_end) ? idx[flat_of(i, T, k, by_choice)] : -1;
    }
#pragma unroll
    for (int c = 0; c < kPrefetch; ++c) {
      const int64_t i = b0 + c * kWave + lane;
      const int64_t a = flat_of(i, T, k, by_choice);
      const int e = ev[c];
      const bool valid = i < a_end && e >= 0 && e < N;
      uint64_t same = __ballot(valid);
      for (int b = 0; b < bits; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t bb = __ballot(bit);
        same &= bit ? bb : ~bb;
      }
      if (valid) {
        const int below = __popcll(same & lt_mask);
        const int base = wcnt[wave][e];  // every lane reads before the leader writes
        if (below == 0) wcnt[wave][e] = base + __popcll(same);
        slot[a] = base + below;
      }
    }
  }
  __syncthreads();

  // ---- B: wave bases per expert, totals, capacity cut, offsets
  int kept = 0;
  if (tid < N) {
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = wcnt[w][tid];
      wcnt[w][tid] = run;
      run += c;
    }
    counts[tid] = run;
    kept = (C >= 0 && run > C) ? C : run;
    scan[tid] = kept;
  }
  __syncthreads();
  for (int d = 1; d < kMaxExperts; d <<= 1) {
    int v = 0;
    if (tid < N && tid >= d) v = scan[tid - d];
    __syncthreads();
    if (tid < N && tid >= d) scan[tid] += v;
    __syncthreads();
  }
  const int ST = S * (int)T;  // rows of the shared experts, in front
  if (tid < N) {
    const int o = ST + (pad ? tid * C : scan[tid] - kept);
    off[tid] = o;
    offsets[S + tid] = o;
  }
  if (tid < S) offsets[tid] = tid * (int)T;
  if (tid == 0) {
    const int total = N > 0 ? scan[N - 1] : 0;  // kept assignments
    off[N] = ST + (pad ? N * C : total);
    offsets[S + N] = ST + (pad ? N * C : total);
    *n_dropped = (int32_t)(A - total);
  }
  // shared rows: token t of shared expert s is row s*T + t, assignment t*k
  for (int64_t r = tid; r < (int64_t)ST; r += kThreads) perm[r] = (int32_t)((r % T) * k);
  if (pad) {
    // padding rows after each expert's kept rows (kept_e = scan[e] - scan[e-1])
    for (int64_t i = tid; i < (int64_t)N * C; i += kThreads) {
      const int e = (int)(i / C), r = (int)(i - (int64_t)e * C);
      const int kept_e = scan[e] - (e > 0 ? scan[e - 1] : 0);
      if (r >= kept_e) perm[ST + i] = 0;
    }
  }
  __syncthreads();

  // ---- C: final ranks -> slot and perm
  for (int64_t b0 = a_begin; b0 < a_end; b0 += kPrefetch * kWave) {
    int ev[kPrefetch], rv[kPrefetch];
#pragma unroll
    for (int c = 0; c < kPrefetch; ++c) {
      const int64_t i = b0 + c * kWave + lane;
      const int64_t a = flat_of(i, T, k, by_choice);
      ev[c] = (i < a_end) ? idx[a] : -1;
      rv[c] = (i < a_end) ? slot[a] : 0;
    }
#pragma unroll
    for (int c = 0; c < kPrefetch; ++c) {
      const int64_t i = b0 + c * kWave + lane;
      const int64_t a = flat_of(i, T, k, by_choice);
      if (i >= a_end) continue;
      const int e = ev[c];
      if (e < 0 || e >= N) {
        slot[a] = -1;
        continue;
      }
      const int rank = wcnt[wave][e] + rv[c];
      if (C < 0 || rank < C) {
        const int s = off[e] + rank;
        slot[a] = s;
        perm[s] = (int32_t)a;
      } else {
        slot[a] = -1;
      }
    }
  }
}

}  // namespace

hipError_t launch_dispatch(const moe_shape& s, const int32_t* idx, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* slot, int32_t* n_dropped,
                           hipStream_t st) {
  const int64_t A = s.T * (int64_t)s.k;
  const int by_choice = (s.flags & MOE_SLOT_MAJOR) && s.k > 1;
  hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(kThreads), 0, st, idx, A, s.T, s.k, by_choice, s.N,
                     s.capacity, s.n_shared, (s.flags & MOE_PADDED) ? 1 : 0, counts, offsets, perm, slot,
                     n_dropped);
  return hipGetLastError();
}

}  // namespace moe
