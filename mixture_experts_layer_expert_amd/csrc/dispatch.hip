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
//     The in-wave rank is parked in slot[a], or, for up to 24 chunks per
//     wave, kept in registers together with the expert id until C (register
//     modes of 1, 4 and 24 chunks: the smallest that holds the batch, since
//     the unrolled code grows with the count).
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
//
// Rerouting (R fallback levels, compact layout): C only records provisional
// rows in slot.  Then, level r = 0 .. R-1: every token with a dropped
// assignment left offers its lowest-j one to its expert of rank k + r
// (fb_idx[t, r]); the offers are ranked per expert in token order with the
// ballot scheme of A over 16 token segments (in-wave ranks parked in the
// routed perm rows, not yet written), and the first `room` of each expert are
// accepted: idx and gate of the assignment are rewritten and slot holds
// -2 - (its place among the expert's rerouted rows).  Finally the offsets
// are the scan of kept + rerouted, and one pass over the assignments writes
// the final slot and perm (kept rows first, then rerouted ones in level and
// token order).
//
// Batches of more than 4096 assignments can instead take the two launches
// of dispatch_count_kernel and dispatch_place_kernel (below), which spread
// the same ranking over one workgroup per 1024-assignment segment.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kPrefetch = 8;  // chunks whose ids are loaded ahead
constexpr int kRegChunks = 24;  // register mode: up to 24 chunks per wave (24576 assignments)

// Flat index a = t*k + j of the i-th assignment in priority order.
__device__ inline int64_t flat_of(int64_t i, int64_t T, int k, bool by_choice) {
  if (!by_choice) return i;
  const int64_t j = i / T;
  return (i - j * T) * k + j;
}

// Rank of each valid lane among the lanes of its wave holding the same
// expert e (lanes below it), plus the wave's running count of e in cnt,
// which the lowest such lane advances.  Every lane reads the count before
// the leader writes it; all lanes of the wave take part.
__device__ inline int wave_rank(bool valid, int e, int bits, uint64_t lt_mask, int* cnt) {
  uint64_t same = __ballot(valid);
  for (int b = 0; b < bits; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const uint64_t bb = __ballot(bit);
    same &= bit ? bb : ~bb;
  }
  int rank = 0;
  if (valid) {
    const int below = __popcll(same & lt_mask);
    const int base = cnt[e];
    if (below == 0) cnt[e] = base + __popcll(same);
    rank = base + below;
  }
  return rank;
}

// wave_rank with the number of expert-id bits fixed at compile time: the
// ballot loop unrolls, so the ballots of independent chunks can interleave.
template <int BITS>
__device__ inline int wave_rank_c(bool valid, int e, uint64_t lt_mask, int* cnt) {
  uint64_t same = __ballot(valid);
#pragma unroll
  for (int b = 0; b < BITS; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const uint64_t bb = __ballot(bit);
    same &= bit ? bb : ~bb;
  }
  int rank = 0;
  if (valid) {
    const int below = __popcll(same & lt_mask);
    const int base = cnt[e];
    if (below == 0) cnt[e] = base + __popcll(same);
    rank = base + below;
  }
  return rank;
}

// Exclusive scan over the waves of each expert's wave counts (in place:
// wcnt[w][e] becomes wave w's base); tot[e] = the expert's total.
__device__ inline void wave_bases(int (*wcnt)[kMaxExperts], int* tot, int N, int tid) {
  if (tid < N) {
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = wcnt[w][tid];
      wcnt[w][tid] = run;
      run += c;
    }
    tot[tid] = run;
  }
}

// Inclusive scan of v[0..N) in LDS (N <= kMaxExperts) by the block's first
// wave, 4 entries per lane (a shuffle scan of the lane totals), then a block
// barrier: one barrier instead of two per doubling step.  Every thread calls
// it, after a barrier that completes v.
__device__ inline void block_scan(int* v, int N, int tid) {
  static_assert(kMaxExperts <= 4 * kWave, "entries per lane");
  if (tid < kWave) {
    int a[4], s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid * 4 + j;
      s += (i < N) ? v[i] : 0;
      a[j] = s;
    }
    int incl = s;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (tid >= off) incl += y;
    }
    const int base = incl - s;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid * 4 + j;
      if (i < N) v[i] = a[j] + base;
    }
  }
  __syncthreads();
}

// BITS >= 0: the expert-id bit count, fixed; -1: computed.  CH > 0: each
// wave keeps its at most CH chunks (ids and in-wave ranks) in registers from
// A to C instead of parking the ranks in slot and loading both again.
template <bool REROUTE, int BITS, int CH>
__global__ __launch_bounds__(kThreads) void dispatch_kernel(int32_t* idx, int64_t A, int64_t T, int k,
                                                            int by_choice, int N, int C, int S, int pad,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ slot,
                                                            int32_t* __restrict__ n_dropped, int R,
                                                            const int32_t* __restrict__ fb_idx,
                                                            const float* __restrict__ fb_gate, float* gate) {
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

  auto rank_of = [&](bool valid, int e) {
    if constexpr (BITS >= 0)
      return wave_rank_c<BITS>(valid, e, lt_mask, wcnt[wave]);
    else
      return wave_rank(valid, e, bits, lt_mask, wcnt[wave]);
  };
  int rev[CH > 0 ? CH : 1], rrk[CH > 0 ? CH : 1];  // register mode: ids, in-wave ranks

  // ---- A: in-wave ranks
  if constexpr (CH > 0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {  // every load in flight at once
      const int64_t i = a_begin + c * kWave + lane;
      rev[c] = (i < a_end) ? idx[flat_of(i, T, k, by_choice)] : -1;
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      rrk[c] = 0;
      if (a_begin + c * kWave < a_end) {  // wave-uniform
        const int64_t i = a_begin + c * kWave + lane;
        const int e = rev[c];
        rrk[c] = rank_of(i < a_end && e >= 0 && e < N, e);
      }
    }
  } else {
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
        const int rank = rank_of(valid, e);
        if (valid) slot[a] = rank;
      }
    }
  }
  __syncthreads();

  // ---- B: wave bases per expert, totals, capacity cut, offsets
  __shared__ int keep[kMaxExperts];
  wave_bases(wcnt, scan, N, tid);
  int kept = 0;
  if (tid < N) {
    const int run = scan[tid];
    counts[tid] = run;
    kept = (C >= 0 && run > C) ? C : run;
    scan[tid] = kept;
    keep[tid] = kept;
  }
  __syncthreads();
  block_scan(scan, N, tid);
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
  if constexpr (CH > 0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t i = a_begin + c * kWave + lane;
      if (i >= a_end) continue;
      const int64_t a = flat_of(i, T, k, by_choice);
      const int e = rev[c];
      if (e < 0 || e >= N) {
        slot[a] = -1;
        continue;
      }
      const int rank = wcnt[wave][e] + rrk[c];
      if (C < 0 || rank < C) {
        const int sr = off[e] + rank;
        slot[a] = sr;
        perm[sr] = (int32_t)a;
      } else {
        slot[a] = -1;
      }
    }
  }
  for (int64_t b0 = a_begin; b0 < (CH > 0 ? a_begin : a_end); b0 += kPrefetch * kWave) {
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
        if constexpr (!REROUTE) perm[s] = (int32_t)a;
      } else {
        slot[a] = -1;
      }
    }
  }
  if constexpr (REROUTE) {
    __shared__ int room[kMaxExperts], rer[kMaxExperts], tot[kMaxExperts], offf[kMaxExperts + 1];
    __syncthreads();  // every wave is done with C's wave bases (wcnt) and slot writes
    if (tid < N) {
      room[tid] = C >= 0 ? C - keep[tid] : 0;
      rer[tid] = 0;
    }
    // token segments of the waves, in whole 64-wide chunks
    const int64_t tchunks = (T + kWave - 1) / kWave;
    const int64_t tper = (tchunks + kWaves - 1) / kWaves;
    const int64_t t_begin = (int64_t)wave * tper * kWave;
    const int64_t t_end = (t_begin + tper * kWave < T) ? t_begin + tper * kWave : T;
    // scratch in the routed perm rows (T*k >= T entries, >= 2T when k >= 2),
    // rewritten by the final pass: in-wave ranks of the offers, and with
    // k >= 2 each token's mask of still-dropped choices (with k = 1 the slot
    // itself says whether the one choice is dropped)
    int32_t* parked = perm + (int64_t)S * T;
    int32_t* dmask = parked + T;
    if (k > 1) {
      for (int64_t t = tid; t < T; t += kThreads) {
        int m = 0;
        for (int j = 0; j < k; ++j) m |= (slot[t * k + j] == -1) ? (1 << j) : 0;
        dmask[t] = m;
      }
    }
    // the offers of a chunk group: lowest still-dropped choice jd[c] of token
    // t0 + c*64 + lane and its expert of rank k + r (-1: no offer); all loads
    // are issued before any is used
    auto offers = [&](int64_t t0, int r, int (&jd)[kPrefetch], int (&ev)[kPrefetch]) {
      int dv[kPrefetch], fv[kPrefetch];
#pragma unroll
      for (int c = 0; c < kPrefetch; ++c) {
        const int64_t t = t0 + c * kWave + lane;
        const int64_t tc = t < t_end ? t : t_begin;  // in range: t_begin < t_end here
        dv[c] = k > 1 ? dmask[tc] : (slot[tc] == -1 ? 1 : 0);
        fv[c] = fb_idx[tc * R + r];
      }
#pragma unroll
      for (int c = 0; c < kPrefetch; ++c) {
        const int64_t t = t0 + c * kWave + lane;
        const bool has = t < t_end && dv[c] != 0;
        jd[c] = has ? __builtin_ctz((unsigned)dv[c]) : -1;
        ev[c] = has ? fv[c] : -1;
      }
    };
    for (int r = 0; r < (C >= 0 ? R : 0); ++r) {
      for (int i = tid; i < kWaves * kMaxExperts; i += kThreads) (&wcnt[0][0])[i] = 0;
      __syncthreads();  // also orders the previous level's writes before these reads
      for (int64_t t0 = t_begin; t0 < t_end; t0 += kPrefetch * kWave) {
        int jd[kPrefetch], ev[kPrefetch];
        offers(t0, r, jd, ev);
#pragma unroll
        for (int c = 0; c < kPrefetch; ++c) {
          const int e = ev[c];
          const bool valid = e >= 0 && e < N;
          const int rank = wave_rank(valid, e, bits, lt_mask, wcnt[wave]);
          if (valid) parked[t0 + c * kWave + lane] = rank;
        }
      }
      __syncthreads();
      wave_bases(wcnt, tot, N, tid);
      __syncthreads();
      for (int64_t t0 = t_begin; t0 < t_end; t0 += kPrefetch * kWave) {
        int jd[kPrefetch], ev[kPrefetch], pv[kPrefetch];
        offers(t0, r, jd, ev);
#pragma unroll
        for (int c = 0; c < kPrefetch; ++c) {
          const int64_t t = t0 + c * kWave + lane;
          pv[c] = parked[t < t_end ? t : t_begin];
        }
#pragma unroll
        for (int c = 0; c < kPrefetch; ++c) {
          const int e = ev[c];
          if (e < 0 || e >= N) continue;
          const int64_t t = t0 + c * kWave + lane;
          const int rank = wcnt[wave][e] + pv[c];
          if (rank < room[e]) {
            const int64_t a = t * k + jd[c];
            slot[a] = -2 - (rer[e] + rank);
            idx[a] = e;
            gate[a] = fb_gate[t * R + r];
            if (k > 1) dmask[t] &= ~(1 << jd[c]);
          }
        }
      }
      __syncthreads();
      if (tid < N) {
        const int acc = tot[tid] < room[tid] ? tot[tid] : room[tid];
        rer[tid] += acc;
        room[tid] -= acc;
      }
    }
    __syncthreads();
    // final offsets: scan of kept + rerouted rows
    if (tid < N) scan[tid] = keep[tid] + rer[tid];
    __syncthreads();
    block_scan(scan, N, tid);
    if (tid < N) {
      const int o = ST + scan[tid] - (keep[tid] + rer[tid]);
      offf[tid] = o;
      offsets[S + tid] = o;
    }
    if (tid == 0) {
      const int total = N > 0 ? scan[N - 1] : 0;
      offsets[S + N] = ST + total;
      *n_dropped = (int32_t)(A - total);
    }
    __syncthreads();
    // final rows: kept ones keep their rank, rerouted ones follow
    for (int64_t a0 = tid; a0 < A; a0 += kPrefetch * kThreads) {
      int sv[kPrefetch], ev[kPrefetch];
#pragma unroll
      for (int c = 0; c < kPrefetch; ++c) {
        const int64_t a = a0 + c * kThreads;
        const int64_t ac = a < A ? a : a0;
        sv[c] = slot[ac];
        ev[c] = idx[ac];
      }
#pragma unroll
      for (int c = 0; c < kPrefetch; ++c) {
        const int64_t a = a0 + c * kThreads;
        const int e = ev[c];
        if (a >= A || sv[c] == -1 || e < 0 || e >= N) continue;
        const int row = sv[c] >= 0 ? offf[e] + (sv[c] - off[e]) : offf[e] + keep[e] + (-2 - sv[c]);
        slot[a] = row;
        perm[row] = (int32_t)a;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Dispatch over many workgroups (the same result as dispatch_kernel).  The
// priority order is cut into segments of kSeg assignments, one per
// workgroup of kSegWaves waves (each wave kSegChunks 64-wide chunks):
//  count: in-segment stable ranks with the ballot scheme (waves in order),
//         parked in slot; the segment's per-expert counts go to
//         bc[seg * N + e] (workspace).
//  place: every workgroup sums bc over the segments in increasing order:
//         its own per-expert base, the totals, the capacity cut and the
//         offsets; segment 0 writes counts, offsets and n_dropped, and the
//         shared rows and padding rows are filled grid-stride; then each
//         workgroup turns its parked ranks into slot and perm.
constexpr int kSegWaves = 4;
constexpr int kSegChunks = 4;
constexpr int kSeg = kSegWaves * kSegChunks * kWave;  // 1024

template <int BITS>
__global__ __launch_bounds__(kSegWaves * kWave) void dispatch_count_kernel(const int32_t* __restrict__ idx, int64_t A,
                                                                           int64_t T, int k, int by_choice, int N,
                                                                           int32_t* __restrict__ slot,
                                                                           int32_t* __restrict__ bc) {
  __shared__ int wcnt[kSegWaves][kMaxExperts];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  for (int i = tid; i < kSegWaves * kMaxExperts; i += kSegWaves * kWave) (&wcnt[0][0])[i] = 0;
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t w0 = (int64_t)blockIdx.x * kSeg + (int64_t)wave * kSegChunks * kWave;
  int ev[kSegChunks], rk[kSegChunks];
#pragma unroll
  for (int c = 0; c < kSegChunks; ++c) {
    const int64_t i = w0 + c * kWave + lane;
    ev[c] = (i < A) ? idx[flat_of(i, T, k, by_choice)] : -1;
  }
#pragma unroll
  for (int c = 0; c < kSegChunks; ++c) {
    const int64_t i = w0 + c * kWave + lane;
    const int e = ev[c];
    rk[c] = wave_rank_c<BITS>(i < A && e >= 0 && e < N, e, lt_mask, wcnt[wave]);
  }
  __syncthreads();
  // wave bases inside the segment, and the segment's counts
  if (tid < N) {
    int run = 0;
    for (int w = 0; w < kSegWaves; ++w) {
      const int c = wcnt[w][tid];
      wcnt[w][tid] = run;
      run += c;
    }
    bc[(int64_t)blockIdx.x * N + tid] = run;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kSegChunks; ++c) {
    const int64_t i = w0 + c * kWave + lane;
    const int e = ev[c];
    if (i < A && e >= 0 && e < N) slot[flat_of(i, T, k, by_choice)] = wcnt[wave][e] + rk[c];
  }
}

__global__ __launch_bounds__(kSegWaves * kWave) void dispatch_place_kernel(
    const int32_t* __restrict__ idx, int64_t A, int64_t T, int k, int by_choice, int N, int C, int S, int pad,
    const int32_t* __restrict__ bc, int nseg, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ slot, int32_t* __restrict__ n_dropped) {
  constexpr int kThr = kSegWaves * kWave;
  __shared__ int base[kMaxExperts], scan[kMaxExperts], off[kMaxExperts + 1];
  const int tid = threadIdx.x;
  const int seg = blockIdx.x;
  // per expert: this segment's base and the total, summed in segment order
  for (int e = tid; e < N; e += kThr) {
    int run = 0, mine = 0;
    for (int g0 = 0; g0 < nseg; g0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = bc[(int64_t)(g0 + u < nseg ? g0 + u : 0) * N + e];  // all in flight
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (g0 + u < nseg) {
          if (g0 + u == seg) mine = run;
          run += v[u];
        }
      }
    }
    base[e] = mine;
    scan[e] = (C >= 0 && run > C) ? C : run;  // kept
    if (seg == 0) counts[e] = run;
  }
  __syncthreads();
  // offsets: exclusive scan of the kept counts (compact) or e*C (padded)
  block_scan(scan, N, tid);
  const int ST = S * (int)T;
  for (int e = tid; e < N; e += kThr) {
    const int kept = scan[e] - (e > 0 ? scan[e - 1] : 0);
    const int o = ST + (pad ? e * C : scan[e] - kept);
    off[e] = o;
    if (seg == 0) offsets[S + e] = o;
  }
  if (seg == 0) {
    if (tid < S) offsets[tid] = tid * (int)T;
    if (tid == 0) {
      const int total = N > 0 ? scan[N - 1] : 0;
      offsets[S + N] = ST + (pad ? N * C : total);
      *n_dropped = (int32_t)(A - total);
    }
  }
  // shared rows and padding rows, grid-stride over all workgroups
  const int64_t gthreads = (int64_t)gridDim.x * kThr;
  for (int64_t r = (int64_t)seg * kThr + tid; r < (int64_t)ST; r += gthreads) perm[r] = (int32_t)((r % T) * k);
  if (pad) {
    for (int64_t i = (int64_t)seg * kThr + tid; i < (int64_t)N * C; i += gthreads) {
      const int e = (int)(i / C), r = (int)(i - (int64_t)e * C);
      const int kept_e = scan[e] - (e > 0 ? scan[e - 1] : 0);
      if (r >= kept_e) perm[ST + i] = 0;
    }
  }
  __syncthreads();
  // place this segment
  const int64_t s0 = (int64_t)seg * kSeg;
#pragma unroll 4
  for (int c = 0; c < kSeg / kThr; ++c) {
    const int64_t i = s0 + c * kThr + tid;
    if (i >= A) continue;
    const int64_t a = flat_of(i, T, k, by_choice);
    const int e = idx[a];
    if (e < 0 || e >= N) {
      slot[a] = -1;
      continue;
    }
    const int rank = base[e] + slot[a];
    if (C < 0 || rank < C) {
      const int sr = off[e] + rank;
      slot[a] = sr;
      perm[sr] = (int32_t)a;
    } else {
      slot[a] = -1;
    }
  }
}

}  // namespace

hipError_t launch_dispatch(const moe_shape& s, const int32_t* idx, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* slot, int32_t* n_dropped,
                           hipStream_t st) {
  const int64_t A = s.T * (int64_t)s.k;
  const int by_choice = (s.flags & MOE_SLOT_MAJOR) && s.k > 1;
  // the plain dispatch never writes idx
  int32_t* idx_rw = const_cast<int32_t*>(idx);
  const int pad = (s.flags & MOE_PADDED) ? 1 : 0;
  int bits = 0;
  while ((1 << bits) < s.N) ++bits;
  const int64_t per = ((A + kWave - 1) / kWave + kWaves - 1) / kWaves;  // chunks per wave
#define MOE_DISPATCH(BITS, CH)                                                                                    \
  hipLaunchKernelGGL((dispatch_kernel<false, BITS, CH>), dim3(1), dim3(kThreads), 0, st, idx_rw, A, s.T, s.k,     \
                     by_choice, s.N, s.capacity, s.n_shared, pad, counts, offsets, perm, slot, n_dropped, 0, nullptr, \
                     nullptr, nullptr)
#define MOE_DISPATCH_BITS(CH)        \
  switch (bits) {                     \
    case 0: MOE_DISPATCH(0, CH); break; \
    case 1: MOE_DISPATCH(1, CH); break; \
    case 2: MOE_DISPATCH(2, CH); break; \
    case 3: MOE_DISPATCH(3, CH); break; \
    case 4: MOE_DISPATCH(4, CH); break; \
    case 5: MOE_DISPATCH(5, CH); break; \
    case 6: MOE_DISPATCH(6, CH); break; \
    case 7: MOE_DISPATCH(7, CH); break; \
    default: MOE_DISPATCH(8, CH); break; \
  }
  // The register mode's chunk loops are unrolled, so the code grows with CH
  // (about 65 KB at 24 chunks).  A launch that follows the expert GEMMs finds
  // its code evicted from every cache, and fetching it took most of a small
  // batch's dispatch (20 us of 6 for 768 assignments): small batches take the
  // smallest register mode that holds them.
  if (per <= 1) {
    MOE_DISPATCH_BITS(1)
  } else if (per <= 4) {
    MOE_DISPATCH_BITS(4)
  } else if (per <= kRegChunks) {
    MOE_DISPATCH_BITS(kRegChunks)
  } else {
    MOE_DISPATCH(-1, 0);
  }
#undef MOE_DISPATCH_BITS
#undef MOE_DISPATCH
  return hipGetLastError();
}

size_t dispatch_ws_bytes(const moe_shape& s) {
  const int64_t A = s.T * (int64_t)s.k;
  return (size_t)((A + kSeg - 1) / kSeg) * (size_t)s.N * sizeof(int32_t);
}

hipError_t launch_dispatch_multi(const moe_shape& s, const int32_t* idx, int32_t* counts, int32_t* offsets,
                                 int32_t* perm, int32_t* slot, int32_t* n_dropped, int32_t* bc, hipStream_t st) {
  const int64_t A = s.T * (int64_t)s.k;
  const int by_choice = (s.flags & MOE_SLOT_MAJOR) && s.k > 1;
  const int pad = (s.flags & MOE_PADDED) ? 1 : 0;
  const int nseg = (int)((A + kSeg - 1) / kSeg);
  int bits = 0;
  while ((1 << bits) < s.N) ++bits;
#define MOE_COUNT(BITS)                                                                                      \
  hipLaunchKernelGGL((dispatch_count_kernel<BITS>), dim3(nseg), dim3(kSegWaves * kWave), 0, st, idx, A, s.T, \
                     s.k, by_choice, s.N, slot, bc)
  switch (bits) {
    case 0: MOE_COUNT(0); break;
    case 1: MOE_COUNT(1); break;
    case 2: MOE_COUNT(2); break;
    case 3: MOE_COUNT(3); break;
    case 4: MOE_COUNT(4); break;
    case 5: MOE_COUNT(5); break;
    case 6: MOE_COUNT(6); break;
    case 7: MOE_COUNT(7); break;
    default: MOE_COUNT(8); break;
  }
#undef MOE_COUNT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dispatch_place_kernel, dim3(nseg), dim3(kSegWaves * kWave), 0, st, idx, A, s.T, s.k, by_choice,
                     s.N, s.capacity, s.n_shared, pad, bc, nseg, counts, offsets, perm, slot, n_dropped);
  return hipGetLastError();
}

hipError_t launch_dispatch_reroute(const moe_shape& s, int R, const int32_t* fb_idx, const float* fb_gate,
                                   int32_t* idx, float* gate, int32_t* counts, int32_t* offsets, int32_t* perm,
                                   int32_t* slot, int32_t* n_dropped, hipStream_t st) {
  const int64_t A = s.T * (int64_t)s.k;
  const int by_choice = (s.flags & MOE_SLOT_MAJOR) && s.k > 1;
  hipLaunchKernelGGL((dispatch_kernel<true, -1, 0>), dim3(1), dim3(kThreads), 0, st, idx, A, s.T, s.k, by_choice, s.N,
                     s.capacity, s.n_shared, 0, counts, offsets, perm, slot, n_dropped, R, fb_idx, fb_gate, gate);
  return hipGetLastError();
}

}  // namespace moe
