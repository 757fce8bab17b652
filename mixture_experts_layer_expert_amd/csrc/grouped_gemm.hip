// Grouped GEMM of the expert MLPs on bf16 MFMA (gfx950).
//
// For every expert e and every row r of its group [offsets[e], offsets[e+1]):
//   C[r, n] = act( sum_k A[row(r), k] * B[e, n, k] + bias[e, n] )
// with row(r) = perm[r] / topk for fc1 (rows of x are gathered on load) and
// row(r) = r for fc2 (rows of the hidden activations).  SwiGLU fuses the
// w1 and w3 products of the same output columns into one tile and writes
// silu(gate) * up.
//
// Work decomposition.  The work list enumerates (expert, row tile, column
// tile) for all experts at once.  A column tile of fc1 is a column shard of
// W1 (and W3); a column tile of fc2 is a column shard of W2^T, i.e. the fc2
// tiles of a row tile cover every output column while each reads one row
// shard of W2^T per k step -- the single-GPU share of the row/column
// decomposition of expert matrices in "Accelerating MoE Model Inference with
// Expert Sharding" (abstract).  Every tile costs the same, so a hot expert
// simply contributes more tiles and the list stays balanced whatever the
// routing skew.  One persistent launch covers the whole list (the pieces of
// all experts fused into one kernel, same abstract).
//
// Scheduling.  Grid = one persistent workgroup per CU, a multiple of 8.
// Workgroups are dealt to the 8 XCDs round-robin by id, so XCD x = id % 8 is
// given a contiguous block of the full rounds' tiles; its workgroups stride
// through it.  Tiles that are adjacent in the list share a weight or row
// panel (row tiles in groups of 8 within an expert), so they meet in the same
// XCD's L2.  A partial last round is dealt round-robin over the XCDs and,
// given a workspace, cut along K (the split, finished by a second launch).
//
// Tile shapes (rows x weight rows, waves): 256x256 (8 waves), 128x256 (8),
// 128x384 (8, down projection only) and 32x256 (4), picked from the rows per
// expert.  Tile pipeline: K is consumed 64 at a time (a "job" is one k step of
// one tile).  Both operand tiles go global -> LDS with
// global_load_lds_dwordx4 (no register staging) into a ring of as many
// stages as fit (2 to 4), fed as one continuous stream of jobs, so the next
// tile's first k steps load while the current tile finishes; a
// wave-instruction fills 1 KiB = 8 rows x 128 B.  Fragments are read from
// LDS one k sub-step ahead of the MFMAs.  Inside a row the eight 16-byte
// chunks are XOR-swizzled by the row index so that the MFMA fragment reads
// (ds_read_b128, one row per lane) are conflict-free.  MFMA
// v_mfma_f32_32x32x16_bf16 with the weight tile as the first operand: each
// lane then owns 4 consecutive output columns of one row; lanes l and l+32
// swap halves so that the epilogue stores 16 bytes per lane.
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {


// Chunk swizzle.  The LDS serves a 64-lane ds_read_b128 16 lanes at a time
// from 64 four-byte banks (256 bytes).  A tile row of CPR 16-byte chunks
// covers CPR*16 bytes, so 256/(CPR*16) consecutive rows share a chunk
// permutation and fall into distinct bank ranges; XOR-ing the chunk index
// with (row / that) makes 16 consecutive rows hit 16 distinct 16-byte bank
// groups.  128-byte rows (BK=64): (row>>1)&7; 64-byte rows (BK=32): (row>>2)&3.
template <int CPR>
__device__ inline int swz(int row) {
  if constexpr (CPR == 16) return row & 15;  // 256-byte rows (BK=128)
  return CPR == 8 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Word 3 of a raw buffer resource: DATA_FORMAT = 32 bits (4 in bits 15-18),
// which untyped loads need non-zero.  Loads at offsets past num_records
// return zeros.
constexpr int kBufferWord3 = 0x00020000;

// HBM -> LDS copy of 16 bytes per lane through a buffer resource
// (buffer_load_dwordx4 ... lds): lane l's bytes at voff + soff land at LDS
// address l + 16 * lane.  The buffer form, unlike global_load_lds, leaves the
// MFMA issue of the SIMD's other wave nearly undisturbed: with one wave per
// SIMD streaming operands and one running MFMAs, the MFMA pipe stays about
// 93% busy with buffer loads against about 62% with global loads (probe on
// gfx950; GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES counters).
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, lds_ptr_t l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, l, 16, voff, soff, 0, 0);
}

// GELU in its erf form, z * Phi(z) with Phi the standard normal CDF, without
// transcendental instructions (the epilogue of short-K tiles is bound by
// them): Phi(z) = 0.5 + z * P(z^2) for |z| <= 4, P of degree 8.  P is a
// least-squares Chebyshev fit of (Phi(sqrt(u)) - 0.5) / sqrt(u) on u in
// [0, 16] (fit_gelu_poly.py in this folder derives it).  Beyond |z| = 4 the
// polynomial is evaluated at u = 16 and the result clamped to [0, 1]: P(16)
// is about 1/8, so 0.5 + z * P(16) leaves [0, 1] by |z| = 4.001, and in
// between it stays within the fit's error of Phi.  The clamp is the free
// output modifier of the last FMA, so there is no branch or select.  The fp32
// evaluation is within 3.2e-5 of Phi everywhere (the largest error is the
// tail beyond |z| = 4), so GELU is within 1.3e-4 absolute, below the bf16
// rounding of the hidden activations it produces.
__device__ inline float gelu_erf(float z) {
  const float u = fminf(z * z, 16.f);
  float p = 9.408924819e-11f;
  p = fmaf(p, u, -7.887303300e-09f);
  p = fmaf(p, u, 2.954978125e-07f);
  p = fmaf(p, u, -6.637191087e-06f);
  p = fmaf(p, u, 1.017005944e-04f);
  p = fmaf(p, u, -1.146868260e-03f);
  p = fmaf(p, u, 9.909445771e-03f);
  p = fmaf(p, u, -6.644644696e-02f);
  p = fmaf(p, u, 3.989348236e-01f);
  return z * __builtin_amdgcn_fmed3f(fmaf(z, p, 0.5f), 0.f, 1.f);
}

template <int BM, int BNB, int WM, int WN, int BK_>
struct Tile {
  static constexpr int BK = BK_;            // k elements per stage
  static constexpr int CPR = BK / 8;        // 16-byte chunks per tile row
  static constexpr int RPI = 64 / CPR;      // tile rows per dma instruction (1 KiB)
  static constexpr int NW = WM * WN;        // waves per workgroup
  static constexpr int THREADS = NW * kWave;
  static constexpr int TM = BM / WM;        // tokens per wave
  static constexpr int TN = BNB / WN;       // weight rows per wave
  static constexpr int FM = TM / 32;        // 32-token MFMA tiles per wave
  static constexpr int FN = TN / 32;        // 32-row MFMA tiles per wave
  static constexpr int QA = BM / (RPI * NW);  // A dma instructions per wave per stage
  static constexpr int QB = BNB / (RPI * NW); // B dma instructions per wave per stage
  static constexpr int kLdsA = BM * BK;     // bf16 elements per stage
  static constexpr int kLdsB = BNB * BK;
  static constexpr int kStageBytes = (kLdsA + kLdsB) * 2;
  // as many stages (2..8) as fit in 150 KiB (room for the work list)
  static constexpr int kFit = (150 * 1024) / kStageBytes;
  static constexpr int kStages = kFit > 8 ? 8 : (kFit < 2 ? 2 : kFit);
  static constexpr size_t kLdsBytes = (size_t)kStages * kStageBytes;
  static_assert(BK == 32 || BK == 64 || BK == 128, "BK 32, 64 or 128");
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile multiple of 32");
  static_assert(QA >= 1 && QB >= 1 && QA * RPI * NW == BM && QB * RPI * NW == BNB, "dma split");
};

struct Params {
  const bf16* A;
  uint32_t a_bytes;  // bytes addressable in A (the buffer resource's range)
  const int32_t* perm;
  int topk;
  const int32_t* offsets;
  int n_experts;
  const bf16* B;
  const bf16* B2;
  const bf16* bias;
  bf16* C;
  int K;
  int n_out;   // output columns of C (F for fc1, D for fc2)
  int act;
  float* part; // split-K partial tiles of the last round, or nullptr: never split
};

// Waits until at most `younger` jobs' worth of DMA instructions (NJ per job)
// are outstanding (younger is clamped to K).  Loads return in issue order,
// so this means every older job has landed in LDS.  Epilogue stores issued
// after a job only make the wait stricter.
template <int NJ, int K>
__device__ inline void wait_dma(int younger) {
  if constexpr (K > 0) {
    if (younger >= K) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K * NJ) : "memory");
      return;
    }
    wait_dma<NJ, K - 1>(younger);
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// Block barrier for the stage ring.  __syncthreads() carries a workgroup
// fence, for which the compiler drains every outstanding vector memory op
// (vmcnt(0)) -- that would also wait for the DMA of jobs still meant to be
// in flight.  Here the caller has already waited for the DMA it needs; this
// only completes the wave's own LDS reads (so no refill can overtake them)
// and synchronises.  The "memory" clobber keeps the compiler from moving
// LDS accesses across it.
__device__ inline void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Persistent grid of the grouped GEMM: one workgroup per CU, a multiple of 8
// (the XCD count) so that every XCD gets the same number of workgroups.
inline int gemm_grid() {
  const int g = device_cu_count();
  return (g + 7) / 8 * 8;
}

__device__ inline float fast_silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + __expf(-z));
}

// ---- work list (shared by the GEMM and its split-K finishing kernel)
//
// Tiles per expert: ceil(rows / BM) row tiles x ceil(n_out / BN_OUT)
// column tiles, numbered expert by expert, row tile fastest.  With G
// persistent workgroups the first rounds*G tiles are full rounds: XCD x
// (= workgroup id % 8) gets the contiguous block of rounds*(G/8) tiles and its
// workgroups stride through it.  The R = total - rounds*G tiles left over
// (dealt round-robin over the XCDs) would keep only R workgroups busy in a
// last, partial round; when a
// workspace for partial sums is given they are instead cut into S = G / R
// chunks along K (S <= KT), one chunk per workgroup; chunks write fp32
// partial tiles and a second kernel sums them in chunk order and applies the
// epilogue.  Every workgroup then gets the same number of jobs to within one
// chunk.
struct TileInfo {
  int e, row0, row_end, n0;
};

constexpr int kMaxSplit = 8;  // K chunks per left-over tile at most

template <int BM, int BN_OUT>
struct WorkList {
  int total, rounds, R, S;

  // Prefix sum of the tiles of each expert into tile_start[0..N]; called by
  // every thread of the block (nthreads >= 64 threads, N <= 256 experts).
  // The expert offsets are copied to off[0..N] (LDS) on the way: the tile
  // lookups inside the pipelined loop then never wait for global memory.
  __device__ void build(const Params& p, int* tile_start, int* scan, int* off, int tid, int nthreads) {
    constexpr int kPer = kMaxExperts / 64;  // experts per thread at 64 threads
    const int N = p.n_experts;
    const int ntiles = (p.n_out + BN_OUT - 1) / BN_OUT;
    int my[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + u * nthreads;
      my[u] = 0;
      if (e < N) {
        const int o0 = p.offsets[e], o1 = p.offsets[e + 1];
        my[u] = ((o1 - o0 + BM - 1) / BM) * ntiles;
        scan[e] = my[u];
        off[e] = o0;
        if (e == N - 1) off[N] = o1;
      }
    }
    __syncthreads();
    // inclusive scan of scan[0..N) by the first wave, kPer entries per lane
    // (a shuffle scan of the lane totals): one barrier instead of two per
    // doubling step, before the first tile's loads can be issued
    if (tid < 64) {
      int a[kPer], sum = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int e = tid * kPer + j;
        sum += (e < N) ? scan[e] : 0;
        a[j] = sum;
      }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (tid >= o) incl += y;
      }
      const int base = incl - sum;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int e = tid * kPer + j;
        if (e < N) scan[e] = a[j] + base;
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + u * nthreads;
      if (e < N) tile_start[e] = scan[e] - my[u];
    }
    if (tid == 0) tile_start[N] = (N > 0) ? scan[N - 1] : 0;
    __syncthreads();
    total = __builtin_amdgcn_readfirstlane(tile_start[N]);
  }

  __device__ void split(int G, int KT, bool can_split) {
    rounds = total / G;
    R = total - rounds * G;
    int s = 1;
    if (can_split && R > 0) {
      s = G / R;
      if (s > KT) s = KT;
      // more chunks shorten the last round less and less, while the partial
      // traffic and the finishing work keep growing
      if (s > kMaxSplit) s = kMaxSplit;
      if (s < 1) s = 1;
    }
    // block-uniform: keep them in scalar registers
    rounds = __builtin_amdgcn_readfirstlane(rounds);
    R = __builtin_amdgcn_readfirstlane(R);
    S = __builtin_amdgcn_readfirstlane(s);
  }

  __device__ TileInfo info(const Params& p, const int* tile_start, const int* off, int L) const {
    const int N = p.n_experts;
    int lo = 0, hi = N - 1;  // expert of tile L: last e with tile_start[e] <= L
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_start[mid] <= L) lo = mid; else hi = mid - 1;
    }
    TileInfo t;
    t.e = lo;
    const int row_begin = off[lo];
    const int rows_e = off[lo + 1] - row_begin;
    const int mtiles = (rows_e + BM - 1) / BM;
    const int local = L - tile_start[lo];
    // Within an expert the tiles go in groups of kGroupM row tiles: a group's
    // row tiles for output columns 0, 1, ... in turn.  An XCD takes a
    // contiguous run of tiles per round, so a run covers at most kGroupM row
    // panels and a few column panels that its L2 shares, instead of every row
    // panel of one column.  Experts with at most kGroupM row tiles keep the
    // plain row-fastest order.
    constexpr int kGroupM = 8;
    const int ntiles = (p.n_out + BN_OUT - 1) / BN_OUT;
    const int g = local / (kGroupM * ntiles);
    const int gm0 = g * kGroupM;
    const int gsize = (mtiles - gm0 < kGroupM) ? mtiles - gm0 : kGroupM;
    const int r = local - g * kGroupM * ntiles;
    t.row0 = row_begin + (gm0 + r % gsize) * BM;
    t.row_end = row_begin + rows_e;
    t.n0 = (r / gsize) * BN_OUT;
    return t;
  }
};

// Stores one 32-feature block of a token row held by lanes l and l+32: lane
// l has features {0-3, 8-11, 16-19, 24-27}, lane l+32 {4-7, 12-15, 20-23,
// 28-31}, as packed bf16 pairs d[q][0..1] (features 8q + 4h + 0..3, h =
// lane / 32).  One cross-half shuffle per dword gives lane l features 16t..
// 16t+7 and lane l+32 features 16t+8..16t+15 (t = 0, 1), so each store is
// 16 bytes per lane and 32 bytes per row.
__device__ inline void store_block32(bf16* crow, int fbase, bool ok, const uint32_t (&d)[4][2], int lane) {
  const bool lower = lane < 32;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint32_t s0 = lower ? d[2 * t + 1][0] : d[2 * t][0];
    const uint32_t s1 = lower ? d[2 * t + 1][1] : d[2 * t][1];
    const uint32_t r0 = (uint32_t)__shfl_xor((int)s0, 32);
    const uint32_t r1 = (uint32_t)__shfl_xor((int)s1, 32);
    uint32_t w[4];
    if (lower) {
      w[0] = d[2 * t][0]; w[1] = d[2 * t][1]; w[2] = r0; w[3] = r1;
    } else {
      w[0] = r0; w[1] = r1; w[2] = d[2 * t + 1][0]; w[3] = d[2 * t + 1][1];
    }
    const int f = fbase + 16 * t + (lower ? 0 : 8);
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    if (ok) *(u32x4*)(crow + f) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  // one round-to-nearest-even conversion of both values
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2_t));
}

// Epilogue of one unit of a wave's share of an output tile: the 32 tokens of
// MFMA block j and 32 output columns, from accumulator a0 (the w1 product
// and a1 the w3 product under SwiGLU; unit u then pairs 32-row groups 2u and
// 2u + 1 of the weight tile, otherwise unit u is group u).  A lane owns token
// column (lane & 31) and output rows (r/4)*8 + (lane/32)*4 + r%4 of the 32x32
// block; rows of one token are gathered into 16-byte stores by store_block32.
// BIAS: add the bias, read from global memory (the split-K finishing kernel;
// the pipelined kernel starts its accumulators at the bias instead).
template <int BM, int BNB, int WM, int WN, int BK, int ACT, bool BIAS>
__device__ inline void store_unit(const Params& p, const TileInfo& tc, const f32x16& a0, const f32x16& a1,
                                  int wm, int wn, int j, int u, int lane) {
  using TL = Tile<BM, BNB, WM, WN, BK>;
  const int h4 = (lane >> 5) * 4;
  const int r_out = tc.row0 + wm * TL::TM + j * 32 + (lane & 31);
  const bool live = r_out < tc.row_end;
  bf16* crow = p.C + (size_t)r_out * p.n_out;
  uint32_t d[4][2];
  int fbase;
  if constexpr (ACT == kActSwiGLU) {
    fbase = tc.n0 + (wn * TL::TN / 64 + u) * 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = fast_silu(a0[q * 4 + t]) * a1[q * 4 + t];
      d[q][0] = pack_bf16x2(v[0], v[1]);
      d[q][1] = pack_bf16x2(v[2], v[3]);
    }
  } else {
    fbase = tc.n0 + wn * TL::TN + u * 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int f = fbase + q * 8 + h4;
      bf16x4 bv = {};
      if constexpr (BIAS)
        if (f < p.n_out) bv = *(const bf16x4*)(p.bias + (size_t)tc.e * p.n_out + f);
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float z = a0[q * 4 + t];
        if constexpr (BIAS) z += (float)bv[t];
        if constexpr (ACT == kActGelu) z = gelu_erf(z);
        if constexpr (ACT == kActRelu) z = fmaxf(z, 0.f);
        v[t] = z;
      }
      d[q][0] = pack_bf16x2(v[0], v[1]);
      d[q][1] = pack_bf16x2(v[2], v[3]);
    }
  }
  store_block32(crow, fbase, live && fbase < p.n_out, d, lane);
}

// Epilogue of a wave's whole share of an output tile (acc: its 32x32
// sub-tiles, weight rows x tokens), unit by unit, for a wave holding FMX
// 32-token blocks, the first of which is block jbase of the tile (with the
// asymmetric split of the token blocks, jbase and FMX differ by wave).  The
// accumulators already hold any bias.
template <int BM, int BNB, int WM, int WN, int BK, int ACT, int FMX>
__device__ inline void store_tile_x(const Params& p, const TileInfo& tc,
                                    f32x16 (&acc)[Tile<BM, BNB, WM, WN, BK>::FN][FMX], int jbase, int wn, int lane) {
  using TL = Tile<BM, BNB, WM, WN, BK>;
  constexpr int PAIR = (ACT == kActSwiGLU) ? 2 : 1;
#pragma unroll
  for (int j = 0; j < FMX; ++j) {
#pragma unroll
    for (int u = 0; u < TL::FN / PAIR; ++u) {
      // wm = 0 with block index jbase + j: the row is row0 + (jbase + j) * 32
      store_unit<BM, BNB, WM, WN, BK, ACT, false>(p, tc, acc[u * PAIR][j], acc[u * PAIR + PAIR - 1][j], 0, wn,
                                                 jbase + j, u, lane);
      __builtin_amdgcn_sched_barrier(0);  // keep accumulator reads chunked
    }
  }
}

// Partial tile q of the split last round: element (wave, i, j, r, lane) of
// the accumulators at a fixed position, so that stores and loads are whole
// 256-byte wave rows.
template <int FN, int FM>
__device__ inline float* part_ptr(const Params& p, int q, int nw, int wave, int lane) {
  return p.part + ((size_t)q * nw + wave) * (FN * FM * 16 * 64) + lane;
}

// Header of the split-K workspace, after the room for G partial tiles:
// [0] = R (left-over tiles), [1] = S (chunks per tile; 1: nothing split),
// then from int 4 on, (expert, first row, end row, first column) of each
// left-over tile.  Written by workgroup 0 of the GEMM, read by the
// finishing kernel, which then needs no work list of its own.
template <int BM, int BNB>
__device__ inline int* split_header(const Params& p, int G) {
  return (int*)(p.part + (size_t)G * BM * BNB);
}
typedef int i32x4 __attribute__((ext_vector_type(4)));

// DW: the waves that issue the operand DMA (all NW, or NW/2 = one per SIMD).
// FMD: 0, or the 32-token MFMA blocks of a DMA wave when the two waves of a
// SIMD split the tile's 2 * FM blocks unevenly (DW = NW/2, WM = 2).
// A wave that issues a job's DMA stalls at issue while the texture unit takes
// the CU's burst of 1 KiB instructions (about 20 cycles each); with one DMA
// wave per SIMD the other wave keeps the MFMA pipe busy meanwhile.
template <int BM, int BNB, int WM, int WN, int BK, int ACT, bool BIAS, int STAGES, int DW, int FMD>
__global__ __launch_bounds__(WM * WN * 64, 1) void grouped_gemm_kernel(Params p) {
  // one row tile per group: each weight panel is streamed by a single tile
  using TL = Tile<BM, BNB, WM, WN, BK>;
  constexpr int CPR = TL::CPR, RPI = TL::RPI;
  constexpr bool kSwiGLU = (ACT == kActSwiGLU);
  constexpr int BN_OUT = kSwiGLU ? BNB / 2 : BNB;  // output columns per tile
  static_assert(DW == TL::NW || DW * 2 == TL::NW, "all waves or half of them issue the DMA");
  constexpr int QA = BM / (RPI * DW);  // A dma instructions per DMA wave per stage
  constexpr int QB = BNB / (RPI * DW); // B dma instructions per DMA wave per stage
  static_assert(QA >= 1 && QB >= 1 && QA * RPI * DW == BM && QB * RPI * DW == BNB, "dma split");
  constexpr int NJ = QA + QB;          // dma instructions per job per DMA wave
  static_assert(STAGES >= 2 && STAGES <= 8, "2..8 stages");
  static_assert((STAGES - 1) * NJ <= 63, "vmcnt range");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16* sA = (bf16*)smem_raw;                       // [STAGES][BM][BK]
  bf16* sB = sA + STAGES * TL::kLdsA;               // [STAGES][BNB][BK]
  __shared__ int s_tile_start[kMaxExperts + 1];
  __shared__ int s_scan[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  // per wave, two slots of the perm entries of its A rows (fc1 gather): the
  // next tile's are brought in by DMA while the current tile is loading
  constexpr int kRowsPerWave = QA * RPI;
  static_assert(kRowsPerWave <= 64, "one dword DMA per wave");
  __shared__ int s_perm[TL::NW][2][64];
  // per wave, a ring of the bias values of its TN columns of a tile: filled by
  // DMA when the tile's loads start, read when the tile's accumulators are
  // initialised.  The DMA side is at most STAGES jobs (so STAGES tiles)
  // ahead, hence STAGES + 1 slots.
  constexpr int kBiasSlots = BIAS ? STAGES + 1 : 1;
  static_assert(!BIAS || TL::TN <= 128, "bias slice of at most 128 columns per wave");
  __shared__ uint32_t s_bias[BIAS ? TL::NW : 1][kBiasSlots][64];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  const int lane = tid % kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int KT = p.K / BK;
  const bool dma_wave = wave < DW;  // wave-uniform

  WorkList<BM, BN_OUT> wl;
  wl.build(p, s_tile_start, s_scan, s_off, tid, TL::THREADS);
  const int G = gridDim.x;  // multiple of 8
  wl.split(G, KT, p.part != nullptr);
  if (p.part && blockIdx.x == 0) {
    // for the finishing kernel (issued before any DMA: an older store only
    // makes the ring's waits stricter)
    int* hdr = split_header<BM, BNB>(p, G);
    if (tid == 0) {
      hdr[0] = wl.R;
      hdr[1] = wl.S;
    }
    if (wl.S > 1)
      for (int r = tid; r < wl.R; r += TL::THREADS) {
        const TileInfo t = wl.info(p, s_tile_start, s_off, wl.rounds * G + r);
        *(i32x4*)(hdr + 4 + 4 * r) = i32x4{t.e, t.row0, t.row_end, t.n0};
      }
  }

  // ---- this workgroup's tiles: `rounds` full ones, then at most one more
  // (a whole left-over tile, or one K chunk of one)
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8, per_xcd = G / 8;
  const int full_base = xcd * wl.rounds * per_xcd + slot;
  // index among the left-over work items: dealt round-robin over the XCDs so
  // that a short last round still spreads over every XCD's memory path
  const int q_rem = slot * 8 + xcd;
  const bool has_rem = q_rem < wl.R * wl.S;
  const int n_mine = wl.rounds + (has_rem ? 1 : 0);
  const int L_rem = __builtin_amdgcn_readfirstlane(wl.rounds * G + q_rem / wl.S);
  const int c_rem = __builtin_amdgcn_readfirstlane(q_rem % wl.S);
  const int k0_rem = __builtin_amdgcn_readfirstlane(c_rem * KT / wl.S);
  const int k1_rem = __builtin_amdgcn_readfirstlane((c_rem + 1) * KT / wl.S);
  auto tile_L = [&](int i) { return i < wl.rounds ? full_base + i * per_xcd : L_rem; };
  auto tile_k0 = [&](int i) { return i < wl.rounds ? 0 : k0_rem; };
  auto tile_k1 = [&](int i) { return i < wl.rounds ? KT : k1_rem; };

  const int lrow = lane / CPR;    // row within the dma instruction's rows
  const int lchunk = lane % CPR;  // physical chunk this lane fills

  // ---- DMA side: per-lane 32-bit byte offsets of the tile being loaded,
  // added to wave-uniform base pointers (saddr + voffset addressing).
  uint32_t offA[QA], offB[QB];
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc((void*)p.A, 0, p.a_bytes, kBufferWord3);
  const uint32_t b_bytes = (uint32_t)p.n_out * (uint32_t)p.K * 2u;  // one expert's weight matrix
  __amdgpu_buffer_rsrc_t rsB1 = __builtin_amdgcn_make_buffer_rsrc((void*)p.B, 0, b_bytes, kBufferWord3);
  __amdgpu_buffer_rsrc_t rsB2 = rsB1;
  // kt_dma counts the k steps of the tile being loaded from its first one
  // (k0_dma) to its end (k1_dma); the step loaded is k0_dma + (kt_dma -
  // k0_dma + rot_dma) mod (k1_dma - k0_dma).  Operand rows lie K*2 bytes
  // apart, and with every workgroup at the same k offset the requests of a
  // 4 KiB or 8 KiB row stride fall on few HBM channels (the decode layer's up
  // projection, K = 2048, streamed 4.5 TB/s against 5.1 TB/s at other
  // strides).  rot_dma therefore rotates the k order: per workgroup for
  // 32-row tiles, whose weight panel no other tile reads; per XCD for larger
  // tiles, which share panels through their XCD's L2, so that the readers of
  // a panel stay in step while the XCDs start at different offsets.
  int i_dma = 0, kt_dma = 0, k0_dma = 0, k1_dma = 0, rot_dma = 0, job_issued = 0;
  // perm DMA for tile i into slot i & 1: lane l fetches the entry of tile
  // row wave*kRowsPerWave + l (clamped to the tile's last row, so always a
  // valid entry); only the first kRowsPerWave lanes' values are used.
  auto fetch_perm = [&](int i) __attribute__((always_inline)) {
    if (!p.perm || i >= n_mine || !dma_wave) return;
    const TileInfo t = wl.info(p, s_tile_start, s_off, tile_L(i));
    int r = t.row0 + wave * kRowsPerWave + (lane < kRowsPerWave ? lane : 0);
    if (r > t.row_end - 1) r = t.row_end - 1;
    __builtin_amdgcn_global_load_lds(p.perm + r, (lds_ptr_t)&s_perm[wave][i & 1][0], 4, 0, 0);
  };
  int jobs_since_fetch = 0;  // DMA jobs issued after the last perm fetch
  auto setup_dma = [&](int i) __attribute__((always_inline)) {
    const TileInfo t = wl.info(p, s_tile_start, s_off, tile_L(i));
    if (p.perm && dma_wave) {
      // the fetch for tile i is older than every job issued since: wait for
      // it to land (in steady state an earlier wait already covered it)
      wait_dma<NJ, STAGES - 1>(jobs_since_fetch);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int trow = (wave * QA + q) * RPI + lrow;  // row within the A tile (DMA waves)
      int src = t.row0 + trow;
      if (src > t.row_end - 1) src = t.row_end - 1;  // tail rows re-load a valid row
      if (p.perm && dma_wave) src = s_perm[wave][i & 1][q * RPI + lrow] / p.topk;
      offA[q] = ((uint32_t)src * (uint32_t)p.K + (uint32_t)((lchunk ^ swz<CPR>(trow)) * 8)) * 2u;
    }
    fetch_perm(i + 1);
    jobs_since_fetch = 0;
    if constexpr (BIAS) {
      // lane l fetches dword min(l, TN/2 - 1) of the wave's slice (two
      // columns); a column past n_out (a ragged last tile) is clamped to the
      // last valid dword, so the address stays valid and is never stored
      int col = t.n0 + wn * TL::TN + 2 * (lane < TL::TN / 2 ? lane : TL::TN / 2 - 1);
      if (col > p.n_out - 2) col = p.n_out - 2;
      const uint32_t* src = (const uint32_t*)(p.bias + (size_t)t.e * p.n_out + col);
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)&s_bias[wave][i % kBiasSlots][0], 4, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int brow = (wave * QB + q) * RPI + lrow;  // row within the B tile (DMA waves)
      int feat = kSwiGLU ? t.n0 + (brow / 64) * 32 + (brow % 32) : t.n0 + brow;
      if (feat > p.n_out - 1) feat = p.n_out - 1;  // column tail
      offB[q] = ((uint32_t)feat * (uint32_t)p.K + (uint32_t)((lchunk ^ swz<CPR>(brow)) * 8)) * 2u;
    }
    const size_t eoff = (size_t)t.e * p.n_out * p.K * 2;
    rsB1 = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)p.B + eoff), 0, b_bytes, kBufferWord3);
    rsB2 = kSwiGLU ? __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)p.B2 + eoff), 0, b_bytes, kBufferWord3)
                   : rsB1;
    kt_dma = tile_k0(i);
    k0_dma = kt_dma;
    k1_dma = tile_k1(i);
    if constexpr (BM <= 32)
      rot_dma = __builtin_amdgcn_readfirstlane((int)((blockIdx.x * 7u + (uint32_t)i * 3u) % (uint32_t)(k1_dma - k0_dma)));
    else  // workgroup b runs on XCD b % 8
      rot_dma = __builtin_amdgcn_readfirstlane((int)(((blockIdx.x & 7u) * (uint32_t)(k1_dma - k0_dma)) / 8u));
  };
  auto issue_next = [&]() __attribute__((always_inline)) {
    if (i_dma >= n_mine) return;
    const int stage = job_issued % STAGES;
    bf16* a_dst = sA + stage * TL::kLdsA;
    bf16* b_dst = sB + stage * TL::kLdsB;
    int kt = kt_dma + rot_dma;
    if (kt >= k1_dma) kt -= k1_dma - k0_dma;
    const uint32_t kbytes = (uint32_t)kt * BK * 2;
    if (dma_wave) {
#pragma unroll
      for (int q = 0; q < QA; ++q)
        dma16(rsA, offA[q], kbytes, (lds_ptr_t)(a_dst + (wave * QA + q) * 512));
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        // SwiGLU: 32-row groups alternate w1 (even) and w3 (odd)
        const bool w3 = kSwiGLU && ((((wave * QB + q) * RPI) / 32) & 1);
        dma16(w3 ? rsB2 : rsB1, offB[q], kbytes, (lds_ptr_t)(b_dst + (wave * QB + q) * 512));
      }
    }
    ++job_issued;
    ++jobs_since_fetch;
    if (++kt_dma == k1_dma) {
      if (++i_dma < n_mine) setup_dma(i_dma);
    }
  };

  // Prologue: fill every stage.  At the barrier of job j the stage of job j
  // is refilled with job j + STAGES, and job j + 1 must already be in flight.
  if (n_mine > 0) {
    fetch_perm(0);
    setup_dma(0);
  }
#pragma unroll
  for (int s = 0; s < STAGES; ++s) issue_next();

  // ---- compute side: one flat loop over the jobs (tile, k step) of this
  // workgroup.  Per job, 4 k sub-steps of 16; fragments are read one
  // sub-step ahead into a second register buffer.  The block barrier sits
  // before the last sub-step: by then every wave has read all fragments of
  // the job, so the stage can be refilled, and the first fragments of the
  // next job are read while the last sub-step's MFMAs run.
  constexpr int KS = BK / 16;
  const int n_jobs = wl.rounds * KT + (has_rem ? k1_rem - k0_rem : 0);
  // Token blocks of this wave: FM 32-token blocks from wm * FM, or with an
  // asymmetric split (FMD > 0) FMD blocks for the DMA wave of a SIMD and the
  // rest of the 2 * FM blocks for the other wave, so that the wave that also
  // issues the operand DMA has fewer MFMAs to issue.
  constexpr int FM_DMA = FMD > 0 ? FMD : TL::FM;
  constexpr int FM_OTHER = FMD > 0 ? 2 * TL::FM - FMD : TL::FM;
  static_assert(FMD == 0 || (WM == 2 && DW * 2 == TL::NW && FMD >= 1 && FMD < 2 * TL::FM), "asymmetric split");
  const int jbase = FMD > 0 ? (dma_wave ? 0 : FMD) : wm * TL::FM;
  auto run = [&](auto fm_tag) __attribute__((always_inline)) {
    constexpr int FMX = decltype(fm_tag)::value;
    bf16x8 bf[2][TL::FN], af[2][FMX];
    auto load_frags = [&](int stage, int ks, int buf) __attribute__((always_inline)) {
      const bf16* a_s = sA + stage * TL::kLdsA;
      const bf16* b_s = sB + stage * TL::kLdsB;
      const int c = 2 * ks + (lane >> 5);
#pragma unroll
      for (int i = 0; i < TL::FN; ++i) {
        const int row = wn * TL::TN + i * 32 + (lane & 31);
        bf[buf][i] = *(const bf16x8*)(b_s + row * BK + ((c ^ swz<CPR>(row)) * 8));
      }
#pragma unroll
      for (int j = 0; j < FMX; ++j) {
        const int row = (jbase + j) * 32 + (lane & 31);
        af[buf][j] = *(const bf16x8*)(a_s + row * BK + ((c ^ swz<CPR>(row)) * 8));
      }
    };
    f32x16 acc[TL::FN][FMX];
    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < TL::FN; ++i)
#pragma unroll
        for (int j = 0; j < FMX; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    };
    // With a bias, a whole tile's accumulators start at its bias values, so
    // the epilogue adds none: row r of a lane's 32-row block is feature
    // (r/4)*8 + (lane/32)*4 + r%4, the same for every token block.  A K chunk
    // of a split tile starts at zero; its finishing kernel adds the bias once.
    // The tile's bias slice has landed by then: DMA waves waited for the
    // tile's first job, which was issued after it, and the other waves wait
    // for all their loads.
    auto init_acc = [&](int i) __attribute__((always_inline)) {
      if constexpr (BIAS) {
        if (i < wl.rounds || wl.S == 1) {
          const bf16* bl = (const bf16*)&s_bias[wave][i % kBiasSlots][0];
          const int h4 = (lane >> 5) * 4;
#pragma unroll
          for (int fi = 0; fi < TL::FN; ++fi)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const bf16x4 bv = *(const bf16x4*)(bl + fi * 32 + q * 8 + h4);
#pragma unroll
              for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int j = 0; j < FMX; ++j) acc[fi][j][q * 4 + t] = (float)bv[t];
            }
          return;
        }
      }
      zero_acc();
    };
    auto mfmas = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < TL::FN; ++i)
#pragma unroll
        for (int j = 0; j < FMX; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[buf][i], af[buf][j], acc[i][j], 0, 0, 0);
    };
    // interleave: one fragment read per (FN*FM)/(FN+FM) MFMAs
    auto interleave = [&]() __attribute__((always_inline)) {
      constexpr int NR = TL::FN + FMX, NM = TL::FN * FMX;
      constexpr int PER = NM / NR > 0 ? NM / NR : 1;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // 1 DS read
        __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // PER MFMAs
      }
    };

    int i_cmp = 0, kt_cmp = 0, len_cmp = 0;
    TileInfo tc;
    if (n_jobs > 0) {
      tc = wl.info(p, s_tile_start, s_off, tile_L(0));
      len_cmp = tile_k1(0) - tile_k0(0);
      if (dma_wave) wait_dma<NJ, STAGES - 1>(job_issued - 1);
      if (BIAS && !dma_wave) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      ring_barrier();
      load_frags(0, 0, 0);
      init_acc(0);
    } else {
      zero_acc();
    }
    for (int job = 0; job < n_jobs; ++job) {
      const int stage = job % STAGES;
#pragma unroll
      for (int ks = 0; ks < KS - 1; ++ks) {
        load_frags(stage, ks + 1, (ks + 1) & 1);
        mfmas(ks & 1);
        interleave();
      }
      // all fragments of this job are in registers: refill its stage later
      const bool more = job + 1 < n_jobs;
      if (dma_wave) wait_dma<NJ, STAGES - 1>(job_issued - (job + 1) - 1);
      ring_barrier();
      issue_next();
      if (more) load_frags((job + 1) % STAGES, 0, KS & 1);
      mfmas((KS - 1) & 1);
      if (more) interleave();
      // a finished tile goes through the epilogue, except a K chunk of a split
      // left-over tile (always this workgroup's last): its partial sums are
      // stored after the loop
      if (++kt_cmp == len_cmp && more) {
        // A wave without tile DMA waits here for the next tile's bias slice,
        // which it fetched when the DMA side moved on to that tile, STAGES
        // jobs ago; waiting before the epilogue leaves its stores in flight.
        if (BIAS && !dma_wave) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        store_tile_x<BM, BNB, WM, WN, BK, ACT, FMX>(p, tc, acc, jbase, wn, lane);
        kt_cmp = 0;
        ++i_cmp;
        tc = wl.info(p, s_tile_start, s_off, tile_L(i_cmp));
        len_cmp = tile_k1(i_cmp) - tile_k0(i_cmp);
        init_acc(i_cmp);
      }
    }
    if (n_jobs > 0) {
      if (!has_rem || wl.S == 1) {
        store_tile_x<BM, BNB, WM, WN, BK, ACT, FMX>(p, tc, acc, jbase, wn, lane);
      } else {
        // in the symmetric layout the finishing kernel reads: block g of the
        // tile's 32-token blocks belongs to wave (g / FM) * WN + wn, slot g % FM
#pragma unroll
        for (int i = 0; i < TL::FN; ++i)
#pragma unroll
          for (int j = 0; j < FMX; ++j) {
            const int g = jbase + j;
            float* d = part_ptr<TL::FN, TL::FM>(p, q_rem, TL::NW, (g / TL::FM) * WN + wn, lane) +
                       (i * TL::FM + g % TL::FM) * 1024;
#pragma unroll
            for (int r = 0; r < 16; ++r) d[r * 64] = acc[i][j][r];
          }
      }
    }
  };
  if constexpr (FMD > 0) {
    if (dma_wave) run(std::integral_constant<int, FM_DMA>{});
    else run(std::integral_constant<int, FM_OTHER>{});
  } else {
    run(std::integral_constant<int, TL::FM>{});
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Second half of the split last round: tile r of the R left-over tiles is
// the sum of its S partial tiles, in chunk order (deterministic), followed by
// the epilogue.  One wave per block; block (x, w, unit) finishes one epilogue
// unit (32 tokens x 32 columns, two accumulator blocks under SwiGLU) of wave
// w's share of tiles x, x + gridDim.x, ..., with the lane layout of the GEMM,
// so a lane reads back exactly the accumulator elements it would have held.
// The chunks' loads go out in batches of kBatch.  R, S and the tiles come
// from the header the GEMM wrote.  G: the GEMM's grid.
template <int BM, int BNB, int WM, int WN, int BK, int ACT, bool BIAS>
__global__ __launch_bounds__(64) void splitk_finish_kernel(Params p, int G) {
  using TL = Tile<BM, BNB, WM, WN, BK>;
  constexpr int PAIR = (ACT == kActSwiGLU) ? 2 : 1;
  constexpr int UPJ = TL::FN / PAIR;  // epilogue units per 32-token block
  constexpr int kBatch = 4;
  const int* hdr = split_header<BM, BNB>(p, G);
  const int R = hdr[0], S = hdr[1];
  if (S <= 1) return;
  const int lane = threadIdx.x;
  const int wave = blockIdx.y;
  const int wm = wave / WN, wn = wave % WN;
  const int j = blockIdx.z / UPJ, u = blockIdx.z % UPJ;
  for (int r = blockIdx.x; r < R; r += gridDim.x) {
    const i32x4 ti = *(const i32x4*)(hdr + 4 + 4 * r);
    const TileInfo tc{ti[0], ti[1], ti[2], ti[3]};
    f32x16 acc[PAIR];
#pragma unroll
    for (int pr = 0; pr < PAIR; ++pr)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[pr][e] = 0.f;
    for (int c0 = 0; c0 < S; c0 += kBatch) {
      f32x16 v[kBatch][PAIR];
#pragma unroll
      for (int b = 0; b < kBatch; ++b)
        if (c0 + b < S)
#pragma unroll
          for (int pr = 0; pr < PAIR; ++pr) {
            const float* src = part_ptr<TL::FN, TL::FM>(p, r * S + c0 + b, TL::NW, wave, lane) +
                               ((u * PAIR + pr) * TL::FM + j) * 1024;
#pragma unroll
            for (int e = 0; e < 16; ++e) v[b][pr][e] = src[e * 64];
          }
      __builtin_amdgcn_sched_barrier(0);  // the batch's loads in flight together
#pragma unroll
      for (int b = 0; b < kBatch; ++b)
        if (c0 + b < S)
#pragma unroll
          for (int pr = 0; pr < PAIR; ++pr) acc[pr] += v[b][pr];
    }
    store_unit<BM, BNB, WM, WN, BK, ACT, BIAS>(p, tc, acc[0], acc[PAIR - 1], wm, wn, j, u, lane);
  }
}

template <int BM, int BNB, int WM, int WN, int BK, int ACT, bool BIAS, int DW, int FMD>
hipError_t launch_cfg(const Params& p, hipStream_t st) {
  using TL = Tile<BM, BNB, WM, WN, BK>;
  constexpr int S = TL::kStages;
  auto kern = grouped_gemm_kernel<BM, BNB, WM, WN, BK, ACT, BIAS, S, DW, FMD>;
  // once per process and instantiation (thread-safe static initialisation)
  static const hipError_t attr_err = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)TL::kLdsBytes);
  if (attr_err != hipSuccess) return attr_err;
  const int grid = gemm_grid();
  hipLaunchKernelGGL(kern, dim3(grid), dim3(TL::THREADS), TL::kLdsBytes, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !p.part) return e;
  // at most grid/2 left-over tiles are ever split (S >= 2), two per block
  // along x; one wave per block
  constexpr int kUnits = TL::FM * (TL::FN / ((ACT == kActSwiGLU) ? 2 : 1));
  hipLaunchKernelGGL((splitk_finish_kernel<BM, BNB, WM, WN, BK, ACT, BIAS>), dim3(grid / 4, TL::NW, kUnits),
                     dim3(64), 0, st, p, grid);
  return hipGetLastError();
}

template <int BM, int BNB, int WM, int WN, int BK, int DW, int FMD = 0>
hipError_t launch_act(const Params& p, hipStream_t st) {
  const bool bias = p.bias != nullptr;
  switch (p.act) {
    case kActGelu:
      return bias ? launch_cfg<BM, BNB, WM, WN, BK, kActGelu, true, DW, FMD>(p, st)
                  : launch_cfg<BM, BNB, WM, WN, BK, kActGelu, false, DW, FMD>(p, st);
    case kActRelu:
      return bias ? launch_cfg<BM, BNB, WM, WN, BK, kActRelu, true, DW, FMD>(p, st)
                  : launch_cfg<BM, BNB, WM, WN, BK, kActRelu, false, DW, FMD>(p, st);
    case kActSwiGLU:
      // the SwiGLU epilogue pairs each wave's w1 and w3 32-row groups
      if constexpr ((BNB / WN / 32) % 2 == 0) return launch_cfg<BM, BNB, WM, WN, BK, kActSwiGLU, false, DW, FMD>(p, st);
      else return hipErrorInvalidValue;
    default:
      return bias ? launch_cfg<BM, BNB, WM, WN, BK, kActNone, true, DW, FMD>(p, st)
                  : launch_cfg<BM, BNB, WM, WN, BK, kActNone, false, DW, FMD>(p, st);
  }
}

}  // namespace

namespace {

// The instantiated tile shapes (BM x BNB, waves, BK).
enum TileCfg { k256x256w8k64, k128x256w8k64, k128x384w8k64, k32x256w4k64, k256x256w8d4, k128x256w8d4,
               k128x384w8d4, k32x256w4k128, k32x128w4k128, k256x256w8a3, kNumCfg };
const char* const kCfgName[] = {"256x256w8k64", "128x256w8k64", "128x384w8k64", "32x256w4k64",
                                "256x256w8d4", "128x256w8d4", "128x384w8d4", "32x256w4k128",
                                "32x128w4k128", "256x256w8a3"};
const int kCfgBM[] = {256, 128, 128, 32, 256, 128, 128, 32, 32, 256};
const int kCfgBN[] = {256, 256, 384, 256, 256, 256, 384, 256, 128, 256};
const int kCfgBK[] = {64, 64, 64, 64, 64, 64, 64, 128, 128, 64};
static_assert(sizeof(kCfgName) / sizeof(kCfgName[0]) == kNumCfg && sizeof(kCfgBM) / sizeof(int) == kNumCfg &&
                  sizeof(kCfgBN) / sizeof(int) == kNumCfg && sizeof(kCfgBK) / sizeof(int) == kNumCfg,
              "one entry per tile shape");

// Tile choice from the mean rows per expert: large groups use 256x256
// tiles (8 waves of 128x64), mid-size groups 128x256 (8 waves of 64x64) --
// or 128x384 (8 waves of 64x96) for the down projection when no group can
// exceed 128 rows (max_rows, from the capacity) -- and small ones 32x256 (4
// waves of 32x64).  Output columns per tile: BN (BN/2
// for SwiGLU, which needs an even number of 32-row groups per wave, so never
// 128x384).  The wider down tile reads each row of the hidden activations
// for 384 output columns instead of 256: the A operand (L2 hits, for the
// most part) is a quarter of the bytes each stage brings in instead of a
// third.  Those hits share each CU's load path with the weight stream: a
// weight stage alone streams at about 6.2 TB/s, with a third of its bytes
// from L2 at about 4.9.  A group of more than 128 rows would need a second,
// mostly empty row tile that reads the wider weight panels again, which
// costs more than the narrower tile (measured).  MOE_GEMM_TILE (tuning) forces one of the
// instantiated shapes for both projections, MOE_GEMM_TILE_UP /
// MOE_GEMM_TILE_DOWN for one.
TileCfg choose_cfg(int64_t expected_rows, int64_t max_rows, bool up, int K) {
  static const char* forced_all = getenv("MOE_GEMM_TILE");
  static const char* forced_up = getenv("MOE_GEMM_TILE_UP");
  static const char* forced_down = getenv("MOE_GEMM_TILE_DOWN");
  const char* forced = up ? (forced_up ? forced_up : forced_all) : (forced_down ? forced_down : forced_all);
  if (forced)
    for (int c = 0; c < kNumCfg; ++c)
      if (!strcmp(forced, kCfgName[c])) return (TileCfg)c;
  // 256x256 up projections split the token blocks 3:5 between the DMA wave
  // and the other wave of each SIMD (Mixtral fc1 3261 -> 3067 us, the
  // shared-expert layer's 420 -> 408 us, the skewed layer's even); the down
  // projections measured slower that way (1685 -> 1822 us, 166 -> 199 us)
  if (expected_rows >= 192) return up ? k256x256w8a3 : k256x256w8d4;
  if (expected_rows >= 48) return (up || max_rows > 128) ? k128x256w8d4 : k128x384w8d4;
  // weight streaming: the up projection's 256-byte row pieces (BK = 128)
  // stream faster than 128-byte ones (decode layer, K = 2048: 146.6 ->
  // 140.6 us); the down projection measured the same either way
  return (up && K % 128 == 0) ? k32x256w4k128 : k32x256w4k64;
}

// Whether to let the kernel split its last round (which costs a second
// launch): only when the expected work is a few rounds of large tiles, where
// a partial last round idles a sizeable share of the GPU.  The estimate uses
// the mean rows per expert; a wrong guess costs time, never correctness
// (without p.part the kernel never splits).  When no group can exceed one
// row tile, the estimate is the most tiles there can be: a whole number of
// rounds then leaves nothing over when every expert is used, and the second
// launch would only find nothing to do.
bool allow_split(TileCfg c, const GroupedGemm& g, int64_t expected_rows, int64_t max_rows) {
  if (kCfgBM[c] < 64) return false;
  const int bn_out = g.act == kActSwiGLU ? kCfgBN[c] / 2 : kCfgBN[c];
  const int64_t est = (int64_t)g.n_experts * ((expected_rows + kCfgBM[c] - 1) / kCfgBM[c]) *
                      ((g.n_out + bn_out - 1) / bn_out);
  const int64_t G = gemm_grid();
  if (max_rows <= kCfgBM[c] && est % G == 0) return false;
  return est < 6 * G;
}

}  // namespace

size_t grouped_gemm_bf16_part_bytes(int64_t expected_rows, int64_t max_rows) {
  // (K only picks between tiles of the same shape)
  const TileCfg u = choose_cfg(expected_rows, max_rows, true, 64), d = choose_cfg(expected_rows, max_rows, false, 64);
  const int a = kCfgBM[u] * kCfgBN[u], b = kCfgBM[d] * kCfgBN[d];
  const size_t G = (size_t)gemm_grid();
  return G * (size_t)(a > b ? a : b) * sizeof(float) + 16 * (G + 1);  // partial tiles + header
}

hipError_t launch_grouped_gemm_bf16(const GroupedGemm& g, int64_t expected_rows, int64_t max_rows,
                                    hipStream_t st) {
  Params p;
  p.A = (const bf16*)g.A;
  p.a_bytes = (uint32_t)(g.a_rows * g.K * 2);
  p.perm = g.perm;
  p.topk = g.topk;
  p.offsets = g.offsets;
  p.n_experts = g.n_experts;
  p.B = (const bf16*)g.B;
  p.B2 = (const bf16*)g.B2;
  p.bias = (const bf16*)g.bias;
  p.C = (bf16*)g.C;
  p.K = g.K;
  p.n_out = g.n_out;
  p.act = g.act;
  TileCfg cfg = choose_cfg(expected_rows, max_rows, g.perm != nullptr, g.K);
  if (g.K % (kCfgBK[cfg]) != 0) cfg = k32x256w4k64;  // a forced BK=128 shape on a K it does not divide
  p.part = (g.part && allow_split(cfg, g, expected_rows, max_rows)) ? g.part : nullptr;
  switch (cfg) {
    case k256x256w8k64: return launch_act<256, 256, 2, 4, 64, 8>(p, st);
    case k128x256w8k64: return launch_act<128, 256, 2, 4, 64, 8>(p, st);
    case k128x384w8k64: return launch_act<128, 384, 2, 4, 64, 8>(p, st);
    case k256x256w8d4: return launch_act<256, 256, 2, 4, 64, 4>(p, st);
    case k256x256w8a3: return launch_act<256, 256, 2, 4, 64, 4, 3>(p, st);
    case k128x256w8d4: return launch_act<128, 256, 2, 4, 64, 4>(p, st);
    case k128x384w8d4: return launch_act<128, 384, 2, 4, 64, 4>(p, st);
    case k32x256w4k128: return launch_act<32, 256, 1, 4, 128, 4>(p, st);
    case k32x128w4k128: return launch_act<32, 128, 1, 4, 128, 4>(p, st);
    default: return launch_act<32, 256, 1, 4, 64, 4>(p, st);
  }
}

}  // namespace moe
