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
// Scheduling.  Grid = a multiple of 8 persistent workgroups.  Workgroups are
// dealt to the 8 XCDs round-robin by id, so XCD x = id % 8 is given the
// contiguous eighth [x*P, (x+1)*P) of the list; its workgroups stride through
// it.  Tiles that are adjacent in the list share a weight panel (row tile
// varies fastest), so they meet in the same XCD's L2.
//
// Tile pipeline.  4 waves.  K is consumed 64 at a time.  Both operand tiles
// go global -> LDS with global_load_lds_dwordx4 (no register staging), into
// a 2-stage ring; a wave-instruction fills 1 KiB = 8 rows x 128 B.  Inside a
// row the eight 16-byte chunks are XOR-swizzled by the row index so that the
// MFMA fragment reads (ds_read_b128, one row per lane) are conflict-free.
// MFMA v_mfma_f32_32x32x16_bf16 with the weight tile as the first operand:
// each lane then owns 4 consecutive output columns of one row, which the
// epilogue stores as 8-byte chunks.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BK = 64;         // k elements per stage (128 bytes per row)
constexpr int kThreads = 256;  // 4 waves
constexpr int kStages = 2;

__device__ inline int swz(int row) { return row & 7; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ inline void dma16(const void* g, lds_ptr_t l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

__device__ inline float gelu_erf(float z) { return 0.5f * z * (1.f + erff(z * 0.70710678118654752f)); }
__device__ inline float silu(float z) { return z / (1.f + expf(-z)); }

template <int BM, int BNB, int WM, int WN>
struct Tile {
  static constexpr int TM = BM / WM;    // tokens per wave
  static constexpr int TN = BNB / WN;   // weight rows per wave
  static constexpr int FM = TM / 32;    // 32-token MFMA tiles per wave
  static constexpr int FN = TN / 32;    // 32-row MFMA tiles per wave
  static constexpr int QA = BM / 32;    // A dma instructions per wave per stage
  static constexpr int QB = BNB / 32;   // B dma instructions per wave per stage
  static constexpr int kLdsA = BM * BK;   // bf16 elements per stage
  static constexpr int kLdsB = BNB * BK;
  static constexpr size_t kLdsBytes = (size_t)kStages * (kLdsA + kLdsB) * 2;
  static_assert(WM * WN == 4, "4 waves");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile multiple of 32");
};

struct Params {
  const bf16* A;
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
};

template <int BM, int BNB, int WM, int WN, int ACT>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(Params p) {
  using TL = Tile<BM, BNB, WM, WN>;
  constexpr bool kSwiGLU = (ACT == kActSwiGLU);
  constexpr int BN_OUT = kSwiGLU ? BNB / 2 : BNB;  // output columns per tile

  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16* sA = (bf16*)smem_raw;                       // [kStages][BM][BK]
  bf16* sB = sA + kStages * TL::kLdsA;              // [kStages][BNB][BK]
  __shared__ int s_tile_start[kMaxExperts + 1];
  __shared__ int s_scan[kMaxExperts];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int N = p.n_experts;
  const int ntiles = (p.n_out + BN_OUT - 1) / BN_OUT;

  // ---- work list: tiles per expert and their prefix sum
  int my_tiles = 0;
  if (tid < N) {
    int rows = p.offsets[tid + 1] - p.offsets[tid];
    my_tiles = ((rows + BM - 1) / BM) * ntiles;
    s_scan[tid] = my_tiles;
  }
  __syncthreads();
  for (int d = 1; d < kMaxExperts; d <<= 1) {
    int v = 0;
    if (tid < N && tid >= d) v = s_scan[tid - d];
    __syncthreads();
    if (tid < N && tid >= d) s_scan[tid] += v;
    __syncthreads();
  }
  if (tid < N) s_tile_start[tid] = s_scan[tid] - my_tiles;
  if (tid == 0) s_tile_start[N] = (N > 0) ? s_scan[N - 1] : 0;
  __syncthreads();
  const int total = s_tile_start[N];

  // ---- XCD-aware assignment of the list
  const int G = gridDim.x;  // multiple of 8
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8, per_xcd = G / 8;
  const int span = (total + 7) / 8;
  const int L_begin = xcd * span + slot;
  const int L_end = min(total, (xcd + 1) * span);

  const int KT = p.K / BK;
  const int lrow = lane / 8;   // row within an 8-row dma group
  const int lchunk = lane % 8; // physical chunk this lane fills

  for (int L = L_begin; L < L_end; L += per_xcd) {
    // expert of tile L: last e with tile_start[e] <= L
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (s_tile_start[mid] <= L) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int row_begin = p.offsets[e];
    const int rows_e = p.offsets[e + 1] - row_begin;
    const int mtiles = (rows_e + BM - 1) / BM;
    const int local = L - s_tile_start[e];
    const int mt = local % mtiles;
    const int nt = local / mtiles;
    const int row0 = row_begin + mt * BM;
    const int row_end = row_begin + rows_e;
    const int n0 = nt * BN_OUT;  // first output column of the tile

    // ---- per-lane source offsets (elements) of the rows this lane loads
    uint32_t offA[TL::QA];
#pragma unroll
    for (int q = 0; q < TL::QA; ++q) {
      const int trow = (wave * TL::QA + q) * 8 + lrow;  // row within the A tile
      int r = row0 + trow;
      if (r > row_end - 1) r = row_end - 1;  // tail rows re-load a valid row
      const int src = p.perm ? (p.perm[r] / p.topk) : r;
      const int c = lchunk ^ swz(trow);
      offA[q] = (uint32_t)src * (uint32_t)p.K + (uint32_t)(c * 8);
    }
    uint32_t offB[TL::QB];
    const bf16* baseB[TL::QB];
#pragma unroll
    for (int q = 0; q < TL::QB; ++q) {
      const int brow = (wave * TL::QB + q) * 8 + lrow;  // row within the B tile
      int feat;
      const bf16* base;
      if constexpr (kSwiGLU) {
        const int g = brow / 32;
        feat = n0 + (g / 2) * 32 + (brow % 32);
        base = (g & 1) ? p.B2 : p.B;
        if (feat > p.n_out - 1) feat = p.n_out - 1;  // column tail
      } else {
        feat = n0 + brow;
        base = p.B;
        if (feat > p.n_out - 1) feat = p.n_out - 1;  // column tail
      }
      const int c = lchunk ^ swz(brow);
      baseB[q] = base + (size_t)e * p.n_out * p.K;
      offB[q] = (uint32_t)feat * (uint32_t)p.K + (uint32_t)(c * 8);
    }

    auto issue = [&](int stage, int kt) {
      bf16* a_dst = sA + stage * TL::kLdsA;
      bf16* b_dst = sB + stage * TL::kLdsB;
      const uint32_t koff = (uint32_t)kt * BK;
#pragma unroll
      for (int q = 0; q < TL::QA; ++q)
        dma16(p.A + offA[q] + koff, (lds_ptr_t)(a_dst + (wave * TL::QA + q) * 512));
#pragma unroll
      for (int q = 0; q < TL::QB; ++q)
        dma16(baseB[q] + offB[q] + koff, (lds_ptr_t)(b_dst + (wave * TL::QB + q) * 512));
    };

    f32x16 acc[TL::FN][TL::FM];
#pragma unroll
    for (int i = 0; i < TL::FN; ++i)
#pragma unroll
      for (int j = 0; j < TL::FM; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    issue(0, 0);
    for (int kt = 0; kt < KT; ++kt) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (kt + 1 < KT) issue((kt + 1) % kStages, kt + 1);
      const bf16* a_s = sA + (kt % kStages) * TL::kLdsA;
      const bf16* b_s = sB + (kt % kStages) * TL::kLdsB;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int c = 2 * ks + (lane >> 5);
        bf16x8 bf[TL::FN], af[TL::FM];
#pragma unroll
        for (int i = 0; i < TL::FN; ++i) {
          const int row = wn * TL::TN + i * 32 + (lane & 31);
          bf[i] = *(const bf16x8*)(b_s + row * BK + ((c ^ swz(row)) * 8));
        }
#pragma unroll
        for (int j = 0; j < TL::FM; ++j) {
          const int row = wm * TL::TM + j * 32 + (lane & 31);
          af[j] = *(const bf16x8*)(a_s + row * BK + ((c ^ swz(row)) * 8));
        }
#pragma unroll
        for (int i = 0; i < TL::FN; ++i)
#pragma unroll
          for (int j = 0; j < TL::FM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[i], af[j], acc[i][j], 0, 0, 0);
      }
    }

    // ---- epilogue: lane owns token column (lane & 31) of each 32x32 tile and
    // output rows (r/4)*8 + (lane/32)*4 + r%4 of it.
#pragma unroll
    for (int j = 0; j < TL::FM; ++j) {
      const int r_out = row0 + wm * TL::TM + j * 32 + (lane & 31);
      const bool live = r_out < row_end;
      bf16* crow = p.C + (size_t)r_out * p.n_out;
      if constexpr (kSwiGLU) {
#pragma unroll
        for (int ip = 0; ip < TL::FN / 2; ++ip) {
          const int fbase = n0 + (wn * TL::TN / 64 + ip) * 32;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int f = fbase + q * 8 + (lane >> 5) * 4;
            bf16x4 v;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float g = acc[2 * ip][j][q * 4 + u];
              const float up = acc[2 * ip + 1][j][q * 4 + u];
              v[u] = (bf16)(silu(g) * up);
            }
            if (live && f < p.n_out) *(bf16x4*)(crow + f) = v;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < TL::FN; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int f = n0 + wn * TL::TN + i * 32 + q * 8 + (lane >> 5) * 4;
            bf16x4 v;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              float z = acc[i][j][q * 4 + u];
              if (p.bias && f < p.n_out) z += (float)p.bias[(size_t)e * p.n_out + f + u];
              if constexpr (ACT == kActGelu) z = gelu_erf(z);
              if constexpr (ACT == kActRelu) z = fmaxf(z, 0.f);
              v[u] = (bf16)z;
            }
            if (live && f < p.n_out) *(bf16x4*)(crow + f) = v;
          }
        }
      }
    }
    __syncthreads();  // LDS ring is refilled by the next tile
  }
}

template <int BM, int BNB, int WM, int WN, int ACT>
hipError_t launch_cfg(const Params& p, hipStream_t st) {
  using TL = Tile<BM, BNB, WM, WN>;
  auto kern = grouped_gemm_kernel<BM, BNB, WM, WN, ACT>;
  // once per process and instantiation (thread-safe static initialisation)
  static const hipError_t attr_err = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)TL::kLdsBytes);
  if (attr_err != hipSuccess) return attr_err;
  int grid = device_cu_count();
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), TL::kLdsBytes, st, p);
  return hipGetLastError();
}

template <int BM, int BNB, int WM, int WN>
hipError_t launch_act(const Params& p, hipStream_t st) {
  switch (p.act) {
    case kActGelu: return launch_cfg<BM, BNB, WM, WN, kActGelu>(p, st);
    case kActRelu: return launch_cfg<BM, BNB, WM, WN, kActRelu>(p, st);
    case kActSwiGLU: return launch_cfg<BM, BNB, WM, WN, kActSwiGLU>(p, st);
    default: return launch_cfg<BM, BNB, WM, WN, kActNone>(p, st);
  }
}

}  // namespace

hipError_t launch_grouped_gemm_bf16(const GroupedGemm& g, int64_t expected_rows, hipStream_t st) {
  Params p;
  p.A = (const bf16*)g.A;
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
  // Tile choice from the mean rows per expert: large groups use 256x256
  // tiles (4 waves of 128x128), mid-size groups 128-row tiles, small ones
  // 32-row tiles.  Output columns per tile: 256 (128 for SwiGLU).
  if (expected_rows >= 192) return launch_act<256, 256, 2, 2>(p, st);
  if (expected_rows >= 48) return launch_act<128, 256, 1, 4>(p, st);
  return launch_act<32, 256, 1, 4>(p, st);
}

}  // namespace moe
