// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace layout, and the stream-ordered launch sequence
//   route -> dispatch -> fc1(+act) -> fc2 -> combine.
// No allocation, no synchronisation, no state beyond a per-device CU count.
#include <atomic>
#include <cmath>
#include <limits>

#include "moe_internal.h"

namespace moe {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline size_t elem_size(const moe_shape& s) { return s.dtype == MOE_DTYPE_BF16 ? 2 : 4; }

int validate(const moe_shape* sp) {
  if (!sp) return MOE_ERR_INVALID_ARG;
  const moe_shape& s = *sp;
  if (s.T < 0 || s.D <= 0 || s.F <= 0 || s.N <= 0 || s.k <= 0) return MOE_ERR_INVALID_ARG;
  if (s.k > s.N || s.capacity < -1) return MOE_ERR_INVALID_ARG;
  if (s.dtype != MOE_DTYPE_F32 && s.dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (s.act != MOE_ACT_GELU && s.act != MOE_ACT_RELU && s.act != MOE_ACT_SWIGLU) return MOE_ERR_INVALID_ARG;
  const uint32_t known = MOE_RENORM | MOE_RESIDUAL | MOE_HAS_BIAS | MOE_ROUTER_BIAS | MOE_FUSED_DECODE |
                         MOE_SLOT_MAJOR | MOE_PADDED;
  if (s.flags & ~known) return MOE_ERR_INVALID_ARG;
  if (s.act == MOE_ACT_SWIGLU && (s.flags & MOE_HAS_BIAS)) return MOE_ERR_UNSUPPORTED;
  if (s.n_shared < 0) return MOE_ERR_INVALID_ARG;
  if ((s.flags & MOE_PADDED) && s.capacity < 0) return MOE_ERR_INVALID_ARG;
  if (s.N + s.n_shared > kMaxExperts || s.k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  const int mult = (s.dtype == MOE_DTYPE_BF16) ? 64 : 16;
  if (s.D % mult || s.F % mult) return MOE_ERR_UNSUPPORTED;
  // 32-bit byte offsets inside the kernels
  const double lim = 4294967295.0;
  const double A = (double)s.T * s.k + (double)s.T * s.n_shared +
                   ((s.flags & MOE_PADDED) ? (double)s.N * s.capacity : 0.0);  // grouped rows (bound)
  if (A > 2147483647.0) return MOE_ERR_UNSUPPORTED;
  if ((double)s.T * s.D * 4 > lim || A * s.F * 4 > lim || A * s.D * 4 > lim || (double)s.F * s.D * 4 > lim)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Rows of the grouped buffers (perm, y_perm, hidden rows): the S*T rows of
// the shared experts, then room for all T*k routed assignments (N*C rows in
// the padded layout).
inline int64_t group_rows(const moe_shape& s) {
  const int64_t routed = (s.flags & MOE_PADDED) ? (int64_t)s.N * s.capacity : s.T * (int64_t)s.k;
  return s.T * (int64_t)s.n_shared + routed;
}

// Mean rows per expert, capped by the capacity (exactly the capacity in the
// padded layout): picks the kernel shape.
int64_t expected_rows(const moe_shape& s) {
  if (s.flags & MOE_PADDED) return s.capacity;
  int64_t expect = (s.T * s.k + s.N - 1) / s.N;
  if (s.capacity >= 0 && expect > s.capacity) expect = s.capacity;
  return expect;
}

// The most rows any group can hold: the capacity (at most T) for routed
// experts, T for a shared one.
int64_t max_rows(const moe_shape& s) {
  if (s.n_shared > 0 || s.capacity < 0) return s.T;
  return s.capacity < s.T ? s.capacity : s.T;
}

bool use_decode(const moe_shape& s) {
  return (s.flags & MOE_FUSED_DECODE) && s.n_shared == 0 && !(s.flags & MOE_PADDED) &&
         decode_applicable(s, expected_rows(s));
}

// Split-K partial tiles of the grouped GEMMs (bf16): the last, partial round
// of tiles is cut along K when this much workspace is given.
size_t part_bytes(const moe_shape& s) {
  if (s.dtype != MOE_DTYPE_BF16) return 0;
  return align_up(grouped_gemm_bf16_part_bytes(expected_rows(s), max_rows(s)));
}

// Workspace of the expert stage: hidden activations H[T*k, F] and the
// split-K partials for the grouped-GEMM path, fp32 shard partials for the
// fused decode path.
size_t ffn_ws_bytes(const moe_shape& s) {
  if (use_decode(s)) return align_up(decode_part_bytes(s));
  return align_up((size_t)group_rows(s) * s.F * elem_size(s)) + part_bytes(s);
}

// Workspace of the whole layer: y_perm[T*k, D] followed by the expert stage.
size_t forward_ws_bytes(const moe_shape& s) {
  return align_up((size_t)group_rows(s) * s.D * elem_size(s)) + ffn_ws_bytes(s);
}

// The split router's partial tiles go in the expert stage's part of the
// workspace (moe_forward) or at its start (moe_route); the one test decides
// for both, so the stage chain and moe_forward run the same kernels.
bool split_route_fits(const moe_shape& s) {
  return use_split_route(s) && route_split_bytes(s) <= ffn_ws_bytes(s);
}

// Expert stage.  With the decode path the fp32 shard partials stay in ws;
// y_perm is produced from them only when y_perm is non-null (stage API).
GemmAct up_act(const moe_shape& s) {
  return s.act == MOE_ACT_GELU ? kActGelu : s.act == MOE_ACT_RELU ? kActRelu : kActSwiGLU;
}

// fc1 (+ activation): H[r] for every kept row r, gathered from x through perm.
hipError_t launch_up(const moe_shape& s, const void* x, const int32_t* perm, const int32_t* offsets,
                     const void* w1, const void* b1, const void* w3, void* h, float* part,
                     hipStream_t st) {
  GroupedGemm g{};
  g.A = x;
  g.perm = perm;
  g.topk = s.k;
  g.offsets = offsets;
  g.n_experts = s.N + s.n_shared;  // the shared groups come first
  g.a_rows = s.T;
  g.B = w1;
  g.B2 = w3;
  g.bias = (s.flags & MOE_HAS_BIAS) ? b1 : nullptr;
  g.C = h;
  g.K = s.D;
  g.n_out = s.F;
  g.act = up_act(s);
  g.part = part;
  return s.dtype == MOE_DTYPE_BF16 ? launch_grouped_gemm_bf16(g, expected_rows(s), max_rows(s), st)
                                   : launch_grouped_gemm_f32(g, expected_rows(s), st);
}

// fc2: y_perm[r] = H[r] . w2[e]^T (+ b2[e]).
hipError_t launch_down(const moe_shape& s, const void* h, const int32_t* offsets, const void* w2,
                       const void* b2, void* y_perm, float* part, hipStream_t st) {
  GroupedGemm g{};
  g.A = h;
  g.perm = nullptr;
  g.topk = 1;
  g.offsets = offsets;
  g.n_experts = s.N + s.n_shared;  // the shared groups come first
  g.a_rows = group_rows(s);
  g.B = w2;
  g.B2 = nullptr;
  g.bias = (s.flags & MOE_HAS_BIAS) ? b2 : nullptr;
  g.C = y_perm;
  g.K = s.F;
  g.n_out = s.D;
  g.act = kActNone;
  g.part = part;
  return s.dtype == MOE_DTYPE_BF16 ? launch_grouped_gemm_bf16(g, expected_rows(s), max_rows(s), st)
                                   : launch_grouped_gemm_f32(g, expected_rows(s), st);
}

int expert_ffn_impl(const moe_shape& s, const void* x, const int32_t* perm, const int32_t* offsets,
                    const void* w1, const void* b1, const void* w3, const void* w2, const void* b2,
                    void* y_perm, void* ws, hipStream_t st) {
  if (use_decode(s)) {
    hipError_t e = launch_decode_ffn(s, x, perm, offsets, w1, b1, w3, w2, b2, (float*)ws, st);
    if (e == hipSuccess && y_perm) e = launch_reduce_shards(s, (const float*)ws, offsets, y_perm, st);
    return hip_status(e);
  }
  float* part = (float*)((unsigned char*)ws + align_up((size_t)group_rows(s) * s.F * elem_size(s)));
  if (s.dtype != MOE_DTYPE_BF16) part = nullptr;
  hipError_t e = launch_up(s, x, perm, offsets, w1, b1, w3, ws, part, st);
  if (e == hipSuccess) e = launch_down(s, ws, offsets, w2, b2, y_perm, part, st);
  return hip_status(e);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int32_t moe_capacity(int64_t T, int32_t k, int32_t N, double cf) {
  if (!(cf >= 0.0) || N <= 0) return -1;
  const double c = (double)T * (double)k / (double)N * cf;
  if (c >= 2147483647.0) return std::numeric_limits<int32_t>::max();
  return (int32_t)std::floor(c);
}

int moe_workspace_bytes(const moe_shape* shape, size_t* bytes) {
  int v = validate(shape);
  if (v != MOE_OK) return v;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = forward_ws_bytes(*shape);
  return MOE_OK;
}

int moe_route(const moe_shape* shape, const void* x, const void* w_router, const float* b_router,
              int32_t* topk_idx, float* topk_gate, float* logits_opt, void* ws, size_t ws_bytes,
              moe_stream_t stream) {
  int v = validate(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if (!x || !w_router || !topk_idx || !topk_gate) return MOE_ERR_INVALID_ARG;
  if ((s.flags & MOE_ROUTER_BIAS) && !b_router) return MOE_ERR_INVALID_ARG;
  if (ws) {
    if (ws_bytes < forward_ws_bytes(s)) return MOE_ERR_WORKSPACE;
    if ((uintptr_t)ws % kAlign) return MOE_ERR_INVALID_ARG;
    if (split_route_fits(s))
      return hip_status(launch_route_split(s, x, w_router, b_router, topk_idx, topk_gate, logits_opt, (float*)ws,
                                           (hipStream_t)stream));
  }
  return hip_status(launch_route(s, x, w_router, b_router, topk_idx, topk_gate, logits_opt, nullptr, 0,
                                 nullptr, nullptr, (hipStream_t)stream));
}

static size_t stats_ws_bytes(const moe_shape& s) {
  // per-block partial sums, then the 8-byte ticket of the second pass
  return align_up((size_t)route_blocks(s) * (size_t)s.N * sizeof(float)) + kAlign;
}

int moe_stats_workspace_bytes(const moe_shape* shape, size_t* bytes) {
  int v = validate(shape);
  if (v != MOE_OK) return v;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = stats_ws_bytes(*shape);
  return MOE_OK;
}

int moe_route_stats(const moe_shape* shape, const void* x, const void* w_router, const float* b_router,
                    int32_t* topk_idx, float* topk_gate, float* logits_opt, void* stats_ws,
                    size_t stats_ws_bytes_, moe_stream_t stream) {
  int v = validate(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if (!x || !w_router || !topk_idx || !topk_gate) return MOE_ERR_INVALID_ARG;
  if ((s.flags & MOE_ROUTER_BIAS) && !b_router) return MOE_ERR_INVALID_ARG;
  if (!stats_ws || stats_ws_bytes_ < stats_ws_bytes(s)) return MOE_ERR_WORKSPACE;
  if ((uintptr_t)stats_ws % kAlign) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_route(s, x, w_router, b_router, topk_idx, topk_gate, logits_opt,
                                 (float*)stats_ws, 0, nullptr, nullptr, (hipStream_t)stream));
}

int moe_router_stats(const moe_shape* shape, const void* stats_ws, size_t stats_ws_bytes_,
                     const int32_t* counts, const int32_t* n_dropped, double* prob_mean, double* frac,
                     double* summary, moe_stream_t stream) {
  int v = validate(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if (!counts || !n_dropped || !prob_mean || !summary) return MOE_ERR_INVALID_ARG;
  if (!stats_ws || stats_ws_bytes_ < stats_ws_bytes(s)) return MOE_ERR_WORKSPACE;
  if ((uintptr_t)stats_ws % kAlign) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_router_stats(s, (const float*)stats_ws, counts, n_dropped, prob_mean, frac,
                                        summary, (hipStream_t)stream));
}

// Fallback ranks: 1 <= R and k + R <= min(8, N); rerouting needs the
// compact layout.
static int check_fallback(const moe_shape& s, int32_t R) {
  if (R < 1) return MOE_ERR_INVALID_ARG;
  if (s.k + R > kMaxTopK || s.k + R > s.N) return MOE_ERR_UNSUPPORTED;
  if (s.flags & MOE_PADDED) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int moe_route_fallback(const moe_shape* shape, const void* x, const void* w_router, const float* b_router,
                       int32_t* topk_idx, float* topk_gate, int32_t n_fallback, int32_t* fb_idx, float* fb_gate,
                       float* logits_opt, moe_stream_t stream) {
  int v = validate(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if ((v = check_fallback(s, n_fallback)) != MOE_OK) return v;
  if (s.T == 0) return MOE_OK;
  if (!x || !w_router || !topk_idx || !topk_gate || !fb_idx || !fb_gate) return MOE_ERR_INVALID_ARG;
  if ((s.flags & MOE_ROUTER_BIAS) && !b_router) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_route(s, x, w_router, b_router, topk_idx, topk_gate, logits_opt, nullptr, n_fallback,
                                 fb_idx, fb_gate, (hipStream_t)stream));
}

int moe_dispatch_reroute(const moe_shape* shape, int32_t n_fallback, const int32_t* fb_idx, const float* fb_gate,
                         int32_t* topk_idx, float* topk_gate, int32_t* counts, int32_t* offsets, int32_t* perm,
                         int32_t* slot, int32_t* n_dropped, moe_stream_t stream) {
  int v = validate(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if ((v = check_fallback(s, n_fallback)) != MOE_OK) return v;
  if (s.T == 0) return MOE_OK;
  if (!fb_idx || !fb_gate || !topk_idx || !topk_gate || !counts || !offsets || !perm || !slot || !n_dropped)
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_dispatch_reroute(s, n_fallback, fb_idx, fb_gate, topk_idx, topk_gate, counts, offsets,
                                            perm, slot, n_dropped, (hipStream_t)stream));
}

// Dispatch over many workgroups when scratch is at hand and the batch has
// more than kSmallDispatch assignments; one workgroup otherwise.  The results
// are identical.  Timed inside the whole layer (graph replays): with 768
// assignments one workgroup (its smallest register mode) beats two launches,
// 0.233 against 0.237 ms per step; with 16384 over 16 experts two launches
// win, 0.427 against 0.436 ms, and over 8 experts they tie.  (Timed alone, one
// workgroup looked better for 16384 assignments over 8 or 16 experts: there
// its 65 KB of unrolled code stays cached, which it does not in the layer.)
constexpr int64_t kSmallDispatch = 4096;
static hipError_t dispatch_any(const moe_shape& s, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                               int32_t* perm, int32_t* slot, int32_t* n_dropped, void* ws, hipStream_t st) {
  if (ws && s.T * (int64_t)s.k > kSmallDispatch)
    return launch_dispatch_multi(s, topk_idx, counts, offsets, perm, slot, n_dropped, (int32_t*)ws, st);
  return launch_dispatch(s, topk_idx, counts, offsets, perm, slot, n_dropped, st);
}

int moe_dispatch(const moe_shape* shape, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                 int32_t* perm, int32_t* slot, int32_t* n_dropped, void* ws, size_t ws_bytes,
                 moe_stream_t stream) {
  int v = validate(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if (!topk_idx || !counts || !offsets || !perm || !slot || !n_dropped) return MOE_ERR_INVALID_ARG;
  if (ws) {
    if (ws_bytes < forward_ws_bytes(s)) return MOE_ERR_WORKSPACE;
    if ((uintptr_t)ws % kAlign) return MOE_ERR_INVALID_ARG;
  }
  return hip_status(dispatch_any(s, topk_idx, counts, offsets, perm, slot, n_dropped, ws, (hipStream_t)stream));
}

int moe_expert_ffn(const moe_shape* shape, const void* x, const int32_t* perm, const int32_t* offsets,
                   const void* w1, const void* b1, const void* w3, const void* w2, const void* b2,
                   void* y_perm, void* ws, size_t ws_bytes, moe_stream_t stream) {
  int v = validate(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if (!x || !perm || !offsets || !w1 || !w2 || !y_perm) return MOE_ERR_INVALID_ARG;
  if (s.act == MOE_ACT_SWIGLU && !w3) return MOE_ERR_INVALID_ARG;
  if ((s.flags & MOE_HAS_BIAS) && (!b1 || !b2)) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < ffn_ws_bytes(s)) return MOE_ERR_WORKSPACE;
  if ((uintptr_t)ws % kAlign) return MOE_ERR_INVALID_ARG;
  return expert_ffn_impl(s, x, perm, offsets, w1, b1, w3, w2, b2, y_perm, ws, (hipStream_t)stream);
}

// Split-K workspace of the stand-alone projections: NULL (never split) or
// at least moe_workspace_bytes(shape) bytes, 256-byte aligned.
static int split_ws(const moe_shape& s, void* ws, size_t ws_bytes, float** part) {
  *part = nullptr;
  if (!ws || s.dtype != MOE_DTYPE_BF16) return MOE_OK;
  if (ws_bytes < forward_ws_bytes(s)) return MOE_ERR_WORKSPACE;
  if ((uintptr_t)ws % kAlign) return MOE_ERR_INVALID_ARG;
  *part = (float*)ws;
  return MOE_OK;
}

int moe_expert_up(const moe_shape* shape, const void* x, const int32_t* perm, const int32_t* offsets,
                  const void* w1, const void* b1, const void* w3, void* h, void* ws, size_t ws_bytes,
                  moe_stream_t stream) {
  int v = validate(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if (!x || !perm || !offsets || !w1 || !h) return MOE_ERR_INVALID_ARG;
  if (s.act == MOE_ACT_SWIGLU && !w3) return MOE_ERR_INVALID_ARG;
  if ((s.flags & MOE_HAS_BIAS) && !b1) return MOE_ERR_INVALID_ARG;
  float* part;
  if ((v = split_ws(s, ws, ws_bytes, &part)) != MOE_OK) return v;
  return hip_status(launch_up(s, x, perm, offsets, w1, b1, w3, h, part, (hipStream_t)stream));
}

int moe_expert_down(const moe_shape* shape, const void* h, const int32_t* offsets, const void* w2,
                    const void* b2, void* y_perm, void* ws, size_t ws_bytes, moe_stream_t stream) {
  int v = validate(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if (!h || !offsets || !w2 || !y_perm) return MOE_ERR_INVALID_ARG;
  if ((s.flags & MOE_HAS_BIAS) && !b2) return MOE_ERR_INVALID_ARG;
  float* part;
  if ((v = split_ws(s, ws, ws_bytes, &part)) != MOE_OK) return v;
  return hip_status(launch_down(s, h, offsets, w2, b2, y_perm, part, (hipStream_t)stream));
}

int moe_combine(const moe_shape* shape, const void* y_perm, const int32_t* slot, const float* topk_gate,
                const void* x_residual, void* out, moe_stream_t stream) {
  int v = validate(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if (!y_perm || !slot || !topk_gate || !out) return MOE_ERR_INVALID_ARG;
  if ((s.flags & MOE_RESIDUAL) && !x_residual) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(s, y_perm, slot, topk_gate, x_residual, out, (hipStream_t)stream));
}

int moe_forward(const moe_shape* shape, const void* x, const void* w_router, const float* b_router,
                const void* w1, const void* b1, const void* w3, const void* w2, const void* b2,
                void* out, int32_t* topk_idx, float* topk_gate, int32_t* counts, int32_t* offsets,
                int32_t* perm, int32_t* slot, int32_t* n_dropped, void* ws, size_t ws_bytes,
                moe_stream_t stream) {
  int v = validate(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if (!x || !w_router || !w1 || !w2 || !out || !topk_idx || !topk_gate || !counts || !offsets ||
      !perm || !slot || !n_dropped)
    return MOE_ERR_INVALID_ARG;
  if (s.act == MOE_ACT_SWIGLU && !w3) return MOE_ERR_INVALID_ARG;
  if ((s.flags & MOE_HAS_BIAS) && (!b1 || !b2)) return MOE_ERR_INVALID_ARG;
  if ((s.flags & MOE_ROUTER_BIAS) && !b_router) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < forward_ws_bytes(s)) return MOE_ERR_WORKSPACE;
  if ((uintptr_t)ws % kAlign) return MOE_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  void* y_perm = ws;
  void* ffn_ws = (unsigned char*)ws + align_up((size_t)group_rows(s) * s.D * elem_size(s));
  // few tokens: the split router, its partial tiles in the expert stage's
  // workspace (dead before the dispatch runs)
  hipError_t e = split_route_fits(s)
                     ? launch_route_split(s, x, w_router, b_router, topk_idx, topk_gate, nullptr, (float*)ffn_ws, st)
                     : launch_route(s, x, w_router, b_router, topk_idx, topk_gate, nullptr, nullptr, 0, nullptr,
                                    nullptr, st);
  // the dispatch scratch lives where the expert stage's workspace will be
  if (e == hipSuccess) e = dispatch_any(s, topk_idx, counts, offsets, perm, slot, n_dropped, ffn_ws, st);
  if (e != hipSuccess) return MOE_ERR_HIP;
  const bool decode = use_decode(s);
  int r = expert_ffn_impl(s, x, perm, offsets, w1, b1, w3, w2, b2, decode ? nullptr : y_perm, ffn_ws, st);
  if (r != MOE_OK) return r;
  if (decode)
    return hip_status(launch_combine_shards(s, (const float*)ffn_ws, decode_shards(s), slot, topk_gate, x,
                                            out, st));
  return hip_status(launch_combine(s, y_perm, slot, topk_gate, x, out, st));
}

// ---- allocation-free forward -------------------------------------------
// moe_forward_noalloc runs moe_forward with its workspace in `scratch`, a
// file-scope device array of kNoAllocScratchBytes that every GPU the library
// runs on holds until the process ends.  Host code never passes the array's
// name to a kernel (in host code it is a stand-in, not a device address):
// the first call on a device, with that device current, looks up the
// array's device address with hipGetSymbolAddress and keeps it per device.
}  // extern "C"

namespace moe {
namespace {

constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// This device's copy of `scratch` (nullptr if the lookup fails).
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  // a concurrent first call stores the same address
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace
}  // namespace moe

extern "C" {

int moe_forward_noalloc(const moe_shape* shape, const void* x, const void* w_router, const float* b_router,
                        const void* w1, const void* b1, const void* w3, const void* w2, const void* b2,
                        void* out, int32_t* topk_idx, float* topk_gate, int32_t* counts, int32_t* offsets,
                        int32_t* perm, int32_t* slot, int32_t* n_dropped, moe_stream_t stream) {
  int v = validate(shape);
  if (v != MOE_OK) return v;
  const size_t need = forward_ws_bytes(*shape);
  if (need > kNoAllocScratchBytes) return MOE_ERR_WORKSPACE;
  if (shape->T == 0) return MOE_OK;
  void* ws = device_scratch();
  if (!ws) return MOE_ERR_HIP;
  // the layer reads nothing from its workspace that it has not written in
  // the same call, so the scratch's previous contents need no clearing
  return moe_forward(shape, x, w_router, b_router, w1, b1, w3, w2, b2, out, topk_idx, topk_gate, counts, offsets,
                     perm, slot, n_dropped, ws, need, stream);
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or option";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
