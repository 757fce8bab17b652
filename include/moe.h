/*
 * moe.h -- C ABI of libmoe_mi355x.so: forward pass of one Mixture-of-Experts
 * FFN layer on one AMD Instinct MI355X (gfx950).
 *
 * The layer is the one described by the notebook "Mixture-of-experts and
 * expert parallelism" (llm-systems-cookbook, serving track): a linear router
 * without bias, a softmax over the N experts and the top-k of it ("Top-k
 * router"); tokens grouped by their chosen expert and run through that
 * expert's MLP, whose outputs are weighted by the gates and summed back into
 * token order ("Dispatch and gather"); an optional per-expert slot budget
 * that drops overflow ("Capacity factor").  The three stages -- input
 * routing, expert computation, result aggregation -- are also the workflow
 * named in "MoE Parallelism for Inference: Tricks and PyTorch Deep Dive"
 * ("Why Parallelism Matters in MoE Inference").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensors are row-major, device memory, allocated and owned by the
 *   caller.  The library never allocates or frees memory and keeps no state
 *   besides a cached device-attribute query per device.
 * - Weights use the nn.Linear layout [out, in], stacked over experts:
 *     x[T,D], out[T,D]             dtype of the shape (fp32 or bf16)
 *     w_router[N,D]                dtype of the shape
 *     b_router[N]                  fp32 (only with MOE_ROUTER_BIAS)
 *     w1[N,F,D], w3[N,F,D]         dtype of the shape (w3 only for SwiGLU)
 *     w2[N,D,F]                    dtype of the shape
 *     b1[N,F], b2[N,D]             dtype of the shape (only with MOE_HAS_BIAS)
 * - An assignment is a (token t, choice j) pair with flat index a = t*k + j.
 *   topk_idx[T,k] and slot[T*k] are int32, topk_gate[T,k] is fp32.
 * - Every call is asynchronous on the caller's HIP stream (NULL = the null
 *   stream): outputs are valid once the stream has reached the call.  Calls
 *   are re-entrant and thread-safe; calls that share output or workspace
 *   buffers must be ordered by the caller.
 * - Return value: MOE_OK (0) or a negative MOE_ERR_* code.  Arguments are
 *   validated on the host before any launch; on error nothing is launched.
 *   T = 0 is a valid no-op.  NaN/Inf inputs give unspecified results.
 *
 * Supported shapes: 1 <= N + S <= 256 (S shared experts), 1 <= k <= min(N, 8),
 * and the row bound B = S*T + T*k (+ N*C with MOE_PADDED, C = capacity) at
 * most 2^31 - 1.  bf16: D and F multiples of 64.  fp32: D and F multiples of
 * 16.  SwiGLU experts carry no biases (MOE_HAS_BIAS with SWIGLU is
 * unsupported).  4*T*D, 4*B*D, 4*B*F and 4*F*D must stay below 2^32 (32-bit
 * byte offsets inside the kernels).  Other shapes return MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* moe_stream_t; /* same type as hipStream_t */

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* bad size, flag, null required pointer */
  MOE_ERR_UNSUPPORTED = -2, /* legal but outside the supported shapes */
  MOE_ERR_WORKSPACE = -3,   /* workspace smaller than moe_workspace_bytes */
  MOE_ERR_HIP = -4          /* a HIP runtime call or launch failed */
};

enum moe_dtype { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 };

/* Expert MLP:
 *   GELU  : y = w2 . gelu(w1 . x + b1) + b2, gelu in its exact erf form
 *           (the notebook's Expert, "Dispatch and gather")
 *   RELU  : same with max(0, .) (Switch-style FFN)
 *   SWIGLU: y = w2 . (silu(w1 . x) * (w3 . x)), silu(z) = z / (1 + e^-z)   */
enum moe_act { MOE_ACT_GELU = 0, MOE_ACT_RELU = 1, MOE_ACT_SWIGLU = 2 };

enum moe_flags {
  MOE_RENORM = 1u,       /* gates divided by their sum over the k choices */
  MOE_RESIDUAL = 2u,     /* out = x + sum of kept, gated expert outputs */
  MOE_HAS_BIAS = 4u,     /* b1 and b2 are present */
  MOE_ROUTER_BIAS = 8u,  /* b_router is added to the router logits */
  /* Algorithm choice for bf16 layers with at most 16 rows per expert: one
   * fused launch per layer over (expert, F-shard) items that streams the
   * weights into registers and writes fp32 shard partials, instead of the
   * two grouped-GEMM launches.  Same results within the bf16 tolerance;
   * ignored where it does not apply.  Off by default (slower on MI355X). */
  MOE_FUSED_DECODE = 16u,
  /* Capacity priority by choice: each expert keeps its assignments in the
   * order (choice j, token t), so every token's first choice is kept before
   * any second choice (the GShard top-2 pattern named among the notebook's
   * references); without it the order is the flat index t*k+j. */
  MOE_SLOT_MAJOR = 32u,
  /* Static capacity layout: every routed expert owns exactly `capacity`
   * rows, expert e rows [S*T + e*C, S*T + (e+1)*C), kept assignments first
   * and padding after; the experts' MLPs run on all N*C rows (padding rows
   * re-use assignment 0 and their outputs are never read).  Without it the
   * rows are sized by the actual counts (the compact, "dynamic gating"
   * layout of "Towards MoE Deployment", abstract).  Needs capacity >= 0. */
  MOE_PADDED = 64u
};

typedef struct moe_shape {
  int64_t T;        /* tokens */
  int32_t D;        /* model dim */
  int32_t F;        /* expert hidden dim */
  int32_t N;        /* experts */
  int32_t k;        /* experts per token */
  int32_t capacity; /* slots per expert; -1 = no limit (see moe_capacity) */
  int32_t dtype;    /* enum moe_dtype */
  int32_t act;      /* enum moe_act */
  uint32_t flags;   /* enum moe_flags, or-ed */
  int32_t n_shared; /* always-on experts S (0 = none), see below */
} moe_shape;

/* Shared (always-on) experts, the notebook's "Exercises" section (a few
 * experts every token goes through, next to the routed ones): with
 * n_shared = S > 0 the expert stacks w1/w3/w2/b1/b2 hold S + N experts, the
 * S shared ones first (slots 0..S-1) and routed expert e in slot S + e; the
 * router (w_router [N, D]) ranks the routed experts only, topk_idx stays in
 * [0, N).  Every token goes to every shared expert with gate 1, uncapped.
 * The grouped rows then hold the shared rows first: row s*T + t is token t
 * of shared expert s (perm = t*k there), then the routed rows, so offsets
 * has S + N + 1 entries (offsets[s] = s*T for s <= S), routed slots are
 * shifted by S*T, perm and the row buffers (y_perm, the hidden rows) hold
 * S*T + T*k rows, and the combine adds the shared rows with gate 1.  counts
 * and n_dropped stay those of the N routed experts.
 *
 * Grouped rows: the row buffers of the expert stage (perm, y_perm and the
 * hidden rows h) hold R = S*T + T*k rows, or R = S*T + N*C with MOE_PADDED
 * (C = capacity); "[R, ...]" below means that count. */

/* Per-expert slot budget of the notebook's "Capacity factor" section:
 * int(T*k/N * cf), evaluated left to right in double and truncated.
 * cf < 0 (or NaN) returns -1 (no limit); results above INT32_MAX saturate. */
int32_t moe_capacity(int64_t T, int32_t k, int32_t N, double cf);

/* Bytes of device workspace that moe_expert_ffn and moe_forward need for
 * this shape (written to *bytes).  The workspace needs 256-byte alignment
 * and holds no state between calls. */
int moe_workspace_bytes(const moe_shape* shape, size_t* bytes);

/* Router ("Top-k router"): logits l = x . w_router^T (+ b_router), softmax
 * over all N, and the k experts with the largest logits in decreasing order,
 * ties to the lower expert index.  topk_gate[t,j] is the softmax probability
 * of expert topk_idx[t,j] (divided by the sum over j with MOE_RENORM).
 * Logits are accumulated in fp32; a token whose top-(k+1) fp32 logits lie
 * within 1e-4 of each other has all N logits recomputed in fp64 from the
 * exact products before it is ranked.  logits_opt (fp32 [T,N], may be NULL)
 * receives the logits used for the ranking, rounded to fp32.
 *
 * ws is optional device scratch, as for moe_dispatch: NULL, or at least
 * moe_workspace_bytes(shape) bytes with 256-byte alignment
 * (MOE_ERR_WORKSPACE or MOE_ERR_INVALID_ARG otherwise).  With it, bf16
 * batches of at most 1024 tokens (D a multiple of 128) take two launches
 * spread over many workgroups: fp32 partial logit tiles of 128-wide slices
 * of D, then their sum in fixed slice order and the ranking.  moe_forward
 * makes the same choice, so a stage chain given the same workspace repeats
 * its results bit for bit.  Without ws the router is one launch; the two
 * can differ in the last bits of the fp32 logits and gates (the selection
 * is the same: it is exact either way). */
int moe_route(const moe_shape* shape, const void* x, const void* w_router,
              const float* b_router, int32_t* topk_idx, float* topk_gate,
              float* logits_opt, void* ws, size_t ws_bytes, moe_stream_t stream);

/* Router load statistics, the notebook's "Switch Transformer auxiliary loss"
 * and "Capacity factor" sections, computed in two steps.
 *
 * moe_route_stats does what moe_route does, with identical outputs. In the
 * same launch, each router block also adds up every expert's softmax
 * probability over the block's tokens. It uses the fp32 logits the ranking
 * used, bias included. The partial sums go to stats_ws, which the caller
 * owns and which must hold moe_stats_workspace_bytes(shape) bytes, 256-byte
 * aligned. The sizes depend on the shape and on the current device's CU
 * count, so query the size on the device that runs the calls. stats_ws also
 * holds a counter that moe_route_stats clears and moe_router_stats advances.
 * Calls that share a stats_ws must therefore be ordered on one stream, and
 * moe_router_stats must follow a moe_route_stats on that stats_ws. It may
 * be repeated, though, without routing again.
 *
 * moe_router_stats runs after moe_dispatch of the same batch. It reads
 * stats_ws, counts and n_dropped and writes device outputs:
 *   prob_mean[e] = P_e = mean over the T tokens of softmax(l_t)[e].
 *     The partials are summed in fp64 in a fixed order, so repeated runs
 *     give the same result.
 *   frac[e] = f_e = counts[e] / T, the share of tokens with expert e among
 *     their choices. This holds because the k choices of a token are
 *     distinct. frac may be NULL.
 *   summary[0] = N * sum_e f_e * P_e, the Switch auxiliary loss. It equals k
 *     for a perfectly balanced router.
 *   summary[1] = max_e counts[e] / (T*k/N), the imbalance.
 *   summary[2] = n_dropped / (T*k), the share of assignments dropped by the
 *     capacity.
 * prob_mean, frac and summary are fp64: N, N and 3 entries.
 *
 * Errors, for both calls:
 *   MOE_ERR_WORKSPACE: stats_ws is NULL or too small.
 *   MOE_ERR_INVALID_ARG: stats_ws is misaligned, or a required pointer is NULL.
 * T = 0 is a no-op. */
int moe_stats_workspace_bytes(const moe_shape* shape, size_t* bytes);
int moe_route_stats(const moe_shape* shape, const void* x, const void* w_router,
                    const float* b_router, int32_t* topk_idx, float* topk_gate,
                    float* logits_opt, void* stats_ws, size_t stats_ws_bytes,
                    moe_stream_t stream);
int moe_router_stats(const moe_shape* shape, const void* stats_ws, size_t stats_ws_bytes,
                     const int32_t* counts, const int32_t* n_dropped, double* prob_mean,
                     double* frac, double* summary, moe_stream_t stream);

/* Dispatch ("Dispatch and gather", "Capacity factor"): counts[e] = number of
 * assignments to expert e (before the capacity cut).  The assignments of
 * expert e are ranked in increasing flat index (with MOE_SLOT_MAJOR: in
 * increasing (j, t)); the first min(counts[e], capacity) are kept.
 * offsets[N+1] is the exclusive scan of the kept counts, perm[offsets[e] ..
 * offsets[e+1]) lists expert e's kept assignments in rank order, slot[a] is
 * the row of assignment a in that grouped order or -1 if it was dropped,
 * and *n_dropped = T*k - offsets[N].  perm must hold T*k entries; entries
 * past offsets[N] are left untouched.  With n_shared = S the S shared groups
 * come first (offsets[S+N+1], perm of S*T + T*k entries, routed rows and
 * slots shifted by S*T; see moe_shape).  With MOE_PADDED expert e's rows
 * start at S*T + e*C and perm holds S*T + N*C entries, padding included.
 * Expert ids outside [0, N) are treated as dropped and not counted.
 * Bit-exact and deterministic.
 *
 * ws is optional device scratch. With ws = NULL, one workgroup does the whole
 * dispatch in one launch. Otherwise ws needs at least
 * moe_workspace_bytes(shape) bytes with 256-byte alignment (MOE_ERR_WORKSPACE
 * or MOE_ERR_INVALID_ARG otherwise). Batches of more than 4096 assignments
 * (T*k) then take two launches over many workgroups: segments of the
 * priority order are ranked apart and placed from their fixed-order counts.
 * The results are identical. */
int moe_dispatch(const moe_shape* shape, const int32_t* topk_idx, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* slot, int32_t* n_dropped,
                 void* ws, size_t ws_bytes, moe_stream_t stream);

/* Overflow fallback. The notebook's "What" section lets capacity overflow
 * take a fallback instead of being dropped; among the first page's tuning
 * tricks is moving rejected tokens to experts with spare room. Two calls implement this with R = n_fallback levels.
 * R must be >= 1 (MOE_ERR_INVALID_ARG otherwise). k + R must not exceed
 * min(8, N), and the layout must be compact, not MOE_PADDED; otherwise the
 * call returns MOE_ERR_UNSUPPORTED. T = 0 is a no-op.
 *
 * moe_route_fallback does what moe_route does, with identical idx. It also
 * writes each token's experts of rank k .. k+R-1 in the same order. Its
 * near-tie test covers the top k+R+1, so more tokens may be re-ranked from
 * fp64 logits. Such a token's gates equal moe_route's only up to fp32
 * rounding. The fallback outputs are:
 *   fb_idx [T, R] int32 receives those experts.
 *   fb_gate [T, R] fp32 receives their softmax probabilities. With
 *     MOE_RENORM they are divided by the same sum over the k choices as the
 *     gates.
 *
 * moe_dispatch_reroute does what moe_dispatch does, then runs R levels.
 * At level r:
 *   - every token with a dropped assignment left offers its lowest-j one to
 *     expert fb_idx[t, r];
 *   - each expert accepts offers in increasing token order while its rows
 *     stay within the capacity;
 *   - for an accepted assignment, topk_idx[t, j] and topk_gate[t, j]
 *     (in/out) are rewritten to that expert and fb_gate[t, r].
 * Results:
 *   - Expert e's rows are its kept assignments in priority order, then the
 *     rerouted ones in (level, token) order. offsets, perm and slot describe
 *     the final rows.
 *   - n_dropped counts what stays dropped. counts keeps the routed counts
 *     before the capacity cut.
 *   - Entries of perm past offsets[S+N] are unspecified: they serve as
 *     scratch.
 * The expert calls and moe_combine then take the rewritten topk_gate. */
int moe_route_fallback(const moe_shape* shape, const void* x, const void* w_router,
                       const float* b_router, int32_t* topk_idx, float* topk_gate,
                       int32_t n_fallback, int32_t* fb_idx, float* fb_gate, float* logits_opt,
                       moe_stream_t stream);
int moe_dispatch_reroute(const moe_shape* shape, int32_t n_fallback, const int32_t* fb_idx,
                         const float* fb_gate, int32_t* topk_idx, float* topk_gate,
                         int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot,
                         int32_t* n_dropped, moe_stream_t stream);

/* Expert MLPs on the grouped rows: for every expert e and every row r in
 * [offsets[e], offsets[e+1]), token t = perm[r] / k,
 *   y_perm[r, :] = MLP_e(x[t, :])       (dtype of the shape, [R, D], R the
 *                                        grouped rows of moe_shape)
 * Rows past the last offset are left untouched.  One launch per layer (fc1+act)
 * and one for fc2, each a persistent grouped GEMM whose work list covers
 * column shards of w1/w3 and row shards of w2 for all experts at once (the
 * row/column expert decomposition of "Accelerating MoE Model Inference with
 * Expert Sharding", abstract), or with MOE_FUSED_DECODE a fused
 * weight-streaming kernel when the rows per expert are few.  fp32
 * accumulation; the hidden activations are held in the shape's dtype.
 * ws/ws_bytes: see moe_workspace_bytes. */
int moe_expert_ffn(const moe_shape* shape, const void* x, const int32_t* perm,
                   const int32_t* offsets, const void* w1, const void* b1, const void* w3,
                   const void* w2, const void* b2, void* y_perm, void* ws, size_t ws_bytes,
                   moe_stream_t stream);

/* The two halves of moe_expert_ffn as separate launches, for callers that
 * keep the hidden activations themselves or time the projections apart.
 * Both always use the grouped GEMM (MOE_FUSED_DECODE is ignored here).
 * ws: NULL, or scratch of at least moe_workspace_bytes(shape) bytes (256-byte
 * aligned) that lets a bf16 projection split its last, partial round of
 * tiles along K (fp32 partial sums, added in a fixed order by a second
 * launch, only where the tile count leaves such a round); results then equal
 * those of moe_expert_ffn and moe_forward, which always hand the kernels
 * their workspace.  A too-small ws returns MOE_ERR_WORKSPACE.
 *
 * moe_expert_up: the expert's first projection and activation (the
 * notebook's Expert: fc1 then GELU or ReLU, biases with MOE_HAS_BIAS; for
 * SwiGLU silu(x w1^T) times x w3^T, w1 the gated branch):
 *   h[r, :] = act(x[perm[r] / k, :] . w1[e]^T + b1[e])     r in [offsets[e], offsets[e+1])
 * h: [R, F] row-major in the shape's dtype (R the grouped rows of
 * moe_shape), caller-owned; rows past the last offset are left untouched.  fp32 accumulation, one rounding to the
 * dtype after the activation.  w3 may be NULL unless the act is SwiGLU. */
int moe_expert_up(const moe_shape* shape, const void* x, const int32_t* perm,
                  const int32_t* offsets, const void* w1, const void* b1, const void* w3,
                  void* h, void* ws, size_t ws_bytes, moe_stream_t stream);

/* moe_expert_down: the expert's second projection (fc2):
 *   y_perm[r, :] = h[r, :] . w2[e]^T + b2[e]                r in [offsets[e], offsets[e+1])
 * h as written by moe_expert_up; y_perm [R, D] in the shape's dtype. */
int moe_expert_down(const moe_shape* shape, const void* h, const int32_t* offsets,
                    const void* w2, const void* b2, void* y_perm, void* ws, size_t ws_bytes,
                    moe_stream_t stream);

/* Combine ("Dispatch and gather"): out[t] = (x[t] with MOE_RESIDUAL, else 0)
 * + sum over j = 0..k-1 with slot[t*k+j] >= 0 of topk_gate[t,j] *
 * y_perm[slot[t*k+j]], summed in fp32 in increasing j and rounded once to
 * the shape's dtype.  A token with every choice dropped gets exactly 0, or
 * exactly x[t] with MOE_RESIDUAL.  x_residual may be NULL without
 * MOE_RESIDUAL. */
int moe_combine(const moe_shape* shape, const void* y_perm, const int32_t* slot,
                const float* topk_gate, const void* x_residual, void* out,
                moe_stream_t stream);

/* The whole layer: moe_route, moe_dispatch, the expert MLPs and the combine,
 * stream-ordered, with the intermediate tensors in ws.  The routing outputs
 * (topk_idx, topk_gate, counts, offsets, perm, slot, n_dropped; sizes as
 * above) are caller buffers so that they can be inspected. */
int moe_forward(const moe_shape* shape, const void* x, const void* w_router,
                const float* b_router, const void* w1, const void* b1, const void* w3,
                const void* w2, const void* b2, void* out, int32_t* topk_idx,
                float* topk_gate, int32_t* counts, int32_t* offsets, int32_t* perm,
                int32_t* slot, int32_t* n_dropped, void* ws, size_t ws_bytes,
                moe_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * layer as moe_forward, same arguments and results, with the workspace
 * taken from a device array inside the library instead of a caller buffer.
 * The array holds MOE_NOALLOC_SCRATCH_BYTES (64 MiB); each GPU the library
 * runs on keeps its own copy until the process ends.  A layer whose
 * moe_workspace_bytes exceeds that returns MOE_ERR_WORKSPACE before any
 * launch.  The call allocates nothing (no hipMalloc, no library routine that
 * allocates); the first call on a device looks up that device's copy of the
 * array.  Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (different streams, or threads) race and must be ordered by the
 * caller.  The array keeps the last call's contents; the layer writes
 * every workspace byte it reads within the same call.  Returns MOE_ERR_HIP
 * if the array's address cannot be looked up. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(const moe_shape* shape, const void* x, const void* w_router,
                        const float* b_router, const void* w1, const void* b1, const void* w3,
                        const void* w2, const void* b2, void* out, int32_t* topk_idx,
                        float* topk_gate, int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* slot, int32_t* n_dropped, moe_stream_t stream);

/* Measurement helper (not a step of the layer): the shader clock the GPU
 * holds, for stating a kernel's throughput against the peak at the clock
 * actually sustained (the MFMA peak scales with the core clock).  Launches
 * `blocks` one-wave workgroups on `stream`; each waits delay_us, then runs
 * a chain of 1024*iters dependent 32-bit integer adds (one per 4 shader
 * clocks on a 16-lane SIMD) and writes stamps[4*b .. 4*b+3] = {100 MHz
 * real-time counter at the chain's start, at its end, adds in the chain,
 * the chain's value} (device memory, uint64, 4*blocks entries,
 * caller-owned).  clock = 4 * adds / (ticks / 100 MHz).  Launched on a second
 * stream while a kernel runs, the waves share that kernel's compute units
 * when its resources leave room for one more wave; a SIMD busy with other
 * vector instructions slows the chain, so the figure is a lower bound.
 * Errors: MOE_ERR_INVALID_ARG for blocks outside [1, 65536], a null stamps,
 * delay_us outside [0, 100000] or iters outside [1, 2^16]. */
int moe_clock_probe(int32_t blocks, double delay_us, int32_t iters, uint64_t* stamps,
                    moe_stream_t stream);

/* Static, human-readable text of a status code. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
