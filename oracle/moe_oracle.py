"""CPU oracle for the forward pass of one Mixture-of-Experts FFN layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check of the entry
module and the benchmark's CPU-baseline leg use it.  It shares no code with
the HIP library; both receive the same seeded inputs from ``workloads``.

What it computes follows the notebook "Mixture-of-experts and expert
parallelism" (llm-systems-cookbook, serving track, notebook 09) plus the
workload statements of the layer configurations:

* "Top-k router": a bias-free linear map from the hidden state to N
  logits, a softmax over all N experts, and the k best experts with their
  gate weights (the softmax probabilities of the chosen experts).
* "Dispatch and gather": each expert is an MLP fc2(gelu(fc1(x))) with
  biases; the layer output starts at zero and, expert by expert, adds the
  expert's output for every token that chose it, scaled by that token's gate
  for the expert.
* "Capacity factor": an expert has a per-batch slot budget of
  tokens*k/N*factor (truncated to an integer); assignments beyond it are
  dropped.  The drop rate is the summed overflow over the summed counts.

Readings where the pages leave a step open (all listed in the design notes):
selection is done on logits with ties to the lower expert index (softmax is
strictly increasing, so this is the exact-arithmetic top-k); the kept
assignments of an expert are its first C in flat order t*k+j; a dropped
assignment contributes zero and the remaining gates are not rescaled;
``renorm`` divides the chosen gates by their sum; ``residual`` adds x; the
SwiGLU expert applies silu to the w1 branch and multiplies by the w3 branch;
GELU is the erf form.

Everything is computed in float64 from the exact stored input values (fp32
and bf16 values widen exactly).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np
from scipy.special import erf as _erf


# ----------------------------------------------------------------- helpers
def f64(a) -> np.ndarray:
    """Exact widening of a numpy array or a CPU torch tensor to float64."""
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        return a.astype(np.float64, copy=False)
    # torch tensor (fp32 or bf16): .double() is exact for both
    return a.detach().cpu().double().numpy()


# ----------------------------------------------------------------- routing
def router_logits(x, w_router, b_router=None) -> np.ndarray:
    """l[t, e] = sum_d x[t, d] * w_router[e, d]  (+ b_router[e]).

    The notebook's router is a linear layer with no bias ("Top-k router");
    the skewed-routing workload adds a fixed per-expert bias.
    """
    l = f64(x) @ f64(w_router).T
    if b_router is not None:
        l = l + f64(b_router)[None, :]
    return l


def softmax(logits: np.ndarray) -> np.ndarray:
    """Softmax over all N experts of each token, max-subtracted."""
    z = logits - logits.max(axis=1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=1, keepdims=True)


def expert_order(logits: np.ndarray) -> np.ndarray:
    """Experts of each token by decreasing logit, ties to the lower index.

    A stable sort of -logit keeps equal keys in ascending expert order.
    """
    return np.argsort(-logits, axis=1, kind="stable")


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """idx[t, :] = the first k experts of ``expert_order`` (int64)."""
    N = logits.shape[1]
    if not 1 <= k <= N:
        raise ValueError(f"k={k} must lie in [1, N={N}]")
    return expert_order(logits)[:, :k].astype(np.int64)


def gate_values(probs: np.ndarray, idx: np.ndarray, renorm: bool) -> np.ndarray:
    """g[t, j] = p[t, idx[t, j]], optionally divided by the sum over j."""
    g = np.take_along_axis(probs, idx, axis=1)
    if renorm:
        g = g / g.sum(axis=1, keepdims=True)
    return g


def topk_margin(logits: np.ndarray, k: int) -> np.ndarray:
    """Smallest gap between consecutive sorted logits among the first k+1.

    For r = 1 .. min(k, N-1) this takes l_(r) - l_(r+1) of the descending
    order; a positive value means both the chosen set and its order are
    decided without ties.  Returns +inf per token when N == 1.
    """
    T, N = logits.shape
    r = min(k, N - 1)
    if r <= 0:
        return np.full(T, np.inf)
    top = -np.sort(-logits, axis=1)[:, : r + 1]
    return (top[:, :-1] - top[:, 1:]).min(axis=1)


def route(x, w_router, b_router, k: int, renorm: bool) -> dict:
    """Router step: logits, softmax probabilities, top-k indices and gates."""
    logits = router_logits(x, w_router, b_router)
    probs = softmax(logits)
    idx = select_topk(logits, k)
    gate = gate_values(probs, idx, renorm)
    return {"logits": logits, "probs": probs, "idx": idx, "gate": gate}


# ---------------------------------------------------------------- dispatch
def expert_counts(idx: np.ndarray, N: int) -> np.ndarray:
    """counts[e] = number of (token, choice) pairs routed to expert e: a
    histogram of the assignments, one increment per assignment.  An id
    outside [0, N) names no expert and is not counted."""
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = np.zeros(N, dtype=np.int64)
    np.add.at(counts, flat[(flat >= 0) & (flat < N)], 1)
    return counts


def capacity(T: int, k: int, N: int, cf: Optional[float]) -> Optional[int]:
    """Per-expert slot budget int(T*k/N * cf); None means no limit.

    Evaluated left to right in double precision and truncated, as the
    notebook's "Capacity factor" section does; a negative factor means no
    limit.
    """
    if cf is None or cf < 0:
        return None
    return int(T * k / N * cf)


def dispatch(idx: np.ndarray, N: int, C: Optional[int], priority: str = "token") -> dict:
    """Group assignments by expert, keep the first C of each.

    Assignment a = t*k + j (token t, choice j).  For expert e its assignments
    are listed in priority order and the first min(count_e, C) are kept:
    ``priority="token"`` orders them by ascending a (token order, the reading
    used for the notebook's capacity cut); ``priority="choice"`` orders them
    by (j, t), i.e. every token's first choice before any second choice (the
    GShard top-2 pattern named in the notebook's references).  ``perm`` lists
    the kept assignments (as flat indices a) expert by expert in that order,
    ``offsets`` delimits each expert's rows, ``slot[a]`` is the row of
    assignment a or -1 when dropped.
    """
    idx = np.asarray(idx, dtype=np.int64)
    if idx.ndim == 1:
        idx = idx[:, None]
    T, k = idx.shape
    flat = idx.reshape(-1)
    A = flat.size
    a_all = np.arange(A)
    if priority == "token":
        key = a_all
    elif priority == "choice":
        key = (a_all % k) * T + a_all // k  # j*T + t
    else:
        raise ValueError(f"unknown priority {priority!r}")
    counts = expert_counts(flat, N)
    slot = np.full(A, -1, dtype=np.int64)
    offsets = np.zeros(N + 1, dtype=np.int64)
    perm_parts = []
    row = 0
    for e in range(N):
        mine = np.nonzero(flat == e)[0]
        mine = mine[np.argsort(key[mine], kind="stable")]  # priority order
        kept = mine if C is None else mine[:C]
        slot[kept] = row + np.arange(kept.size)
        perm_parts.append(kept)
        row += kept.size
        offsets[e + 1] = row
    perm = np.concatenate(perm_parts) if perm_parts else np.zeros(0, dtype=np.int64)
    n_dropped = A - perm.size
    return {"counts": counts, "offsets": offsets, "perm": perm, "slot": slot,
            "n_dropped": int(n_dropped)}


def fallback_choices(logits: np.ndarray, probs: np.ndarray, k: int, R: int, renorm: bool):
    """The R next-best experts of every token after its k choices (ranks
    k .. k+R-1 of ``expert_order``) and their gates: the softmax probability,
    divided by the same sum over the k choices as the k gates when
    ``renorm``."""
    N = logits.shape[1]
    if not 1 <= k + R <= N:
        raise ValueError(f"k + R = {k + R} must lie in [1, N={N}]")
    order = expert_order(logits)[:, :k + R].astype(np.int64)
    p = np.take_along_axis(probs, order, axis=1)
    fb = p[:, k:]
    if renorm:
        fb = fb / p[:, :k].sum(axis=1, keepdims=True)
    return order[:, k:], fb


def reroute(disp: dict, idx: np.ndarray, gate: np.ndarray, fb_idx: np.ndarray, fb_gate: np.ndarray,
            N: int, C: Optional[int]) -> dict:
    """Overflow fallback after the capacity cut: a dropped assignment is sent
    to the token's next-best expert that still has room (the notebook's
    "What" section allows a fallback for the overflow; moving rejected tokens
    to experts with spare room is one of the first page's tuning tricks).

    Level r = 0 .. R-1: every token with a dropped assignment left offers its
    lowest-j one to its expert of rank k + r (``fb_idx[t, r]``); each expert
    accepts the offers in increasing token order while its rows stay within
    C.  An accepted assignment (t, j) takes that expert and the gate
    ``fb_gate[t, r]``.  Expert e's rows are its kept assignments in priority
    order (``disp``), then the accepted ones in (level, token) order.  Returns
    ``disp`` updated (counts keep the routed counts before the cut, n_dropped
    counts what stays dropped) plus the rewritten ``idx`` and ``gate`` and
    ``n_rerouted``.
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    R = fb_idx.shape[1]
    idx2 = idx.copy()
    gate2 = np.array(gate, dtype=np.float64, copy=True)
    off = disp["offsets"]
    rows = [list(disp["perm"][off[e]:off[e + 1]]) for e in range(N)]
    if C is not None:
        room = [C - len(rows[e]) for e in range(N)]
        dropped = [[j for j in range(k) if disp["slot"][t * k + j] < 0] for t in range(T)]
        for r in range(R):
            for t in range(T):
                if not dropped[t]:
                    continue
                e = int(fb_idx[t, r])
                if room[e] > 0:
                    j = dropped[t].pop(0)
                    room[e] -= 1
                    rows[e].append(t * k + j)
                    idx2[t, j] = e
                    gate2[t, j] = fb_gate[t, r]
    offsets = np.zeros(N + 1, dtype=np.int64)
    slot = np.full(T * k, -1, dtype=np.int64)
    for e in range(N):
        offsets[e + 1] = offsets[e] + len(rows[e])
        for i, a in enumerate(rows[e]):
            slot[a] = offsets[e] + i
    perm = np.array([a for e in range(N) for a in rows[e]], dtype=np.int64)
    out = dict(disp)
    out.update({"offsets": offsets, "perm": perm, "slot": slot, "n_dropped": int(T * k - perm.size),
                "n_rerouted": int(perm.size - disp["perm"].size), "idx": idx2, "gate": gate2})
    return out


def padded(disp: dict, N: int, C: int) -> dict:
    """The static capacity layout: every expert owns exactly C rows, expert e
    rows e*C .. e*C + C - 1, its kept assignments first in rank order and
    padding after (the fixed per-expert buffer the notebook's "Capacity
    factor" section sizes; the compact, count-sized layout of ``dispatch``
    is the "dynamic gating" alternative of "Towards MoE Deployment").
    ``perm`` holds -1 on padding rows; ``slot`` and ``offsets`` follow the
    new rows; counts and drops are unchanged.
    """
    if C is None:
        raise ValueError("the padded layout needs a capacity")
    off = disp["offsets"]
    perm = np.full(N * C, -1, dtype=np.int64)
    slot = np.full_like(disp["slot"], -1)
    for e in range(N):
        kept = disp["perm"][off[e]:off[e + 1]]
        perm[e * C:e * C + kept.size] = kept
        slot[kept] = e * C + np.arange(kept.size)
    out = dict(disp)
    out.update({"offsets": np.arange(N + 1) * C, "perm": perm, "slot": slot})
    return out


def with_shared(disp: dict, T: int, k: int, n_shared: int) -> dict:
    """Dispatch of a layer with ``n_shared`` always-on experts (the notebook's
    "Exercises" section: shared experts next to the routed ones).  Every
    token goes to every shared expert, uncapped, with gate 1.  Their rows come
    first: row s*T + t belongs to token t of shared expert s (``perm`` holds
    t*k there, the assignment index of the token's first choice, so that
    perm // k is the token), then the routed rows of ``disp`` shifted by
    n_shared*T.  ``offsets`` gains the n_shared groups in front; ``counts``
    and ``n_dropped`` stay those of the routed assignments.
    """
    if n_shared == 0:
        return disp
    ST = n_shared * T
    offsets = np.concatenate([np.arange(n_shared) * T, disp["offsets"] + ST])
    perm = np.concatenate([np.tile(np.arange(T) * k, n_shared), disp["perm"]])
    slot = np.where(disp["slot"] >= 0, disp["slot"] + ST, -1)
    out = dict(disp)
    out.update({"offsets": offsets, "perm": perm, "slot": slot})
    return out


def drop_rate(counts: np.ndarray, C: Optional[int]) -> float:
    """Share of the assignments that do not fit: each expert overflows by
    max(0, count - C), and the total overflow is divided by the number of
    assignments (the sum of the counts)."""
    if C is None:
        return 0.0
    overflow = sum(max(0, int(c) - C) for c in counts)
    return float(overflow / int(np.sum(counts)))


def imbalance(counts: np.ndarray, T: int, k: int, N: int) -> float:
    """Largest expert load over the perfectly balanced load T*k/N."""
    return float(np.max(counts) / (T * k / N))


def _choice_fraction(idx: np.ndarray, N: int) -> np.ndarray:
    """f[e] = share of tokens that have expert e among their choices: mark
    each (token, chosen expert) cell of a T x N table, then average each
    column."""
    idx = np.asarray(idx, dtype=np.int64)
    T = idx.shape[0]
    chosen = np.zeros((T, N), dtype=bool)
    chosen[np.repeat(np.arange(T), idx.shape[1]), idx.reshape(-1)] = True
    return chosen.sum(axis=0) / T


def switch_aux_loss(idx: np.ndarray, probs: np.ndarray, N: int) -> float:
    """The load-balancing loss of the notebook section "Switch Transformer
    auxiliary loss": N times the sum over experts of f_e (the share of tokens
    that chose e) times P_e (e's softmax probability averaged over the
    tokens)."""
    f = _choice_fraction(idx, N)
    P = np.asarray(probs, dtype=np.float64).sum(axis=0) / np.asarray(probs).shape[0]
    return float(N * np.dot(f, P))


def router_stats(idx: np.ndarray, probs: np.ndarray, counts: np.ndarray, N: int, C: Optional[int]) -> dict:
    """The router's load statistics for one batch: per expert the share f_e
    of tokens with expert e among their choices and the mean softmax
    probability P_e over all N experts, the auxiliary loss N * sum f_e P_e
    (notebook section "Switch Transformer auxiliary loss"), the imbalance
    max count / (T*k/N) and the drop rate at capacity C (section "Capacity
    factor")."""
    idx = np.asarray(idx)
    T, k = idx.shape
    f = _choice_fraction(idx, N)
    P = np.asarray(probs, dtype=np.float64).sum(axis=0) / T
    return {"frac": f, "prob_mean": P, "aux_loss": switch_aux_loss(idx, probs, N),
            "imbalance": imbalance(counts, T, k, N), "drop_rate": drop_rate(counts, C)}


# ----------------------------------------------------------------- experts
def gelu_erf(z: np.ndarray) -> np.ndarray:
    """GELU in its exact form z * Phi(z), Phi the standard normal CDF."""
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def relu(z: np.ndarray) -> np.ndarray:
    return np.maximum(z, 0.0)


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z)."""
    return z / (1.0 + np.exp(-z))


def expert_hidden(X, act: str, w1, b1=None, w3=None) -> np.ndarray:
    """First half of one expert on rows X[m, D] -> H[m, F].

    gelu/relu: H = act(X w1^T + b1) (the notebook's Expert: fc1, then the
    activation).  swiglu: H = silu(X w1^T) * (X w3^T).
    Weights use the nn.Linear layout [out, in].
    """
    X = f64(X)
    Z = X @ f64(w1).T
    if b1 is not None:
        Z = Z + f64(b1)[None, :]
    if act == "gelu":
        return gelu_erf(Z)
    if act == "relu":
        return relu(Z)
    if act == "swiglu":
        return silu(Z) * (X @ f64(w3).T)
    raise ValueError(f"unknown activation {act!r}")


def expert_output(H, w2, b2=None) -> np.ndarray:
    """Second half of one expert (fc2 of the notebook's Expert):
    Y[m, D] = H w2^T + b2."""
    Y = f64(H) @ f64(w2).T
    if b2 is not None:
        Y = Y + f64(b2)[None, :]
    return Y


def expert_mlp(X, act: str, w1, b1=None, w3=None, w2=None, b2=None) -> np.ndarray:
    """One expert on rows X[m, D] -> Y[m, D]: expert_output of expert_hidden."""
    return expert_output(expert_hidden(X, act, w1, b1, w3), w2, b2)


def _expert_params(params: dict, e: int) -> dict:
    def sl(name):
        t = params.get(name)
        return None if t is None else t[e]
    return {"w1": sl("w1"), "b1": sl("b1"), "w3": sl("w3"), "w2": sl("w2"), "b2": sl("b2")}


# ----------------------------------------------------------------- forward
def combine_from_experts(x, params: dict, act: str, k: int, gate: np.ndarray,
                         disp: dict, residual: bool,
                         tokens: Optional[Sequence[int]] = None, n_shared: int = 0) -> dict:
    """Per-expert loop of "Dispatch and gather" over the kept assignments.

    out starts at zero (or at x with ``residual``); for each expert e the
    rows of its kept assignments are gathered, run through expert e, scaled
    by their gates and added to their tokens' outputs.  With ``n_shared``
    (``disp`` from ``with_shared``) the first n_shared groups are the shared
    experts, weight slots 0..n_shared-1, gate 1; routed expert e is weight
    slot n_shared + e.  With ``tokens`` only those tokens' outputs are
    produced (rows of other tokens are skipped).  Returns ``y`` (float64,
    [T, D] or [len(tokens), D]) and ``y_perm`` (ungated expert output of
    every computed kept row; NaN elsewhere).
    """
    xs = x
    T = xs.shape[0]
    D = xs.shape[1]
    perm = disp["perm"]
    offsets = disp["offsets"]
    N = offsets.size - 1
    if tokens is None:
        want = np.ones(T, dtype=bool)
        out_rows = np.arange(T)
    else:
        tokens = np.asarray(tokens, dtype=np.int64)
        want = np.zeros(T, dtype=bool)
        want[tokens] = True
        out_rows = tokens
    where = np.full(T, -1, dtype=np.int64)
    where[out_rows] = np.arange(out_rows.size)
    out = np.zeros((out_rows.size, D), dtype=np.float64)
    if residual:
        out += f64(xs[out_rows] if tokens is not None else xs)
    y_perm = np.full((perm.size, D), np.nan)
    for e in range(N):
        rows = np.arange(offsets[e], offsets[e + 1])
        a = perm[rows]
        rows, a = rows[a >= 0], a[a >= 0]  # padding rows of the static layout carry nothing
        t = a // k
        sel = want[t]
        if not sel.any():
            continue
        rows, a, t = rows[sel], a[sel], t[sel]
        j = a % k
        Ye = expert_mlp(f64(xs[t]), act, **_expert_params(params, e))
        y_perm[rows] = Ye
        g = np.ones(t.size) if e < n_shared else gate[t, j]
        np.add.at(out, where[t], Ye * g[:, None])
    return {"y": out, "y_perm": y_perm}


def combine_rows(y_perm, slot, gate, k: int, x=None, n_shared: int = 0) -> np.ndarray:
    """Aggregation alone, from given expert output rows: out[t] is the sum
    over choices j whose assignment t*k+j was kept of gate[t, j] times row
    slot[t*k+j] of y_perm, plus rows s*T + t of the n_shared shared experts
    (gate 1), plus x[t] when x is given."""
    y_perm = f64(y_perm)
    slot = np.asarray(slot).reshape(-1)
    gate = np.asarray(gate, dtype=np.float64)
    T = gate.shape[0]
    out = np.zeros((T, y_perm.shape[1])) if x is None else f64(x).copy()
    for t in range(T):
        for s_ in range(n_shared):
            out[t] += y_perm[s_ * T + t]
        for j in range(k):
            s = slot[t * k + j]
            if s >= 0:
                out[t] += gate[t, j] * y_perm[s]
    return out


def moe_forward(x, params: dict, *, k: int, act: str, renorm: bool = False,
                capacity_slots: Optional[int] = None, residual: bool = False,
                tokens: Optional[Sequence[int]] = None, priority: str = "token",
                n_shared: int = 0, layout: str = "compact", n_fallback: int = 0) -> dict:
    """Whole layer: route, dispatch with capacity, experts, combine.

    ``params`` holds w_router, b_router, w1, b1, w3, w2, b2 (numpy arrays or
    CPU tensors in the C-ABI layouts; absent entries are None); the expert
    stacks hold n_shared shared experts first, then the routed ones.
    ``priority`` is the capacity order of ``dispatch``; ``layout`` is
    "compact" (rows sized by the counts) or "padded" (``padded``: C rows
    per expert); ``n_fallback`` = R > 0 reroutes dropped assignments over R
    levels (``reroute``, compact layout).
    """
    r = route(x, params["w_router"], params.get("b_router"), k, renorm)
    N = r["logits"].shape[1]
    d = dispatch(r["idx"], N, capacity_slots, priority)
    if n_fallback:
        if layout != "compact":
            raise ValueError("rerouting uses the compact layout")
        fb_idx, fb_gate = fallback_choices(r["logits"], r["probs"], k, n_fallback, renorm)
        d = reroute(d, r["idx"], r["gate"], fb_idx, fb_gate, N, capacity_slots)
        r = dict(r)
        r.update({"idx": d.pop("idx"), "gate": d.pop("gate"), "fb_idx": fb_idx, "fb_gate": fb_gate})
    if layout == "padded":
        d = padded(d, N, capacity_slots)
    elif layout != "compact":
        raise ValueError(f"unknown layout {layout!r}")
    d = with_shared(d, f64(x).shape[0], k, n_shared)
    c = combine_from_experts(x, params, act, k, r["gate"], d, residual, tokens, n_shared)
    out = dict(r)
    out.update(d)
    out.update(c)
    return out


def brute_forward(x, params: dict, *, k: int, act: str, renorm: bool = False,
                  capacity_slots: Optional[int] = None, residual: bool = False,
                  priority: str = "token", n_shared: int = 0) -> np.ndarray:
    """Second formulation for tiny inputs: every expert on every token.

    Builds the sparse gate matrix G[t, e] (the gate of each kept assignment,
    zero elsewhere) and contracts it with the dense stack of all experts'
    outputs.  Kept assignments are found by counting, for each (t, j), the
    assignments to the same expert that come before it in the priority order
    (O(A^2)): earlier flat index (token order) or earlier (choice, token).
    """
    X = f64(x)
    T = X.shape[0]
    logits = router_logits(X, params["w_router"], params.get("b_router"))
    N = logits.shape[1]
    # selection by explicit comparison: expert e precedes e' when its logit is
    # larger, or equal with a smaller index
    idx = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        order = sorted(range(N), key=lambda e: (-logits[t, e], e))
        idx[t] = order[:k]
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    g = np.array([[p[t, idx[t, j]] for j in range(k)] for t in range(T)])
    if renorm:
        g = g / g.sum(axis=1, keepdims=True)
    flat = idx.reshape(-1)
    G = np.zeros((T, N))
    for a in range(flat.size):
        t, j = divmod(a, k)
        if priority == "token":
            rank = int((flat[:a] == flat[a]).sum())
        else:
            rank = sum(1 for b in range(flat.size)
                       if flat[b] == flat[a] and (b % k, b // k) < (j, t))
        if capacity_slots is None or rank < capacity_slots:
            G[a // k, flat[a]] += g[a // k, a % k]
    Yall = np.stack([expert_mlp(X, act, **_expert_params(params, n_shared + e)) for e in range(N)])
    y = np.einsum("te,ted->td", G, Yall.transpose(1, 0, 2))
    for s_ in range(n_shared):  # always-on experts, gate 1
        y = y + expert_mlp(X, act, **_expert_params(params, s_))
    if residual:
        y = y + X
    return y
