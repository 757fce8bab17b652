"""Python binding of the C ABI (include/moe.h): argument marshalling only.

Each function takes torch tensors that already live on the GPU, checks that
their dtype, device and contiguity match what the C entry point reads, and
passes raw pointers plus the current HIP stream.  Every step of the layer runs
in the HIP library; nothing here computes.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as L

_DT = {"fp32": (L.MOE_DTYPE_F32, torch.float32), "bf16": (L.MOE_DTYPE_BF16, torch.bfloat16)}
_ACT = {"gelu": L.MOE_ACT_GELU, "relu": L.MOE_ACT_RELU, "swiglu": L.MOE_ACT_SWIGLU}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = L.load().moe_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


@dataclass(frozen=True)
class MoeShape:
    T: int
    D: int
    F: int
    N: int
    k: int
    capacity: int = -1
    dtype: str = "bf16"
    act: str = "swiglu"
    renorm: bool = False
    residual: bool = False
    has_bias: bool = False
    router_bias: bool = False
    fused_decode: bool = False  # MOE_FUSED_DECODE algorithm choice
    slot_major: bool = False    # MOE_SLOT_MAJOR capacity priority (choice, token)
    n_shared: int = 0           # always-on experts (expert slots 0..n_shared-1)
    padded: bool = False        # MOE_PADDED static capacity layout (N*capacity rows)

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DT[self.dtype][1]

    @property
    def group_rows(self) -> int:
        """Rows of the grouped buffers (perm, y_perm, hidden rows)."""
        routed = self.N * self.capacity if self.padded else self.T * self.k
        return self.T * self.n_shared + routed

    def c(self) -> L.MoeShapeC:
        flags = ((L.MOE_RENORM if self.renorm else 0) | (L.MOE_RESIDUAL if self.residual else 0)
                 | (L.MOE_HAS_BIAS if self.has_bias else 0)
                 | (L.MOE_ROUTER_BIAS if self.router_bias else 0)
                 | (L.MOE_FUSED_DECODE if self.fused_decode else 0)
                 | (L.MOE_SLOT_MAJOR if self.slot_major else 0)
                 | (L.MOE_PADDED if self.padded else 0))
        return L.MoeShapeC(self.T, self.D, self.F, self.N, self.k, self.capacity,
                           _DT[self.dtype][0], _ACT[self.act], flags, self.n_shared)

    @staticmethod
    def from_config(cfg, T: Optional[int] = None, fused_decode: bool = False) -> "MoeShape":
        T = cfg.T if T is None else T
        cap = capacity(T, cfg.k, cfg.N, -1.0 if cfg.cf is None else cfg.cf)
        return MoeShape(T=T, D=cfg.D, F=cfg.F, N=cfg.N, k=cfg.k, capacity=cap, dtype=cfg.dtype,
                        act=cfg.act, renorm=cfg.renorm, residual=cfg.residual,
                        has_bias=cfg.expert_bias, router_bias=cfg.router_bias is not None,
                        fused_decode=fused_decode, n_shared=getattr(cfg, "n_shared", 0))


def _ptr(t: Optional[torch.Tensor], dtype: Optional[torch.dtype] = None, name: str = "",
         n: Optional[int] = None) -> Optional[int]:
    """Device address of t after checking device, layout, dtype and, when n is
    given, that t holds at least n elements (the library trusts its sizes)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if n is not None and t.numel() < n:
        raise ValueError(f"{name}: {t.numel()} elements, the shape needs {n}")
    return t.data_ptr()


def _slots(shape: "MoeShape") -> int:
    return shape.n_shared + shape.N  # expert slots of the weight stacks


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != L.MOE_OK:
        raise MoeError(fn, status)


def capacity(T: int, k: int, N: int, cf: float) -> int:
    return int(L.load().moe_capacity(T, k, N, float(cf)))


def workspace_bytes(shape: MoeShape) -> int:
    n = ctypes.c_size_t(0)
    sc = shape.c()
    _check("moe_workspace_bytes", L.load().moe_workspace_bytes(ctypes.byref(sc), ctypes.byref(n)))
    return int(n.value)


def route(shape: MoeShape, x, w_router, b_router, topk_idx, topk_gate, logits=None, stream=None, ws=None):
    """ws (optional, >= workspace_bytes) lets few-token bf16 batches use the
    two-launch split router, as moe_forward does."""
    dt = shape.torch_dtype
    sc = shape.c()
    wp, wn = _ws_arg(ws)
    _check("moe_route", L.load().moe_route(
        ctypes.byref(sc), _ptr(x, dt, "x", shape.T * shape.D), _ptr(w_router, dt, "w_router", shape.N * shape.D),
        _ptr(b_router, torch.float32, "b_router", shape.N), _ptr(topk_idx, torch.int32, "topk_idx", shape.T * shape.k),
        _ptr(topk_gate, torch.float32, "topk_gate", shape.T * shape.k), _ptr(logits, torch.float32, "logits", shape.T * shape.N),
        wp, wn, _stream(stream)))


def stats_workspace_bytes(shape: MoeShape) -> int:
    n = ctypes.c_size_t(0)
    sc = shape.c()
    _check("moe_stats_workspace_bytes", L.load().moe_stats_workspace_bytes(ctypes.byref(sc), ctypes.byref(n)))
    return int(n.value)


def route_stats(shape: MoeShape, x, w_router, b_router, topk_idx, topk_gate, stats_ws, logits=None,
                stream=None):
    dt = shape.torch_dtype
    sc = shape.c()
    _check("moe_route_stats", L.load().moe_route_stats(
        ctypes.byref(sc), _ptr(x, dt, "x", shape.T * shape.D), _ptr(w_router, dt, "w_router", shape.N * shape.D),
        _ptr(b_router, torch.float32, "b_router", shape.N), _ptr(topk_idx, torch.int32, "topk_idx", shape.T * shape.k),
        _ptr(topk_gate, torch.float32, "topk_gate", shape.T * shape.k), _ptr(logits, torch.float32, "logits", shape.T * shape.N),
        *_ws_arg(stats_ws), _stream(stream)))


def router_stats(shape: MoeShape, stats_ws, counts, n_dropped, prob_mean, frac, summary, stream=None):
    i32, f64 = torch.int32, torch.float64
    sc = shape.c()
    _check("moe_router_stats", L.load().moe_router_stats(
        ctypes.byref(sc), *_ws_arg(stats_ws), _ptr(counts, i32, "counts", shape.N),
        _ptr(n_dropped, i32, "n_dropped", 1), _ptr(prob_mean, f64, "prob_mean", shape.N), _ptr(frac, f64, "frac", shape.N),
        _ptr(summary, f64, "summary", 3), _stream(stream)))


def route_fallback(shape: MoeShape, x, w_router, b_router, topk_idx, topk_gate, n_fallback, fb_idx, fb_gate,
                   logits=None, stream=None):
    dt = shape.torch_dtype
    sc = shape.c()
    _check("moe_route_fallback", L.load().moe_route_fallback(
        ctypes.byref(sc), _ptr(x, dt, "x", shape.T * shape.D), _ptr(w_router, dt, "w_router", shape.N * shape.D),
        _ptr(b_router, torch.float32, "b_router", shape.N), _ptr(topk_idx, torch.int32, "topk_idx", shape.T * shape.k),
        _ptr(topk_gate, torch.float32, "topk_gate", shape.T * shape.k), int(n_fallback), _ptr(fb_idx, torch.int32, "fb_idx", shape.T * int(n_fallback)),
        _ptr(fb_gate, torch.float32, "fb_gate", shape.T * int(n_fallback)), _ptr(logits, torch.float32, "logits", shape.T * shape.N), _stream(stream)))


def dispatch_reroute(shape: MoeShape, n_fallback, fb_idx, fb_gate, topk_idx, topk_gate, counts, offsets, perm,
                     slot, n_dropped, stream=None):
    i32 = torch.int32
    sc = shape.c()
    _check("moe_dispatch_reroute", L.load().moe_dispatch_reroute(
        ctypes.byref(sc), int(n_fallback), _ptr(fb_idx, i32, "fb_idx", shape.T * int(n_fallback)), _ptr(fb_gate, torch.float32, "fb_gate", shape.T * int(n_fallback)),
        _ptr(topk_idx, i32, "topk_idx", shape.T * shape.k), _ptr(topk_gate, torch.float32, "topk_gate", shape.T * shape.k),
        _ptr(counts, i32, "counts", shape.N), _ptr(offsets, i32, "offsets", shape.n_shared + shape.N + 1), _ptr(perm, i32, "perm", shape.group_rows),
        _ptr(slot, i32, "slot", shape.T * shape.k), _ptr(n_dropped, i32, "n_dropped", 1), _stream(stream)))


def dispatch(shape: MoeShape, topk_idx, counts, offsets, perm, slot, n_dropped, stream=None, ws=None):
    """ws (optional, >= workspace_bytes) lets large batches use the
    multi-workgroup dispatch; the results are the same."""
    i32 = torch.int32
    sc = shape.c()
    wp, wn = _ws_arg(ws)
    _check("moe_dispatch", L.load().moe_dispatch(
        ctypes.byref(sc), _ptr(topk_idx, i32, "topk_idx", shape.T * shape.k), _ptr(counts, i32, "counts", shape.N),
        _ptr(offsets, i32, "offsets", shape.n_shared + shape.N + 1), _ptr(perm, i32, "perm", shape.group_rows),
        _ptr(slot, i32, "slot", shape.T * shape.k), _ptr(n_dropped, i32, "n_dropped", 1), wp, wn, _stream(stream)))


def expert_ffn(shape: MoeShape, x, perm, offsets, w1, b1, w3, w2, b2, y_perm, ws, stream=None):
    dt = shape.torch_dtype
    i32 = torch.int32
    sc = shape.c()
    _check("moe_expert_ffn", L.load().moe_expert_ffn(
        ctypes.byref(sc), _ptr(x, dt, "x", shape.T * shape.D), _ptr(perm, i32, "perm", shape.group_rows), _ptr(offsets, i32, "offsets", shape.n_shared + shape.N + 1),
        _ptr(w1, dt, "w1", _slots(shape) * shape.F * shape.D), _ptr(b1, dt, "b1", _slots(shape) * shape.F), _ptr(w3, dt, "w3", _slots(shape) * shape.F * shape.D), _ptr(w2, dt, "w2", _slots(shape) * shape.D * shape.F),
        _ptr(b2, dt, "b2", _slots(shape) * shape.D), _ptr(y_perm, dt, "y_perm", shape.group_rows * shape.D), _ptr(ws, None, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)))


def _ws_arg(ws):
    if ws is None:
        return None, 0
    return _ptr(ws, None, "ws"), ws.numel() * ws.element_size()


def expert_up(shape: MoeShape, x, perm, offsets, w1, b1, w3, h, ws=None, stream=None):
    """fc1 + activation into h; ws (optional, >= workspace_bytes) allows the
    split of the last round of tiles, as moe_expert_ffn does."""
    dt = shape.torch_dtype
    i32 = torch.int32
    sc = shape.c()
    wp, wn = _ws_arg(ws)
    _check("moe_expert_up", L.load().moe_expert_up(
        ctypes.byref(sc), _ptr(x, dt, "x", shape.T * shape.D), _ptr(perm, i32, "perm", shape.group_rows), _ptr(offsets, i32, "offsets", shape.n_shared + shape.N + 1),
        _ptr(w1, dt, "w1", _slots(shape) * shape.F * shape.D), _ptr(b1, dt, "b1", _slots(shape) * shape.F), _ptr(w3, dt, "w3", _slots(shape) * shape.F * shape.D), _ptr(h, dt, "h", shape.group_rows * shape.F), wp, wn,
        _stream(stream)))


def expert_down(shape: MoeShape, h, offsets, w2, b2, y_perm, ws=None, stream=None):
    """fc2 of the hidden rows into y_perm; ws as for expert_up."""
    dt = shape.torch_dtype
    sc = shape.c()
    wp, wn = _ws_arg(ws)
    _check("moe_expert_down", L.load().moe_expert_down(
        ctypes.byref(sc), _ptr(h, dt, "h", shape.group_rows * shape.F), _ptr(offsets, torch.int32, "offsets", shape.n_shared + shape.N + 1),
        _ptr(w2, dt, "w2", _slots(shape) * shape.D * shape.F), _ptr(b2, dt, "b2", _slots(shape) * shape.D), _ptr(y_perm, dt, "y_perm", shape.group_rows * shape.D), wp, wn, _stream(stream)))


def combine(shape: MoeShape, y_perm, slot, topk_gate, x_residual, out, stream=None):
    dt = shape.torch_dtype
    sc = shape.c()
    _check("moe_combine", L.load().moe_combine(
        ctypes.byref(sc), _ptr(y_perm, dt, "y_perm", shape.group_rows * shape.D), _ptr(slot, torch.int32, "slot", shape.T * shape.k),
        _ptr(topk_gate, torch.float32, "topk_gate", shape.T * shape.k), _ptr(x_residual, dt, "x_residual", shape.T * shape.D),
        _ptr(out, dt, "out", shape.T * shape.D), _stream(stream)))


def forward(shape: MoeShape, x, w_router, b_router, w1, b1, w3, w2, b2, out, topk_idx, topk_gate,
            counts, offsets, perm, slot, n_dropped, ws, stream=None):
    dt = shape.torch_dtype
    i32 = torch.int32
    sc = shape.c()
    _check("moe_forward", L.load().moe_forward(
        ctypes.byref(sc), _ptr(x, dt, "x", shape.T * shape.D), _ptr(w_router, dt, "w_router", shape.N * shape.D),
        _ptr(b_router, torch.float32, "b_router", shape.N), _ptr(w1, dt, "w1", _slots(shape) * shape.F * shape.D), _ptr(b1, dt, "b1", _slots(shape) * shape.F),
        _ptr(w3, dt, "w3", _slots(shape) * shape.F * shape.D), _ptr(w2, dt, "w2", _slots(shape) * shape.D * shape.F), _ptr(b2, dt, "b2", _slots(shape) * shape.D), _ptr(out, dt, "out", shape.T * shape.D),
        _ptr(topk_idx, i32, "topk_idx", shape.T * shape.k), _ptr(topk_gate, torch.float32, "topk_gate", shape.T * shape.k),
        _ptr(counts, i32, "counts", shape.N), _ptr(offsets, i32, "offsets", shape.n_shared + shape.N + 1), _ptr(perm, i32, "perm", shape.group_rows),
        _ptr(slot, i32, "slot", shape.T * shape.k), _ptr(n_dropped, i32, "n_dropped", 1), _ptr(ws, None, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)))


def forward_noalloc(shape: MoeShape, x, w_router, b_router, w1, b1, w3, w2, b2, out, topk_idx, topk_gate,
                    counts, offsets, perm, slot, n_dropped, stream=None):
    """moe_forward with the library's own device scratch as the workspace
    (no workspace argument; layers up to MOE_NOALLOC_SCRATCH_BYTES)."""
    dt = shape.torch_dtype
    i32 = torch.int32
    sc = shape.c()
    _check("moe_forward_noalloc", L.load().moe_forward_noalloc(
        ctypes.byref(sc), _ptr(x, dt, "x", shape.T * shape.D), _ptr(w_router, dt, "w_router", shape.N * shape.D),
        _ptr(b_router, torch.float32, "b_router", shape.N), _ptr(w1, dt, "w1", _slots(shape) * shape.F * shape.D), _ptr(b1, dt, "b1", _slots(shape) * shape.F),
        _ptr(w3, dt, "w3", _slots(shape) * shape.F * shape.D), _ptr(w2, dt, "w2", _slots(shape) * shape.D * shape.F), _ptr(b2, dt, "b2", _slots(shape) * shape.D), _ptr(out, dt, "out", shape.T * shape.D),
        _ptr(topk_idx, i32, "topk_idx", shape.T * shape.k), _ptr(topk_gate, torch.float32, "topk_gate", shape.T * shape.k),
        _ptr(counts, i32, "counts", shape.N), _ptr(offsets, i32, "offsets", shape.n_shared + shape.N + 1), _ptr(perm, i32, "perm", shape.group_rows),
        _ptr(slot, i32, "slot", shape.T * shape.k), _ptr(n_dropped, i32, "n_dropped", 1), _stream(stream)))


def clock_probe(blocks: int, delay_us: float, iters: int, stamps, stream=None):
    """Shader-clock probe (moe_clock_probe): a chain of 1024*iters dependent
    adds per workgroup; stamps is a device int64 tensor of at least 4*blocks
    entries, filled with {realtime start, realtime end, adds in the chain,
    chain value} per workgroup."""
    _check("moe_clock_probe", L.load().moe_clock_probe(
        int(blocks), float(delay_us), int(iters), _ptr(stamps, torch.int64, "stamps", 4 * int(blocks)),
        _stream(stream)))


def probe_clock_ghz(stamps) -> float:
    """Median core clock in GHz over the probe's workgroups: 4 shader clocks
    per dependent add, over the elapsed ticks of the 100 MHz real-time
    counter (host arithmetic on the copied-back stamps)."""
    s = stamps.view(-1, 4).cpu().tolist()
    rates = sorted(4.0 * n / ((r1 - r0) * 10.0) for r0, r1, n, _ in s if r1 > r0)
    return rates[len(rates) // 2] if rates else float("nan")


class MoeBuffers:
    """Device buffers of one layer call (outputs, routing tensors, workspace),
    allocated once with torch so that repeated calls allocate nothing."""

    def __init__(self, shape: MoeShape, device="cuda"):
        self.shape = shape
        A = shape.T * shape.k
        i32 = dict(dtype=torch.int32, device=device)
        self.out = torch.empty(shape.T, shape.D, dtype=shape.torch_dtype, device=device)
        self.topk_idx = torch.empty(shape.T, shape.k, **i32)
        self.topk_gate = torch.empty(shape.T, shape.k, dtype=torch.float32, device=device)
        self.counts = torch.empty(shape.N, **i32)
        self.offsets = torch.empty(shape.n_shared + shape.N + 1, **i32)
        self.perm = torch.empty(max(shape.group_rows, 1), **i32)
        self.slot = torch.empty(max(A, 1), **i32)
        self.n_dropped = torch.empty(1, **i32)
        self.ws = torch.empty(max(workspace_bytes(shape), 256), dtype=torch.uint8, device=device)

    def forward(self, x, p: dict, stream=None):
        forward(self.shape, x, p["w_router"], p.get("b_router"), p["w1"], p.get("b1"), p.get("w3"),
                p["w2"], p.get("b2"), self.out, self.topk_idx, self.topk_gate, self.counts,
                self.offsets, self.perm, self.slot, self.n_dropped, self.ws, stream)
        return self.out
