"""The C-ABI library loads, exports every entry point that include/moe.h
declares, and rejects bad arguments on the host before any launch.  No call
here reaches the GPU (every call fails validation or is host-only)."""
import ctypes
import os
import re

import pytest

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(moe_[a-z_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    from mixture_experts_layer_expert_amd import _lib
    return _lib.load()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_expert_up", "moe_expert_down",
              "moe_combine", "moe_forward", "moe_route_stats", "moe_router_stats", "moe_route_fallback",
              "moe_dispatch_reroute",
              "moe_capacity", "moe_workspace_bytes", "moe_stats_workspace_bytes", "moe_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in _declared_functions():
        assert hasattr(lib, n), n
        assert isinstance(getattr(lib, n), ctypes._CFuncPtr)


def test_status_strings(lib):
    from mixture_experts_layer_expert_amd import _lib as L
    for code in (L.MOE_OK, L.MOE_ERR_INVALID_ARG, L.MOE_ERR_UNSUPPORTED, L.MOE_ERR_WORKSPACE, L.MOE_ERR_HIP):
        assert lib.moe_status_string(code).decode() not in ("", "unknown status")
    assert lib.moe_status_string(12345).decode() == "unknown status"


def test_capacity_helper_matches_the_notebook_rule(lib):
    assert lib.moe_capacity(16384, 1, 128, 1.0) == 128
    assert lib.moe_capacity(16384, 1, 128, 1.5) == 192
    assert lib.moe_capacity(1024, 2, 8, 1.0) == 256
    assert lib.moe_capacity(10, 1, 3, 1.0) == 3   # truncation
    assert lib.moe_capacity(10, 2, 3, 0.0) == 0
    assert lib.moe_capacity(10, 2, 3, -1.0) == -1
    assert lib.moe_capacity(10, 2, 3, float("nan")) == -1
    assert lib.moe_capacity(2**40, 8, 1, 1.0) == 2**31 - 1


def _shape(**kw):
    from mixture_experts_layer_expert_amd import _lib as L
    base = dict(T=64, D=128, F=256, N=8, k=2, capacity=-1, dtype=L.MOE_DTYPE_BF16,
                act=L.MOE_ACT_SWIGLU, flags=0)
    base.update(kw)
    return L.MoeShapeC(**base)


def _ws(lib, s):
    n = ctypes.c_size_t(0)
    rc = lib.moe_workspace_bytes(ctypes.byref(s), ctypes.byref(n))
    return rc, n.value


def test_workspace_bytes_and_validation(lib):
    from mixture_experts_layer_expert_amd import _lib as L
    # prefill-shaped (many rows per expert): y_perm[T*k, D] + H[T*k, F], bf16,
    # + fp32 split-K partial tiles, one 256x256 tile per workgroup of the
    # persistent grid (one per CU; 256 without a device), + the split header
    # (16 bytes per workgroup and 16 more, rounded up to 256)
    grid = 256
    hdr = (16 * (grid + 1) + 255) // 256 * 256
    rc, n = _ws(lib, _shape(T=4096))
    assert rc == L.MOE_OK
    assert n == 4096 * 2 * 128 * 2 + 4096 * 2 * 256 * 2 + grid * 256 * 256 * 4 + hdr
    # decode-shaped (<= 16 rows per expert): grouped GEMM by default (32x256
    # tiles) ...
    rc, n = _ws(lib, _shape(T=64))
    assert rc == L.MOE_OK
    assert n == 64 * 2 * 128 * 2 + 64 * 2 * 256 * 2 + grid * 32 * 256 * 4 + hdr
    # two shared experts: the grouped rows grow by 2*T
    rc, n = _ws(lib, _shape(T=4096, n_shared=2))
    assert rc == L.MOE_OK
    assert n == 4096 * 4 * 128 * 2 + 4096 * 4 * 256 * 2 + grid * 256 * 256 * 4 + hdr
    # padded layout, capacity 1536: N*C = 12288 grouped rows instead of T*k
    rc, n = _ws(lib, _shape(T=4096, capacity=1536, flags=L.MOE_PADDED))
    assert rc == L.MOE_OK
    assert n == 12288 * 128 * 2 + 12288 * 256 * 2 + grid * 256 * 256 * 4 + hdr
    # mid-size groups bounded by a capacity of at most 128 rows: 128x256 tiles
    # up, 128x384 down (the larger partial tile)
    rc, n = _ws(lib, _shape(T=4096, N=64, capacity=128, act=L.MOE_ACT_RELU))
    assert rc == L.MOE_OK
    assert n == 4096 * 2 * 128 * 2 + 4096 * 2 * 256 * 2 + grid * 128 * 384 * 4 + hdr
    # ... not bounded (capacity 192): 128x256 both ways
    rc, n = _ws(lib, _shape(T=4096, N=64, capacity=192, act=L.MOE_ACT_RELU))
    assert rc == L.MOE_OK
    assert n == 4096 * 2 * 128 * 2 + 4096 * 2 * 256 * 2 + grid * 128 * 256 * 4 + hdr
    assert _ws(lib, _shape(n_shared=-1))[0] == L.MOE_ERR_INVALID_ARG
    assert _ws(lib, _shape(N=250, n_shared=7))[0] == L.MOE_ERR_UNSUPPORTED
    # fp32 layers never split
    rc, n = _ws(lib, _shape(T=64, dtype=L.MOE_DTYPE_F32, act=L.MOE_ACT_GELU))
    assert rc == L.MOE_OK
    assert n == 64 * 2 * 128 * 4 + 64 * 2 * 256 * 4
    # ... and with the fused decode kernel y_perm + fp32 partials of the F
    # shards; 8 experts -> 32 shards wanted, reduced until the shard is one
    # of the compiled widths (128, 256, 352, 384 columns) -> 2 shards of 128
    rc, n = _ws(lib, _shape(T=64, flags=L.MOE_FUSED_DECODE))
    assert rc == L.MOE_OK
    assert n == 64 * 2 * 128 * 2 + 2 * 64 * 2 * 128 * 4
    bad = [
        (dict(k=0), L.MOE_ERR_INVALID_ARG), (dict(k=9, N=16), L.MOE_ERR_UNSUPPORTED),
        (dict(k=9), L.MOE_ERR_INVALID_ARG), (dict(N=300, k=2), L.MOE_ERR_UNSUPPORTED),
        (dict(T=-1), L.MOE_ERR_INVALID_ARG), (dict(capacity=-2), L.MOE_ERR_INVALID_ARG),
        (dict(dtype=7), L.MOE_ERR_INVALID_ARG), (dict(act=5), L.MOE_ERR_INVALID_ARG),
        (dict(flags=1 << 7), L.MOE_ERR_INVALID_ARG), (dict(D=100), L.MOE_ERR_UNSUPPORTED),
        (dict(flags=L.MOE_PADDED), L.MOE_ERR_INVALID_ARG),  # padded layout without a capacity
        (dict(F=96), L.MOE_ERR_UNSUPPORTED), (dict(flags=L.MOE_HAS_BIAS), L.MOE_ERR_UNSUPPORTED),
        (dict(T=2**31, D=4096), L.MOE_ERR_UNSUPPORTED),
    ]
    for kw, want in bad:
        assert _ws(lib, _shape(**kw))[0] == want, kw
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_bytes(None, ctypes.byref(n)) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_workspace_bytes(ctypes.byref(_shape()), None) == L.MOE_ERR_INVALID_ARG
    # fp32 needs multiples of 16
    assert _ws(lib, _shape(dtype=L.MOE_DTYPE_F32, D=48, F=80))[0] == L.MOE_OK
    assert _ws(lib, _shape(dtype=L.MOE_DTYPE_F32, D=40, F=80))[0] == L.MOE_ERR_UNSUPPORTED


def test_fused_decode_flag_applies_only_to_the_compiled_shapes(lib):
    """The fused decode kernel takes bf16 layers of at most 16 rows per
    expert, D a multiple of 128 and an F shard of 128, 256, 352 or 384
    columns; elsewhere the flag falls back to the grouped GEMMs, whose
    workspace then equals the one without the flag."""
    from mixture_experts_layer_expert_amd import _lib as L
    decode = dict(T=128, D=2048, F=1408, N=64, k=6)

    def ws(flags, **kw):
        rc, n = _ws(lib, _shape(**{**decode, **kw, "flags": flags}))
        assert rc == L.MOE_OK
        return n

    F = L.MOE_FUSED_DECODE
    # taken: 4 shards of 352 columns, fp32 partials of every assignment row
    assert ws(F) == 768 * 2048 * 2 + 4 * 768 * 2048 * 4
    assert ws(F) != ws(0)
    for kw in (dict(D=192), dict(F=1600), dict(T=4096), dict(dtype=L.MOE_DTYPE_F32, act=L.MOE_ACT_GELU)):
        assert ws(F, **kw) == ws(0, **kw), kw


def test_stats_workspace_bytes_and_validation(lib):
    """One fp32 partial per (router block, expert), rounded up to 256 bytes,
    then 256 bytes for the ticket of the second pass: bf16 with D % 128 == 0
    uses 16 tokens per block below 32 tokens per CU (256 CUs without a
    device) and for at most 16 experts, fp32 32 tokens per block."""
    from mixture_experts_layer_expert_amd import _lib as L
    n = ctypes.c_size_t(0)
    assert lib.moe_stats_workspace_bytes(ctypes.byref(_shape(T=4096)), ctypes.byref(n)) == L.MOE_OK
    assert n.value == (4096 // 16) * 8 * 4 + 256
    # 64 tokens per block from 64 per CU on, for more than 16 experts
    assert lib.moe_stats_workspace_bytes(ctypes.byref(_shape(T=4096 * 4, N=32)), ctypes.byref(n)) == L.MOE_OK
    assert n.value == (4096 * 4 // 64) * 32 * 4 + 256
    # at most 16 experts: always 16 tokens per block
    assert lib.moe_stats_workspace_bytes(ctypes.byref(_shape(T=4096 * 4)), ctypes.byref(n)) == L.MOE_OK
    assert n.value == (4096 * 4 // 16) * 8 * 4 + 256
    s32 = _shape(T=1000, dtype=L.MOE_DTYPE_F32, act=L.MOE_ACT_GELU)
    assert lib.moe_stats_workspace_bytes(ctypes.byref(s32), ctypes.byref(n)) == L.MOE_OK
    assert n.value == 1024 + 256  # 32 blocks * 8 experts * 4 bytes, rounded up to 256 bytes
    assert lib.moe_stats_workspace_bytes(ctypes.byref(_shape(k=0)), ctypes.byref(n)) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_stats_workspace_bytes(ctypes.byref(_shape()), None) == L.MOE_ERR_INVALID_ARG
    s = ctypes.byref(_shape())
    fake = ctypes.c_void_p(0x1000)
    assert lib.moe_route_stats(s, fake, fake, None, fake, fake, None, None, 1 << 20,
                               None) == L.MOE_ERR_WORKSPACE
    assert lib.moe_route_stats(s, fake, fake, None, fake, fake, None, fake, 16, None) == L.MOE_ERR_WORKSPACE
    assert lib.moe_route_stats(s, fake, fake, None, fake, fake, None, ctypes.c_void_p(0x1001), 1 << 20,
                               None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_route_stats(s, None, fake, None, fake, fake, None, fake, 1 << 20,
                               None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_router_stats(s, fake, 1 << 20, None, fake, fake, None, fake, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_router_stats(s, fake, 1 << 20, fake, fake, fake, None, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_router_stats(s, fake, 8, fake, fake, fake, None, fake, None) == L.MOE_ERR_WORKSPACE
    z = ctypes.byref(_shape(T=0))
    assert lib.moe_route_stats(z, fake, fake, None, fake, fake, None, None, 0, None) == L.MOE_OK
    assert lib.moe_router_stats(z, None, 0, fake, fake, fake, None, fake, None) == L.MOE_OK


def test_reroute_entry_points_validate(lib):
    """Fallback depth R: >= 1, k + R <= min(8, N); compact layout only;
    T = 0 is a no-op once the arguments are valid."""
    from mixture_experts_layer_expert_amd import _lib as L
    fake = ctypes.c_void_p(0x1000)
    s = ctypes.byref(_shape(k=2, N=8, capacity=10))
    route = lambda sh, R, fb=fake: lib.moe_route_fallback(sh, fake, fake, None, fake, fake, R, fb, fb, None, None)
    disp = lambda sh, R, fb=fake: lib.moe_dispatch_reroute(sh, R, fb, fb, fake, fake, fake, fake, fake, fake, fake,
                                                           None)
    for f in (route, disp):
        assert f(s, 0) == L.MOE_ERR_INVALID_ARG
        assert f(s, 7) == L.MOE_ERR_UNSUPPORTED  # k + R = 9 > 8
        assert f(ctypes.byref(_shape(k=2, N=3, capacity=10)), 2) == L.MOE_ERR_UNSUPPORTED  # k + R > N
        assert f(ctypes.byref(_shape(k=2, N=8, capacity=10, flags=L.MOE_PADDED)), 1) == L.MOE_ERR_UNSUPPORTED
        assert f(s, 2, None) == L.MOE_ERR_INVALID_ARG
        assert f(ctypes.byref(_shape(T=0, k=2, N=8, capacity=10)), 2) == L.MOE_OK


def test_entry_points_reject_null_pointers_before_launch(lib):
    from mixture_experts_layer_expert_amd import _lib as L
    s = ctypes.byref(_shape())
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    assert lib.moe_route(s, None, fake, None, fake, fake, None, None, 0, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(_shape(flags=L.MOE_ROUTER_BIAS)), fake, fake, None, fake, fake,
                         None, None, 0, None) == L.MOE_ERR_INVALID_ARG
    # the router's optional scratch: too small, misaligned
    assert lib.moe_route(s, fake, fake, None, fake, fake, None, fake, 16, None) == L.MOE_ERR_WORKSPACE
    assert lib.moe_route(s, fake, fake, None, fake, fake, None, ctypes.c_void_p(0x1001), 1 << 40,
                         None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(s, fake, None, fake, fake, fake, fake, None, 0, None) == L.MOE_ERR_INVALID_ARG
    # optional scratch: too small, misaligned
    assert lib.moe_dispatch(s, fake, fake, fake, fake, fake, fake, fake, 16, None) == L.MOE_ERR_WORKSPACE
    assert lib.moe_dispatch(s, fake, fake, fake, fake, fake, fake, ctypes.c_void_p(0x1001), 1 << 40,
                            None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn(s, fake, fake, fake, fake, None, None, fake, None, fake, fake, 1 << 30,
                              None) == L.MOE_ERR_INVALID_ARG  # SwiGLU without w3
    assert lib.moe_expert_ffn(s, fake, fake, fake, fake, None, fake, fake, None, fake, fake, 16,
                              None) == L.MOE_ERR_WORKSPACE
    assert lib.moe_expert_up(s, fake, fake, fake, fake, None, None, fake, None, 0,
                             None) == L.MOE_ERR_INVALID_ARG  # SwiGLU without w3
    assert lib.moe_expert_up(s, fake, fake, fake, fake, None, fake, None, None, 0,
                             None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_down(s, fake, fake, fake, None, None, None, 0, None) == L.MOE_ERR_INVALID_ARG
    sb = ctypes.byref(_shape(act=L.MOE_ACT_GELU, flags=L.MOE_HAS_BIAS))
    assert lib.moe_expert_down(sb, fake, fake, fake, None, fake, None, 0, None) == L.MOE_ERR_INVALID_ARG
    # an optional split-K workspace that is too small, or misaligned
    assert lib.moe_expert_up(s, fake, fake, fake, fake, None, fake, fake, fake, 16,
                             None) == L.MOE_ERR_WORKSPACE
    assert lib.moe_expert_down(s, fake, fake, fake, None, fake, ctypes.c_void_p(0x1001), 1 << 40,
                               None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctypes.byref(_shape(flags=L.MOE_RESIDUAL)), fake, fake, fake, None, fake,
                           None) == L.MOE_ERR_INVALID_ARG
    args = [fake] * 16
    args[8] = None  # out
    assert lib.moe_forward(s, *args, fake, 1 << 30, None) == L.MOE_ERR_INVALID_ARG
    ok = [fake] * 16
    ok[2] = None  # b_router unused
    ok[4] = None  # b1
    ok[7] = None  # b2
    assert lib.moe_forward(s, *ok, fake, 10, None) == L.MOE_ERR_WORKSPACE
    # misaligned workspace
    assert lib.moe_forward(s, *ok, ctypes.c_void_p(0x1001), 1 << 30, None) == L.MOE_ERR_INVALID_ARG


def test_zero_tokens_is_a_no_op(lib):
    from mixture_experts_layer_expert_amd import _lib as L
    s = ctypes.byref(_shape(T=0))
    fake = ctypes.c_void_p(0x1000)
    assert lib.moe_route(s, fake, fake, None, fake, fake, None, None, 0, None) == L.MOE_OK
    assert lib.moe_dispatch(s, fake, fake, fake, fake, fake, fake, None, 0, None) == L.MOE_OK
    assert lib.moe_combine(s, fake, fake, fake, None, fake, None) == L.MOE_OK
    assert lib.moe_expert_up(s, fake, fake, fake, fake, None, fake, fake, None, 0, None) == L.MOE_OK
    assert lib.moe_expert_down(s, fake, fake, fake, None, fake, None, 0, None) == L.MOE_OK


def test_library_has_no_undefined_internal_symbols():
    """Every kernel stub the library references is defined in it (a kernel
    whose host stub is not emitted leaves an undefined moe:: symbol and the
    library fails to load)."""
    import shutil
    import subprocess
    from mixture_experts_layer_expert_amd import _lib
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    bad = [l for l in out.splitlines() if "3moe" in l]
    assert not bad, bad[:5]


def test_binding_rejects_undersized_buffers():
    """The Python binding checks every buffer against the shape before the
    library sees a pointer (the library itself trusts its sizes)."""
    import torch
    from mixture_experts_layer_expert_amd import api

    class FakeGpuTensor:  # stands in for a device tensor on a host without a GPU
        is_cuda = True

        def __init__(self, n, dtype=torch.bfloat16):
            self.n, self.dtype = n, dtype

        def is_contiguous(self):
            return True

        def numel(self):
            return self.n

        def data_ptr(self):
            return 0x1000

    assert api._ptr(FakeGpuTensor(64 * 128), torch.bfloat16, "x", 64 * 128) == 0x1000
    with pytest.raises(ValueError, match="the shape needs"):
        api._ptr(FakeGpuTensor(64 * 128 - 1), torch.bfloat16, "x", 64 * 128)
    with pytest.raises(ValueError, match="expected torch.float32"):
        api._ptr(FakeGpuTensor(10), torch.float32, "topk_gate", 10)
    shape = api.MoeShape(T=64, D=128, F=256, N=8, k=2, capacity=-1, act="relu")
    with pytest.raises(ValueError, match="x: 4096 elements"):
        api.route(shape, FakeGpuTensor(4096), FakeGpuTensor(8 * 128), None,
                  FakeGpuTensor(128, torch.int32), FakeGpuTensor(128, torch.float32))


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """With no built library the binding raises ImportError at the first
    call; there is no CPU fallback to hide it."""
    from mixture_experts_layer_expert_amd import _lib as L
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "absent" / "libmoe_mi355x.so"))
    with pytest.raises(ImportError, match="not found"):
        L.load()


def test_clock_probe_validates_on_the_host(lib):
    from mixture_experts_layer_expert_amd import _lib as L
    dummy = ctypes.c_void_p(0x1000)  # never dereferenced: each call fails validation
    assert lib.moe_clock_probe(0, 0.0, 10, dummy, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_clock_probe(65537, 0.0, 10, dummy, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_clock_probe(4, 0.0, 10, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_clock_probe(4, -1.0, 10, dummy, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_clock_probe(4, 0.0, 0, dummy, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_clock_probe(4, 0.0, (1 << 16) + 1, dummy, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_clock_probe(4, 200000.0, 10, dummy, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_clock_probe(4, float("nan"), 10, dummy, None) == L.MOE_ERR_INVALID_ARG
