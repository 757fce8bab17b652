"""The bf16 GEMM's GELU epilogue evaluates Phi(z) = 0.5 + z * P(u) with a
degree-8 P at u = min(z^2, 16), clamped to [0, 1] (so Phi = [z > 0] once
|z| is a little above 4).  These host checks read
the coefficients out of the kernel source and hold them against the normal
CDF computed independently (scipy's erf): the kernel's evaluation order in
fp32 stays within 4e-5 of Phi, and its GELU within 1.5e-4, on [-6, 6].  They
also check that the source carries the fit that csrc/fit_gelu_poly.py
derives."""
import importlib.util
import os
import re

import numpy as np
from scipy.special import erf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "mixture_experts_layer_expert_amd", "csrc", "grouped_gemm.hip")


def kernel_coefficients():
    text = open(SRC, encoding="utf-8").read()
    body = text[text.index("__device__ inline float gelu_erf(float z) {"):]
    body = body[:body.index("\n}\n")]
    first = re.search(r"float p = ([-+0-9.e]+)f;", body).group(1)
    rest = re.findall(r"p = fmaf\(p, u, ([-+0-9.e]+)f\);", body)
    hi_to_lo = [float(first)] + [float(v) for v in rest]
    assert len(hi_to_lo) == 9, hi_to_lo
    assert "fminf(z * z, 16.f)" in body and "fmed3f(fmaf(z, p, 0.5f), 0.f, 1.f)" in body
    return np.array(hi_to_lo[::-1])  # c0 .. c8


def phi(z):
    return 0.5 * (1.0 + erf(z / np.sqrt(2.0)))


def kernel_phi_fp32(z, c):
    c32 = c.astype(np.float32)
    z = z.astype(np.float32)
    u = np.minimum((z * z).astype(np.float32), np.float32(16.0))
    p = np.full_like(u, c32[8])
    for ck in c32[7::-1]:
        # an fp32 FMA: the product of two fp32 values is exact in fp64
        p = (p.astype(np.float64) * u + ck).astype(np.float32)
    ph = (z.astype(np.float64) * p + 0.5).astype(np.float32)
    return np.clip(ph, np.float32(0.0), np.float32(1.0))


def test_phi_and_gelu_error_bounds():
    c = kernel_coefficients()
    z = np.linspace(-6.0, 6.0, 240001)
    got = kernel_phi_fp32(z, c).astype(np.float64)
    want = phi(z)
    assert np.abs(got - want).max() <= 4e-5
    gelu_err = np.abs(z * got - z * want).max()
    assert gelu_err <= 1.5e-4, gelu_err
    # the pieces meet: just inside |z| = 4 the polynomial is within the bound
    # of 0 and 1, and the clamp reaches them exactly by |z| = 4.002
    inner = kernel_phi_fp32(np.array([3.9999, -3.9999]), c).astype(np.float64)
    assert abs(inner[0] - 1.0) <= 1e-4 and abs(inner[1]) <= 1e-4
    outer = kernel_phi_fp32(np.array([4.002, -4.002, 30.0, -30.0]), c)
    assert list(outer) == [1.0, 0.0, 1.0, 0.0]


def test_source_carries_the_derived_fit():
    spec = importlib.util.spec_from_file_location(
        "fit_gelu_poly", os.path.join(ROOT, "mixture_experts_layer_expert_amd", "csrc", "fit_gelu_poly.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    derived = mod.fit()
    c = kernel_coefficients()
    assert np.allclose(c, derived, rtol=1e-6, atol=0.0), (c, derived)
