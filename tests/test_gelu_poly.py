"""The bf16 GEMM's GELU epilogue evaluates Phi(z) = 0.5 + z * P(z^2) with a
degree-8 P for |z| <= 4 and Phi = [z > 0] beyond.  These host checks read
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
    assert "fmaf(z, p, 0.5f)" in body and "u > 16.f" in body
    return np.array(hi_to_lo[::-1])  # c0 .. c8


def phi(z):
    return 0.5 * (1.0 + erf(z / np.sqrt(2.0)))


def kernel_phi_fp32(z, c):
    c32 = c.astype(np.float32)
    z = z.astype(np.float32)
    u = (z * z).astype(np.float32)
    p = np.full_like(u, c32[8])
    for ck in c32[7::-1]:
        p = (p * u + ck).astype(np.float32)
    ph = (np.float32(0.5) + z * p).astype(np.float32)
    return np.where(u > np.float32(16.0), (z > 0).astype(np.float32), ph)


def test_phi_and_gelu_error_bounds():
    c = kernel_coefficients()
    z = np.linspace(-6.0, 6.0, 240001)
    got = kernel_phi_fp32(z, c).astype(np.float64)
    want = phi(z)
    assert np.abs(got - want).max() <= 4e-5
    gelu_err = np.abs(z * got - z * want).max()
    assert gelu_err <= 1.5e-4, gelu_err
    # the pieces meet: just inside |z| = 4 the polynomial is within the bound
    # of the value the [z > 0] branch takes just outside
    inner = kernel_phi_fp32(np.array([3.9999, -3.9999]), c).astype(np.float64)
    assert abs(inner[0] - 1.0) <= 1e-4 and abs(inner[1]) <= 1e-4


def test_source_carries_the_derived_fit():
    spec = importlib.util.spec_from_file_location(
        "fit_gelu_poly", os.path.join(ROOT, "mixture_experts_layer_expert_amd", "csrc", "fit_gelu_poly.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    derived = mod.fit()
    c = kernel_coefficients()
    assert np.allclose(c, derived, rtol=1e-6, atol=0.0), (c, derived)
