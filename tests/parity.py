"""Error metrics and tolerance bars for comparing the HIP path with the fp64 oracle.

Bars (stated once, used by every GPU parity test):
  * fp32 O:   max |gpu - ref| <= 1e-5
  * bf16 O:   max |gpu - ref| <= 1e-2 after discounting the output's own rounding to
              bf16: |gpu - ref| <= 1e-2 + half_ulp_bf16(ref). A correctly rounded bf16
              result of a value in [4, 8) is already up to 2^-6 = 0.0156 away from it,
              so the 1e-2 bar is applied to the error the kernel adds before that final,
              unavoidable rounding. Where |ref| < 2 (half an ulp <= 2^-8 there) the plain
              bar max |gpu - ref| <= 1e-2 is asserted as well, and the raw max-abs error
              over all elements is returned so that callers can report it.
  * lse:      max |gpu - ref| <= 1e-3 on rows with an allowed key; rows without one
              must be -inf on both sides.
  * dQ/dK/dV: relative L2 error ||gpu - ref||_2 / ||ref||_2 <= 2e-2 over the compared
              elements; where the exact tensor is zero by cancellation, max |gpu| <= 1e-4.
"""
import numpy as np
import torch

O_TOL_F32 = 1e-5
O_TOL_BF16 = 1e-2
LSE_TOL = 1e-3
GRAD_REL_L2 = 2e-2
# When the exact gradient is zero by cancellation, relative error is undefined; the bar is
# then absolute. Structural zeros (keys nobody may attend to) are tested for exact 0.
ZERO_REF_ABS = 1e-4


def to64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def half_ulp_bf16(ref: np.ndarray) -> np.ndarray:
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def o_excess(gpu, ref, dtype: str) -> float:
    """max(|gpu - ref| - allowance); <= bar means pass."""
    g, r = to64(gpu), to64(ref)
    err = np.abs(g - r)
    if dtype == "bf16":
        err = err - half_ulp_bf16(r)
    return float(err.max()) if err.size else 0.0


# Below this magnitude half a bf16 ulp is at most 2^-8, and the plain max-abs bar is asserted.
PLAIN_BAR_BELOW = 2.0


def check_o(gpu, ref, dtype: str, what: str = "O") -> float:
    """Asserts the O bar; returns the raw max |gpu - ref| over all elements."""
    bar = O_TOL_BF16 if dtype == "bf16" else O_TOL_F32
    g, r = to64(gpu), to64(ref)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    ex = o_excess(g, r, dtype)
    assert ex <= bar, f"{what}: max error beyond allowance {ex:.3e} > {bar:.1e}"
    err = np.abs(g - r)
    small = np.abs(r) < PLAIN_BAR_BELOW
    if small.any():
        m = float(err[small].max())
        assert m <= bar, f"{what}: max |gpu - ref| {m:.3e} > {bar:.1e} where |ref| < {PLAIN_BAR_BELOW}"
    return float(err.max()) if err.size else 0.0


def check_lse(gpu, ref, what: str = "lse"):
    g, r = to64(gpu), to64(ref)
    empty = np.isneginf(r)
    assert np.all(np.isneginf(g[empty])), f"{what}: rows without allowed keys must be -inf"
    if (~empty).any():
        err = np.abs(g[~empty] - r[~empty])
        assert np.all(np.isfinite(g[~empty])), f"{what}: non-finite on live rows"
        m = float(err.max())
        assert m <= LSE_TOL, f"{what}: max abs error {m:.3e} > {LSE_TOL:.0e}"
        return m
    return 0.0


def rel_l2(gpu, ref) -> float:
    g, r = to64(gpu), to64(ref)
    den = np.linalg.norm(r)
    num = np.linalg.norm(g - r)
    return float(num / den) if den > 0 else float(num)


def check_grad(gpu, ref, what: str):
    g = to64(gpu)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    e = rel_l2(g, ref)
    assert e <= GRAD_REL_L2, f"{what}: relative L2 error {e:.3e} > {GRAD_REL_L2:.0e}"
    return e
