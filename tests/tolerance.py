"""Tolerance checks for GPU outputs against the fp64 oracle.

W4A16 / W8A16 (the decode layer's accuracy target): with an fp32 output,
    max |y - ref| <= 1e-2 * mean|ref| + 1e-3   and   mean|y - ref| / mean|ref| <= 2e-3.
With a bf16 output the stored value is the fp32 result rounded to bf16, whose
half-ulp alone can exceed the first bound at large |y|; the elementwise bound
then adds half a bf16 ulp of ref, and the mean-relative bound is unchanged.

W4A8 against the W4A16 reference: the precision class of executorch
test_int4_quantized_gemm.py `_check_close` (rtol 0.03, atol 8.0, mean
relative error below 0.02), and the three checks of its
Int4QuantizedGemmPrecisionTest against the unquantized (dense) product:
the W4A8 error against dense may be at most 1.10x the W4A16 error in the
mean, the W4A8 - W4A16 difference at most 2% of mean|W4A16|, and the largest
W4A8 error at most the largest W4A16 error + max(2, 2% of max|dense|).
"""
from __future__ import annotations

import numpy as np
import torch


def _as_f64(y) -> np.ndarray:
    if isinstance(y, torch.Tensor):
        y = y.detach().float().cpu().numpy()
    return np.asarray(y, dtype=np.float64)


def bf16_half_ulp(ref: np.ndarray) -> np.ndarray:
    a = np.abs(ref)
    _, e = np.frexp(np.maximum(a, np.finfo(np.float32).tiny))   # a in [2^(e-1), 2^e)
    return np.ldexp(1.0, e - 9)                                    # ulp = 2^(e-8)


def check_w16(y, ref: np.ndarray, label: str = "") -> dict:
    y = _as_f64(y)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.isfinite(y).all(), f"{label}: non-finite output"
    err = np.abs(y - ref)
    mean_ref = float(np.abs(ref).mean())
    bound = 1e-2 * mean_ref + 1e-3
    mean_rel = float(err.mean() / max(mean_ref, 1e-30))
    return {"max_err": float(err.max()), "bound": bound, "mean_rel": mean_rel, "err": err}


def assert_w16(y, ref, label: str = "") -> None:
    """W4A16 / W8A16 bound; bf16 outputs get half a bf16 ulp of slack per element."""
    is_bf16 = isinstance(y, torch.Tensor) and y.dtype == torch.bfloat16
    r = check_w16(y, ref, label)
    ref = np.asarray(ref, np.float64)
    slack = bf16_half_ulp(ref) if is_bf16 else 0.0
    over = r["err"] > r["bound"] + slack
    assert not over.any(), (
        f"{label}: {int(over.sum())} elements over the bound; max|dy| = {r['max_err']:.4g}, "
        f"bound = {r['bound']:.4g} (+ half bf16 ulp: {is_bf16})")
    assert r["mean_rel"] <= 2e-3, f"{label}: mean relative error {r['mean_rel']:.3g} > 2e-3"


def assert_w4a8_class(y, ref_w4a16, label: str = "") -> None:
    """rtol 0.03 / atol 8.0 elementwise, mean relative error < 0.02, all finite."""
    y = _as_f64(y)
    ref = np.asarray(ref_w4a16, np.float64)
    assert np.isfinite(y).all(), f"{label}: non-finite output"
    err = np.abs(y - ref)
    over = err > 8.0 + 0.03 * np.abs(ref)
    assert not over.any(), f"{label}: {int(over.sum())} elements outside rtol 0.03 / atol 8"
    mean_rel = err.mean() / np.abs(ref).mean()
    assert mean_rel < 0.02, f"{label}: mean relative error {mean_rel:.3g} >= 0.02"


def precision_class_failures(a8, a16, dense) -> list[str]:
    """The dense-reference checks of the pages' W4A8 precision test; returns
    the failed ones (empty when the case passes)."""
    a8, a16, dense = _as_f64(a8), _as_f64(a16), _as_f64(dense)
    bad = []
    if not np.isfinite(a8).all():
        return ["non-finite"]
    e8 = np.abs(a8 - dense)
    e16 = np.abs(a16 - dense)
    ratio = e8.mean() / max(e16.mean(), 1e-6)
    mean_rel = np.abs(a8 - a16).mean() / max(np.abs(a16).mean(), 1e-6)
    allowance = max(2.0, 0.02 * np.abs(dense).max())
    if ratio > 1.10:
        bad.append(f"dense error ratio {ratio:.3f} > 1.10")
    if mean_rel > 0.02:
        bad.append(f"mean relative difference {mean_rel:.4f} > 0.02")
    if e8.max() > e16.max() + allowance:
        bad.append(f"max error {e8.max():.3g} > {e16.max():.3g} + {allowance:.3g}")
    return bad
