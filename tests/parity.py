"""Comparison gates shared by the GPU parity tests (not collected by pytest).

Attention gate (tolerance of the decode-attention output against the fp64
oracle value b, per element):
    |a - b| <= 2e-3 (+ half a bf16 ulp at |b| + 2e-3 when the output is bf16)
    |a - b| <= 1e-2 * |b| + 1e-5
The half-ulp term is the representation error of storing the fp32 result in
bf16 (up to 3.9e-3 for magnitudes in [1, 2)).  It is taken at the largest
magnitude an fp32 result within 2e-3 of b can have, so it depends on the
oracle value alone: an output that is wrong cannot widen its own bound by
landing in a coarser binade.  The relative bound is untouched by it.  The
1e-5 floor admits fp32 summation noise on elements that cancel to ~0.
"""
from __future__ import annotations

import numpy as np

ABS_TOL = 2e-3
REL_TOL = 1e-2
REL_FLOOR = 1e-5


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at magnitude |x| (8 significant bits)."""
    m = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    _, e = np.frexp(m)                    # m = f * 2^e, f in [0.5, 1)
    return np.ldexp(1.0, e - 9)


def attention_gate(a: np.ndarray, b: np.ndarray, out_dtype: str) -> dict:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = np.abs(a - b)
    abs_tol = ABS_TOL + (half_ulp_bf16(np.abs(b) + ABS_TOL) if out_dtype == "bf16" else 0.0)
    ok = (err <= abs_tol) & (err <= REL_TOL * np.abs(b) + REL_FLOOR)
    big = np.abs(b) >= 1e-3
    return {
        "ok": bool(ok.all()),
        "n": int(err.size),
        "n_fail": int((~ok).sum()),
        "max_abs": float(err.max()) if err.size else 0.0,
        "max_rel": float((err[big] / np.abs(b[big])).max()) if big.any() else 0.0,
        "n_small": int((~big).sum()),
        "plain_abs_ok": bool((err <= ABS_TOL).all()),
        "first_fail": (np.argwhere(~ok)[0].tolist() if (~ok).any() else None),
    }


def assert_gate(a, b, out_dtype, what=""):
    r = attention_gate(a, b, out_dtype)
    assert r["ok"], f"{what}: {r}"
    return r
