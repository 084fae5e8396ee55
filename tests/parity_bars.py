"""Parity bars of the GPU tests, and a record of how close each check came.

The bars (review page, §2.3 output and §2.6 gradients; the acceptance
tolerances of the path):
- selected indices and counts: bit-exact (checked where they are compared);
- float32 workloads: 1e-5 max-abs on o and lse, 1e-5 relative L2 on gradients;
- bf16 workloads: o within 1e-2 max-abs of the float64 oracle plus the exact
  bf16 half-ulp of the oracle's value (a bf16 output is the float32 result
  rounded to nearest even for storage, which alone moves it by up to that
  half-ulp: 2^-9 |o| < h <= 2^-8 |o|, so storage alone exceeds 1e-2 only at
  |o| >= 4); dq, dk, dv, ds within 2e-2 relative L2; lse within 2e-3 max-abs.

Every check records its worst error as a fraction of its bar under the
running test's id; the test session prints the table at its end.
"""
from __future__ import annotations

import numpy as np

O_ABS = {"f32": 1e-5, "bf16": 1e-2}
GRAD_REL = {"f32": 1e-5, "bf16": 2e-2}
LSE_ABS = {"f32": 1e-5, "bf16": 2e-3}

RECORD: dict[str, dict[str, float]] = {}
CURRENT = [""]


def bf16_half_ulp(x) -> np.ndarray:
    """Half the spacing of bf16 numbers at |x| (8 significant bits): for
    2^e <= |x| < 2^(e+1) it is 2^(e-8); 0 at x = 0."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, ex = np.frexp(a)            # a = m * 2^ex with 0.5 <= m < 1, so e = ex - 1
    return np.where(a > 0, np.ldexp(1.0, ex - 9), 0.0)


def o_bound(ref, dtype: str) -> np.ndarray:
    ref = np.asarray(ref, dtype=np.float64)
    if dtype == "bf16":
        return O_ABS["bf16"] + bf16_half_ulp(ref)
    return np.full(ref.shape, O_ABS[dtype])


def _note(what, frac: float) -> None:
    key = what if isinstance(what, str) else str(what[0]) if isinstance(what, tuple) else str(what)
    row = RECORD.setdefault(CURRENT[0] or "?", {})
    row[key] = max(row.get(key, 0.0), float(frac))


def assert_o(got, ref, dtype: str, what="o") -> float:
    """Element-wise output check; returns the worst error / bar."""
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    bound = o_bound(ref, dtype)
    frac = err / bound
    worst = np.unravel_index(np.argmax(frac), frac.shape) if frac.size else ()
    w = float(frac[worst]) if frac.size else 0.0
    _note(what, w)
    assert np.all(err <= bound), (what, "err", float(err[worst]), "ref", float(ref[worst]),
                                  "bar", float(bound[worst]), worst)
    return w


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def assert_rel(got, ref, bar: float, what) -> float:
    e = rel_l2(got, ref)
    _note(what, e / bar)
    assert e <= bar, (what, e, bar)
    return e


def assert_maxabs(got, ref, bar: float, what) -> float:
    e = float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)))) \
        if np.size(ref) else 0.0
    _note(what, e / bar)
    assert e <= bar, (what, e, bar)
    return e


def summary_lines() -> list[str]:
    if not RECORD:
        return []
    kinds = sorted({k for row in RECORD.values() for k in row})
    out = ["worst error as a fraction of its bar (1.0 = at the bar)",
           "  " + " ".join(f"{k:>8s}" for k in kinds) + "  test"]
    for test, row in RECORD.items():
        cells = " ".join(f"{row[k]:8.3f}" if k in row else f"{'':8s}" for k in kinds)
        out.append(f"  {cells}  {test}")
    return out
