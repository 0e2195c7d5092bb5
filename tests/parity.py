"""Comparison helpers for GPU-vs-oracle parity (tolerances written here, in one place).

Tolerances (from the target's statement of the bar):
  * fp32 inputs:      max |O - O_ref| <= 1e-5.
  * bf16/fp16 inputs: max |X - X_ref| <= 1e-2 and mean |X - X_ref| <= 1e-3 for
                      X in O, dQ, dK, dV, against the oracle run on the same rounded inputs.
  * LSE:              |lse - lse_ref| <= 1e-4 * max(1, |lse_ref|)  (relative, with a floor
                      of 1 because a causal row 0 has lse = s_00, which can be ~0).
fp16 is held to the bf16 bounds (the bar names none for it); the achieved error is
reported by the tests either way.

Output rounding floor.  A result stored in a 16-bit type cannot be closer to the exact
value than the rounding of that exact value: for |O| in [4, 8) a bf16 half-ulp is 2^-6 =
0.0156, above the 1e-2 bar.  The max bar is therefore applied to the error each element
shows beyond its own floor,
    |x_i - ref_i| <= 1e-2 + |round_out(ref_i) - ref_i|,
where round_out rounds to the output's storage type (for fp32 outputs the floor is ~1e-8
and the bar is the plain one).  The mean bar is applied as written.  Edge cases (tiny N,
a handful of visible keys) can have |O| ~ 1 everywhere, where the floor alone has a mean
near 1e-3; ``floor_aware=True`` then allows a mean of max(bar, 3 x the floor's mean).
The named full-size workloads always use the mean bar as written.
"""

from __future__ import annotations

import numpy as np
import torch

TOL = {
    "f32": {"max": 1e-5, "mean": 1e-5},
    "bf16": {"max": 1e-2, "mean": 1e-3},
    "f16": {"max": 1e-2, "mean": 1e-3},
}
LSE_REL = 1e-4


def to64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, np.float64)


def errors(x, ref):
    x, ref = to64(x), to64(ref)
    d = np.abs(x - ref)
    return float(d.max()), float(d.mean())


def rounding_floor(ref, dtype: str) -> float:
    """max |round_dtype(ref) - ref|: the error a perfect kernel would still show after
    storing its result in the output dtype."""
    ref = to64(ref)
    td = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    r = torch.from_numpy(ref).to(td).to(torch.float64).numpy()
    return float(np.abs(r - ref).max())


def rounding_floor_stats(ref, dtype: str):
    """(max, mean) of |round_dtype(ref) - ref|."""
    ref = to64(ref)
    td = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    d = np.abs(torch.from_numpy(ref).to(td).to(torch.float64).numpy() - ref)
    return float(d.max()), float(d.mean())


def _round_to(ref64: np.ndarray, dtype: str) -> np.ndarray:
    td = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return torch.from_numpy(ref64).to(td).to(torch.float64).numpy()


def assert_close(name, x, ref, dtype: str, out_dtype: str | None = None, floor_aware: bool = False):
    """Check x against the fp64 reference.  ``dtype`` selects the bar (input type);
    ``out_dtype`` is the storage type of x (defaults to ``dtype``).  Returns
    (max error, mean error, max error beyond the rounding floor, max floor)."""
    x64, r64 = to64(x), to64(ref)
    d = np.abs(x64 - r64)
    fl = np.abs(_round_to(r64, out_dtype or dtype) - r64)
    mx, mean = float(d.max()), float(d.mean())
    excess = float((d - fl).max())
    tmax, tmean = TOL[dtype]["max"], TOL[dtype]["mean"]
    if floor_aware:
        tmean = max(tmean, 3 * float(fl.mean()))
    assert np.isfinite(mx), f"{name}: non-finite values"
    assert excess <= tmax, (f"{name}: error beyond the output rounding floor {excess:.3e} > {tmax:.0e} "
                            f"(max {mx:.3e}, mean {mean:.3e}, floor max {fl.max():.3e})")
    assert mean <= tmean, f"{name}: mean abs err {mean:.3e} > {tmean:.2e} (max {mx:.3e})"
    return mx, mean, excess, float(fl.max())


def assert_lse(lse, ref):
    lse, ref = to64(lse), to64(ref)
    err = np.abs(lse - ref) / np.maximum(1.0, np.abs(ref))
    worst = float(err.max())
    assert np.isfinite(worst), "lse: non-finite values"
    assert worst <= LSE_REL, f"lse: relative err {worst:.3e} > {LSE_REL:.0e}"
    return worst


class ErrorStats:
    """Running error statistics of one output tensor over many heads: raw max and mean
    |x - ref|, the output-rounding floor |round_out(ref) - ref| (max and mean), the largest
    error beyond each element's own floor, and max |ref|.  For lse the error is the
    relative one, |x - ref| / max(1, |ref|), and no floor applies."""

    def __init__(self, out_dtype: str | None, relative: bool = False):
        self.out_dtype, self.relative = out_dtype, relative
        self.max = self.floor_max = self.excess_max = self.ref_max = 0.0
        self.sum = self.floor_sum = 0.0
        self.count = 0
        self.nonfinite = 0

    def add(self, x, ref):
        x64, r64 = to64(x), to64(ref)
        fin = np.isfinite(r64)
        same_inf = ~fin & (x64 == r64)  # an empty row's lse = -inf on both sides
        self.nonfinite += int((~np.isfinite(x64) & ~same_inf).sum())
        x64, r64 = np.where(same_inf, 0.0, x64), np.where(same_inf, 0.0, r64)
        d = np.abs(x64 - r64)
        if self.relative:
            d = d / np.maximum(1.0, np.abs(r64))
            fl = np.zeros_like(d)
        else:
            fl = np.abs(_round_to(r64, self.out_dtype) - r64) if self.out_dtype else np.zeros_like(d)
        self.max = max(self.max, float(d.max()))
        self.sum += float(d.sum())
        self.count += d.size
        self.floor_max = max(self.floor_max, float(fl.max()))
        self.floor_sum += float(fl.sum())
        self.excess_max = max(self.excess_max, float((d - fl).max()))
        self.ref_max = max(self.ref_max, float(np.abs(r64).max()))

    def merge(self, other: "ErrorStats"):
        self.max = max(self.max, other.max)
        self.floor_max = max(self.floor_max, other.floor_max)
        self.excess_max = max(self.excess_max, other.excess_max)
        self.ref_max = max(self.ref_max, other.ref_max)
        self.sum += other.sum
        self.floor_sum += other.floor_sum
        self.count += other.count
        self.nonfinite += other.nonfinite

    @property
    def mean(self) -> float:
        return self.sum / max(self.count, 1)

    @property
    def floor_mean(self) -> float:
        return self.floor_sum / max(self.count, 1)

    def as_dict(self):
        return {"max": self.max, "mean": self.mean, "floor_max": self.floor_max, "floor_mean": self.floor_mean,
                "beyond_floor_max": self.excess_max, "max_abs_ref": self.ref_max, "elements": self.count,
                "nonfinite": self.nonfinite}

    def check(self, name: str, bar_dtype: str):
        """The bars of this module: lse relative <= LSE_REL; otherwise the max bar on the
        error beyond the floor and the mean bar as written."""
        assert self.nonfinite == 0, f"{name}: {self.nonfinite} non-finite values"
        if self.relative:
            assert self.max <= LSE_REL, f"{name}: relative err {self.max:.3e} > {LSE_REL:.0e}"
            return
        tmax, tmean = TOL[bar_dtype]["max"], TOL[bar_dtype]["mean"]
        assert self.excess_max <= tmax, (f"{name}: error beyond the output rounding floor {self.excess_max:.3e} > "
                                         f"{tmax:.0e} (raw max {self.max:.3e}, floor max {self.floor_max:.3e})")
        assert self.mean <= tmean, f"{name}: mean abs err {self.mean:.3e} > {tmean:.0e} (max {self.max:.3e})"
