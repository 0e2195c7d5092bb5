"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant below is the oracle's per-head forward or backward with one plausible
error (a dropped term, a wrong sign or index, a transposed operand).  If a mutant
passed every pin, the pins would not be strong enough to trust the oracle.
"""

import numpy as np
import pytest

from oracle import naive, tiled_ref
from oracle_pins import BACKWARD_PINS, FORWARD_PINS


def _fwd(mut):
    def fwd(q, k, v, scale, causal):
        q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
        s = scale * (q @ k.T)
        if mut == "no_scale":
            s = q @ k.T
        if causal:
            hidden = naive.causal_mask(*s.shape)
            if mut == "mask_off_by_one":
                hidden = np.arange(s.shape[1])[None, :] > np.arange(s.shape[0])[:, None] + 1
            s = np.where(hidden, -np.inf, s)
        m = s.max(axis=1, keepdims=True)
        with np.errstate(over="ignore", invalid="ignore"):
            e = np.exp(s) if mut == "no_max_shift" else np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        p = e / l
        if mut == "transposed_pv":
            o = p.T @ v
        elif mut == "unnormalised":
            o = e @ v
        else:
            o = p @ v
        with np.errstate(divide="ignore", invalid="ignore"):
            lse = (np.log(l) if mut == "no_max_shift" else m + np.log(l))[:, 0]
        if mut == "lse_log2":
            lse = (m + np.log2(l))[:, 0]
        if mut == "lse_missing_m":
            lse = np.log(l)[:, 0]
        return o, lse
    return fwd


def _bwd(mut):
    def bwd(q, k, v, do, scale, causal):
        q, k, v, do = (np.asarray(a, np.float64) for a in (q, k, v, do))
        p = naive.probabilities(q, k, scale, causal)
        dv = (p @ do) if mut == "dv_untransposed" else (p.T @ do)
        dp = do @ v.T
        dsum = np.sum(p * dp, axis=-1, keepdims=True)
        ds = p * dp if mut == "ds_missing_D" else p * (dp - dsum)
        dq = scale * (ds @ (q if mut == "dq_wrong_operand" else k))
        dk = scale * (ds.T @ q)
        if mut == "dk_sign":
            dk = -dk
        if mut == "dq_no_scale":
            dq = ds @ k
        return dq, dk, dv
    return bwd


FWD_MUTANTS = ["no_scale", "mask_off_by_one", "no_max_shift", "transposed_pv", "unnormalised",
               "lse_log2", "lse_missing_m"]
BWD_MUTANTS = ["dv_untransposed", "ds_missing_D", "dq_wrong_operand", "dk_sign", "dq_no_scale"]


def test_unmutated_copies_pass():
    """The harness itself: the copies without a planted mistake pass every pin."""
    f, b = _fwd(None), _bwd(None)
    for _, pin in FORWARD_PINS:
        pin(f)
    for _, pin in BACKWARD_PINS:
        pin(f, b)


@pytest.mark.parametrize("mut", FWD_MUTANTS)
def test_forward_mutant_is_caught(mut):
    f = _fwd(mut)
    failed = []
    for name, pin in FORWARD_PINS:
        try:
            pin(f)
        except (AssertionError, FloatingPointError, ValueError):
            failed.append(name)
    assert failed, f"mutant {mut} passed every forward pin"


@pytest.mark.parametrize("mut", BWD_MUTANTS)
def test_backward_mutant_is_caught(mut):
    f, b = naive.forward_head, _bwd(mut)
    failed = []
    for name, pin in BACKWARD_PINS:
        try:
            pin(f, b)
        except (AssertionError, FloatingPointError, ValueError):
            failed.append(name)
    assert failed, f"mutant {mut} passed every backward pin"


def test_tiled_wrong_rescale_is_caught():
    """A tiled recurrence that rescales by e^(m_new - m_old) instead of e^(m_old - m_new)
    disagrees with the two-block worked example."""
    row = np.array([1.0, 2.0, 0.0, 3.0])
    m, l = -np.inf, 0.0
    for start in (0, 2):
        x = row[start:start + 2]
        m_new = max(m, x.max())
        alpha = np.exp(m_new - m) if np.isfinite(m) else 0.0
        l = alpha * l + np.exp(x - m_new).sum()
        m = m_new
    good = tiled_ref.online_stats(row, 2)[-1][1]
    assert round(l, 3) != round(good, 3) == 1.553
