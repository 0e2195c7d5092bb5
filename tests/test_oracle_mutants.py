"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant below is the oracle's per-head forward or backward with one plausible
error (a dropped term, a wrong sign or index, a transposed operand).  If a mutant
passed every pin, the pins would not be strong enough to trust the oracle.
"""

import numpy as np
import pytest

from oracle import naive, tiled_ref
from oracle_pins import (BACKWARD_PINS, CROSS_BACKWARD_PINS, CROSS_FORWARD_PINS, FORWARD_PINS, GQA_BACKWARD_PINS,
                         GQA_FORWARD_PINS, MASK_PINS, pin_block_geometry)


def _fwd(mut):
    def fwd(q, k, v, scale, causal):
        q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
        s = scale * (q @ k.T)
        if mut == "no_scale":
            s = q @ k.T
        if causal:
            hidden = naive.causal_mask(*s.shape)
            if mut == "top_left":  # ignores the offset of the query positions when N_q < N_k
                hidden = np.arange(s.shape[1])[None, :] > np.arange(s.shape[0])[:, None]
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
        if mut == "top_left" and causal:
            s = scale * (q @ k.T)
            s = np.where(np.arange(s.shape[1])[None, :] > np.arange(s.shape[0])[:, None], -np.inf, s)
            p = naive.softmax_rows(s)[0]
        else:
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


def _caught(pins, call):
    failed = []
    for name, pin in pins:
        try:
            call(pin)
        except (AssertionError, FloatingPointError, ValueError):
            failed.append(name)
    return failed


def test_cross_top_left_mask_is_caught():
    """A causal mask aligned at the first key instead of the last query fails the
    suffix pins (forward and backward); the unmutated copies pass them."""
    assert not _caught(CROSS_FORWARD_PINS, lambda pin: pin(_fwd(None)))
    assert not _caught(CROSS_BACKWARD_PINS, lambda pin: pin(_bwd(None)))
    assert _caught(CROSS_FORWARD_PINS, lambda pin: pin(_fwd("top_left")))
    assert _caught(CROSS_BACKWARD_PINS, lambda pin: pin(_bwd("top_left")))


def _fwd_mh(mut):
    def fwd(q, k, v, scale, causal):
        B, H, nq, _ = q.shape
        hkv = k.shape[1]
        o = np.zeros(q.shape[:3] + (v.shape[-1],))
        lse = np.zeros(q.shape[:3])
        for b in range(B):
            for h in range(H):
                g = h % hkv if mut == "head_mod" else h // (H // hkv)
                o[b, h], lse[b, h] = naive.forward_head(q[b, h], k[b, g], v[b, g], scale, causal)
        return o, lse
    return fwd


def _bwd_mh(mut):
    def bwd(q, k, v, do, scale, causal):
        B, H = q.shape[:2]
        hkv = k.shape[1]
        dq = np.zeros(q.shape)
        dk = np.zeros(k.shape)
        dv = np.zeros(v.shape)
        for b in range(B):
            for h in range(H):
                g = h // (H // hkv)
                dq[b, h], dkh, dvh = naive.backward_head(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal)
                if mut == "no_group_sum":
                    dk[b, g], dv[b, g] = dkh, dvh
                else:
                    dk[b, g] += dkh
                    dv[b, g] += dvh
        return dq, dk, dv
    return bwd


def test_gqa_mutants_are_caught():
    """Query head h reading key/value head h % H_kv instead of h // G, and a shared
    head's gradient taken from one query head instead of the group's sum, each fail."""
    assert not _caught(GQA_FORWARD_PINS, lambda pin: pin(_fwd_mh(None)))
    assert not _caught(GQA_BACKWARD_PINS, lambda pin: pin(_bwd_mh(None)))
    assert _caught(GQA_FORWARD_PINS, lambda pin: pin(_fwd_mh("head_mod")))
    assert _caught(GQA_BACKWARD_PINS, lambda pin: pin(_bwd_mh("no_group_sum")))


def test_mask_mutants_are_caught():
    """Blocks of 127 instead of 128 fail the geometry pin; a softmax that divides an empty
    row by its zero sum (NaN instead of 0) fails the empty-row pin; ignoring the mask
    fails the SDPA pin."""
    def expand127(bm, n_q, n_k):
        bm = np.asarray(bm)
        keep = np.repeat(np.repeat(bm != 0, 127, axis=0), 127, axis=1)
        if keep.shape[0] < n_q or keep.shape[1] < n_k:
            raise AssertionError("too small")
        return ~keep[:n_q, :n_k]
    with pytest.raises(AssertionError):
        pin_block_geometry(expand127)

    def fwd_nan(q, k, v, scale, causal, hidden=None):
        s = naive.scores(q, k, scale, causal, hidden)
        m = s.max(axis=1, keepdims=True)
        with np.errstate(invalid="ignore", divide="ignore"):
            e = np.exp(s - m)
            l = e.sum(axis=1, keepdims=True)
            return (e / l) @ v, (m + np.log(l))[:, 0]

    def fwd_nomask(q, k, v, scale, causal, hidden=None):
        return naive.forward_head(q, k, v, scale, causal)

    assert _caught(MASK_PINS, lambda pin: pin(naive.forward_head, naive.backward_head)) == []
    assert "empty_row" in _caught(MASK_PINS, lambda pin: pin(fwd_nan, naive.backward_head))
    assert "mask_sdpa" in _caught(MASK_PINS, lambda pin: pin(fwd_nomask, naive.backward_head))


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
