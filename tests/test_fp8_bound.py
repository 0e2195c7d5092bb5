"""The FP8 forward's error bound (tests/fp8_bound.py) pinned on the CPU: a model of the
kernel's arithmetic (fp32 sums and exponent, exponentials with 2^-22 error, P rounded to
E4M3 relative to a running max updated every 64 keys, bf16 output) stays inside it on
varied inputs, and the bound is tight enough that a coarser rounding of P, or a bound
that forgets the P rounding, is caught."""

import math

import numpy as np
import pytest

from oracle import fp8
from fp8_bound import E4M3_REL, E4M3_SUB, head_bound, simulate_head


def _case(seed, nq, nk, d, outliers=False, vscale=1.0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((1, 1, nq, d))
    k = r.standard_normal((1, 1, nk, d))
    v = r.standard_normal((1, 1, nk, d)) * vscale
    if outliers:
        q[0, 0, r.choice(nq, max(1, nq // 20), replace=False)] *= 8
        k[0, 0, r.choice(nk, max(1, nk // 20), replace=False)] *= 8
    q8, qs = fp8.quantize_rows(q)
    k8, ks = fp8.quantize_rows(k)
    v8, vs = fp8.quantize_channels(v)
    qrow = np.repeat(qs, 128, axis=2)[0, 0, :nq]
    krow = np.repeat(ks, 128, axis=2)[0, 0, :nk]
    return q8[0, 0], qrow, k8[0, 0], krow, v8[0, 0], vs[0, 0]


CASES = [(1, 70, 70, 64, False, True), (2, 130, 300, 64, True, False), (3, 200, 200, 128, True, True),
         (4, 1, 500, 128, False, True), (5, 64, 64, 16, False, False), (6, 96, 257, 32, True, True)]


@pytest.mark.parametrize("seed,nq,nk,d,outliers,causal", CASES)
def test_kernel_model_stays_inside_the_bound(seed, nq, nk, d, outliers, causal):
    args = _case(seed, nq, nk, d, outliers)
    sc = 1 / math.sqrt(d)
    o, lse, bound, lse_bound = head_bound(*args, sc, causal)
    rng = np.random.default_rng(seed + 100)
    for _ in range(3):
        o_sim, lse_sim = simulate_head(*args, sc, causal, rng)
        err = np.abs(o_sim - o)
        assert (err <= bound).all(), f"max excess {(err - bound).max():.3e}"
        assert (np.abs(lse_sim - lse) <= lse_bound).all()
    # the bound is dominated by the E4M3 rounding of P, not by the fp32 terms: about 2^-4
    # of sum_j P_j |v_j|, a few percent of |O|
    assert 1e-3 < float(np.median(bound)) < 0.2


@pytest.mark.parametrize("seed,nq,nk,d,outliers,causal", [CASES[i] for i in (0, 1, 2, 5)])
def test_bound_catches_a_coarser_rounding_of_p(seed, nq, nk, d, outliers, causal):
    """Rounding P to 3 significant bits (E4M3 has 4) leaves the E4M3 bound somewhere."""
    def round3(x):
        x = np.asarray(x, np.float64)
        e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -6)))
        step = 2.0 ** (e - 2)
        return np.round(x / step) * step

    args = _case(seed, nq, nk, d, outliers)
    sc = 1 / math.sqrt(d)
    o, _, bound, _ = head_bound(*args, sc, causal)
    o_sim, _ = simulate_head(*args, sc, causal, np.random.default_rng(0), p_round=round3)
    assert (np.abs(o_sim - o) > bound).any()


@pytest.mark.parametrize("seed,nq,nk,d,outliers,causal", [CASES[i] for i in (0, 1, 2, 5)])
def test_bound_without_the_p_rounding_term_is_violated(seed, nq, nk, d, outliers, causal):
    """The fp32 terms alone do not cover a kernel that rounds P to E4M3, and they do cover
    one that does not round P."""
    args = _case(seed, nq, nk, d, outliers)
    sc = 1 / math.sqrt(d)
    o, _, bound0, _ = head_bound(*args, sc, causal, p_rel=0.0, p_sub=0.0)
    o_sim, _ = simulate_head(*args, sc, causal, np.random.default_rng(1))
    assert (np.abs(o_sim - o) > bound0).any()
    o_exact_p, _ = simulate_head(*args, sc, causal, np.random.default_rng(2), p_round=lambda x: np.asarray(x))
    assert (np.abs(o_exact_p - o) <= bound0).all()


def test_bound_holds_for_a_wide_value_range():
    """V scaled by 1000 and K rows with large scores: the bound scales with the values."""
    args = _case(9, 100, 333, 64, True, vscale=1000.0)
    o, lse, bound, lse_bound = head_bound(*args, 0.125, True)
    o_sim, lse_sim = simulate_head(*args, 0.125, True, np.random.default_rng(9))
    assert (np.abs(o_sim - o) <= bound).all()
    assert (np.abs(lse_sim - lse) <= lse_bound).all()
    assert E4M3_REL == 2.0 ** -4 and E4M3_SUB == 2.0 ** -10
