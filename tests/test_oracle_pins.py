"""The fp64 oracle pinned to what the pages and the mathematics fix (CPU only)."""

import math

import numpy as np
import pytest

from oracle import naive, tiled_ref
from oracle_pins import (BACKWARD_PINS, CROSS_BACKWARD_PINS, CROSS_FORWARD_PINS, FORWARD_PINS, GQA_BACKWARD_PINS,
                         GQA_FORWARD_PINS, MASK_PINS, golden, pin_block_geometry, pin_block_sparse_causal)


@pytest.mark.parametrize("name,pin", FORWARD_PINS, ids=[n for n, _ in FORWARD_PINS])
def test_forward_pin(name, pin):
    pin(naive.forward_head)


@pytest.mark.parametrize("name,pin", BACKWARD_PINS, ids=[n for n, _ in BACKWARD_PINS])
def test_backward_pin(name, pin):
    pin(naive.forward_head, naive.backward_head)


@pytest.mark.parametrize("name,pin", CROSS_FORWARD_PINS, ids=[n for n, _ in CROSS_FORWARD_PINS])
def test_cross_forward_pin(name, pin):
    pin(naive.forward_head)


@pytest.mark.parametrize("name,pin", CROSS_BACKWARD_PINS, ids=[n for n, _ in CROSS_BACKWARD_PINS])
def test_cross_backward_pin(name, pin):
    pin(naive.backward_head)


@pytest.mark.parametrize("name,pin", GQA_FORWARD_PINS, ids=[n for n, _ in GQA_FORWARD_PINS])
def test_gqa_forward_pin(name, pin):
    pin(naive.forward)


@pytest.mark.parametrize("name,pin", GQA_BACKWARD_PINS, ids=[n for n, _ in GQA_BACKWARD_PINS])
def test_gqa_backward_pin(name, pin):
    pin(naive.backward)


@pytest.mark.parametrize("name,pin", MASK_PINS, ids=[n for n, _ in MASK_PINS])
def test_mask_pin(name, pin):
    pin(naive.forward_head, naive.backward_head)


def test_block_geometry_pin():
    pin_block_geometry(naive.expand_block_mask)


def test_block_sparse_causal_pin():
    pin_block_sparse_causal(naive.forward)


def test_causal_rejects_more_queries_than_keys():
    with pytest.raises(ValueError):
        naive.causal_mask(5, 4)


def test_softmax_rows_worked_example():
    g = golden("softmax_2_1_3.json")
    p, m, l = naive.softmax_rows(np.array([g["row"]]))
    np.testing.assert_array_equal(np.round(p[0], g["weights_decimals"]), g["weights"])
    assert m[0] == 3.0
    # l is the sum after the max shift; times e^m it is the page's sum of exponentials
    assert round(float(l[0] * math.exp(m[0])), g["sum_decimals"]) == g["sum"]


def test_online_two_block_worked_example():
    g = golden("online_two_block.json")
    trace = tiled_ref.online_stats(g["row"], g["block"])
    (m1, l1, _), (m2, l2, _) = trace
    d = g["decimals"]
    assert m1 == g["after_block_1"]["m"] and round(l1, d) == g["after_block_1"]["l"]
    assert m2 == g["after_block_2"]["m"] and round(l2, d) == g["after_block_2"]["l"]
    # the merge as written with the block's own (m~, l~) agrees with the streaming form
    mb, lb = tiled_ref.block_stats(g["row"][2:])
    mm, lm = tiled_ref.merge_stats(m1, l1, mb, lb)
    assert mm == m2 and abs(lm - l2) < 1e-15
    # and with the direct normaliser of the whole row
    _, m, l = naive.softmax_rows(np.array([g["row"]]))
    assert m[0] == m2 and abs(l[0] - l2) < 1e-15


def test_rescale_factor_worked_example():
    g = golden("rescale_factor.json")
    trace = tiled_ref.online_stats(g["row"], g["block"])
    assert trace[0][0] == 3.0 and trace[1][0] == 5.0
    assert round(trace[1][2], g["decimals"]) == g["alpha"]


def _brute_cases():
    for n in range(1, 9):
        for causal in (False, True):
            yield n, causal


@pytest.mark.parametrize("n,causal", list(_brute_cases()))
def test_tiled_equals_untiled_brute_force(n, causal):
    """Every (Br, Bc) in [1..N]^2: the tiled recurrence reaches the definition's O and LSE
    to rounding, including the skipped fully-masked causal blocks."""
    r = np.random.default_rng(100 + n)
    for d in (1, 3):
        q, k, v = (r.standard_normal((n, d)) * 3 for _ in range(3))
        o_ref, lse_ref = naive.forward_head(q, k, v, 0.7, causal)
        for br in range(1, n + 1):
            for bc in range(1, n + 1):
                o, lse = tiled_ref.tiled_forward_head(q, k, v, 0.7, causal, br, bc)
                np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def test_tiled_forward_matches_sdpa_at_tile_scale():
    """A few multi-tile shapes with a ragged tail, against the definition."""
    r = np.random.default_rng(7)
    for n, br, bc, causal in ((200, 64, 32, True), (130, 32, 64, False), (97, 128, 64, True)):
        q, k, v = (r.standard_normal((1, 2, n, 16)) for _ in range(3))
        o, lse = tiled_ref.tiled_forward(q, k, v, 0.25, causal, br, bc)
        o_ref, lse_ref = naive.forward(q, k, v, 0.25, causal)
        np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def test_head_selection_and_batching():
    """forward/backward over (B, H) equal the per-head functions, and a head subset
    leaves the other heads NaN."""
    r = np.random.default_rng(8)
    q, k, v, do = (r.standard_normal((2, 3, 11, 4)) for _ in range(4))
    o, lse = naive.forward(q, k, v, 0.5, True)
    dq, dk, dv = naive.backward(q, k, v, do, 0.5, True)
    for b in range(2):
        for h in range(3):
            o1, l1 = naive.forward_head(q[b, h], k[b, h], v[b, h], 0.5, True)
            np.testing.assert_array_equal(o[b, h], o1)
            np.testing.assert_array_equal(lse[b, h], l1)
            g = naive.backward_head(q[b, h], k[b, h], v[b, h], do[b, h], 0.5, True)
            np.testing.assert_array_equal(dq[b, h], g[0])
            np.testing.assert_array_equal(dk[b, h], g[1])
            np.testing.assert_array_equal(dv[b, h], g[2])
    o2, _ = naive.forward(q, k, v, 0.5, True, heads=[(1, 2)])
    assert np.isnan(o2[0]).all() and np.array_equal(o2[1, 2], o[1, 2])
