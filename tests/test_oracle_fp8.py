"""The FP8 oracle (oracle/fp8.py) pinned to the E4M3 format's definition, the page's claims
about block scales and rotations, the definition of attention, and a rounding bound."""

import math

import numpy as np
import pytest
import torch

from oracle import fp8, naive


def test_e4m3_grid_from_the_format():
    """256 patterns, two NaNs (0x7F, 0xFF), largest value 448 at 0x7E, smallest positive
    2^-9 (subnormal), symmetric, and every finite value distinct except +-0."""
    t = fp8.e4m3_decode()
    assert t.shape == (256,)
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and np.isnan(t).sum() == 2
    fin = t[np.isfinite(t)]
    assert fin.max() == 448.0 == t[0x7E] and fin.min() == -448.0
    assert np.sort(fin[fin > 0])[0] == 2.0 ** -9
    np.testing.assert_array_equal(t[0x80:0xFF], -t[0x00:0x7F])
    assert len(np.unique(fin)) == 253  # 254 finite patterns, +0 and -0 equal
    # the page's two numbers: 256 bit patterns, largest value 448
    assert fp8.E4M3_MAX == 448.0


def test_e4m3_round_is_nearest_even():
    t = fp8.e4m3_decode()
    grid = np.unique(t[np.isfinite(t)])
    np.testing.assert_array_equal(fp8.e4m3_round(grid), grid)            # grid points are fixed
    pos = grid[grid >= 0]
    mids = (pos[:-1] + pos[1:]) / 2                                        # exact ties
    got = fp8.e4m3_round(mids)
    codes = {float(v): c for c, v in enumerate(t[:0x7F])}
    for mid, g, lo, hi in zip(mids, got, pos[:-1], pos[1:]):
        even = lo if codes[float(lo)] % 2 == 0 else hi
        assert g == even, (mid, g, lo, hi)
    r = np.random.default_rng(0)
    x = r.uniform(-460, 460, 20000) * r.choice([1, 1e-2, 1e-4], 20000)
    got = fp8.e4m3_round(x)
    xc = np.clip(x, -448, 448)
    nearest = grid[np.abs(xc[:, None] - grid[None, :]).argmin(axis=1)]
    dist_got, dist_best = np.abs(got - xc), np.abs(nearest - xc)
    np.testing.assert_array_equal(dist_got, dist_best)
    assert fp8.e4m3_round(1000.0) == 448.0 and fp8.e4m3_round(-1e9) == -448.0


def test_block_scales_confine_an_outlier():
    """The page: each block gets its own scale, so an outlier only coarsens its own
    block.  Also: the block's largest magnitude maps to exactly +-448 x scale, and the
    per-element error is at most half an E4M3 step."""
    r = np.random.default_rng(1)
    x = r.standard_normal((1, 2, 300, 64))
    c1, s1 = fp8.quantize_rows(x)
    y = x.copy()
    y[0, 0, 5, 7] = 1000.0                                  # outlier in block 0 of head 0
    c2, s2 = fp8.quantize_rows(y)
    np.testing.assert_array_equal(c2[0, 0, 128:], c1[0, 0, 128:])
    np.testing.assert_array_equal(c2[0, 1], c1[0, 1])
    assert s2[0, 0, 0] > 100 * s1[0, 0, 0] and (s2[0, 0, 1:] == s1[0, 0, 1:]).all()
    d = fp8.dequantize_rows(c1, s1)
    for i in range(3):
        blk = slice(i * 128, (i + 1) * 128)
        assert math.isclose(np.abs(d[:, :, blk]).max(), np.abs(x[:, :, blk]).max(), rel_tol=1e-15)
    xs = x / np.repeat(s1, 128, axis=2)[:, :, :300, None]
    err = np.abs(d - x) / np.repeat(s1, 128, axis=2)[:, :, :300, None]
    bound = np.where(np.abs(xs) >= 2 ** -6, 2 ** -4 * np.abs(xs), 2 ** -10)
    assert (err <= bound * (1 + 1e-12)).all()


def test_channel_scales():
    r = np.random.default_rng(2)
    v = r.standard_normal((1, 1, 50, 8)) * np.arange(1, 9)
    c, s = fp8.quantize_channels(v)
    d = fp8.dequantize_channels(c, s)
    np.testing.assert_allclose(np.abs(d).max(axis=2), np.abs(v).max(axis=2), rtol=1e-15)
    assert (np.abs(d - v) <= 2 ** -4 * np.abs(v) + 2 ** -10 * s[:, :, None, :] + 1e-15).all()


def test_rotation_is_free_before_rounding_and_spreads_an_outlier():
    for d in (64, 128):
        R = fp8.rotation(d, seed=3)
        np.testing.assert_allclose(R @ R.T, np.eye(d), rtol=0, atol=1e-13)
        r = np.random.default_rng(4)
        q, k = r.standard_normal((5, d)), r.standard_normal((7, d))
        np.testing.assert_allclose((q @ R) @ (k @ R).T, q @ k.T, rtol=0, atol=1e-12)
        e = np.zeros(d)
        e[11] = 40.0
        np.testing.assert_allclose(np.abs(e @ R), 40.0 / math.sqrt(d), rtol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk,bc", [(37, 37, 64), (50, 203, 64), (20, 100, 17), (1, 300, 64)])
def test_tiled_recurrence_without_rounding_is_attention(causal, nq, nk, bc):
    r = np.random.default_rng(nq + nk + bc)
    q = r.standard_normal((nq, 8)) * 2
    k, v = r.standard_normal((nk, 8)) * 2, r.standard_normal((nk, 8))
    o, lse = fp8.tiled_forward_head(q, k, v, 0.5, causal, bc, round_p=False)
    o_ref, lse_ref = naive.forward_head(q, k, v, 0.5, causal)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_rounded_p_within_its_bound(causal):
    """Rounding P to E4M3 changes O by at most sum_j |v_j| max(2^-4 P_ij l_i, 2^-10) / l_i
    (half a step, relative for normal values and absolute for subnormal ones, in units
    where the running max is 1), and leaves the logsumexp unchanged."""
    r = np.random.default_rng(5)
    n, d = 260, 16
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    o, lse = fp8.tiled_forward_head(q, k, v, 0.25, causal, 64, round_p=True)
    o_x, lse_x = fp8.tiled_forward_head(q, k, v, 0.25, causal, 64, round_p=False)
    s = naive.scores(q, k, 0.25, causal)
    p, m, l = naive.softmax_rows(s)
    bound = (np.abs(v)[None, :, :] * np.maximum(2 ** -4 * (p * l[:, None])[:, :, None], 2 ** -10)
             * (p > 0)[:, :, None]).sum(axis=1) / l[:, None]
    err = np.abs(o - o_x)
    assert (err <= bound + 1e-12).all()
    assert err.max() > 1e-4                                   # the rounding does act
    np.testing.assert_allclose(lse, lse_x, rtol=0, atol=1e-12)


def test_forward_maps_groups_and_channel_scales():
    r = np.random.default_rng(6)
    B, H, Hkv, nq, nk, d = 1, 4, 2, 70, 150, 16
    q = r.standard_normal((B, H, nq, d))
    k, v = r.standard_normal((B, Hkv, nk, d)), r.standard_normal((B, Hkv, nk, d)) * 3
    q8, sq = fp8.quantize_rows(q)
    k8, sk = fp8.quantize_rows(k)
    v8, sv = fp8.quantize_channels(v)
    o, lse = fp8.forward(q8, sq, k8, sk, v8, sv, 0.3, True, round_p=False)
    qd, kd, vd = fp8.dequantize_rows(q8, sq), fp8.dequantize_rows(k8, sk), fp8.dequantize_channels(v8, sv)
    o_ref, lse_ref = naive.forward(qd, kd, vd, 0.3, True)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_fp8_mutants_are_caught():
    """A decode table with exponent bias 8, a recurrence that forgets to rescale o, and a
    single per-tensor scale each fail one of the checks above."""
    t = fp8.e4m3_decode()
    wrong = t / 2  # bias 8 instead of 7
    assert np.nanmax(wrong) != 448.0
    r = np.random.default_rng(7)
    q, k, v = (r.standard_normal((40, 4)) * 3 for _ in range(3))

    def no_rescale(q, k, v, scale, causal, bc):
        m = np.full(q.shape[0], -np.inf)
        l = np.zeros(q.shape[0])
        o = np.zeros((q.shape[0], v.shape[1]))
        for j0 in range(0, k.shape[0], bc):
            s = scale * q @ k[j0:j0 + bc].T
            m_new = np.maximum(m, s.max(axis=1))
            alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
            p = np.exp(s - m_new[:, None])
            l = l * alpha + p.sum(axis=1)
            o = o + p @ v[j0:j0 + bc]               # the planted mistake: o not rescaled
            m = m_new
        return o / l[:, None]
    assert not np.allclose(no_rescale(q, k, v, 0.5, False, 16), naive.forward_head(q, k, v, 0.5, False)[0], atol=1e-6)
    x = r.standard_normal((1, 1, 300, 8))
    x[0, 0, 3, 0] = 1000.0
    amax = np.abs(x).max()
    per_tensor = fp8.e4m3_codes(x / (amax / 448))
    c, _ = fp8.quantize_rows(x)
    assert (per_tensor[0, 0, 128:] != c[0, 0, 128:]).any()  # a per-tensor scale coarsens every block


def test_near_tie_marks_midpoints():
    t = fp8.e4m3_decode()
    grid = np.unique(t[np.isfinite(t) & (t >= 0)])
    mids = (grid[:-1] + grid[1:]) / 2
    amb, step = fp8.near_tie(mids, 1e-9)
    assert amb.all()
    np.testing.assert_allclose(step, np.diff(grid), rtol=0, atol=0)
    amb, _ = fp8.near_tie(grid[1:], 1e-3)                       # grid points are not ties
    assert not amb.any()
    amb, _ = fp8.near_tie(mids * (1 + 1e-4), 1e-5)
    assert not amb.any()


def test_tie_slack_bounds_a_perturbed_rounding():
    """Perturbing every probability by at most 1e-6 (relative) before rounding moves O by
    no more than the slack computed with tie_rel = 1e-6."""
    r = np.random.default_rng(8)
    q, k, v = (r.standard_normal((90, 8)) for _ in range(3))
    o, lse, slack = fp8.tiled_forward_head(q, k, v, 0.5, True, 64, True, tie_rel=1e-6)
    orig = fp8.e4m3_round
    try:
        fp8.e4m3_round = lambda x: orig(np.asarray(x) * (1 + 1e-6 * r.uniform(-1, 1, np.shape(x))))
        o2, _ = fp8.tiled_forward_head(q, k, v, 0.5, True, 64, True)
    finally:
        fp8.e4m3_round = orig
    assert (np.abs(o2 - o) <= slack + 1e-12).all()


# Two rows whose exact E4M3 outcome follows from the format's grid by hand, and which
# fix the model's schedule: keys in 64-key tiles aligned at key 0, the running max
# updated at every tile, P rounded relative to it.  One query q = 1 (d = 1, scale 1),
# key scores are the k values; "far" keys score -1000 (p = 0 exactly).
A = math.log(0.515625)  # e^A = 0.515625 = 33/64, between the E4M3 values 0.5 and 0.5625


def _row(nk, scores):
    k = np.full((nk, 1), -1000.0)
    v = np.zeros((nk, 2))
    for j, (s, col) in scores.items():
        k[j, 0] = s
        v[j, col] = 1.0
    return np.ones((1, 1)), k, v


def test_schedule_pin_one_tile():
    """Keys 0 (score A) and 40 (score 0) share the first 64-key tile: the tile max is 0, so
    p_0 = 0.515625 is rounded to E4M3 before the P V product -> 0.5 (the nearer grid
    value; the midpoint is 0.53125); the denominator uses the unrounded p.
    O = (0.5, 1) / 1.515625, lse = ln 1.515625."""
    q, k, v = _row(64, {0: (A, 0), 40: (0.0, 1)})
    o, lse = fp8.tiled_forward_head(q, k, v, 1.0, False, bc=64, round_p=True)
    np.testing.assert_allclose(o[0], [0.5 / 1.515625, 1 / 1.515625], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0], math.log(1.515625), rtol=0, atol=1e-15)


def test_schedule_pin_two_tiles():
    """Keys 0 (score A) and 64 (score 0) in consecutive tiles: tile 1 sees only key 0 (max A,
    p_0 = 1, exact in E4M3), tile 2 raises the max to 0 and rescales o by e^A; p_64 = 1.
    Nothing is rounded: O = (0.515625, 1) / 1.515625, the exact attention."""
    q, k, v = _row(128, {0: (A, 0), 64: (0.0, 1)})
    o, lse = fp8.tiled_forward_head(q, k, v, 1.0, False, bc=64, round_p=True)
    np.testing.assert_allclose(o[0], [0.515625 / 1.515625, 1 / 1.515625], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0], math.log(1.515625), rtol=0, atol=1e-15)


def test_schedule_pins_catch_other_schedules():
    """A 32-key tiling puts keys 0 and 40 in different tiles (first pin fails: nothing is
    rounded), and a lazily updated max (moved only when a tile's max exceeds it by 8 in
    log2 units) keeps the reference at A in the second pin, so p_64 = 1/0.515625 = 1.939
    is rounded to 2.0 (second pin fails)."""
    q, k, v = _row(64, {0: (A, 0), 40: (0.0, 1)})
    o32, _ = fp8.tiled_forward_head(q, k, v, 1.0, False, bc=32, round_p=True)
    assert abs(o32[0, 0] - 0.5 / 1.515625) > 1e-3

    def lazy(q, k, v, bc=64, slack=8.0):
        m, l, o = -np.inf, 0.0, np.zeros(v.shape[1])
        for j0 in range(0, k.shape[0], bc):
            s = (q @ k[j0:j0 + bc].T)[0]
            mx = s.max()
            if mx * math.log2(math.e) > m * math.log2(math.e) + slack or m == -np.inf:
                a = 0.0 if m == -np.inf else math.exp(m - mx)
                l, o, m = l * a, o * a, max(m, mx)
            p = np.exp(s - m)
            l += p.sum()
            o = o + fp8.e4m3_round(p) @ v[j0:j0 + bc]
        return o / l

    q, k, v = _row(128, {0: (A, 0), 64: (0.0, 1)})
    ol = lazy(q, k, v)
    np.testing.assert_allclose(ol, [1 / (1 + 1 / 0.515625), 2 / (1 + 1 / 0.515625)], rtol=0, atol=1e-12)
    assert abs(ol[1] - 1 / 1.515625) > 1e-2
