"""Pins for the fp64 oracle, written as functions of the implementation under test.

Each pin takes callables ``fwd(q, k, v, scale, causal) -> (O, LSE)`` and/or
``bwd(q, k, v, dO, scale, causal) -> (dQ, dK, dV)`` for one head (2-D arrays) and
raises AssertionError when the implementation disagrees with something the pages
or the mathematics fix.  ``test_oracle_pins.py`` runs them on the oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with a planted mistake
and checks that some pin fails.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- forward pins


def pin_worked_softmax(fwd):
    """Softmax of [2, 1, 3] embedded in an attention head: q0 = e1, k_j = x_j e1,
    v_j = e_(j+1), scale 1.  Row 0 of O is the softmax weights; exp(LSE_0) is the sum."""
    g = golden("softmax_2_1_3.json")
    x = np.array(g["row"])
    n, d = 3, 4
    q = np.zeros((n, d)); q[:, 0] = 1.0
    k = np.zeros((n, d)); k[:, 0] = x
    v = np.zeros((n, d)); v[np.arange(n), np.arange(n) + 1] = 1.0
    o, lse = fwd(q, k, v, 1.0, False)
    np.testing.assert_array_equal(np.round(o[0, 1:4], g["weights_decimals"]), g["weights"])
    assert o[0, 0] == 0.0
    assert round(float(np.exp(lse[0])), g["sum_decimals"]) == g["sum"]
    # each exponential: weight * sum
    np.testing.assert_array_equal(np.round(o[0, 1:4] * np.exp(lse[0]), g["exp_decimals"]), g["exp"])


def pin_worked_two_block(fwd):
    """[1, 2, 0, 3] as the score row of query 0: the direct normaliser with m = 3 is the
    value the two-block example reaches, 1.553, so LSE_0 = 3 + ln(1.553...)."""
    g = golden("online_two_block.json")
    x = np.array(g["row"])
    n, d = 4, 2
    q = np.zeros((n, d)); q[:, 0] = 1.0
    k = np.zeros((n, d)); k[:, 0] = x
    v = np.zeros((n, d)); v[:, 1] = np.arange(n)
    _, lse = fwd(q, k, v, 1.0, False)
    m = g["after_block_2"]["m"]
    assert round(float(np.exp(lse[0] - m)), g["decimals"]) == g["after_block_2"]["l"]


def pin_overflow(fwd):
    """Scores far beyond the fp32 exp limit stay finite: a row [1000, 999] gives weights
    e/(e+1) and 1/(e+1) (closed form)."""
    g = golden("fp32_exp_limit.json")
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(np.exp(np.float32(g["overflow_exponent"]))))
    assert round(math.log(np.finfo(np.float32).max), g["limit_decimals"]) == g["limit_exponent"]
    q = np.array([[1.0, 0.0], [1.0, 0.0]])
    k = np.array([[1000.0, 0.0], [999.0, 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    o, lse = fwd(q, k, v, 1.0, False)
    w = math.e / (math.e + 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    np.testing.assert_allclose(o[0], [w, 1.0 - w], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0], 1000.0 + math.log1p(math.exp(-1.0)), rtol=1e-15, atol=0)


def pin_q_zero(fwd, causal):
    """Q = 0: every visible key has the same score, so O_i is the mean of the visible
    V rows and LSE_i = ln(number of visible keys)."""
    r = _rng(11)
    n, d = 9, 5
    q = np.zeros((n, d)); k = r.standard_normal((n, d)); v = r.standard_normal((n, d))
    o, lse = fwd(q, k, v, 0.3, causal)
    for i in range(n):
        vis = i + 1 if causal else n
        np.testing.assert_allclose(o[i], v[:vis].mean(axis=0), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[i], math.log(vis), rtol=0, atol=1e-13)


def pin_single_key(fwd):
    """N = 1: O = V and LSE = scale q.k."""
    r = _rng(12)
    q, k, v = (r.standard_normal((1, 7)) for _ in range(3))
    o, lse = fwd(q, k, v, 0.7, True)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0], 0.7 * float(q[0] @ k[0]), rtol=1e-14, atol=1e-14)


def pin_constant_v(fwd, causal):
    """All V rows equal c: O_i = c for every row."""
    r = _rng(13)
    n, d = 8, 6
    q, k = r.standard_normal((n, d)), r.standard_normal((n, d))
    c = r.standard_normal(d)
    o, _ = fwd(q, k, np.tile(c, (n, 1)), 0.5, causal)
    np.testing.assert_allclose(o, np.tile(c, (n, 1)), rtol=0, atol=1e-13)


def pin_key_shift(fwd, causal):
    """K_j -> K_j + u for every key: each score row moves by a constant, so O is
    unchanged and LSE_i moves by scale q_i.u."""
    r = _rng(14)
    n, d = 10, 4
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    u = r.standard_normal(d)
    o1, l1 = fwd(q, k, v, 0.4, causal)
    o2, l2 = fwd(q, k + u, v, 0.4, causal)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + 0.4 * (q @ u), rtol=0, atol=1e-12)


def pin_rows_sum_to_one(fwd, causal):
    """P rows sum to 1 and, with causal masking, vanish above the diagonal: with V = I,
    O = P."""
    r = _rng(15)
    n = 7
    q, k = r.standard_normal((n, 3)), r.standard_normal((n, 3))
    p, _ = fwd(q, k, np.eye(n), 0.9, causal)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(p >= 0)
    if causal:
        assert np.all(np.triu(p, 1) == 0.0)
        assert np.all(np.diag(p) > 0)


def pin_sdpa(fwd, causal, n=33, d=16, seed=16):
    """torch's scaled_dot_product_attention (CPU, float64, math path) as an
    independent library routine; LSE against torch.logsumexp of the masked scores."""
    r = _rng(seed)
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    scale = 1.0 / math.sqrt(d)
    o, lse = fwd(q, k, v, scale, causal)
    tq, tk, tv = (torch.from_numpy(a)[None, None] for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)[0, 0]
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    s = torch.from_numpy(q) @ torch.from_numpy(k).T * scale
    if causal:
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- backward pins


def pin_autograd(bwd, causal, n=21, d=8, seed=17):
    """Gradients of torch's fp64 SDPA (autograd on CPU) against the oracle's."""
    r = _rng(seed)
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    tq, tk, tv = (torch.from_numpy(a)[None, None].requires_grad_(True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    out.backward(torch.from_numpy(do)[None, None])
    dq, dk, dv = bwd(q, k, v, do, scale, causal)
    np.testing.assert_allclose(dq, tq.grad[0, 0].numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dk, tk.grad[0, 0].numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dv, tv.grad[0, 0].numpy(), rtol=0, atol=1e-10)


def pin_finite_differences(fwd, bwd, causal, n=6, d=3, seed=18):
    """Central differences of L = sum(O * dO) against dQ, dK, dV at every entry."""
    r = _rng(seed)
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    scale = 0.8
    dq, dk, dv = bwd(q, k, v, do, scale, causal)
    h = 1e-6

    def loss(qq, kk, vv):
        return float(np.sum(fwd(qq, kk, vv, scale, causal)[0] * do))

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=0, atol=1e-7, err_msg=f"d{name}")


def pin_backward_invariants(bwd, causal, n=12, d=5, seed=19):
    """sum_j dK_j = 0 (rows of dS sum to zero); sum_j dV_j = sum_i dO_i (rows of P sum
    to one); with causal masking dQ_0 = 0 (row 0 sees only key 0)."""
    r = _rng(seed)
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    dq, dk, dv = bwd(q, k, v, do, 0.6, causal)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=0, atol=1e-12)
    if causal:
        np.testing.assert_allclose(dq[0], 0.0, rtol=0, atol=1e-14)


def pin_backward_scaling(bwd, causal, n=9, d=4, seed=20):
    """(Q, scale) -> (aQ, scale/a) leaves S unchanged: dK and dV unchanged, dQ -> dQ/a;
    K -> K + u leaves dQ, dK, dV unchanged."""
    r = _rng(seed)
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    a = 2.5
    g1 = bwd(q, k, v, do, 0.5, causal)
    g2 = bwd(a * q, k, v, do, 0.5 / a, causal)
    np.testing.assert_allclose(g2[0] * a, g1[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(g2[1], g1[1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(g2[2], g1[2], rtol=0, atol=1e-12)
    u = r.standard_normal(d)
    g3 = bwd(q, k + u, v, do, 0.5, causal)
    for x, y in zip(g3, g1):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)


# ------------------------------------------------ query/key lengths that differ, grouped heads


def pin_cross_sdpa(fwd, nq=7, nk=19, d=8, seed=21):
    """N_q != N_k without a mask: torch SDPA (fp64, CPU) as the library routine."""
    r = _rng(seed)
    q = r.standard_normal((nq, d))
    k, v = (r.standard_normal((nk, d)) for _ in range(2))
    scale = 1.0 / math.sqrt(d)
    o, lse = fwd(q, k, v, scale, False)
    tq, tk, tv = (torch.from_numpy(a)[None, None] for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)[0, 0]
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    s = torch.from_numpy(q) @ torch.from_numpy(k).T * scale
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


def pin_causal_suffix(fwd, n=23, nq=5, d=6, seed=22):
    """Causal with N_q < N_k: the queries are the last N_q positions, so the result is
    the last N_q rows of causal self-attention over the whole sequence (whose square
    case the SDPA pin fixes).  Any other alignment of the mask fails this."""
    r = _rng(seed)
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    o_full, lse_full = fwd(q, k, v, 0.4, True)
    for m in (nq, 1, n - 1):
        o, lse = fwd(q[n - m:], k, v, 0.4, True)
        np.testing.assert_allclose(o, o_full[n - m:], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, lse_full[n - m:], rtol=0, atol=1e-13)


def pin_decode_row(fwd, nk=17, d=5, seed=23):
    """One causal query against N_k keys (a decode step) sees every key: it equals the
    unmasked result."""
    r = _rng(seed)
    q = r.standard_normal((1, d))
    k, v = (r.standard_normal((nk, d)) for _ in range(2))
    o_c, lse_c = fwd(q, k, v, 0.9, True)
    o_f, lse_f = fwd(q, k, v, 0.9, False)
    np.testing.assert_array_equal(o_c, o_f)
    np.testing.assert_array_equal(lse_c, lse_f)


def pin_cross_autograd(bwd, nq=6, nk=15, d=4, seed=24):
    """N_q != N_k gradients against torch autograd through fp64 SDPA (no mask)."""
    r = _rng(seed)
    q, do = (r.standard_normal((nq, d)) for _ in range(2))
    k, v = (r.standard_normal((nk, d)) for _ in range(2))
    scale = 0.7
    tq, tk, tv = (torch.from_numpy(a)[None, None].requires_grad_(True) for a in (q, k, v))
    torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale).backward(torch.from_numpy(do)[None, None])
    dq, dk, dv = bwd(q, k, v, do, scale, False)
    for x, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(x, t.grad[0, 0].numpy(), rtol=0, atol=1e-10)


def pin_backward_suffix(bwd, n=14, nq=4, d=3, seed=25):
    """Causal N_q < N_k gradients equal those of causal self-attention over the whole
    sequence when only the last N_q rows of O carry a gradient (dO = 0 elsewhere)."""
    r = _rng(seed)
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    do = r.standard_normal((nq, d))
    do_full = np.zeros((n, d))
    do_full[n - nq:] = do
    dq_f, dk_f, dv_f = bwd(q, k, v, do_full, 0.5, True)
    dq, dk, dv = bwd(q[n - nq:], k, v, do, 0.5, True)
    np.testing.assert_allclose(dq, dq_f[n - nq:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, dk_f, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, dv_f, rtol=0, atol=1e-12)


def _gqa_inputs(seed, B=2, hkv=2, g=3, nq=9, nk=11, d=4):
    r = _rng(seed)
    q = r.standard_normal((B, hkv * g, nq, d))
    k, v = (r.standard_normal((B, hkv, nk, d)) for _ in range(2))
    do = r.standard_normal((B, hkv * g, nq, d))
    return q, k, v, do


def pin_gqa_sdpa(fwd_mh, causal, seed=26):
    """Grouped heads (H_q = 3 H_kv) against torch SDPA with enable_gqa (fp64, CPU), and
    against the one-head-per-group computation with K, V repeated per query head."""
    q, k, v, _ = _gqa_inputs(seed)
    g = q.shape[1] // k.shape[1]
    o, lse = fwd_mh(q, k, v, 0.6, causal)
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    if causal:  # top-left and bottom-right coincide only when N_q == N_k
        tk, tv = tk[:, :, :q.shape[2]], tv[:, :, :q.shape[2]]
        o, lse = fwd_mh(q, k[:, :, :q.shape[2]], v[:, :, :q.shape[2]], 0.6, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.6, enable_gqa=True)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    o_r, lse_r = fwd_mh(q, np.repeat(tk.numpy(), g, axis=1), np.repeat(tv.numpy(), g, axis=1), 0.6, causal)
    np.testing.assert_array_equal(o, o_r)
    np.testing.assert_array_equal(lse, lse_r)


def pin_gqa_autograd(bwd_mh, causal, seed=27):
    """Grouped-head gradients against torch autograd through fp64 SDPA with enable_gqa:
    dK and dV of a shared head are the sums over its group."""
    q, k, v, do = _gqa_inputs(seed, nk=9)
    tq, tk, tv = (torch.from_numpy(a).requires_grad_(True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.6, enable_gqa=True)
    out.backward(torch.from_numpy(do))
    dq, dk, dv = bwd_mh(q, k, v, do, 0.6, causal)
    for x, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(x, t.grad.numpy(), rtol=0, atol=1e-10)


# ------------------------------------------------ block-sparse masks, empty rows


def _random_hidden(r, nq, nk, keep=0.6):
    """A random hidden-key mask in which every query keeps at least one key."""
    hid = r.random((nq, nk)) > keep
    hid[np.arange(nq), r.integers(0, nk, nq)] = False
    return hid


def pin_mask_sdpa(fwd, nq=11, nk=23, d=6, seed=31):
    """An arbitrary hidden-key mask against torch SDPA with the boolean attn_mask
    (fp64, CPU); LSE against torch.logsumexp of the masked scores."""
    r = _rng(seed)
    q = r.standard_normal((nq, d))
    k, v = (r.standard_normal((nk, d)) for _ in range(2))
    hid = _random_hidden(r, nq, nk)
    o, lse = fwd(q, k, v, 0.5, False, hid)
    tq, tk, tv = (torch.from_numpy(a)[None, None] for a in (q, k, v))
    keep = torch.from_numpy(~hid)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=keep, scale=0.5)[0, 0]
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    sm = (torch.from_numpy(q) @ torch.from_numpy(k).T * 0.5).masked_fill(~keep, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(sm, dim=-1).numpy(), rtol=0, atol=1e-12)


def pin_mask_autograd(bwd, nq=9, nk=14, d=4, seed=32):
    """Gradients with an arbitrary hidden-key mask against autograd through fp64 SDPA."""
    r = _rng(seed)
    q, do = (r.standard_normal((nq, d)) for _ in range(2))
    k, v = (r.standard_normal((nk, d)) for _ in range(2))
    hid = _random_hidden(r, nq, nk)
    tq, tk, tv = (torch.from_numpy(a)[None, None].requires_grad_(True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(~hid), scale=0.8)
    out.backward(torch.from_numpy(do)[None, None])
    dq, dk, dv = bwd(q, k, v, do, 0.8, False, hid)
    for x, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(x, t.grad[0, 0].numpy(), rtol=0, atol=1e-10)


def pin_empty_row(fwd, bwd, nq=7, nk=9, d=3, seed=33):
    """A query row with every key hidden: O = 0, LSE = -inf and zero dQ; the other rows
    are exactly what they are without that row, and dK, dV do not change."""
    r = _rng(seed)
    q, do = (r.standard_normal((nq, d)) for _ in range(2))
    k, v = (r.standard_normal((nk, d)) for _ in range(2))
    hid = _random_hidden(r, nq, nk)
    hid[3] = True
    o, lse = fwd(q, k, v, 0.6, False, hid)
    assert np.all(o[3] == 0.0) and lse[3] == -np.inf
    rest = [i for i in range(nq) if i != 3]
    o2, lse2 = fwd(q[rest], k, v, 0.6, False, hid[rest])
    np.testing.assert_array_equal(o[rest], o2)
    np.testing.assert_array_equal(lse[rest], lse2)
    dq, dk, dv = bwd(q, k, v, do, 0.6, False, hid)
    assert np.all(dq[3] == 0.0)
    dq2, dk2, dv2 = bwd(q[rest], k, v, do[rest], 0.6, False, hid[rest])
    np.testing.assert_allclose(dk, dk2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv, dv2, rtol=0, atol=1e-14)


def pin_block_geometry(expand):
    """128 x 128 blocks, ragged at the ends: a 2 x 3 block mask over 130 queries and 260
    keys, checked at block edges and in the ragged last block."""
    bm = np.array([[1, 0, 1], [0, 1, 0]], np.uint8)
    hid = expand(bm, 130, 260)
    assert hid.shape == (130, 260)
    expect = {(0, 0): False, (127, 127): False, (127, 128): True, (128, 127): True, (128, 128): False,
              (129, 255): False, (129, 256): True, (0, 256): False, (0, 259): False, (129, 259): True}
    for (i, j), h in expect.items():
        assert bool(hid[i, j]) == h, (i, j)
    assert hid[:128, 128:256].all() and not hid[:128, :128].any()
    try:
        expand(bm, 257, 260)
    except ValueError:
        pass
    else:
        raise AssertionError("a block mask of the wrong shape must be rejected")


def pin_block_sparse_causal(fwd_mh, seed=34):
    """A block mask that keeps exactly the blocks on or below the diagonal changes
    nothing under causal masking; an all-ones block mask changes nothing at all."""
    r = _rng(seed)
    B, H, N, d = 1, 2, 300, 4
    q, k, v = (r.standard_normal((B, H, N, d)) for _ in range(3))
    nb = -(-N // 128)
    lower = np.tril(np.ones((nb, nb), np.uint8))[None]
    o_c, l_c = fwd_mh(q, k, v, 0.5, True)
    o_b, l_b = fwd_mh(q, k, v, 0.5, True, block_mask=lower)
    np.testing.assert_array_equal(o_b, o_c)
    np.testing.assert_array_equal(l_b, l_c)
    ones = np.ones((H, nb, nb), np.uint8)
    o_f, l_f = fwd_mh(q, k, v, 0.5, False)
    o_1, l_1 = fwd_mh(q, k, v, 0.5, False, block_mask=ones)
    np.testing.assert_array_equal(o_1, o_f)
    np.testing.assert_array_equal(l_1, l_f)


MASK_PINS = [
    ("mask_sdpa", lambda f, b: pin_mask_sdpa(f)),
    ("mask_autograd", lambda f, b: pin_mask_autograd(b)),
    ("empty_row", lambda f, b: pin_empty_row(f, b)),
]


CROSS_FORWARD_PINS = [
    ("cross_sdpa", pin_cross_sdpa),
    ("causal_suffix", pin_causal_suffix),
    ("decode_row", pin_decode_row),
]

CROSS_BACKWARD_PINS = [
    ("cross_autograd", pin_cross_autograd),
    ("backward_suffix", pin_backward_suffix),
]

GQA_FORWARD_PINS = [(f"gqa_sdpa_{'causal' if c else 'full'}", (lambda c: (lambda f: pin_gqa_sdpa(f, c)))(c))
                    for c in (False, True)]
GQA_BACKWARD_PINS = [(f"gqa_autograd_{'causal' if c else 'full'}", (lambda c: (lambda b: pin_gqa_autograd(b, c)))(c))
                     for c in (False, True)]


FORWARD_PINS = [
    ("worked_softmax", lambda f: pin_worked_softmax(f)),
    ("worked_two_block", lambda f: pin_worked_two_block(f)),
    ("overflow", lambda f: pin_overflow(f)),
    ("single_key", lambda f: pin_single_key(f)),
] + [
    (f"{name}_{'causal' if c else 'full'}", (lambda p, c: (lambda f: p(f, c)))(p, c))
    for name, p in (("q_zero", pin_q_zero), ("constant_v", pin_constant_v), ("key_shift", pin_key_shift),
                    ("rows_sum_to_one", pin_rows_sum_to_one), ("sdpa", pin_sdpa))
    for c in (False, True)
]

BACKWARD_PINS = [
    (f"{name}_{'causal' if c else 'full'}", (lambda p, c: (lambda f, b: p(b, c)))(p, c))
    for name, p in (("autograd", pin_autograd), ("invariants", pin_backward_invariants),
                    ("scaling", pin_backward_scaling))
    for c in (False, True)
] + [
    (f"finite_differences_{'causal' if c else 'full'}", (lambda c: (lambda f, b: pin_finite_differences(f, b, c)))(c))
    for c in (False, True)
]
