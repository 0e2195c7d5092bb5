"""GPU parity on a seeded sweep of random shapes: batch, grouped heads, query and key
lengths that differ and cross tile edges, both head dimensions and all storage types,
launched whole, split over the key range and under random block masks, forward and
backward, every element against the fp64 oracle.

The named workloads and the hand-picked cases elsewhere pin each path at chosen shapes;
this sweep draws the combinations nobody picked (a short ragged group under a split, a
mask with an empty block row on a grouped head, ...).  The case list is fixed by its seed,
so every run checks the same cases and a failure names one by its id.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_forward_amd as fa
from exact_tiled_attention_forward_amd.workloads import make_cross_inputs
from oracle import naive
from parity import assert_close, assert_lse, to64

pytestmark = pytest.mark.gpu


def _draw_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(["bf16", "f16", "f32"], p=[0.45, 0.4, 0.15]))
        B = int(rng.integers(1, 3))
        Hkv = int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 4, 8]))
        # lengths from 1 to about 1500, biased to the small end and to tile edges +- 1
        def length():
            if rng.random() < 0.3:
                return int(max(1, rng.choice([32, 64, 128, 256, 512, 1024]) + rng.integers(-1, 2)))
            return int(np.exp(rng.uniform(0, np.log(1500))))
        Nq, Nk = length(), length()
        causal = bool(rng.random() < 0.5)
        if causal and Nq > Nk:
            Nq, Nk = Nk, Nq
        launch = str(rng.choice(["whole", "split", "mask"], p=[0.4, 0.35, 0.25]))
        if dt == "f32" and launch == "mask":
            launch = "whole"  # block masks take 16-bit inputs
        nsplit = int(rng.integers(2, 9)) if launch == "split" else None
        cases.append((i, B, Hkv * G, Hkv, Nq, Nk, d, dt, causal, launch, nsplit))
    return cases


CASES = _draw_cases(160, seed=20240601)


def _id(c):
    i, B, Hq, Hkv, Nq, Nk, d, dt, causal, launch, nsplit = c
    extra = f"_s{nsplit}" if nsplit else ""
    return f"{i:03d}_B{B}_Hq{Hq}_Hkv{Hkv}_Nq{Nq}_Nk{Nk}_d{d}_{dt}_{'causal' if causal else 'full'}_{launch}{extra}"


def _check_lse(lse, ref):
    lse, ref = to64(lse), to64(ref)
    empty = ~np.isfinite(ref)
    assert np.array_equal(~np.isfinite(lse), empty), "rows without a visible key differ"
    if (~empty).any():
        assert_lse(lse[~empty], ref[~empty])


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_shape(case):
    i, B, Hq, Hkv, Nq, Nk, d, dt, causal, launch, nsplit = case
    inp = make_cross_inputs(B, Hq, Hkv, Nq, Nk, d, dt, seed_base=31000 + 37 * i, with_do=dt != "f32")
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    bm = None
    if launch == "mask":
        rng = np.random.default_rng(500 + i)
        heads = int(rng.choice([1, Hq]))
        bm = (rng.random((heads, -(-Nq // 128), -(-Nk // 128))) < rng.uniform(0.3, 0.9)).astype(np.uint8)
    bmg = torch.from_numpy(bm).cuda() if bm is not None else None
    o, lse = fa.fa_forward(q, k, v, causal=causal, split=nsplit, block_mask=bmg)
    torch.cuda.synchronize()
    ref_in = [to64(inp[x]) for x in ("q", "k", "v")]
    scale = 1 / math.sqrt(d)
    o_ref, lse_ref = naive.forward(*ref_in, scale, causal, block_mask=bm)
    mx, mean, ex, _ = assert_close(_id(case) + " O", o.cpu(), o_ref, dt, floor_aware=True)
    _check_lse(lse.cpu(), lse_ref)
    msg = f"O max {mx:.2e} (beyond floor {ex:.2e}) mean {mean:.2e}"
    if dt != "f32" and Nq > 1:
        do = inp["do"].cuda()
        dq, dk, dv = fa.fa_backward(q, k, v, o, do, lse, causal=causal, block_mask=bmg)
        torch.cuda.synchronize()
        ref = naive.backward(*ref_in, to64(inp["do"]), scale, causal, block_mask=bm)
        for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            gmx, gmean, _, _ = assert_close(f"{_id(case)} {name}", g.cpu(), r, dt, out_dtype="f32")
            msg += f"; {name} max {gmx:.2e}"
    print(_id(case) + ": " + msg)


def _draw_fp8_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.integers(1, 3))
        G = int(rng.choice([1, 2, 4]))
        Nq, Nk = (int(np.exp(rng.uniform(0, np.log(1200)))) for _ in range(2))
        causal = bool(rng.random() < 0.5)
        if causal and Nq > Nk:
            Nq, Nk = Nk, Nq
        cases.append((i, int(rng.integers(1, 3)), Hkv * G, Hkv, Nq, Nk, d, causal))
    return cases


FP8_CASES = _draw_fp8_cases(24, seed=20240602)


def _fp8_id(c):
    i, B, Hq, Hkv, Nq, Nk, d, causal = c
    return f"{i:02d}_B{B}_Hq{Hq}_Hkv{Hkv}_Nq{Nq}_Nk{Nk}_d{d}_{'causal' if causal else 'full'}"


@pytest.mark.parametrize("case", FP8_CASES, ids=[_fp8_id(c) for c in FP8_CASES])
def test_random_shape_fp8(case):
    """The E4M3 path on random shapes: quantize Q, K (128-row blocks) and V (channels),
    then every element of O within the per-element bound derived for E4M3 probabilities,
    fp32 arithmetic and the bf16 output, against exact attention on the dequantized
    inputs; lse within its bound and the relative lse bar."""
    from fp8_bound import forward_bound

    i, B, Hq, Hkv, Nq, Nk, d, causal = case
    inp = make_cross_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", seed_base=33000 + 41 * i)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    q8, qs = fa.fa_quantize_fp8(q)
    k8, ks = fa.fa_quantize_fp8(k)
    v8, vs = fa.fa_quantize_fp8(v, per_channel=True)
    o, lse = fa.fa_forward_fp8(q8, qs, k8, ks, v8, vs, causal=causal)
    torch.cuda.synchronize()
    args = [a.cpu().numpy() for a in (q8, qs, k8, ks, v8, vs)]
    o_ex, lse_ex, bound, lse_bound = forward_bound(*args, 1 / math.sqrt(d), causal)
    err = np.abs(to64(o.cpu()) - o_ex)
    assert (err <= bound).all(), f"{(err > bound).sum()} elements beyond the bound, worst excess {(err - bound).max():.3e}"
    lse_out = to64(lse.cpu())
    assert (np.abs(lse_out - lse_ex) <= lse_bound).all()
    assert_lse(lse_out, lse_ex)
    print(_fp8_id(case) + f": max {err.max():.2e}, max error/bound {(err / bound).max():.2f}")
