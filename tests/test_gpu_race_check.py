"""Race check: the release library against its race-check build, bit for bit.

The race-check build (libfa_racecheck.so, compiled with FA_RACE_CHECK=1) computes the
same arithmetic on a perturbed schedule: after every workgroup barrier each wave sleeps
for a time that grows with its index modulo 4 (up to about 12000 cycles, longer than a
tile fill takes to land), and every LDS tile fill waits for itself as soon as it is
issued.  A tile buffer refilled while some wave may still read it, or read before
its fill has landed, changes the output under one schedule or the other.  Every kernel
path is exercised: the two-phase d = 128 forward, the lock-step forward (d = 64, block
masks, split key ranges), the key-parallel decode kernel, the fp32 and FP8 forwards, and
both backward kernels.
"""

import contextlib

import numpy as np
import pytest
import torch

import exact_tiled_attention_forward_amd as fa
from exact_tiled_attention_forward_amd.workloads import make_cross_inputs

pytestmark = pytest.mark.gpu

_racecheck = None


def racecheck_library():
    global _racecheck
    if _racecheck is None:
        _racecheck = fa.load_library(fa.RACECHECK_LIB_PATH)
    return _racecheck


@contextlib.contextmanager
def using(lib):
    """Route the binding's calls to `lib` for the duration of the block."""
    saved = fa._lib
    fa._lib = lib
    try:
        yield
    finally:
        fa._lib = saved


def both_builds(run):
    """run() -> dict of tensors, once per build; the two must agree bit for bit."""
    with using(fa.library()):
        ref = {k: t.clone() for k, t in run().items()}
    with using(racecheck_library()):
        got = run()
    torch.cuda.synchronize()
    for k in ref:
        a, b = ref[k].contiguous(), got[k].contiguous()
        same = torch.equal(a.view(torch.uint8), b.view(torch.uint8))
        assert same, (f"{k}: release and race-check builds differ "
                      f"(max |diff| {(a.float() - b.float()).abs().nan_to_num(0.0).max().item():.3e})")


# (B, Hq, Hkv, Nq, Nk, d, dtype, causal, split)
FWD = [
    (1, 4, 4, 1100, 1100, 128, "bf16", True, 1),     # two-phase kernel, ragged
    (2, 2, 2, 700, 700, 128, "f16", False, 1),       # two-phase kernel, one partial block
    (1, 8, 2, 600, 900, 128, "bf16", True, 1),       # two-phase kernel, grouped heads, Nq < Nk
    (2, 3, 3, 1000, 1000, 64, "bf16", True, 1),      # lock-step d = 64
    (1, 2, 2, 2048, 2048, 64, "f16", True, 5),       # split key range and merge
    (1, 2, 2, 1500, 1500, 128, "bf16", False, 4),    # split at d = 128
    (2, 8, 2, 1, 3000, 128, "bf16", True, None),     # decode: key-parallel kernel
    (1, 2, 2, 300, 300, 64, "f32", False, None),     # fp32, split
]


def _id(c):
    B, Hq, Hkv, Nq, Nk, d, dt, causal, split = c
    return f"B{B}_Hq{Hq}_Hkv{Hkv}_Nq{Nq}_Nk{Nk}_d{d}_{dt}_{'causal' if causal else 'full'}_split{split}"


@pytest.mark.parametrize("case", FWD, ids=[_id(c) for c in FWD])
def test_forward_same_under_a_perturbed_schedule(case):
    B, Hq, Hkv, Nq, Nk, d, dt, causal, split = case
    inp = make_cross_inputs(B, Hq, Hkv, Nq, Nk, d, dt, seed_base=15000 + Nq + d)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))

    def run():
        o, lse = fa.fa_forward(q, k, v, causal=causal, split=split)
        return {"o": o, "lse": lse}

    both_builds(run)


# (B, Hq, Hkv, N, d, dtype, causal)
BWD = [
    (1, 2, 2, 1000, 128, "bf16", True),
    (1, 4, 2, 700, 64, "f16", True),
    (2, 2, 2, 333, 128, "bf16", False),
]


@pytest.mark.parametrize("case", BWD, ids=[f"B{c[0]}_Hq{c[1]}_Hkv{c[2]}_N{c[3]}_d{c[4]}_{c[5]}_{c[6]}" for c in BWD])
def test_backward_same_under_a_perturbed_schedule(case):
    B, Hq, Hkv, N, d, dt, causal = case
    inp = make_cross_inputs(B, Hq, Hkv, N, N, d, dt, seed_base=16000 + N + d, with_do=True)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    o, lse = fa.fa_forward(q, k, v, causal=causal)

    def run():
        dq, dk, dv = fa.fa_backward(q, k, v, o, do, lse, causal=causal)
        return {"dq": dq, "dk": dk, "dv": dv}

    both_builds(run)


@pytest.mark.parametrize("split", [None, 1], ids=["library_split", "one_pass"])
def test_block_sparse_same_under_a_perturbed_schedule(split):
    """split=None lets this small grid split over the key range and merge the chunks;
    split=1 keeps one pass over the needed tiles of each query block."""
    B, H, N, d = 1, 4, 1024, 128
    inp = make_cross_inputs(B, H, H, N, N, d, "bf16", seed_base=17000, with_do=True)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    nb = N // 128
    m = (np.random.default_rng(3).random((H, nb, nb)) < 0.5).astype(np.uint8)
    mask = torch.from_numpy(m).cuda()

    def run():
        o, lse = fa.fa_forward(q, k, v, block_mask=mask, split=split)
        dq, dk, dv = fa.fa_backward(q, k, v, o, do, lse, block_mask=mask)
        return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}

    both_builds(run)


def test_fp8_same_under_a_perturbed_schedule():
    inp = make_cross_inputs(1, 4, 2, 900, 900, 128, "bf16", seed_base=18000)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))

    def run():
        q8, qs = fa.fa_quantize_fp8(q)
        k8, ks = fa.fa_quantize_fp8(k)
        v8, vs = fa.fa_quantize_fp8(v, per_channel=True)
        o, lse = fa.fa_forward_fp8(q8, qs, k8, ks, v8, vs, causal=True)
        return {"q8": q8, "o": o, "lse": lse}

    both_builds(run)
