"""GPU parity of block-sparse attention (128 x 128 blocks of a byte mask) against the fp64
oracle with the expanded dense mask, forward and backward."""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_forward_amd as fa
from exact_tiled_attention_forward_amd.workloads import make_cross_inputs
from oracle import naive
from parity import assert_close, assert_lse, to64

pytestmark = pytest.mark.gpu


def random_block_mask(heads, nq, nk, density, seed, empty_block_row=None):
    nb = (-(-nq // 128), -(-nk // 128))
    r = np.random.default_rng(seed)
    m = (r.random((heads,) + nb) < density).astype(np.uint8)
    if empty_block_row is not None:
        m[:, empty_block_row, :] = 0   # every query of that block sees no key
    return m


def check_lse(lse, ref):
    lse, ref = to64(lse), to64(ref)
    empty = ~np.isfinite(ref)
    assert np.array_equal(~np.isfinite(lse), empty), "rows without a visible key differ"
    if (~empty).any():
        assert_lse(lse[~empty], ref[~empty])


# (B, Hq, Hkv, Nq, Nk, d, dtype, causal, mask heads (1 or Hq), density, split, empty block row)
CASES = [
    (1, 4, 2, 300, 500, 128, "bf16", False, 4, 0.5, 1, None),
    (2, 2, 2, 700, 700, 64, "f16", True, 1, 0.6, 1, 2),
    (1, 4, 4, 640, 640, 128, "bf16", True, 4, 0.4, 3, None),
    (1, 2, 1, 1, 1000, 128, "bf16", True, 2, 0.5, None, None),
    (1, 2, 2, 260, 130, 64, "bf16", False, 2, 0.7, 1, 0),
    # d = 128, lengths that are multiples of the mask block, one pass: grouped heads, Nq < Nk,
    # an empty block row, a mask with no visible block at all, one that keeps everything
    (1, 4, 2, 512, 640, 128, "bf16", False, 4, 0.5, 1, None),
    (2, 4, 4, 768, 768, 128, "f16", True, 1, 0.5, 1, 3),
    (1, 8, 2, 256, 1024, 128, "bf16", True, 8, 0.3, 1, None),
    (1, 2, 1, 384, 384, 128, "bf16", False, 1, 0.0, 1, None),
    (1, 2, 2, 1280, 1280, 128, "bf16", True, 2, 1.0, 1, None),
]


def _id(c):
    B, Hq, Hkv, Nq, Nk, d, dt, causal, mh, dens, sp, empty = c
    return f"B{B}_Hq{Hq}_Hkv{Hkv}_Nq{Nq}_Nk{Nk}_d{d}_{dt}_{'causal' if causal else 'full'}_mh{mh}_p{dens}_s{sp}_e{empty}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_block_sparse_forward_and_backward(case):
    B, Hq, Hkv, Nq, Nk, d, dt, causal, mh, dens, sp, empty = case
    bm = random_block_mask(mh, Nq, Nk, dens, seed=Nq + Nk + mh, empty_block_row=empty)
    inp = make_cross_inputs(B, Hq, Hkv, Nq, Nk, d, dt, seed_base=13000 + Nq + Nk, with_do=True)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    bmg = torch.from_numpy(bm).cuda()
    o, lse = fa.fa_forward(q, k, v, causal=causal, split=sp, block_mask=bmg)
    torch.cuda.synchronize()
    ref_in = [to64(inp[x]) for x in ("q", "k", "v")]
    o_ref, lse_ref = naive.forward(*ref_in, 1 / math.sqrt(d), causal, block_mask=bm)
    assert_close(_id(case) + " O", o.cpu(), o_ref, dt)
    check_lse(lse.cpu(), lse_ref)
    if Nq == 1:
        return  # the backward of a decode step is not a training shape; covered by the others
    dq, dk, dv = fa.fa_backward(q, k, v, o, do, lse, causal=causal, block_mask=bmg)
    torch.cuda.synchronize()
    ref = naive.backward(*ref_in, to64(inp["do"]), 1 / math.sqrt(d), causal, block_mask=bm)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        assert_close(f"{_id(case)} {name}", g.cpu(), r, dt, out_dtype="f32")


def test_all_ones_mask_equals_dense():
    B, H, N, d = 1, 4, 520, 128
    inp = make_cross_inputs(B, H, H, N, N, d, "bf16", seed_base=13500, with_do=True)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    ones = torch.ones((1, 5, 5), dtype=torch.uint8, device="cuda")
    o1, l1 = fa.fa_forward(q, k, v, causal=True, split=1)
    o2, l2 = fa.fa_forward(q, k, v, causal=True, split=1, block_mask=ones)
    g1 = fa.fa_backward(q, k, v, o1, do, l1, causal=True)
    g2 = fa.fa_backward(q, k, v, o2, do, l2, causal=True, block_mask=ones)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_butterfly_mask_forward_and_backward(causal):
    """The flat butterfly block pattern (block i sees block j iff i XOR j is 0 or a power
    of two) at a ragged length, grouped heads, one mask layer for every head."""
    from exact_tiled_attention_forward_amd.workloads import butterfly_block_mask
    B, Hq, Hkv, N, d = 1, 4, 2, 1000, 128
    bm = butterfly_block_mask(N)
    assert bm.shape == (1, 8, 8) and int(bm[0].sum(1).min()) == 4
    inp = make_cross_inputs(B, Hq, Hkv, N, N, d, "bf16", seed_base=13700, with_do=True)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    bmg = bm.cuda()
    o, lse = fa.fa_forward(q, k, v, causal=causal, block_mask=bmg)
    dq, dk, dv = fa.fa_backward(q, k, v, o, do, lse, causal=causal, block_mask=bmg)
    torch.cuda.synchronize()
    ref_in = [to64(inp[x]) for x in ("q", "k", "v")]
    o_ref, lse_ref = naive.forward(*ref_in, 1 / math.sqrt(d), causal, block_mask=bm.numpy())
    assert_close("butterfly O", o.cpu(), o_ref, "bf16")
    check_lse(lse.cpu(), lse_ref)
    ref = naive.backward(*ref_in, to64(inp["do"]), 1 / math.sqrt(d), causal, block_mask=bm.numpy())
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        assert_close(f"butterfly {name}", g.cpu(), r, "bf16", out_dtype="f32")
