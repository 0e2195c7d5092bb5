"""GPU parity of attention with grouped key/value heads and query/key lengths that differ
(cross-attention, a decode step against a cached K/V) against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_forward_amd as fa
from exact_tiled_attention_forward_amd.workloads import make_cross_inputs
from oracle import naive
from parity import assert_close, assert_lse, to64

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, Nq, Nk, d, dtype, causal): grouped heads, Nq < Nk and Nq > Nk (non-causal),
# one decode row, ragged lengths that cross tile edges
FWD_CASES = [
    (1, 4, 2, 37, 129, 64, "bf16", True),
    (1, 4, 1, 1, 300, 128, "bf16", True),
    (2, 6, 3, 200, 77, 64, "f16", False),
    (1, 8, 2, 300, 300, 128, "bf16", True),
    (1, 4, 4, 129, 513, 128, "f16", True),
    (1, 2, 1, 65, 64, 64, "f32", False),
    (1, 2, 2, 33, 97, 128, "f32", True),
    (2, 4, 2, 260, 1030, 128, "bf16", False),
]


def _case_id(c):
    B, Hq, Hkv, Nq, Nk, d, dt, causal = c
    return f"B{B}_Hq{Hq}_Hkv{Hkv}_Nq{Nq}_Nk{Nk}_d{d}_{dt}_{'causal' if causal else 'full'}"


@pytest.mark.parametrize("case", FWD_CASES, ids=[_case_id(c) for c in FWD_CASES])
def test_forward_matches_oracle(case):
    B, Hq, Hkv, Nq, Nk, d, dt, causal = case
    inp = make_cross_inputs(B, Hq, Hkv, Nq, Nk, d, dt, seed_base=9100 + Nq + Nk)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o, lse = fa.fa_forward(q, k, v, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = naive.forward(*(to64(inp[x]) for x in ("q", "k", "v")), 1 / math.sqrt(d), causal)
    assert_close(_case_id(case) + " O", o.cpu(), o_ref, dt)
    assert_lse(lse.cpu(), lse_ref)


BWD_CASES = [
    (1, 4, 2, 37, 129, 64, "bf16", True),
    (2, 4, 1, 100, 100, 128, "bf16", True),
    (1, 6, 2, 64, 200, 64, "f16", False),
    (1, 2, 1, 1, 257, 128, "bf16", True),
    (1, 4, 2, 300, 65, 128, "bf16", False),
    (1, 8, 4, 190, 640, 128, "f16", True),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[_case_id(c) for c in BWD_CASES])
def test_backward_matches_oracle(case):
    B, Hq, Hkv, Nq, Nk, d, dt, causal = case
    inp = make_cross_inputs(B, Hq, Hkv, Nq, Nk, d, dt, seed_base=9500 + Nq + Nk, with_do=True)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    o, lse = fa.fa_forward(q, k, v, causal=causal)
    dq, dk, dv = fa.fa_backward(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    assert dk.shape == k.shape and dv.shape == v.shape and dq.shape == q.shape
    ref = naive.backward(*(to64(inp[x]) for x in ("q", "k", "v", "do")), 1 / math.sqrt(d), causal)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        assert_close(f"{_case_id(case)} {name}", g.cpu(), r, dt, out_dtype="f32")


def test_square_ex_equals_square_entry_points():
    """fa_forward with Hkv = Hq and Nk = Nq goes through the same kernels: bitwise equal
    to a call that passes k and v as separate but identical tensors."""
    inp = make_cross_inputs(2, 4, 4, 300, 300, 128, "bf16", seed_base=9900, with_do=True)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    o1, l1 = fa.fa_forward(q, k, v, causal=True)
    o2, l2 = fa.fa_forward(q, k.clone(), v.clone(), causal=True)
    g1 = fa.fa_backward(q, k, v, o1, do, l1, causal=True)
    g2 = fa.fa_backward(q, k.clone(), v.clone(), o2, do, l2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_grouped_heads_equal_repeated_heads():
    """Grouped key/value heads give the same O and dQ as the same heads repeated per query
    head; the grouped dK, dV equal the repeated ones summed over each group."""
    B, Hq, Hkv, N, d = 1, 6, 2, 160, 64
    inp = make_cross_inputs(B, Hq, Hkv, N, N, d, "bf16", seed_base=9950, with_do=True)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    G = Hq // Hkv
    kr, vr = (x.repeat_interleave(G, dim=1).contiguous() for x in (k, v))
    o1, l1 = fa.fa_forward(q, k, v, causal=True)
    o2, l2 = fa.fa_forward(q, kr, vr, causal=True)
    dq1, dk1, dv1 = fa.fa_backward(q, k, v, o1, do, l1, causal=True)
    dq2, dk2, dv2 = fa.fa_backward(q, kr, vr, o2, do, l2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(dq1, dq2)
    dk2s = dk2.view(B, Hkv, G, N, d).sum(dim=2)
    dv2s = dv2.view(B, Hkv, G, N, d).sum(dim=2)
    np.testing.assert_allclose(dk1.cpu().numpy(), dk2s.cpu().numpy(), rtol=0, atol=1e-5)
    np.testing.assert_allclose(dv1.cpu().numpy(), dv2s.cpu().numpy(), rtol=0, atol=1e-5)
