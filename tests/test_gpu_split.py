"""GPU parity of the split key-range forward (decode steps and other small grids) against
the fp64 oracle: every chunk's partial (m, l, o) merged with the (m, l) rule."""

import math

import pytest
import torch

import exact_tiled_attention_forward_amd as fa
from exact_tiled_attention_forward_amd.workloads import make_cross_inputs
from oracle import naive
from parity import assert_close, assert_lse, to64

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, Nq, Nk, d, dtype, causal, split): split None = the library's choice
CASES = [
    (2, 8, 2, 1, 3000, 128, "bf16", True, None),      # decode step, grouped heads
    (1, 4, 4, 1, 4097, 64, "f16", False, None),
    (2, 16, 2, 3, 2500, 128, "bf16", True, None),     # 8 query heads x 3 rows packed per group
    (1, 2, 2, 700, 700, 64, "bf16", True, 3),
    (1, 4, 1, 130, 900, 128, "f16", True, 5),
    (2, 2, 2, 300, 300, 128, "bf16", False, 7),
    (1, 2, 2, 64, 64, 64, "bf16", True, 1024),        # more splits than key tiles
    (1, 2, 1, 257, 1000, 64, "bf16", False, 2),
    # groups of at most 32 packed rows run key-parallel; 33 rows go to the 256-row kernel
    (1, 8, 1, 4, 1000, 128, "bf16", True, None),     # 8 x 4 = 32 rows, causal
    (1, 8, 1, 4, 1000, 64, "f16", False, 3),         # 32 rows, forced split
    (1, 3, 1, 11, 777, 128, "bf16", True, 2),        # 3 x 11 = 33 rows
    (2, 4, 2, 1, 70, 128, "bf16", True, 1024),       # decode, more splits than key tiles
    # fp32: 64-row blocks per query head split over their 32-key tiles
    (1, 1, 1, 256, 256, 64, "f32", False, None),      # the fp32 single-head workload's shape
    (1, 2, 1, 300, 300, 128, "f32", True, 4),
    (2, 4, 2, 65, 700, 64, "f32", True, None),
    (1, 2, 2, 100, 33, 64, "f32", False, 1024),       # more splits than key tiles
]


def _id(c):
    B, Hq, Hkv, Nq, Nk, d, dt, causal, sp = c
    return f"B{B}_Hq{Hq}_Hkv{Hkv}_Nq{Nq}_Nk{Nk}_d{d}_{dt}_{'causal' if causal else 'full'}_split{sp}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_split_forward_matches_oracle(case):
    B, Hq, Hkv, Nq, Nk, d, dt, causal, sp = case
    inp = make_cross_inputs(B, Hq, Hkv, Nq, Nk, d, dt, seed_base=12000 + Nq + Nk)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    if sp is None:
        assert fa.fa_forward_split_count(q, k, causal) > 1, "expected the library to split this grid"
    o, lse = fa.fa_forward(q, k, v, causal=causal, split=sp)
    torch.cuda.synchronize()
    o_ref, lse_ref = naive.forward(*(to64(inp[x]) for x in ("q", "k", "v")), 1 / math.sqrt(d), causal)
    assert_close(_id(case) + " O", o.cpu(), o_ref, dt)
    assert_lse(lse.cpu(), lse_ref)


def test_split_is_deterministic_and_close_to_one_pass():
    inp = make_cross_inputs(1, 8, 8, 4096, 4096, 64, "bf16", seed_base=12500)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o1, l1 = fa.fa_forward(q, k, v, causal=True, split=4)
    o2, l2 = fa.fa_forward(q, k, v, causal=True, split=4)
    o0, l0 = fa.fa_forward(q, k, v, causal=True, split=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert float((o1.float() - o0.float()).abs().max()) <= 2e-2
    assert float((l1 - l0).abs().max()) <= 1e-4 * max(1.0, float(l0.abs().max()))
