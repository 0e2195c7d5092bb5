"""GPU parity at a million keys, on sampled rows the oracle computes one by one.

A query row's O, lse and dQ depend only on that row of Q (and dO) and on the keys it
sees, so the oracle evaluates a row as a one-row head over keys 0..i (causal) or all
keys: O(N d) work per row instead of O(N^2 d).  The rows sit at the edges of tiles,
query blocks and the sequence, plus a few drawn at random.  These shapes are far past
the named workloads: 16384 key tiles per row, byte offsets up to 2^27 per head, and
running sums over 2^20 terms.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_forward_amd as fa
from exact_tiled_attention_forward_amd.workloads import make_cross_inputs, make_inputs
from oracle import naive
from parity import assert_close, assert_lse, to64

pytestmark = pytest.mark.gpu


def sample_rows(n, seed):
    edges = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 4095, 4096, n // 2, n - 257, n - 256, n - 2, n - 1]
    rng = np.random.default_rng(seed)
    return sorted(set(edges) | set(int(x) for x in rng.integers(0, n, 4)))


@pytest.mark.parametrize("dtype,d,causal,log2n,with_bwd", [
    ("bf16", 64, True, 20, True),     # 2^20 keys, causal, forward and dQ
    ("f16", 128, False, 19, False),   # 2^19 keys, every row sees every key
], ids=["bf16_d64_causal_1M", "f16_d128_full_512K"])
def test_long_sequence_sampled_rows(dtype, d, causal, log2n, with_bwd):
    n = 1 << log2n
    inp = make_inputs(1, 1, n, d, dtype, seed_base=19000 + log2n + d, with_do=with_bwd)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o, lse = fa.fa_forward(q, k, v, causal=causal)
    if with_bwd:
        do = inp["do"].cuda()
        dq, _, _ = fa.fa_backward(q, k, v, o, do, lse, causal=causal)
        dq = dq.cpu()
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()

    scale = 1 / math.sqrt(d)
    q64, k64, v64 = (to64(inp[x][0, 0]) for x in ("q", "k", "v"))
    do64 = to64(inp["do"][0, 0]) if with_bwd else None
    rows = sample_rows(n, seed=log2n)
    o_ref, lse_ref, dq_ref = [], [], []
    for i in rows:
        last = i + 1 if causal else n  # keys the row sees
        oi, li = naive.forward_head(q64[i:i + 1], k64[:last], v64[:last], scale, False)
        o_ref.append(oi[0])
        lse_ref.append(li[0])
        if with_bwd:
            dqi, _, _ = naive.backward_head(q64[i:i + 1], k64[:last], v64[:last], do64[i:i + 1], scale, False)
            dq_ref.append(dqi[0])
    mx, mean, ex, _ = assert_close(f"O rows of N={n}", o[0, 0, rows], np.array(o_ref), dtype, floor_aware=True)
    worst = assert_lse(lse[0, 0, rows], np.array(lse_ref))
    msg = f"N={n} d={d} {dtype} causal={causal}: O max {mx:.2e} (beyond floor {ex:.2e}) lse rel {worst:.2e}"
    if with_bwd:
        gmx, gmean, _, _ = assert_close(f"dQ rows of N={n}", dq[0, 0, rows], np.array(dq_ref), dtype, out_dtype="f32")
        msg += f"; dQ max {gmx:.2e} mean {gmean:.2e}"
    print(msg + f" over {len(rows)} rows")


def test_decode_over_a_million_cached_keys():
    """One query row per head against 2^20 cached keys, grouped heads (8 query heads on 2
    key/value heads): the key-parallel kernel with its split and merge, every row checked."""
    B, Hq, Hkv, Nk, d = 1, 8, 2, 1 << 20, 128
    inp = make_cross_inputs(B, Hq, Hkv, 1, Nk, d, "bf16", seed_base=19500)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o, lse = fa.fa_forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    scale = 1 / math.sqrt(d)
    G = Hq // Hkv
    for b in range(B):
        for kvh in range(Hkv):
            k64, v64 = to64(inp["k"][b, kvh]), to64(inp["v"][b, kvh])
            for h in range(kvh * G, (kvh + 1) * G):
                o_ref, lse_ref = naive.forward_head(to64(inp["q"][b, h]), k64, v64, scale, True)
                assert_close(f"O b={b} h={h}", o[b, h], o_ref, "bf16", floor_aware=True)
                assert_lse(lse[b, h], lse_ref)
