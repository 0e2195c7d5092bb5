"""GPU parity of fa_forward against the fp64 oracle (needs an MI355X)."""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_forward_amd as fa
from exact_tiled_attention_forward_amd.workloads import WORKLOADS, make_inputs, workload_inputs
from oracle import naive
from oracle_pins import golden
from parity import assert_close, assert_lse, to64

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def run_fwd(inp, causal, scale=None):
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o, lse = fa.fa_forward(q, k, v, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


SMALL_N = [1, 2, 3, 17, 63, 64, 65, 127, 128, 129, 255, 300, 511, 577]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_small_shapes_all_rows(dtype, d, causal):
    """Every N in a sweep that spans one to several tiles with ragged tails; all rows of
    all heads against the oracle."""
    for n in SMALL_N:
        inp = make_inputs(2, 3, n, d, dtype, seed_base=7000 + n)
        o, lse = run_fwd(inp, causal)
        o_ref, lse_ref = naive.forward(to64(inp["q"]), to64(inp["k"]), to64(inp["v"]), 1 / math.sqrt(d), causal)
        mx, mean, ex, _ = assert_close(f"O n={n}", o, o_ref, dtype, floor_aware=True)
        worst = assert_lse(lse, lse_ref)
        print(f"{dtype} d={d} causal={causal} N={n}: O max {mx:.2e} (beyond floor {ex:.2e}) mean {mean:.2e} "
              f"lse rel {worst:.2e}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_outlier_rows_move_the_running_max(dtype, d, causal):
    """5% of the Q and K rows scaled by 8 (as in the large-head workload): scores reach
    hundreds in log2 units, so the running max of a row jumps by very different amounts
    from one key tile to the next, and the lazy rescale fires with a different factor on
    every row.  All rows of all heads against the oracle."""
    for n in (300, 700, 1100):
        inp = make_inputs(1, 2, n, d, dtype, seed_base=7500 + n + d, outlier_frac=0.05, outlier_scale=8.0)
        o, lse = run_fwd(inp, causal)
        o_ref, lse_ref = naive.forward(to64(inp["q"]), to64(inp["k"]), to64(inp["v"]), 1 / math.sqrt(d), causal)
        mx, mean, ex, _ = assert_close(f"O n={n}", o, o_ref, dtype, floor_aware=True)
        worst = assert_lse(lse, lse_ref)
        print(f"{dtype} d={d} causal={causal} N={n} outliers: O max {mx:.2e} (beyond floor {ex:.2e}) "
              f"mean {mean:.2e} lse rel {worst:.2e}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_scores_far_above_the_first_tile(dtype, d, causal):
    """Two keys (300 and 301, past the first key tile of every kernel) whose scores lie 18 to
    60 above every earlier score, in log2 units, with weights 4 : 1 or 2 : 1 between them.
    A kernel that exponentiates against a stale reference would send their probabilities
    past what the 16-bit P holds (fp16 stops at 65504) or flatten their ratio.  The shapes
    run the 256-row kernel whole (16 heads of 1024) and split over the key range (2 heads
    of 4096); every row against the oracle."""
    cs = math.log2(math.e) / math.sqrt(d)  # score -> log2 units
    for h, n in ((16, 1024), (2, 4096)):
        for gaps in ((20.0, 18.0), (40.0, 39.0), (60.0, 58.0)):
            g = torch.Generator().manual_seed(int(gaps[0]) + n + d)
            q = 0.1 * torch.randn(1, h, n, d, generator=g)
            k = 0.1 * torch.randn(1, h, n, d, generator=g)
            v = torch.randn(1, h, n, d, generator=g)
            q[..., 0] = 1.0
            k[..., 0] = torch.linspace(-1.0, 1.0, n)
            k[..., 300, 0] = gaps[0] / cs
            k[..., 301, 0] = gaps[1] / cs
            inp = {x: t.to(DT[dtype]) for x, t in (("q", q), ("k", k), ("v", v))}
            o, lse = run_fwd(inp, causal)
            assert not torch.isnan(o).any(), f"NaN in O ({h}x{n}, gaps {gaps})"
            o_ref, lse_ref = naive.forward(to64(inp["q"]), to64(inp["k"]), to64(inp["v"]), 1 / math.sqrt(d),
                                           causal)
            mx, mean, ex, _ = assert_close(f"O {h}x{n} gaps {gaps}", o, o_ref, dtype, floor_aware=True)
            worst = assert_lse(lse, lse_ref)
            print(f"{dtype} d={d} causal={causal} {h}x{n} gaps {gaps}: O max {mx:.2e} (beyond floor {ex:.2e}) "
                  f"lse rel {worst:.2e}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("slope", [0.25, -0.25, 3.0], ids=["rising", "falling", "steep"])
def test_monotone_scores_and_other_scales(dtype, d, slope):
    """Scores that rise (or fall) steadily along the keys, by `slope` log2 units per key:
    rising, every key tile passes the running max by 16 or more (the steep case by
    hundreds), so each tile rescales o and both sums; falling, everything after the first
    tile fades to nothing.  Run at three softmax scales (the default 1/sqrt(d), 1 and
    1/64), causal and not, every row against the oracle."""
    h, n = 4, 1024
    g = torch.Generator().manual_seed(4000 + d + int(100 * slope))
    q = 0.05 * torch.randn(1, h, n, d, generator=g)
    k = 0.05 * torch.randn(1, h, n, d, generator=g)
    v = torch.randn(1, h, n, d, generator=g)
    for scale in (1 / math.sqrt(d), 1.0, 1 / 64):
        cs = scale * math.log2(math.e)
        qq, kk = q.clone(), k.clone()
        # score of key j: 16 * k_j0 plus a little noise; the key values stay within fp16 range
        qq[..., 0] = 16.0
        kk[..., 0] = slope * (torch.arange(n, dtype=torch.float32) - n / 2) / (16.0 * cs)
        inp = {x: t.to(DT[dtype]) for x, t in (("q", qq), ("k", kk), ("v", v))}
        for causal in (False, True):
            o, lse = run_fwd(inp, causal, scale=scale)
            assert torch.isfinite(o).all(), f"non-finite O (scale {scale}, causal {causal})"
            o_ref, lse_ref = naive.forward(to64(inp["q"]), to64(inp["k"]), to64(inp["v"]), scale, causal)
            mx, mean, ex, _ = assert_close(f"O scale {scale} causal {causal}", o, o_ref, dtype, floor_aware=True)
            worst = assert_lse(lse, lse_ref)
            print(f"{dtype} d={d} slope {slope} scale {scale:.4f} causal={causal}: O max {mx:.2e} "
                  f"(beyond floor {ex:.2e}) lse rel {worst:.2e}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_worked_examples_through_the_kernel(dtype):
    """The page examples embedded in a d = 64 head, scale 1, non-causal: softmax of
    [2, 1, 3] appears as row 0 of O, and exp(lse_0) is 30.19; the [1, 2, 0, 3] row gives
    exp(lse_0 - 3) = 1.553."""
    g = golden("softmax_2_1_3.json")
    n, d = 3, 64
    q = torch.zeros(1, 1, n, d); q[..., 0] = 1.0
    k = torch.zeros(1, 1, n, d); k[0, 0, :, 0] = torch.tensor(g["row"])
    v = torch.zeros(1, 1, n, d); v[0, 0, torch.arange(n), torch.arange(n) + 1] = 1.0
    inp = {x: t.to(DT[dtype]) for x, t in (("q", q), ("k", k), ("v", v))}
    o, lse = run_fwd(inp, False, scale=1.0)
    w = o[0, 0, 0, 1:4].double().numpy()
    tol = 1e-5 if dtype == "f32" else 4e-3  # bf16 output carries 2^-9 relative rounding
    np.testing.assert_allclose(w, g["weights"], atol=tol + 5e-4)
    assert round(math.exp(float(lse[0, 0, 0])), 2) == g["sum"]

    g2 = golden("online_two_block.json")
    n = 4
    q = torch.zeros(1, 1, n, d); q[..., 0] = 1.0
    k = torch.zeros(1, 1, n, d); k[0, 0, :, 0] = torch.tensor(g2["row"])
    v = torch.randn(1, 1, n, d, generator=torch.Generator().manual_seed(3))
    inp = {x: t.to(DT[dtype]) for x, t in (("q", q), ("k", k), ("v", v))}
    _, lse = run_fwd(inp, False, scale=1.0)
    assert round(math.exp(float(lse[0, 0, 0]) - 3.0), 3) == g2["after_block_2"]["l"]


def test_deterministic_and_no_writes_past_the_end():
    """Two runs give bitwise-identical O and lse, and nothing is written beyond the
    (B, H, N, d) output or the (B, H, N) lse."""
    B, H, N, d = 2, 4, 333, 128
    inp = make_inputs(B, H, N, d, "bf16", 9100)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    sentinel = -12345.0
    obuf = torch.full((B * H * N * d + 4096,), sentinel, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((B * H * N + 1024,), sentinel, dtype=torch.float32, device="cuda")
    o = obuf[: B * H * N * d].view(B, H, N, d)
    lse = lbuf[: B * H * N].view(B, H, N)
    fa.fa_forward(q, k, v, o, lse, causal=True)
    o1, l1 = o.clone(), lse.clone()
    fa.fa_forward(q, k, v, o, lse, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o) and torch.equal(l1, lse)
    assert torch.all(obuf[B * H * N * d:] == sentinel)
    assert torch.all(lbuf[B * H * N:] == sentinel)


def test_smoke_shape_from_the_article():
    """Seed 0, (2, 4, 512, 64) bf16, non-causal: the consistency check shape of the cf-1.com
    article (section 3.3), held to this library's tolerances rather than its 1e-2."""
    w = WORKLOADS["smoke_2x4x512"]
    inp = workload_inputs(w)
    o, lse = run_fwd(inp, w.causal)
    o_ref, lse_ref = naive.forward(to64(inp["q"]), to64(inp["k"]), to64(inp["v"]), w.scale, w.causal)
    assert_close("O", o, o_ref, w.dtype)
    assert_lse(lse, lse_ref)
