"""GPU parity of fa_backward (after fa_forward) against the fp64 oracle (needs an MI355X)."""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_forward_amd as fa
from exact_tiled_attention_forward_amd.workloads import make_inputs
from oracle import naive
from parity import assert_close, to64

pytestmark = pytest.mark.gpu


def run_fwd_bwd(inp, causal, scale=None):
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    o, lse = fa.fa_forward(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = fa.fa_backward(q, k, v, o, do, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def check_grads(tag, got, ref, dtype, floor_aware=False):
    out = []
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        mx, mean, ex, _ = assert_close(f"{tag} {name}", g, r, dtype, out_dtype="f32", floor_aware=floor_aware)
        out.append(f"{name} max {mx:.2e} mean {mean:.2e}")
    return "; ".join(out)


SMALL_N = [1, 2, 17, 64, 65, 127, 128, 129, 200, 300, 511, 577]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_small_shapes_all_rows(dtype, d, causal):
    """Ragged N spanning one to several key and query tiles; every gradient entry of
    every head against the oracle's backward computed from Q, K, V, dO alone."""
    failures = []
    for n in SMALL_N:
        inp = make_inputs(2, 2, n, d, dtype, seed_base=8000 + n, with_do=True)
        got = run_fwd_bwd(inp, causal)
        ref = naive.backward(*(to64(inp[x]) for x in ("q", "k", "v", "do")), 1 / math.sqrt(d), causal)
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            x, r = to64(g), to64(r)
            e = np.abs(x - r)
            print(f"{dtype} d={d} causal={causal} N={n} {name}: max {e.max():.2e} mean {e.mean():.2e} "
                  f"max|ref| {np.abs(r).max():.2e} mean|ref| {np.abs(r).mean():.2e}")
        try:
            check_grads(f"N={n}", got, ref, dtype)
        except AssertionError as exc:
            failures.append(str(exc))
    assert not failures, failures


def test_backward_alone_from_oracle_statistics():
    """fa_backward fed the oracle's O (rounded to bf16) and lse rather than the kernel's."""
    n, d, causal = 257, 64, True
    inp = make_inputs(1, 3, n, d, "bf16", seed_base=8500, with_do=True)
    q, k, v, do = (to64(inp[x]) for x in ("q", "k", "v", "do"))
    o_ref, lse_ref = naive.forward(q, k, v, 1 / math.sqrt(d), causal)
    tq, tk, tv, tdo = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    o = torch.from_numpy(o_ref).to(torch.bfloat16).cuda()
    lse = torch.from_numpy(lse_ref).float().cuda()
    dq, dk, dv = fa.fa_backward(tq, tk, tv, o, tdo, lse, causal=causal)
    torch.cuda.synchronize()
    ref = naive.backward(q, k, v, to64(inp["do"]), 1 / math.sqrt(d), causal)
    print(check_grads("oracle stats", (dq.cpu(), dk.cpu(), dv.cpu()), ref, "bf16"))


def test_backward_deterministic_and_no_writes_past_the_end():
    B, H, N, d = 1, 3, 333, 128
    inp = make_inputs(B, H, N, d, "bf16", 9200, with_do=True)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    o, lse = fa.fa_forward(q, k, v, causal=True)
    sentinel = -7777.0
    n = B * H * N * d
    bufs = [torch.full((n + 2048,), sentinel, dtype=torch.float32, device="cuda") for _ in range(3)]
    grads = [b[:n].view(B, H, N, d) for b in bufs]
    fa.fa_backward(q, k, v, o, do, lse, *grads, causal=True)
    first = [g.clone() for g in grads]
    fa.fa_backward(q, k, v, o, do, lse, *grads, causal=True)
    torch.cuda.synchronize()
    for a, b, buf in zip(first, grads, bufs):
        assert torch.equal(a, b)
        assert torch.all(buf[n:] == sentinel)


def test_values_beyond_fp16_range():
    """bf16 inputs with one entry of 2^17 (beyond the fp16 range) in V, then in dO, then
    none, through one workspace.  The large entry makes a few scores' dP, D and dS large
    beside ordinary ones, so the hi + lo products must keep the small terms, and a call
    after such inputs must not depend on what they left in the workspace.  The large
    entry scales the gradients, so the bars scale with max|ref|."""
    B, H, N, d, causal = 1, 2, 200, 64, True
    ws = torch.empty(fa.fa_backward_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    for where in ("v", "do", None):
        inp = make_inputs(B, H, N, d, "bf16", seed_base=9300, with_do=True)
        if where == "v":
            inp["v"][0, 1, 37, 5] = 2.0 ** 17
        elif where == "do":
            inp["do"][0, 0, 150, 3] = -(2.0 ** 17)
        q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
        o, lse = fa.fa_forward(q, k, v, causal=causal)
        got = fa.fa_backward(q, k, v, o, do, lse, causal=causal, workspace=ws)
        torch.cuda.synchronize()
        ref = naive.backward(*(to64(inp[x]) for x in ("q", "k", "v", "do")), 1 / math.sqrt(d), causal)
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            x = to64(g.cpu())
            assert np.isfinite(x).all(), f"{where} {name}: non-finite gradient"
            s = max(1.0, float(np.abs(r).max()))
            e = np.abs(x - r)
            print(f"large entry in {where}: {name} max {e.max():.2e} mean {e.mean():.2e} max|ref| {s:.2e}")
            assert e.max() <= 1e-2 * s and e.mean() <= 1e-3 * s, f"{where} {name}"
        if where is None:
            check_grads("after the large entries", tuple(g.cpu() for g in got), ref, "bf16")


def _adversarial_scores(kind, h, n, d, dtype, seed):
    """Q, K whose scores (log2 units at the default scale) either hold two keys 40 and 39
    above every other score ("far") or rise by 0.75 per key ("steep", 48 per 64-key tile,
    up to about 770 at the end); V and dO N(0,1)."""
    g = torch.Generator().manual_seed(seed)
    cs = math.log2(math.e) / math.sqrt(d)
    q = 0.1 * torch.randn(1, h, n, d, generator=g)
    k = 0.1 * torch.randn(1, h, n, d, generator=g)
    v = torch.randn(1, h, n, d, generator=g)
    do = torch.randn(1, h, n, d, generator=g)
    if kind == "far":
        q[..., 0] = 1.0
        k[..., 0] = torch.linspace(-1.0, 1.0, n)
        k[..., 300, 0] = 40.0 / cs
        k[..., 301, 0] = 39.0 / cs
    else:
        q[..., 0] = 16.0
        k[..., 0] = 0.75 * (torch.arange(n, dtype=torch.float32) - n / 2) / (16.0 * cs)
    dt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return {"q": q.to(dt), "k": k.to(dt), "v": v.to(dt), "do": do.to(dt)}


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("kind", ["far", "steep"])
def test_far_and_steep_scores(kind, dtype, d, causal):
    """The backward under scores far from the ordinary range: two keys 40 and 39 above every
    other score, or scores rising by 0.75 (log2 units) per key.  P is recomputed from lse,
    so the forward's lse must carry these rows exactly; most probabilities underflow to
    zero and a few rows saturate on one key.  Keys in the hundreds make the gradients
    large, so dO is first divided by the largest oracle gradient (the gradients are linear
    in dO), which puts them at unit scale where the bar applies as written.
    The slope stays moderate because dQ is ill-conditioned here: its terms dS_ij K_j cancel
    (sum_j dS_ij = 0) against keys in the hundreds, and any fp32 kernel's lse, rounded at a
    magnitude in the thousands, scales a row's P by 1 + 2^-13 or so and breaks that
    cancellation.  At 3 per key (scores up to about 3000) a plain fp32 emulation on the CPU
    already shows dQ errors of 2.4e-3 to 4.3e-3 against fp64, and the kernel, whose lse
    carries the forward's few-ulp rounding, 5.6e-3 to 1.4e-2."""
    h, n = 2, 1024
    inp = _adversarial_scores(kind, h, n, d, dtype, seed=6100 + d)
    q, k, v = (to64(inp[x]) for x in ("q", "k", "v"))
    ref = naive.backward(q, k, v, to64(inp["do"]), 1 / math.sqrt(d), causal)
    s = max(float(np.abs(r).max()) for r in ref)
    inp["do"] = (inp["do"].float() / s).to(inp["do"].dtype)
    ref = naive.backward(q, k, v, to64(inp["do"]), 1 / math.sqrt(d), causal)
    got = run_fwd_bwd(inp, causal)
    for name, gr in zip(("dQ", "dK", "dV"), got):
        assert torch.isfinite(gr).all(), f"{name}: non-finite gradient"
    print(f"{kind} {dtype} d={d} causal={causal} (dO / {s:.1f}): " + check_grads(kind, got, ref, dtype))
