"""GPU parity of the FP8 path: the quantizer (bit-exact codes and scales, decisions in fp32
as on the GPU) and the E4M3 forward against the oracle's model of the same recurrence."""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_forward_amd as fa
from exact_tiled_attention_forward_amd.workloads import make_cross_inputs
from oracle import fp8, naive
from parity import assert_lse, to64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("per_channel", [False, True], ids=["rows", "channels"])
def test_quantizer_is_bit_exact(dtype, per_channel):
    inp = make_cross_inputs(2, 3, 3, 300, 300, 64, dtype, seed_base=14000)
    x = inp["q"].clone()
    x[0, 1, 17, 5] = 200.0 if dtype != "f32" else 1234.5  # an outlier in one block
    x[1, 2, 128:256] = 0                                   # an all-zero block
    codes, scales = fa.fa_quantize_fp8(x.cuda(), per_channel=per_channel)
    torch.cuda.synchronize()
    xr = x.float().numpy()
    if per_channel:
        c_ref, s_ref = fp8.quantize_channels(xr, dtype=np.float32)
    else:
        c_ref, s_ref = fp8.quantize_rows(xr, dtype=np.float32)
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)


# (B, Hq, Hkv, Nq, Nk, d, causal)
CASES = [
    (1, 4, 2, 300, 300, 128, True),
    (2, 2, 2, 257, 400, 64, False),
    (1, 8, 8, 1024, 1024, 128, True),
    (1, 4, 1, 1, 700, 128, True),
    (1, 2, 2, 130, 1000, 64, True),
]


def _id(c):
    B, Hq, Hkv, Nq, Nk, d, causal = c
    return f"B{B}_Hq{Hq}_Hkv{Hkv}_Nq{Nq}_Nk{Nk}_d{d}_{'causal' if causal else 'full'}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_fp8_forward_matches_the_model(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    inp = make_cross_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", seed_base=14500 + Nq + Nk)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    q8, qs = fa.fa_quantize_fp8(q)
    k8, ks = fa.fa_quantize_fp8(k)
    v8, vs = fa.fa_quantize_fp8(v, per_channel=True)
    o, lse = fa.fa_forward_fp8(q8, qs, k8, ks, v8, vs, causal=causal)
    torch.cuda.synchronize()
    args = [a.cpu().numpy() for a in (q8, qs, k8, ks, v8, vs)]
    sc = 1 / math.sqrt(d)
    # the model's probabilities carry the exact exponential; the kernel's carry fp32 score
    # rounding and v_exp_f32's error (a few 1e-7 relative), so a probability within 1e-5
    # of an E4M3 rounding midpoint may round either way: the slack bounds that
    o_ref, lse_ref, slack = fp8.forward(*args, sc, causal, tie_rel=1e-5)
    out = to64(o.cpu())
    floor = np.abs(to64(torch.from_numpy(o_ref).to(torch.bfloat16)) - o_ref)
    err = np.abs(out - o_ref)
    excess = err - floor - slack
    mx, mean = float(err.max()), float(err.mean())
    assert excess.max() <= 1e-2, f"{_id(case)}: error beyond floor and tie slack {excess.max():.3e} (max {mx:.3e})"
    assert mean <= 1e-3, f"{_id(case)}: mean error {mean:.3e}"
    assert_lse(lse.cpu(), lse_ref)
    # and against exact attention on the dequantized inputs: within the P-rounding bound
    qd = fp8.dequantize_rows(args[0], args[1])
    kd = fp8.dequantize_rows(args[2], args[3])
    vd = fp8.dequantize_channels(args[4], args[5])
    G = Hq // Hkv
    o_ex = np.empty(o_ref.shape)
    bound = np.empty(o_ref.shape)
    for b in range(B):
        for h in range(Hq):
            kk, vv = kd[b, h // G], vd[b, h // G]
            s = naive.scores(qd[b, h], kk, sc, causal)
            p, m, l = naive.softmax_rows(s)
            o_ex[b, h] = p @ vv
            bound[b, h] = (np.abs(vv)[None] * np.maximum(2 ** -4 * (p * l[:, None])[:, :, None], 2 ** -10)
                           * (p > 0)[:, :, None]).sum(axis=1) / l[:, None]
    floor_ex = np.abs(to64(torch.from_numpy(o_ex).to(torch.bfloat16)) - o_ex)
    assert (np.abs(out - o_ex) <= bound + floor_ex + 1e-3).all()
    print(f"{_id(case)}: vs model max {mx:.2e} mean {mean:.2e} (slack max {slack.max():.2e}, excess max "
          f"{excess.max():.2e}); vs exact max {np.abs(out - o_ex).max():.2e} mean {np.abs(out - o_ex).mean():.2e}")
