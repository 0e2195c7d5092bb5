"""GPU parity of the FP8 path.

* The quantizer: codes and scales bit-exact against the oracle's quantizer taking its
  decisions (the scale amax/448 and the quotient x/scale that decides a code) in fp32,
  the precision the kernel takes them in.
* The E4M3 forward: against exact attention on the dequantized inputs (``naive``) within
  the per-element bound derived in ``fp8_bound.py`` (E4M3 rounding of P, fp32
  arithmetic, bf16 output), and lse within that bound and the 1e-4 relative lse bar; as
  a second bar, also against the oracle's model of the kernel's recurrence
  (``oracle/fp8.py``, schedule pinned by hand-computed rows): max 1e-2 and mean 1e-3
  beyond the bf16 floor plus the slack of probabilities that sit on an E4M3 rounding
  midpoint.
* The two hand-computed rows that pin that schedule, through the kernel itself."""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_forward_amd as fa
from exact_tiled_attention_forward_amd.workloads import make_cross_inputs
from fp8_bound import forward_bound
from oracle import fp8
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
def test_fp8_forward_within_the_derived_bound(case):
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
    out, lse_out = to64(o.cpu()), to64(lse.cpu())
    # the bar: exact attention on the dequantized inputs, per-element derived bound
    o_ex, lse_ex, bound, lse_bound = forward_bound(*args, sc, causal)
    err = np.abs(out - o_ex)
    assert (err <= bound).all(), (f"{_id(case)}: {(err > bound).sum()} elements beyond the bound, worst excess "
                                  f"{(err - bound).max():.3e}")
    assert (np.abs(lse_out - lse_ex) <= lse_bound).all()
    assert_lse(lse_out, lse_ex)
    # second bar: the model of the kernel's recurrence (oracle/fp8.py), beyond the bf16
    # floor and a tie slack: a probability within 1e-5 (relative) of an E4M3 rounding
    # midpoint may round either way in the kernel (fp32 scores, v_exp_f32)
    o_ref, lse_ref, slack = fp8.forward(*args, sc, causal, tie_rel=1e-5)
    floor = np.abs(to64(torch.from_numpy(o_ref).to(torch.bfloat16)) - o_ref)
    err_m = np.abs(out - o_ref)
    excess = err_m - floor - slack
    assert excess.max() <= 1e-2, f"{_id(case)}: vs model beyond floor and tie slack {excess.max():.3e}"
    assert err_m.mean() <= 1e-3, f"{_id(case)}: vs model mean error {err_m.mean():.3e}"
    print(f"{_id(case)}: vs exact max {err.max():.2e} mean {err.mean():.2e} (bound median {np.median(bound):.2e}, "
          f"max error/bound {(err / bound).max():.2f}); vs model max {err_m.max():.2e} mean {err_m.mean():.2e}")


E4M3_ONE, E4M3_MINUS_ONE, E4M3_MINUS_448 = 0x38, 0xB8, 0xFE


@pytest.mark.parametrize("second", [40, 64], ids=["one_tile", "two_tiles"])
def test_schedule_pins_through_the_kernel(second):
    """The hand-computed rows of tests/test_oracle_fp8.py on the GPU.  One query (code 1.0),
    key 0 with code -1.0, key `second` with code 0, every other key -448; unit scales and
    scale = -ln(0.515625), so p_0 = 0.515625 relative to key `second`.  V picks channel 0
    for key 0 and channel 1 for key `second`.  Keys 0 and 40 share a 64-key tile, so p_0 is
    rounded to E4M3 (0.5); keys 0 and 64 do not, and nothing is rounded."""
    d, nk = 64, 128
    sigma = np.float32(-math.log(0.515625))
    q8 = torch.zeros((1, 1, 1, d), dtype=torch.uint8)
    q8[0, 0, 0, 0] = E4M3_ONE
    k8 = torch.zeros((1, 1, nk, d), dtype=torch.uint8)
    k8[0, 0, :, 0] = E4M3_MINUS_448
    k8[0, 0, 0, 0] = E4M3_MINUS_ONE
    k8[0, 0, second, 0] = 0
    v8 = torch.zeros((1, 1, nk, d), dtype=torch.uint8)
    v8[0, 0, 0, 0] = E4M3_ONE
    v8[0, 0, second, 1] = E4M3_ONE
    ones = lambda *s: torch.ones(s, dtype=torch.float32, device="cuda")  # noqa: E731
    o, lse = fa.fa_forward_fp8(q8.cuda(), ones(1, 1, 1), k8.cuda(), ones(1, 1, 1), v8.cuda(), ones(1, 1, d),
                               scale=float(sigma))
    torch.cuda.synchronize()
    p0 = math.exp(-float(sigma))                   # 0.515625 up to the fp32 rounding of sigma
    l = 1.0 + p0
    want = [0.5 / l, 1 / l] if second == 40 else [p0 / l, 1 / l]
    got = to64(o.cpu())[0, 0, 0]
    np.testing.assert_allclose(got[:2], want, rtol=2.0 ** -8, atol=1e-6)
    assert (got[2:] == 0).all()
    assert abs(float(lse.cpu()[0, 0, 0]) - math.log(l)) <= 1e-6
