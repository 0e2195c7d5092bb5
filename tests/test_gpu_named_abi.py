"""The square entry points fa_forward / fa_backward called directly through ctypes, and the
method's memory claim: no N x N buffer is ever allocated (needs an MI355X).

The memory claim is the pages' reason for the tiled method: the naive path writes the
N x N score matrix to device memory (8.59 GB for 4 x 16 heads at N = 8192 in fp16; the
cf-1.com article, section 1.1, and "大模型数学速成（17）", sections 一 and 四), while
the tiled path keeps it on chip.  Here the device memory that the forward and the
backward take beyond their inputs is measured at that shape and must equal the outputs
(and the backward's per-row workspace).
"""

import ctypes
import math

import pytest
import torch

import exact_tiled_attention_forward_amd as fa
from exact_tiled_attention_forward_amd.workloads import make_inputs
from oracle import naive
from parity import assert_close, assert_lse, to64

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, True), ("f16", 64, False)])
def test_square_symbols_through_ctypes(dtype, d, causal):
    """lib.fa_forward and lib.fa_backward with caller-allocated outputs and workspace, on
    torch's current stream; every row of every head against the oracle."""
    lib = fa.library()
    B, H, N = 2, 3, 700
    inp = make_inputs(B, H, N, d, dtype, seed_base=16000 + d, with_do=True)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    code = {"bf16": fa.FA_BF16, "f16": fa.FA_F16}[dtype]
    sc = 1 / math.sqrt(d)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    st = lib.fa_forward(_p(q), _p(k), _p(v), _p(o), _p(lse), B, H, N, d, ctypes.c_float(sc), int(causal), code,
                        stream)
    assert st == 0, lib.fa_status_string(st).decode()
    nbytes = lib.fa_backward_workspace_bytes(B, H, N, d)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dq, dk, dv = (torch.empty((B, H, N, d), dtype=torch.float32, device="cuda") for _ in range(3))
    st = lib.fa_backward(_p(q), _p(k), _p(v), _p(o), _p(do), _p(lse), _p(dq), _p(dk), _p(dv), _p(ws), nbytes,
                         B, H, N, d, ctypes.c_float(sc), int(causal), code, stream)
    assert st == 0, lib.fa_status_string(st).decode()
    torch.cuda.synchronize()
    a = {x: to64(inp[x]) for x in ("q", "k", "v", "do")}
    o_ref, lse_ref = naive.forward(a["q"], a["k"], a["v"], sc, causal)
    assert_close("O", o.cpu(), o_ref, dtype)
    assert_lse(lse.cpu(), lse_ref)
    ref = naive.backward(a["q"], a["k"], a["v"], a["do"], sc, causal)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        assert_close(name, g.cpu(), r, dtype, out_dtype="f32")


def _rounded(nbytes, unit=2 << 20):
    return -(-nbytes // unit) * unit


def test_no_quadratic_device_memory():
    """At 4 x 16 heads, N = 8192, d = 64, fp16 (naive S: 4*16*8192^2*2 B = 8.59 GB), the
    forward's device memory high-water mark grows by O and lse only, and the backward's by
    dQ, dK, dV and the 8-byte-per-row workspace only (each rounded up to the caching
    allocator's 2 MiB segments); the device's free memory drops by no more than that."""
    B, H, N, d = 4, 16, 8192, 64
    naive_s = B * H * N * N * 2
    assert naive_s == 8_589_934_592
    inp = make_inputs(B, H, N, d, "f16", seed_base=41000, with_do=True)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    def measure(fn, outputs_bytes):
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        free0 = torch.cuda.mem_get_info()[0]
        res = fn()
        torch.cuda.synchronize()
        grew = torch.cuda.max_memory_allocated() - base
        took = free0 - torch.cuda.mem_get_info()[0]
        allowed = sum(_rounded(b) for b in outputs_bytes)
        print(f"high-water growth {grew / 2**20:.1f} MiB, device free memory taken {took / 2**20:.1f} MiB, "
              f"outputs {sum(outputs_bytes) / 2**20:.1f} MiB, naive S {naive_s / 2**30:.2f} GiB")
        assert grew <= allowed
        assert took <= allowed + (64 << 20)  # the allocator's own segment rounding
        return res

    rows = B * H * N
    o, lse = measure(lambda: fa.fa_forward(q, k, v, causal=False), [rows * d * 2, rows * 4])
    grads = measure(lambda: fa.fa_backward(q, k, v, o, do, lse, causal=False),
                    [rows * d * 4] * 3 + [fa.fa_backward_workspace_bytes(B, H, N, d)])
    for g in grads:
        assert torch.isfinite(g).all()
