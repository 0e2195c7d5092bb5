"""Full-size parity: every head and every row of every named workload against the fp64
oracle, in the launch configuration the benchmark times (needs an MI355X).

Each workload runs once on the GPU (forward, and the backward where the workload has
one) exactly as ``bench.py`` launches it: the library's suggested split count, the
workload's block mask, the square entry points for square shapes.  The oracle then
computes every (batch, key/value head) group on the host, several groups at a time on
threads (numpy releases the interpreter lock inside its array loops), and the errors of
O, lse, dQ, dK and dV are gathered over all heads.

The bars are those of ``parity.py``.  The raw maximum, the mean, the output rounding
floor and the error beyond the floor are reported for each tensor; with the environment
variable FA_PARITY_RECORD set to a file name, one JSON line per workload is appended to
it (``parity_table.py`` turns such a file into a table).
"""

import json
import math
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import exact_tiled_attention_forward_amd as fa
from exact_tiled_attention_forward_amd.workloads import WORKLOADS, workload_block_mask, workload_inputs
from oracle import naive
from parity import ErrorStats, to64

pytestmark = pytest.mark.gpu

FULL = ["single_head_f32", "prefill_bf16", "gpt2_medium_train", "long_f16", "long_bf16", "large_head_causal",
        "smoke_2x4x512", "gqa_causal_train", "decode_gqa", "block_sparse_local", "block_sparse_butterfly"]

HOST_BYTES = 64 << 30  # host memory the concurrent oracle heads may use together


def _record(entry):
    path = os.environ.get("FA_PARITY_RECORD")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(entry) + "\n")


def _workers(w):
    """Threads for the oracle: about eight N_q x N_k float64 arrays live per head (S, P and
    their temporaries; dP and dS in the backward)."""
    per_head = 8 * 8 * w.N * w.Nk
    cores = len(os.sched_getaffinity(0))
    return max(1, min(cores, 16, HOST_BYTES // per_head))


def _gpu(w, inp, bm):
    """The workload's passes on the GPU, launched as bench.py launches them."""
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    ns = fa.fa_forward_split_count(q, k, w.causal)
    bmd = bm.to(dev) if bm is not None else None
    o, lse = fa.fa_forward(q, k, v, causal=w.causal, split=ns, block_mask=bmd)
    out = {"o": o, "lse": lse}
    if w.backward:
        do = inp["do"].to(dev)
        out["dq"], out["dk"], out["dv"] = fa.fa_backward(q, k, v, o, do, lse, causal=w.causal, block_mask=bmd)
    torch.cuda.synchronize()
    return {name: t.cpu() for name, t in out.items()}, ns


@pytest.mark.parametrize("name", FULL)
def test_full_size_every_head(name):
    w = WORKLOADS[name]
    t0 = time.perf_counter()
    inp = workload_inputs(w)
    bm = workload_block_mask(w)
    got, ns = _gpu(w, inp, bm)
    t_gpu = time.perf_counter() - t0
    q, k, v = (inp[x] for x in ("q", "k", "v"))
    do = inp.get("do")
    G = w.H // w.Hkv
    out16 = None if w.dtype == "f32" else w.dtype
    hidden = None if bm is None else naive.expand_block_mask(bm[0].numpy(), w.N, w.Nk)

    def group(bg):
        b, g = bg
        st = {"O": ErrorStats(out16 or "f32"), "lse": ErrorStats(None, relative=True)}
        if w.backward:
            st.update({"dQ": ErrorStats("f32"), "dK": ErrorStats("f32"), "dV": ErrorStats("f32")})
        kk, vv = to64(k[b, g]), to64(v[b, g])
        dk_ref = dv_ref = 0.0
        for h in range(g * G, (g + 1) * G):
            qq = to64(q[b, h])
            o_ref, lse_ref = naive.forward_head(qq, kk, vv, w.scale, w.causal, hidden)
            st["O"].add(got["o"][b, h], o_ref)
            st["lse"].add(got["lse"][b, h], lse_ref)
            del o_ref, lse_ref
            if w.backward:
                dq_ref, dkh, dvh = naive.backward_head(qq, kk, vv, to64(do[b, h]), w.scale, w.causal, hidden)
                st["dQ"].add(got["dq"][b, h], dq_ref)
                dk_ref = dk_ref + dkh
                dv_ref = dv_ref + dvh
        if w.backward:
            st["dK"].add(got["dk"][b, g], dk_ref)
            st["dV"].add(got["dv"][b, g], dv_ref)
        return st

    groups = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    total = {}
    with ThreadPoolExecutor(max_workers=_workers(w)) as ex:
        for i, st in enumerate(ex.map(group, groups)):
            for key, s in st.items():
                if key in total:
                    total[key].merge(s)
                else:
                    total[key] = s
            if (i + 1) % max(1, len(groups) // 4) == 0:
                print(f"{name}: {i + 1}/{len(groups)} head groups checked ({time.perf_counter() - t0:.0f} s)",
                      flush=True)
    entry = {"workload": name, "shape": [w.B, w.H, w.Hkv, w.N, w.Nk, w.d], "dtype": w.dtype, "causal": w.causal,
             "split": ns, "block_mask": bm is not None, "heads": w.B * w.H, "gpu_seconds": round(t_gpu, 2),
             "seconds": round(time.perf_counter() - t0, 2),
             "errors": {key: s.as_dict() for key, s in total.items()}}
    _record(entry)
    for key, s in total.items():
        print(f"{name} {key}: max {s.max:.3e} mean {s.mean:.3e} floor max {s.floor_max:.3e} "
              f"beyond floor {s.excess_max:.3e} max|ref| {s.ref_max:.3e}")
    bar = w.dtype
    for key, s in total.items():
        s.check(f"{name} {key}", bar)
