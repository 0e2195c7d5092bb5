"""Seeded synthetic workloads for exact attention: shapes, dtypes and input recipes.

This module holds no attention arithmetic.  It only draws Q, K, V (and dO) from a
seeded CPU generator and rounds them to the storage dtype, so that the HIP path
and the fp64 CPU checker receive bit-identical inputs.

Workloads (B, H, N, d, storage dtype, causal):

* ``single_head_f32``      1, 1,   256,  64, fp32, no   -- forward only, O and LSE.
* ``prefill_bf16``         1, 8,  4096,  64, bf16, yes  -- 4,096-token, 8-head prefill.
* ``gpt2_medium_train``   16, 16, 1024,  64, bf16, yes  -- forward + backward, dO ~ N(0,1).
* ``long_f16``             4, 16, 8192,  64, fp16, no   -- naive S would be 8.59 GB.
* ``long_bf16``            1, 16, 16384, 64, bf16, no
* ``large_head_causal``    2, 16, 8192, 128, bf16, yes  -- forward + backward; in Q and K,
  for each (b, h) independently, round(0.05 N) row indices drawn without replacement
  are scaled by 8 (exact in bf16) to stress the running-max rescaling.
* ``smoke_2x4x512``        2, 4,   512,  64, bf16, no   -- the consistency smoke test
  shape and seed 0 from the cf-1.com article, section 3.3.
* ``gqa_causal_train``     1, 32 query / 8 key-value heads, 8192, 128, bf16, yes -- forward +
  backward with grouped heads.
* ``decode_gqa``           8, 32 query / 8 key-value heads, 1 query row against 8192 cached
  keys, 128, bf16, causal (the query is the newest position) -- forward only.
* ``block_sparse_local``   1, 16, 16384, 128, bf16, no   -- forward + backward under the
  local_global_block_mask pattern (9 of 128 key blocks per query block, about 7%).
* ``block_sparse_butterfly`` 1, 16, 16384, 128, bf16, no -- forward + backward under the
  butterfly_block_mask pattern (8 of 128 key blocks per query block, 6.25%).

Recipe: each tensor is drawn i.i.d. N(0, 1) in fp32 on the CPU with
``torch.Generator().manual_seed(seed)`` and cast (round-to-nearest-even) to the storage
dtype.  Seeds are ``seed_base + t`` with t = 1 (Q), 2 (K), 3 (V), 4 (dO), 5 (Q outlier
rows), 6 (K outlier rows).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_cross_inputs", "local_global_block_mask",
           "butterfly_block_mask", "workload_block_mask", "torch_dtype", "elem_bytes", "fwd_flops", "bwd_flops"]

_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _DTYPES[name]


def elem_bytes(name: str) -> int:
    return {"f32": 4, "f16": 2, "bf16": 2}[name]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool
    backward: bool
    seed_base: int
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    note: str = field(default="", compare=False)
    Hkv_: int = 0  # key/value heads (0: H, one per query head)
    Nk_: int = 0   # key rows (0: N)
    block_pattern: str = ""  # "" (dense), "local_global" or "butterfly" (128 x 128 block mask)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def Hkv(self) -> int:
        return self.Hkv_ or self.H

    @property
    def Nk(self) -> int:
        return self.Nk_ or self.N

    def visible_pairs(self) -> float:
        """(query, key) pairs per head that the work convention counts: N^2/2 for square
        causal attention (the usual halving), the exact count when N_q < N_k."""
        nq, nk = self.N, self.Nk
        if not self.causal:
            return float(nq * nk)
        if nq == nk:
            return nq * nk / 2.0
        return float(nq * nk - nq * (nq - 1) // 2)

    def shape(self):
        return (self.B, self.H, self.N, self.d)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_head_f32", 1, 1, 256, 64, "f32", False, False, 1000),
        Workload("prefill_bf16", 1, 8, 4096, 64, "bf16", True, False, 2000),
        Workload("gpt2_medium_train", 16, 16, 1024, 64, "bf16", True, True, 3000),
        Workload("long_f16", 4, 16, 8192, 64, "f16", False, False, 41000),
        Workload("long_bf16", 1, 16, 16384, 64, "bf16", False, False, 42000),
        Workload("large_head_causal", 2, 16, 8192, 128, "bf16", True, True, 5000, 0.05, 8.0),
        Workload("smoke_2x4x512", 2, 4, 512, 64, "bf16", False, False, 0),
        Workload("gqa_causal_train", 1, 32, 8192, 128, "bf16", True, True, 6000, Hkv_=8),
        Workload("decode_gqa", 8, 32, 1, 128, "bf16", True, False, 7000, Hkv_=8, Nk_=8192),
        Workload("block_sparse_local", 1, 16, 16384, 128, "bf16", False, True, 8000, block_pattern="local_global"),
        Workload("block_sparse_butterfly", 1, 16, 16384, 128, "bf16", False, True, 8100, block_pattern="butterfly"),
    ]
}


def _randn(shape, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(int(seed))
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def _scale_rows(x: torch.Tensor, frac: float, factor: float, seed: int) -> torch.Tensor:
    """Scale round(frac*N) rows of every (b, h) slice of x by ``factor``."""
    B, H, N, _ = x.shape
    count = int(round(frac * N))
    if count == 0:
        return x
    g = torch.Generator().manual_seed(int(seed))
    x = x.clone()
    for b in range(B):
        for h in range(H):
            rows = torch.randperm(N, generator=g)[:count]
            x[b, h, rows] *= factor
    return x


def make_inputs(B: int, H: int, N: int, d: int, dtype: str, seed_base: int,
                outlier_frac: float = 0.0, outlier_scale: float = 1.0, with_do: bool = False):
    """Return dict of CPU tensors q, k, v (and do) in the storage dtype.

    Shapes are (B, H, N, d), contiguous.  Values are N(0,1) fp32 draws rounded to the
    storage dtype; with ``outlier_frac`` the chosen Q and K rows are multiplied by
    ``outlier_scale`` before rounding (a power of two, so the product is exact).
    """
    shape = (B, H, N, d)
    td = torch_dtype(dtype)
    q = _randn(shape, seed_base + 1)
    k = _randn(shape, seed_base + 2)
    v = _randn(shape, seed_base + 3)
    if outlier_frac > 0:
        q = _scale_rows(q, outlier_frac, outlier_scale, seed_base + 5)
        k = _scale_rows(k, outlier_frac, outlier_scale, seed_base + 6)
    out = {"q": q.to(td).contiguous(), "k": k.to(td).contiguous(), "v": v.to(td).contiguous()}
    if with_do:
        out["do"] = _randn(shape, seed_base + 4).to(td).contiguous()
    return out


def local_global_block_mask(N: int, window: int = 4):
    """uint8 (1, nb, nb) block mask (128 x 128 blocks, nb = ceil(N/128)): every query block
    sees the key blocks within ``window`` of its own and the first key block -- a local
    window plus one global block, the kind of fixed sparsity pattern block-sparse attention
    serves."""
    nb = -(-N // 128)
    i = torch.arange(nb)[:, None]
    j = torch.arange(nb)[None, :]
    keep = ((i - j).abs() <= window) | (j == 0)
    return keep.to(torch.uint8)[None].contiguous()


def butterfly_block_mask(N: int):
    """uint8 (1, nb, nb) block mask (128 x 128 blocks, nb = ceil(N/128)) with the flat
    butterfly pattern: query block i sees key block j iff i XOR j is 0 or a power of two,
    i.e. the two block indices differ in at most one bit.  This is the union of the
    supports of the log2(nb) butterfly factors (each pairs blocks whose indices differ in
    one bit), so every block row holds 1 + log2(nb) visible blocks when nb is a power of
    two: 8 of 128 (6.25%) at N = 16384."""
    nb = -(-N // 128)
    i = torch.arange(nb)[:, None]
    j = torch.arange(nb)[None, :]
    x = i ^ j
    keep = (x & (x - 1)) == 0  # x == 0 or a power of two
    return keep.to(torch.uint8)[None].contiguous()


def workload_block_mask(w: "Workload"):
    """The workload's block mask (CPU uint8 tensor), or None for a dense workload."""
    if w.block_pattern == "local_global":
        return local_global_block_mask(w.N)
    if w.block_pattern == "butterfly":
        return butterfly_block_mask(w.N)
    return None


def make_cross_inputs(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, dtype: str, seed_base: int,
                      with_do: bool = False):
    """Like make_inputs for attention with grouped heads and/or different lengths:
    q (and do) are (B, Hq, Nq, d), k and v are (B, Hkv, Nk, d); same seeds per tensor."""
    td = torch_dtype(dtype)
    out = {"q": _randn((B, Hq, Nq, d), seed_base + 1).to(td).contiguous(),
           "k": _randn((B, Hkv, Nk, d), seed_base + 2).to(td).contiguous(),
           "v": _randn((B, Hkv, Nk, d), seed_base + 3).to(td).contiguous()}
    if with_do:
        out["do"] = _randn((B, Hq, Nq, d), seed_base + 4).to(td).contiguous()
    return out


def workload_inputs(w: Workload, with_do: bool | None = None):
    """Inputs of a named workload at its full size."""
    with_do = w.backward if with_do is None else with_do
    if w.Hkv != w.H or w.Nk != w.N:
        return make_cross_inputs(w.B, w.H, w.Hkv, w.N, w.Nk, w.d, w.dtype, w.seed_base, with_do=with_do)
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed_base, w.outlier_frac, w.outlier_scale, with_do=with_do)


def fwd_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Forward work convention: 4 B H N^2 d (two N x N x d products), halved for causal."""
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def bwd_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Backward work convention: 10 B H N^2 d (five N x N x d products, including the
    recomputation of S), halved for causal."""
    f = 10.0 * B * H * N * N * d
    return f / 2 if causal else f
