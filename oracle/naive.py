"""Plain fp64 attention: the definition written out, S and P materialised.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py`` for who may import this.

Definition ([FA-17] section 二, [FA-blog] section 1.1, [FA-ch] intro):

    S = scale * Q K^T              (N x N per batch and head)
    P = softmax(S)  row by row     (safe softmax: subtract the row max first,
                                    [FA-ch] section 地基：流式 softmax)
    O = P V

Readings where the pages are silent (each also listed in the design doc):

* causal: key j is visible to query i iff j <= i (lower triangle, diagonal
  included; [FA-17] section 四 and the mask remark in section 五, [FA-ch]
  FlashAttention-2 section on fully masked blocks).  Masked scores are -inf.
* LSE_i = m_i + ln(l_i): the natural-log logsumexp of the scaled, masked row; the
  pages save (m, l) per row ([FA-ch] FlashAttention section on recomputation,
  [FA-nips] 方法细节), and m + ln l carries the same information.
* backward: the pages state only that it recomputes S/P from Q, K and the saved
  statistics.  The gradients here are the calculus of O = softmax(S) V:
      dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
      dS = P * (dP - D 1^T),  dQ = scale dS K,  dK = scale dS^T Q.

All arithmetic is numpy float64.  Inputs are whatever the GPU receives (fp32, or
bf16/fp16 values already rounded), upcast to float64 by the caller or here.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "causal_mask",
    "scores",
    "softmax_rows",
    "probabilities",
    "forward",
    "forward_head",
    "backward",
    "backward_head",
]


def causal_mask(n_q: int, n_k: int) -> np.ndarray:
    """Boolean (n_q, n_k) array, True where key j is hidden from query i (j > i)."""
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    return j > i


def scores(q: np.ndarray, k: np.ndarray, scale: float, causal: bool) -> np.ndarray:
    """S = scale * Q K^T for one head, masked scores set to -inf.

    q: (N, d), k: (N, d) -> (N, N) float64.
    """
    s = scale * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    if causal:
        s = np.where(causal_mask(s.shape[0], s.shape[1]), -np.inf, s)
    return s


def softmax_rows(s: np.ndarray):
    """Row-wise safe softmax of a score matrix ([FA-ch] 地基：流式 softmax).

    Subtracts the row max m before exponentiating so nothing overflows, then divides
    by the row sum l.  Returns (P, m, l).  Rows may contain -inf (masked) entries but
    at least one finite entry.
    """
    s = np.asarray(s, np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=-1, keepdims=True)
    return e / l, m[..., 0], l[..., 0]


def probabilities(q, k, scale: float, causal: bool) -> np.ndarray:
    """P = softmax(scale * Q K^T) for one head (N x N, float64)."""
    p, _, _ = softmax_rows(scores(q, k, scale, causal))
    return p


def forward_head(q, k, v, scale: float, causal: bool):
    """One head: returns (O (N, d), LSE (N,)) in float64."""
    s = scores(q, k, scale, causal)
    p, m, l = softmax_rows(s)
    o = p @ np.asarray(v, np.float64)
    lse = m + np.log(l)
    return o, lse


def forward(q, k, v, scale: float, causal: bool, heads=None):
    """Attention forward over (B, H, N, d) inputs.

    Returns (O, LSE) as float64 arrays of shapes (B, H, N, d) and (B, H, N).  With
    ``heads`` (an iterable of (b, h) pairs) only those heads are computed and the
    other entries are NaN -- used to check sampled heads at full problem sizes.
    """
    q = np.asarray(q)
    B, H, N, d = q.shape
    o = np.full((B, H, N, v.shape[-1]), np.nan)
    lse = np.full((B, H, N), np.nan)
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for b, h in todo:
        o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], scale, causal)
    return o, lse


def backward_head(q, k, v, do, scale: float, causal: bool):
    """One head: returns (dQ, dK, dV) in float64 from Q, K, V and dO alone."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    p = probabilities(q, k, scale, causal)
    dv = p.T @ do
    dp = do @ v.T
    dsum = np.sum(p * dp, axis=-1, keepdims=True)  # D_i = sum_j P_ij dP_ij
    ds = p * (dp - dsum)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def backward(q, k, v, do, scale: float, causal: bool, heads=None):
    """Attention backward over (B, H, N, d) inputs -> (dQ, dK, dV) float64.

    ``heads`` restricts the computation to the listed (b, h) pairs (others NaN).
    """
    q = np.asarray(q)
    B, H, N, d = q.shape
    dq = np.full(q.shape, np.nan)
    dk = np.full(q.shape, np.nan)
    dv = np.full(np.asarray(v).shape, np.nan)
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for b, h in todo:
        dq[b, h], dk[b, h], dv[b, h] = backward_head(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
    return dq, dk, dv
