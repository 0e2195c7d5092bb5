"""Plain fp64 attention: the definition written out, S and P materialised.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py`` for who may import this.

Definition ([FA-17] section 二, [FA-blog] section 1.1, [FA-ch] intro):

    S = scale * Q K^T              (N x N per batch and head)
    P = softmax(S)  row by row     (safe softmax: subtract the row max first,
                                    [FA-ch] section 地基：流式 softmax)
    O = P V

Readings where the pages are silent:

* causal: key j is visible to query i iff j <= i (lower triangle, diagonal
  included; [FA-17] section 四 and the mask remark in section 五, [FA-ch]
  FlashAttention-2 section on fully masked blocks).  Masked scores are -inf.
* query and key lengths may differ ([FA-blog] section 3.4: Q from the decoder,
  K/V from the encoder or a growing cache).  With causal masking the N_q queries
  are the last N_q positions of the N_k-long sequence (a decode step's query is the
  newest token and sees the whole cache, [FA-17] section 五 on decode): key j is
  visible to query i iff j <= i + (N_k - N_q).  N_q > N_k with causal masking
  would leave rows with no visible key and is rejected.
* grouped heads ([FA-17] section 四 names GQA as a mask-like variant orthogonal to
  the tiling): H_q query heads share H_kv key/value heads, H_q = G * H_kv; query
  head h reads key/value head h // G (consecutive query heads form a group).  In
  the backward, the gradient of a shared K or V head is the sum over its group.
* block-sparse masks ([FA-nips] 方法细节 and its LRA results: block-sparse
  FlashAttention skips whole zero blocks of a given block mask): a mask of
  (heads, ceil(N_q/128), ceil(N_k/128)) bytes, shared by the batch, one layer or
  one per query head; block (i//128, j//128) == 0 hides key j from query i (on top
  of the causal mask).  A query row with no visible key has P = 0, O = 0 and
  LSE = -inf (and zero gradients), the usual reading of an empty softmax in
  masked attention.
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
    "BLOCK",
    "causal_mask",
    "expand_block_mask",
    "kv_head",
    "scores",
    "softmax_rows",
    "probabilities",
    "forward",
    "forward_head",
    "backward",
    "backward_head",
]


def causal_mask(n_q: int, n_k: int) -> np.ndarray:
    """Boolean (n_q, n_k) array, True where key j is hidden from query i.

    The queries are the last n_q positions of an n_k-long sequence, so query i sits at
    position i + (n_k - n_q) and sees keys j <= i + (n_k - n_q); for n_q == n_k this is
    the plain lower triangle j <= i.
    """
    if n_q > n_k:
        raise ValueError("causal attention needs n_q <= n_k (otherwise some query sees no key)")
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    return j > i + (n_k - n_q)


def kv_head(h: int, h_q: int, h_kv: int) -> int:
    """Key/value head read by query head h: consecutive groups of h_q // h_kv query heads
    share one key/value head."""
    if h_q % h_kv:
        raise ValueError("the query head count must be a multiple of the key/value head count")
    return h // (h_q // h_kv)


BLOCK = 128  # rows and columns of one block of a block-sparse mask


def expand_block_mask(block_mask_head, n_q: int, n_k: int, block: int = BLOCK) -> np.ndarray:
    """Boolean (n_q, n_k) array, True where key j is hidden from query i because block
    (i // block, j // block) of the (ceil(n_q/block), ceil(n_k/block)) block mask is 0."""
    bm = np.asarray(block_mask_head)
    nb_q, nb_k = -(-n_q // block), -(-n_k // block)
    if bm.shape != (nb_q, nb_k):
        raise ValueError(f"block mask must be ({nb_q}, {nb_k}) for n_q={n_q}, n_k={n_k}")
    keep = np.repeat(np.repeat(bm != 0, block, axis=0), block, axis=1)[:n_q, :n_k]
    return ~keep


def scores(q: np.ndarray, k: np.ndarray, scale: float, causal: bool, hidden=None) -> np.ndarray:
    """S = scale * Q K^T for one head, masked scores set to -inf.

    q: (N_q, d), k: (N_k, d) -> (N_q, N_k) float64.  ``hidden`` (bool (N_q, N_k)) hides
    more keys on top of the causal mask.
    """
    s = scale * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    if causal:
        s = np.where(causal_mask(s.shape[0], s.shape[1]), -np.inf, s)
    if hidden is not None:
        s = np.where(hidden, -np.inf, s)
    return s


def softmax_rows(s: np.ndarray):
    """Row-wise safe softmax of a score matrix ([FA-ch] 地基：流式 softmax).

    Subtracts the row max m before exponentiating so nothing overflows, then divides
    by the row sum l.  Returns (P, m, l).  Rows may contain -inf (masked) entries; a row
    with no finite entry gets P = 0, m = -inf and l = 0.
    """
    s = np.asarray(s, np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    empty = ~np.isfinite(m)
    e = np.exp(s - np.where(empty, 0.0, m))
    l = np.sum(e, axis=-1, keepdims=True)
    p = e / np.where(empty, 1.0, l)
    return p, m[..., 0], l[..., 0]


def probabilities(q, k, scale: float, causal: bool, hidden=None) -> np.ndarray:
    """P = softmax(scale * Q K^T) for one head (N_q x N_k, float64)."""
    p, _, _ = softmax_rows(scores(q, k, scale, causal, hidden))
    return p


def forward_head(q, k, v, scale: float, causal: bool, hidden=None):
    """One head: returns (O (N_q, d), LSE (N_q,)) in float64; an empty row gives O = 0 and
    LSE = -inf."""
    s = scores(q, k, scale, causal, hidden)
    p, m, l = softmax_rows(s)
    o = p @ np.asarray(v, np.float64)
    with np.errstate(divide="ignore"):
        lse = m + np.log(l)
    return o, lse


def _hidden(block_mask, h: int, n_q: int, n_k: int):
    """Dense hidden-key mask of query head h from a (1 or H_q, nb_q, nb_k) block mask."""
    if block_mask is None:
        return None
    bm = np.asarray(block_mask)
    return expand_block_mask(bm[0 if bm.shape[0] == 1 else h], n_q, n_k)


def forward(q, k, v, scale: float, causal: bool, heads=None, block_mask=None):
    """Attention forward: q (B, H_q, N_q, d), k and v (B, H_kv, N_k, d).

    Returns (O, LSE) as float64 arrays of shapes (B, H_q, N_q, d) and (B, H_q, N_q).
    With ``heads`` (an iterable of (b, h) query-head pairs) only those heads are
    computed and the other entries are NaN -- used to check sampled heads at full
    problem sizes.  ``block_mask`` ((1 or H_q, ceil(N_q/128), ceil(N_k/128)), 0 =
    hidden block) applies a block-sparse mask.
    """
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    o = np.full((B, H, N, v.shape[-1]), np.nan)
    lse = np.full((B, H, N), np.nan)
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for b, h in todo:
        g = kv_head(h, H, Hkv)
        hid = _hidden(block_mask, h, N, k.shape[2])
        o[b, h], lse[b, h] = forward_head(q[b, h], k[b, g], v[b, g], scale, causal, hid)
    return o, lse


def backward_head(q, k, v, do, scale: float, causal: bool, hidden=None):
    """One head: returns (dQ, dK, dV) in float64 from Q, K, V and dO alone."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    p = probabilities(q, k, scale, causal, hidden)
    dv = p.T @ do
    dp = do @ v.T
    dsum = np.sum(p * dp, axis=-1, keepdims=True)  # D_i = sum_j P_ij dP_ij
    ds = p * (dp - dsum)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def backward(q, k, v, do, scale: float, causal: bool, heads=None, block_mask=None):
    """Attention backward: q, dO (B, H_q, N_q, d), k, v (B, H_kv, N_k, d) ->
    (dQ, dK, dV) float64 in the shapes of q, k and v.

    The gradient of a key/value head shared by a group of query heads is the sum of
    the group's per-head gradients.  ``heads`` restricts the computation to the listed
    (b, h_kv) key/value heads and every query head of their groups (others NaN); with
    one query head per key/value head these are the (b, h) heads themselves.
    """
    q, k, v, do = np.asarray(q), np.asarray(k), np.asarray(v), np.asarray(do)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    kv_head(0, H, Hkv)  # validates the grouping
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    todo = [(b, g) for b in range(B) for g in range(Hkv)] if heads is None else list(heads)
    for b, g in todo:
        dk[b, g] = 0.0
        dv[b, g] = 0.0
        for h in range(g * G, (g + 1) * G):
            hid = _hidden(block_mask, h, N, k.shape[2])
            dq[b, h], dkh, dvh = backward_head(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal, hid)
            dk[b, g] += dkh
            dv[b, g] += dvh
    return dq, dk, dv
