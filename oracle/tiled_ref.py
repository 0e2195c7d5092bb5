"""CPU tiled online-softmax recurrence, in the pages' order -- TEST INFRASTRUCTURE ONLY.

This is not a second oracle for the GPU results (``naive`` is).  It spells out the
recurrence the pages describe, so that tests can pin the worked examples the pages
print and check, by brute force on tiny inputs, that tiling reaches the same O and
LSE as the untiled definition ([FA-ch] intro: equal up to floating-point rounding;
[FA-blog] section 2.2; [FA-nips] 方法细节, the correctness theorem).

Recurrence for one query block (rows i), streaming key/value blocks j in order
([FA-blog] section 2.2, [FA-17] section 三, [FA-nips] 基准/方法设计):

    m_new   = max(m_old, rowmax(S_ij))
    alpha   = exp(m_old - m_new)                 (the rescale patch, [FA-ch] 地基)
    l_new   = alpha * l_old + rowsum(exp(S_ij - m_new))
    acc_new = alpha * acc_old + exp(S_ij - m_new) @ V_j
    ...
    O_i = acc / l   (one division at the end, [FA-ch] FlashAttention-2 section)
    LSE_i = m + ln(l)

``merge_stats`` is the block-to-block merge as written in [FA-nips] 基准/方法设计:
m_new = max(m, m~), l_new = e^(m - m_new) l + e^(m~ - m_new) l~, where (m~, l~) are
the new block's own max and sum.
"""

from __future__ import annotations

import numpy as np

__all__ = ["block_stats", "merge_stats", "online_stats", "tiled_forward_head", "tiled_forward"]


def block_stats(x: np.ndarray):
    """(m~, l~) of one block of a score row: its own max and sum of exp(x - m~)."""
    x = np.asarray(x, np.float64)
    m = np.max(x)
    return m, float(np.sum(np.exp(x - m)))


def merge_stats(m: float, l: float, m_blk: float, l_blk: float):
    """Merge running (m, l) with a block's (m~, l~) ([FA-nips] 基准/方法设计)."""
    m_new = max(m, m_blk)
    l_new = np.exp(m - m_new) * l + np.exp(m_blk - m_new) * l_blk
    return m_new, l_new


def online_stats(row, block: int):
    """Stream one score row in blocks of ``block`` entries.

    Returns the list of (m, l, alpha) after each block, where alpha is the factor the
    previous running sum was multiplied by ([FA-17] worked example; [FA-ch] rescale
    e^(old max - new max)).
    """
    row = np.asarray(row, np.float64)
    m, l = -np.inf, 0.0
    trace = []
    for start in range(0, row.size, block):
        x = row[start:start + block]
        m_new = max(m, float(np.max(x)))
        alpha = float(np.exp(m - m_new))
        l = alpha * l + float(np.sum(np.exp(x - m_new)))
        m = m_new
        trace.append((m, l, alpha))
    return trace


def tiled_forward_head(q, k, v, scale: float, causal: bool, br: int, bc: int):
    """One head, tiled: query blocks of ``br`` rows outer, key/value blocks of ``bc``
    rows inner.  Returns (O, LSE) in float64.  Fully masked key blocks of a causal
    query block are skipped, as the FlashAttention-2 section of [FA-ch] describes."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n = q.shape[0]
    o = np.empty((n, v.shape[1]))
    lse = np.empty(n)
    for i0 in range(0, n, br):
        rows = np.arange(i0, min(i0 + br, n))
        m = np.full(rows.size, -np.inf)
        l = np.zeros(rows.size)
        acc = np.zeros((rows.size, v.shape[1]))
        for j0 in range(0, n, bc):
            cols = np.arange(j0, min(j0 + bc, n))
            if causal and cols[0] > rows[-1]:
                break  # every key of this and later blocks is in the future of every row
            s = scale * (q[rows] @ k[cols].T)
            if causal:
                s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
            m_new = np.maximum(m, np.max(s, axis=1))
            alpha = np.exp(m - m_new)
            p = np.exp(s - m_new[:, None])
            l = alpha * l + np.sum(p, axis=1)
            acc = alpha[:, None] * acc + p @ v[cols]
            m = m_new
        o[rows] = acc / l[:, None]
        lse[rows] = m + np.log(l)
    return o, lse


def tiled_forward(q, k, v, scale: float, causal: bool, br: int, bc: int):
    """(B, H, N, d) wrapper around ``tiled_forward_head``."""
    q = np.asarray(q)
    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[-1]))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = tiled_forward_head(q[b, h], k[b, h], v[b, h], scale, causal, br, bc)
    return o, lse
