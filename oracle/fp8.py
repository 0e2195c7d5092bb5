"""FP8 (E4M3) attention forward with block scales -- TEST INFRASTRUCTURE ONLY (see
``oracle/__init__.py`` for who may import this).

Source: [FA-ch] "Flash Attention", section FlashAttention-3 (the second lever, FP8): an
E4M3 number has 256 bit patterns and a largest value of 448; block quantization gives
every small block its own scale so that an outlier only coarsens its own block; an
optional fixed random rotation of Q and K spreads an outlier's energy over every
dimension before rounding and leaves the dot products unchanged before rounding.

What is computed here, step by step (all arithmetic fp64 unless stated):

* ``e4m3_decode`` -- the value of each of the 256 bit patterns from the format's
  definition (sign, 4-bit exponent with bias 7, 3-bit mantissa; exponent 0 is
  subnormal; 0x7F and 0xFF are NaN, so 448 = 0x7E is the largest value).
* ``e4m3_round`` -- nearest representable value, ties to the even mantissa; inputs
  beyond +-448 are first clamped to +-448 (the quantizer never produces NaN).
* ``quantize_rows`` -- per (batch, head, block of 128 rows) scale s = amax / 448
  (1 for an all-zero block) and codes e4m3_round(x / s); ``quantize_channels`` -- per
  (batch, head, channel) scale over all rows (used for V, applied to O at the end).
* ``rotation`` -- a fixed random orthogonal d x d matrix (a Sylvester Hadamard matrix
  with a seeded random sign on every row, over sqrt(d)).
* ``tiled_forward_head`` -- the tiled online-softmax forward the FP8 kernel computes:
  keys in tiles of ``bc`` (aligned at key 0), running max m per row updated at every
  tile (m = max(m, tile max)), o and l rescaled by e^(m_old - m_new), probabilities
  p = e^(s - m) summed into l unrounded, and rounded to E4M3 (``round_p``) before they
  multiply V.  O = o / l and lse = m + ln l.  With ``round_p=False`` this is the exact
  tiled recurrence of ``tiled_ref`` (pinned to the definition).

Reading where the pages are silent: which tensors get which scales, the block size,
and whether P is rounded.  Here Q and K get 128-row block scales, V a per-channel
scale, and P (in [0, 1] relative to the running max) is rounded to E4M3 as the PV
product's input, which is what makes the product an 8-bit one.
"""

from __future__ import annotations

import math

import numpy as np
import torch

__all__ = ["E4M3_MAX", "e4m3_decode", "e4m3_round", "quantize_rows", "quantize_channels", "dequantize_rows",
           "dequantize_channels", "rotation", "tiled_forward_head", "forward"]

E4M3_MAX = 448.0
BLOCK = 128


def e4m3_decode() -> np.ndarray:
    """Values of the 256 E4M3 bit patterns (index = pattern), NaN for 0x7F and 0xFF."""
    out = np.empty(256)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            out[code] = np.nan
        elif exp == 0:
            out[code] = sign * (man / 8.0) * 2.0 ** (1 - 7)
        else:
            out[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return out


def e4m3_round(x) -> np.ndarray:
    """Round to the nearest E4M3 value (ties to even), after clamping to +-448.

    The rounding itself is torch's float8_e4m3fn cast (a library routine); the pins check
    it against the decoded grid."""
    x = np.asarray(x, np.float64)
    xc = np.ascontiguousarray(np.clip(np.atleast_1d(x), -E4M3_MAX, E4M3_MAX))
    return torch.from_numpy(xc).to(torch.float8_e4m3fn).to(torch.float64).numpy().reshape(x.shape)


def e4m3_codes(x) -> np.ndarray:
    """Bit patterns (uint8) of e4m3_round(x)."""
    x = np.asarray(x, np.float64)
    xc = np.ascontiguousarray(np.clip(np.atleast_1d(x), -E4M3_MAX, E4M3_MAX))
    return torch.from_numpy(xc).to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(x.shape)


def quantize_rows(x, block: int = BLOCK, dtype=np.float64):
    """x (B, H, N, d) -> (codes uint8 (B, H, N, d), scales (B, H, ceil(N/block))), with
    x ~= decode(codes) * scale of the row's block.  ``dtype`` is the precision of the
    scale and of x / scale (np.float32 takes the rounding decisions as a GPU computing in
    fp32 would)."""
    x = np.asarray(x, dtype)
    B, H, N, d = x.shape
    nb = -(-N // block)
    scales = np.ones((B, H, nb), dtype)
    codes = np.zeros(x.shape, np.uint8)
    for i in range(nb):
        blk = x[:, :, i * block:(i + 1) * block]
        amax = np.abs(blk).max(axis=(2, 3))
        s = np.where(amax > 0, amax / dtype(E4M3_MAX), dtype(1.0)).astype(dtype)
        scales[:, :, i] = s
        codes[:, :, i * block:(i + 1) * block] = e4m3_codes(blk / s[:, :, None, None])
    return codes, scales


def quantize_channels(x, dtype=np.float64):
    """x (B, H, N, d) -> (codes (B, H, N, d), scales (B, H, d)): one scale per channel."""
    x = np.asarray(x, dtype)
    amax = np.abs(x).max(axis=2)
    s = np.where(amax > 0, amax / dtype(E4M3_MAX), dtype(1.0)).astype(dtype)
    return e4m3_codes(x / s[:, :, None, :]), s


def dequantize_rows(codes, scales, block: int = BLOCK):
    vals = e4m3_decode()[np.asarray(codes)]
    s = np.repeat(np.asarray(scales, np.float64), block, axis=2)[:, :, :vals.shape[2]]
    return vals * s[..., None]


def dequantize_channels(codes, scales):
    return e4m3_decode()[np.asarray(codes)] * np.asarray(scales, np.float64)[:, :, None, :]


def rotation(d: int, seed: int = 0) -> np.ndarray:
    """Fixed random orthogonal d x d matrix: random signs times a Sylvester Hadamard
    matrix, over sqrt(d).  d must be a power of two."""
    if d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    signs = np.where(np.random.default_rng(seed).random(d) < 0.5, -1.0, 1.0)
    return (signs[:, None] * h) / math.sqrt(d)


def near_tie(p, rel: float):
    """(mask, step): where p >= 0 lies within rel * p of a midpoint between two E4M3 values
    (so that a rounding of p computed with that much error may land on either), and the
    grid step there."""
    p = np.asarray(p, np.float64)
    step = np.where(p >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(p, 2.0 ** -6))) - 3), 2.0 ** -9)
    frac = p / step - np.floor(p / step)
    return (np.abs(frac - 0.5) * step <= rel * p) & (p > 0), step


def tiled_forward_head(q, k, v, scale: float, causal: bool, bc: int = 64, round_p: bool = True,
                       tie_rel: float = 0.0):
    """One head of the FP8 kernel's recurrence on already-dequantized q (N_q, d), k, v
    (N_k, d); v here excludes its per-channel scale (the caller multiplies O by it).
    Returns (O, lse), and with ``tie_rel`` > 0 also a (N_q, d) slack: how far O could move
    if every probability within tie_rel (relative) of an E4M3 rounding midpoint rounded the
    other way -- the room a computation whose exponentials carry that much error needs."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    nq, nk = q.shape[0], k.shape[0]
    off = nk - nq
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    o = np.zeros((nq, v.shape[1]))
    slack = np.zeros((nq, v.shape[1]))
    rows = np.arange(nq)[:, None]
    for j0 in range(0, nk, bc):
        kj, vj = k[j0:j0 + bc], v[j0:j0 + bc]
        s = scale * (q @ kj.T)
        if causal:
            keys = np.arange(j0, j0 + kj.shape[0])[None, :]
            s = np.where(keys > rows + off, -np.inf, s)
        m_new = np.maximum(m, s.max(axis=1))
        seen = np.isfinite(m_new)
        alpha = np.where(np.isfinite(m), np.exp(m - np.where(seen, m_new, 0.0)), 0.0)
        p = np.where(seen[:, None], np.exp(s - np.where(seen, m_new, 0.0)[:, None]), 0.0)
        l = l * alpha + p.sum(axis=1)
        pr = e4m3_round(p) if round_p else p
        o = o * alpha[:, None] + pr @ vj
        if tie_rel > 0:
            amb, step = near_tie(p, tie_rel)
            slack = slack * alpha[:, None] + (amb * step) @ np.abs(vj)
        m = m_new
    if tie_rel > 0:
        return o / l[:, None], m + np.log(l), slack / l[:, None]
    return o / l[:, None], m + np.log(l)


def forward(q8, q_scale, k8, k_scale, v8, v_scale, scale: float, causal: bool, bc: int = 64, heads=None,
            round_p: bool = True, tie_rel: float = 0.0):
    """FP8 forward over codes and scales: q8 (B, H_q, N_q, d) with (B, H_q, ceil(N_q/128))
    scales, k8 likewise over (B, H_kv, N_k, d), v8 (B, H_kv, N_k, d) with (B, H_kv, d)
    channel scales.  Query head h reads key/value head h // (H_q // H_kv).  Returns
    (O, lse) float64 (and the tie slack of ``tiled_forward_head``, scaled like O, when
    ``tie_rel`` > 0); with ``heads`` only those (b, h) query heads (others NaN)."""
    qd = dequantize_rows(q8, q_scale)
    kd = dequantize_rows(k8, k_scale)
    vd = e4m3_decode()[np.asarray(v8)]
    vs = np.asarray(v_scale, np.float64)
    B, H, N, d = qd.shape
    G = H // kd.shape[1]
    o = np.full(qd.shape, np.nan)
    lse = np.full((B, H, N), np.nan)
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    slack = np.full(qd.shape, np.nan)
    for b, h in todo:
        g = h // G
        res = tiled_forward_head(qd[b, h], kd[b, g], vd[b, g], scale, causal, bc, round_p, tie_rel)
        o[b, h] = res[0] * vs[b, g][None, :]
        lse[b, h] = res[1]
        if tie_rel > 0:
            slack[b, h] = res[2] * vs[b, g][None, :]
    if tie_rel > 0:
        return o, lse, slack
    return o, lse
