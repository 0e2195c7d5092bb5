"""Per-element error bound of the FP8 (E4M3) forward against exact attention on the
dequantized inputs.  Test logic: the bar the GPU's FP8 output is held to.

Source of the approximation: "Flash Attention" (mlx.void.app), section FlashAttention-3:
the products run on E4M3 values (4 significant bits, largest value 448) with block
scales.  Q, K and V are given as codes and scales, so the exact result on those inputs
is plain attention of the dequantized tensors (``naive``); what the FP8 kernel adds on
top is (a) rounding each probability to E4M3 before the P V product, and (b) fp32
arithmetic: accumulated code products, the exponent's multiply-add, ``v_exp_f32``, the
running sums, the rescaling and the final division, and (c) the bf16 rounding of O.

Derivation (one query row; j runs over visible keys; E_j = exp(s_j - m) with the final
row max m, l = sum_j E_j, O = sum_j E_j v_j / l exactly):

1. Exponent.  The kernel forms x_j = t_j * cs - m_run in fp32 from the fp32 sum t_j of d
   exact code products (|error| <= gamma_d sum_c |q_c k_c|, gamma_n = n u / (1 - n u),
   u = 2^-24), with cs = scale * log2(e) * s_q * s_k rounded in a few steps (<= 6u
   relative) and one rounding of the fused multiply-add (<= u |x_j|).  m_run is common
   to every key of a tile and cancels in O and lse (the rescale by exp2(m_old - m_new)
   reconciles any reference), so the exponent error is
       dx_j <= cs gamma_d T_j + 8u |t_j cs| + u (|t_j cs| + max_j' |t_j' cs|),
   T_j = sum_c |q_c k_jc| (base-2 units).
2. Probability.  p~_j = exp2(x_j) (1 + e), |e| <= 2^-22 for v_exp_f32 (two ulps); every
   rescale of the running o and l by exp2(m_old - m_new) multiplies both by the same
   computed factor (one more exp error and two roundings per tile, n_t tiles).  So
   p~_j = E_j a (1 + delta_j) for a common a with
       delta_j <= ln(2) dx_j (1.01) + 2^-22 + (n_t + 1)(2^-22 + 2u).
3. E4M3 rounding of P (the method's own approximation).  p~_j is rounded relative to the
   running max, which never exceeds the final one (factor a_j <= 1 to final-max units).
   Half an E4M3 step is 2^-4 p for p >= 2^-6 and 2^-10 below (subnormals, step 2^-9); a
   p below 2^-10 rounds to 0 and loses exactly itself.  With E~_j = E_j (1 + delta_j) =
   a_j p~_j, in final-max units
       |a_j E4M3(p~_j) - E~_j| <= max(2^-4 E~_j, min(E~_j, 2^-10)).
   (A p~_j near a rounding midpoint may round either way; the bound holds for either
   neighbour.)
4. Sums.  The numerator sum_j pr_j v_jc and the denominator l~ = sum_j p~_j accumulate in
   fp32: <= gamma_{n_k + n_t + 2} times the sums of absolute values.
   With A_c = sum_j |v_jc| (max(2^-4 E~_j, min(E~_j, 2^-10)) + delta_j E_j),
   B = sum_j delta_j E_j + gamma (l + sum_j delta_j E_j) (the denominator error) and
   C_c = gamma sum_j (E~_j (1 + 2^-4) + min(E~_j, 2^-10)) |v_jc|:
       |O~_c - O_c| <= (A_c + |O_c| B + C_c) / (l - B) + 4u |O_c|        (fp32 result)
5. Output.  bf16 rounding adds at most 2^-8 of the value (8 significant bits):
       bound_c = err_c + 2^-8 (|O_c| + err_c).
6. lse = m + ln l~ (the unrounded fp32 sum): |lse~ - lse| <= B / (l - B) + 8u (|lse| + 1).

The dominant term is step 3: about 2^-4 sum_j P_j |v_jc| plus 2^-10 |v_jc| / l for each
probability in the subnormal range, far above the fp32 terms.
"""

from __future__ import annotations

import math

import numpy as np

from oracle import fp8, naive

U = 2.0 ** -24          # fp32 unit roundoff
EXP_REL = 2.0 ** -22    # v_exp_f32 relative error allowance
E4M3_REL = 2.0 ** -4    # E4M3 unit roundoff (4 significant bits)
E4M3_SUB = 2.0 ** -10   # half the E4M3 subnormal step 2^-9
BF16_REL = 2.0 ** -8    # bf16 unit roundoff (8 significant bits)
LOG2E = 1.4426950408889634


def gamma(n: int) -> float:
    return n * U / (1 - n * U)


def head_bound(q8, qs, k8, ks, v8, vs, scale: float, causal: bool, bc: int = 64, p_rel: float = E4M3_REL,
               p_sub: float = E4M3_SUB):
    """One query head against its key/value head.  q8 (N_q, d) codes with per-row scales
    qs (N_q,) (each row's 128-row block scale), k8 (N_k, d) with ks (N_k,), v8 (N_k, d)
    with channel scales vs (d,).  Returns (O exact, lse exact, O bound, lse bound), all
    float64.  ``p_rel``/``p_sub`` are the probability rounding's relative and subnormal
    half steps (the E4M3 values by default)."""
    dec = fp8.e4m3_decode()
    qc, kc, vc = dec[np.asarray(q8)], dec[np.asarray(k8)], dec[np.asarray(v8)]
    qs, ks, vs = (np.asarray(a, np.float64) for a in (qs, ks, vs))
    nq, d = qc.shape
    nk = kc.shape[0]
    qd, kd, vd = qc * qs[:, None], kc * ks[:, None], vc * vs[None, :]
    s = naive.scores(qd, kd, scale, causal)
    p, m, l = naive.softmax_rows(s)
    o = p @ vd
    lse = m + np.log(l)
    vis = np.isfinite(s)
    E = p * l[:, None]                               # exp(s - m), 0 where hidden
    t = qc @ kc.T                                    # code products (exact in fp64)
    T = np.abs(qc) @ np.abs(kc).T
    cs = scale * LOG2E * qs[:, None] * ks[None, :]
    tcs = np.abs(t * cs)
    tmax = np.where(vis, tcs, 0.0).max(axis=1, keepdims=True)
    dx = cs * gamma(d) * T + 8 * U * tcs + U * (tcs + tmax)
    n_t = -(-nk // bc)
    delta = math.log(2) * dx * 1.01 + EXP_REL + (n_t + 1) * (EXP_REL + 2 * U)
    delta = np.where(vis, delta, 0.0)
    g = gamma(nk + n_t + 2)
    av = np.abs(vd)
    Et = E * (1 + delta)
    rnd = np.where(vis, np.maximum(p_rel * Et, np.minimum(Et, p_sub)), 0.0)
    A = (rnd + delta * E) @ av
    dE = (delta * E).sum(axis=1)
    B = dE + g * (l + dE)
    C = g * (np.where(vis, Et * (1 + p_rel) + np.minimum(Et, p_sub), 0.0) @ av)
    err = (A + np.abs(o) * B[:, None] + C) / (l - B)[:, None] + 4 * U * np.abs(o)
    bound = err + BF16_REL * (np.abs(o) + err)
    lse_bound = B / (l - B) + 8 * U * (np.abs(lse) + 1)
    return o, lse, bound, lse_bound


def forward_bound(q8, q_scale, k8, k_scale, v8, v_scale, scale: float, causal: bool, heads=None, **kw):
    """head_bound over (B, H_q, N_q, d) codes with (B, H_q, ceil(N_q/128)) row-block scales,
    (B, H_kv, N_k, d) codes with row-block scales, and (B, H_kv, N_k, d) V codes with
    (B, H_kv, d) channel scales; query head h reads key/value head h // (H_q // H_kv).
    Returns (O, lse, O bound, lse bound); with ``heads`` only those (b, h) (others NaN)."""
    q8, k8, v8 = np.asarray(q8), np.asarray(k8), np.asarray(v8)
    B, H, nq, d = q8.shape
    Hkv, nk = k8.shape[1], k8.shape[2]
    G = H // Hkv
    qrow = np.repeat(np.asarray(q_scale, np.float64), fp8.BLOCK, axis=2)[:, :, :nq]
    krow = np.repeat(np.asarray(k_scale, np.float64), fp8.BLOCK, axis=2)[:, :, :nk]
    out = [np.full((B, H, nq, d), np.nan), np.full((B, H, nq), np.nan), np.full((B, H, nq, d), np.nan),
           np.full((B, H, nq), np.nan)]
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for b, h in todo:
        gh = h // G
        res = head_bound(q8[b, h], qrow[b, h], k8[b, gh], krow[b, gh], v8[b, gh], np.asarray(v_scale)[b, gh],
                         scale, causal, **kw)
        for arr, r in zip(out, res):
            arr[b, h] = r
    return tuple(out)


def simulate_head(q8, qs, k8, ks, v8, vs, scale: float, causal: bool, rng, bc: int = 64, p_round=None):
    """A CPU model of the kernel's arithmetic for testing the bound: fp32 code-product
    sums, an fp32 exponent per tile relative to the running max (updated every tile),
    exponentials with a random relative error up to 2^-22, probabilities rounded by
    ``p_round`` (E4M3 by default) for the numerator and summed unrounded in fp32 for the
    denominator, fp32 accumulation, bf16 output.  Returns (O, lse)."""
    p_round = p_round or fp8.e4m3_round
    dec = fp8.e4m3_decode()
    f = np.float32
    qc, kc, vc = (dec[np.asarray(a)].astype(f) for a in (q8, k8, v8))
    nq, d = qc.shape
    nk = kc.shape[0]
    c = f(f(scale) * f(LOG2E))
    off = nk - nq
    m = np.full(nq, -np.inf, f)
    lsum = np.zeros(nq, f)
    o = np.zeros((nq, vc.shape[1]), f)
    for j0 in range(0, nk, bc):
        t = (qc @ kc[j0:j0 + bc].T).astype(f)
        cs = (c * np.asarray(qs, f)[:, None] * np.asarray(ks, f)[None, j0:j0 + bc]).astype(f)
        if causal:
            keys = np.arange(j0, min(j0 + bc, nk))[None, :]
            t = np.where(keys > np.arange(nq)[:, None] + off, -np.inf, t).astype(f)
        mx = (t * cs).astype(f).max(axis=1)
        m_new = np.maximum(m, mx)
        with np.errstate(invalid="ignore"):
            alpha = np.where(np.isfinite(m), np.exp2(m - m_new) * (1 + EXP_REL * rng.uniform(-1, 1, nq)), 0.0)
        alpha = alpha.astype(f)
        mu = np.where(np.isfinite(m_new), m_new, 0.0).astype(f)
        x = (t * cs - mu[:, None]).astype(f)
        pt = (np.exp2(x.astype(np.float64)) * (1 + EXP_REL * rng.uniform(-1, 1, x.shape))).astype(f)
        lsum = (lsum * alpha + pt.sum(axis=1, dtype=f)).astype(f)
        pr = p_round(pt.astype(np.float64)).astype(f)
        o = (o * alpha[:, None] + pr @ vc[j0:j0 + bc]).astype(f)
        m = m_new
    out = (o / lsum[:, None] * np.asarray(vs, f)[None, :]).astype(f)
    import torch
    out = torch.from_numpy(out).to(torch.bfloat16).to(torch.float64).numpy()
    lse = (m.astype(np.float64) + np.log2(lsum.astype(np.float64))) * math.log(2)
    return out, lse
