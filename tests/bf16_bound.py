"""Per-element error bound of the bf16 kernels against exact attention.

Exactness is what the method promises ("IO-4 FlashAttention" note, problem setup;
DSBA seminar review: exact attention, no approximation), so every difference
between a kernel's output and the fp64 oracle comes from the kernels' own
roundings, which are documented and fixed:

  * scores S = Q K^T from exact bf16 products summed in fp32, scaled and shifted
    by one fma, exponentiated by exp2 (about 1 ulp);
  * the probabilities P are rounded to bf16 (unit roundoff u = 2^-8) before the
    P V product, and the forward's row sum is taken over exactly those values;
  * O is accumulated in fp32 over the keys and rounded to bf16 once;
  * the backward recomputes P in fp32 from the forward's LSE (whose error scales
    every P of its row), forms D = rowsum(dO o O) in fp32 from the bf16 O, dP =
    dO V^T in fp32, dS = P (dP - D) rounded to bf16, and sums dQ, dK, dV in fp32;
    the key side also rounds P to bf16 for its dV product.

First-order propagation.  Let e_ij be the bf16 rounding of the forward's P_ij,
rho_ik that of O_ik, r_ij that of dS_ij and p_ij that of the key side's P_ij (all
relative, |.| <= u), and write dev_ij = dP_ij - D_i.  Then
  dO_ik   = sum_j P_ij e_ij (v_jk - O_ik)                      (+ rho_ik O_ik, once)
  dLSE_i  = sum_j P_ij e_ij
  dD_i    = sum_j P_ij e_ij dev_ij + sum_k dO_ik O_ik rho_ik
  ddS_ij  = -P_ij (dLSE_i dev_ij + dD_i) + r_ij dS_ij
  ddQ_ik  = scale sum_j ddS_ij K_jk,  ddK_jk = scale sum_i ddS_ij Q_ik,
  ddV_jk  = sum_i P_ij (p_ij - dLSE_i) dO_ik,
so every output error is one linear form  sum_t a_t x_t  in the independent
rounding variables x_t.  The bound treats them as independent, mean-zero and
bounded by u (the model of probabilistic rounding-error analysis, Higham and
Mary, SIAM J. Sci. Comput. 41(5), 2019): by Hoeffding's inequality the form
exceeds  LAMBDA * u * sqrt(sum_t a_t^2)  with probability at most
2 exp(-LAMBDA^2 / 2), about 2.5e-14 per element at LAMBDA = 8.  The sums of
squares are evaluated in closed form below.  The final bf16 rounding of an output,
the fp32 sums (n 2^-24 sum of |terms|) and the fp32 score/exponent arguments are
added in full, worst case.  Everything comes from the oracle's exact P, O, LSE and
plain magnitudes, so the bound scales with the values: a sharper softmax gives
larger gradients and a proportionally larger bound.
"""
import numpy as np

import oracle

U = 2.0 ** -8       # bf16 unit roundoff (8-bit significand, round to nearest even)
W = 2.0 ** -24      # fp32 unit roundoff
LAMBDA = 8.0
LN2 = np.log(2.0)
LOG2E = 1.0 / LN2


def _f64(t):
    return t.detach().cpu().double().numpy() if hasattr(t, "detach") else np.asarray(t, dtype=np.float64)


def _hoeffding(sum_sq):
    return LAMBDA * U * np.sqrt(np.maximum(sum_sq, 0.0))


def bounds(q, k, v, do=None, scale=None, causal=False, grad_bf16=False):
    """One head ([N, d] each).  Returns a dict of bounds shaped like the outputs:
    O, LSE (and dQ, dK, dV when do is given)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape
    if scale is None:
        scale = oracle.default_scale(d)
    sc = abs(scale)
    O, L, P = oracle.fwd_probs(q, k, v, scale=scale, causal=causal)
    seen = P > 0.0
    c = sc * LOG2E                               # the kernels' log2-domain scale
    s = scale * (q @ k.T)                        # exact scores
    qk_abs = np.abs(q) @ np.abs(k).T             # sum_k |q_ik k_jk|
    m = np.where(seen, s, -np.inf).max(axis=1, keepdims=True) * LOG2E
    g_n = N * W                                  # fp32 sums of up to N terms (worst case)
    absv, absO = np.abs(v), np.abs(O)
    P2 = P * P
    a = P2.sum(axis=1)                           # sum_j P_ij^2: dLSE_i's sum of squares / u^2
    # worst-case relative error of one p from its fp32 argument (score sum, fma, exp2)
    d_arg = np.where(seen, LN2 * (c * d * W * qk_abs + 2 * W * (np.abs(s) * LOG2E + np.abs(m))) + 2 * W, 0.0)
    Pd = P * d_arg

    ss_o = P2 @ (v * v) - 2 * O * (P2 @ v) + O * O * a[:, None]
    small_o = Pd @ absv + absO * Pd.sum(axis=1, keepdims=True) + g_n * (P @ absv + absO) + 6 * W * absO
    bO = np.minimum(_hoeffding(ss_o), U * (P @ absv + absO)) + small_o
    bO = bO * (1 + U) + U * absO                                  # + the final bf16 rounding of O
    small_l = Pd.sum(axis=1) + g_n + 3 * W * (np.abs(L) + 1.0)
    bL = np.minimum(_hoeffding(a), U) + small_l
    bL = -np.log1p(-np.minimum(bL, 0.5))
    out = {"O": bO, "LSE": bL}
    if do is None:
        return out

    do = _f64(do)
    absdo, absq, absk = np.abs(do), np.abs(q), np.abs(k)
    dP = do @ v.T
    D = (P * dP).sum(axis=1)
    dev = dP - D[:, None]
    dS = P * dev
    absdS = np.abs(dS)
    A = ((do * O) ** 2).sum(axis=1)              # D's O roundings: sum_k (dO_ik O_ik)^2
    b = (P2 * dev).sum(axis=1)
    cc = (P2 * dev * dev).sum(axis=1)
    # sum over the forward roundings e_ij' of row i of (P_ij' (dev_ij + dev_ij'))^2
    F = dev * dev * a[:, None] + 2 * dev * b[:, None] + cc[:, None]
    PK = P @ k
    dSK = dS @ k
    # worst-case parts: the fp32 argument of the recomputed P, dP's and D's fp32 sums, LSE's own fp32 error
    d_arg_b = np.where(seen, LN2 * (c * d * W * qk_abs + 2 * W * (np.abs(s) + np.abs(L)[:, None]) * LOG2E) + 2 * W,
                       0.0)
    e_small = (np.exp(small_l) - 1)[:, None] + d_arg_b
    bdP = d * W * (absdo @ absv.T)
    bD_small = d * W * (absdo * absO).sum(axis=1) + (Pd * np.abs(dev)).sum(axis=1)
    ds_small = P * (e_small * np.abs(dev) + bdP + bD_small[:, None])
    ds_mag = absdS + P * U * (np.abs(dev) * np.sqrt(a)[:, None] + np.sqrt(A + cc)[:, None]) * LAMBDA + ds_small

    ss_dq = (dS * dS) @ (k * k) + PK * PK * A[:, None] + dSK * dSK * a[:, None] + 2 * dSK * PK * b[:, None] \
        + PK * PK * cc[:, None]
    bdQ = sc * (_hoeffding(ss_dq) + ds_small @ absk + g_n * (ds_mag @ absk)) + W * sc * np.abs(dSK)
    ss_dk = (dS * dS).T @ (q * q) + (P2 * A[:, None]).T @ (q * q) + (P2 * F).T @ (q * q)
    bdK = sc * (_hoeffding(ss_dk) + ds_small.T @ absq + g_n * (ds_mag.T @ absq)) + W * sc * np.abs(dS.T @ q)
    ss_dv = (P2 * (1.0 + a[:, None])).T @ (do * do)
    bdV = _hoeffding(ss_dv) + (P * e_small).T @ absdo + g_n * (P.T @ absdo) * (1 + 2 * U)
    if grad_bf16:
        dV = P.T @ do
        bdQ = bdQ + U * (sc * np.abs(dSK) + bdQ)
        bdK = bdK + U * (sc * np.abs(dS.T @ q) + bdK)
        bdV = bdV + U * (np.abs(dV) + bdV)
    out.update(dQ=bdQ, dK=bdK, dV=bdV)
    return out
