"""Stage-1 alpha fitting — plain fp64 CPU oracle (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import, call or run
anything in this package. The GPU path shares no code with it and never calls it.

"SLA2: Sparse-Linear Attention v2 for Diffusion Transformers" fits the router and alpha in a
first stage with an MSE loss against full attention on Q/K/V tensors, and notes that alpha then
lands close to the kept row mass P_1 1 (§4 six checks item 5; §5 training table; §3 mixing
O = alpha O_s + (1 - alpha) O_l). Readings taken here (listed with their reasons in the design
notes of the repository):

  * the alpha part only, with the router held fixed: O is affine in alpha, so the MSE
    sum over the block's rows and all batches of |alpha O_s + (1 - alpha) O_l - O_full|^2 is a
    quadratic in each query block's alpha, minimised by
        alpha* = <O_full - O_l, O_s - O_l> / |O_s - O_l|^2
    (inner products over the 128 rows x d of the block, summed over the batch, since alpha is
    one value per head and query block);
  * alpha is kept in [0, 1] (the convex combination of §4 check 2): alpha* is clipped;
  * a block whose branches agree (|O_s - O_l| = 0) gets alpha = 1.
"""

from __future__ import annotations

import numpy as np

from oracle import sla2 as _f   # the forward's steps

BQ = 128


def fit_alpha(O_full, O_s, O_l):
    """alpha* per (head, query block) for [B, H, N, d] arrays; returns [H, N/128] (fp64)."""
    O_full = np.asarray(O_full, np.float64)
    O_s = np.asarray(O_s, np.float64)
    O_l = np.asarray(O_l, np.float64)
    B, H, N, d = O_s.shape
    diff = (O_s - O_l).reshape(B, H, N // BQ, BQ * d)
    res = (O_full - O_l).reshape(B, H, N // BQ, BQ * d)
    num = (res * diff).sum(axis=(0, 3))
    den = (diff * diff).sum(axis=(0, 3))
    alpha = np.ones((H, N // BQ))
    ok = den > 0
    alpha[ok] = num[ok] / den[ok]
    return np.clip(alpha, 0.0, 1.0)


def mse(alpha, O_full, O_s, O_l):
    """The stage-1 loss for a given alpha [H, N/128] (sum of squares over everything)."""
    a = np.repeat(np.asarray(alpha, np.float64), BQ, axis=1)[None, :, :, None]
    O = a * np.asarray(O_s, np.float64) + (1.0 - a) * np.asarray(O_l, np.float64)
    return float(((O - np.asarray(O_full, np.float64)) ** 2).sum())


# ----------------------------------------------------------------------------- router part
# Stage 1 also fits the router (proj_q, proj_k) with the same loss, and in training the hard
# Top-k is replaced by SoftTop-k so that gradients reach the router ("SLA2: Sparse-Linear
# Attention with Learnable Routing and QAT", summary page, novelty paragraph and step 1;
# "SLA2: Sparse-Linear Attention v2 for Diffusion Transformers", §4 Eq. 17, §5 training
# table, stage 1). The pages do not say how the soft mask enters the attention. Readings
# taken here:
#
#   * the mask relaxation: for a block mask M with entries in [0, 1], key block j of query
#     block i enters the sparse branch with weight M_ij on its exponentials and the linear
#     branch with weight 1 - M_ij on its h_j, z_j:
#         O_s = sum_k M_i,j(k) e^{S_qk} V_k / sum_k M_i,j(k) e^{S_qk}
#         O_l = phi(q) sum_j (1 - M_ij) h_j / phi(q) . sum_j (1 - M_ij) z_j
#     which is the method's own forward (softmax over the kept keys, linear attention over
#     the dropped blocks) when M is 0/1;
#   * straight-through: the forward uses the hard Top-k mask (the inference forward, without
#     quantisation: stage 1 precedes the quantisation-aware stage), and the gradient of the
#     loss with respect to the soft mask is taken to be dL/dM at the hard mask;
#   * the soft mask is SoftTop-k of the router's P_c with the hard rule's kept count (the
#     `soft_topk` reading); its gradient treats lambda_i as the function of P_c fixed by the
#     row-sum constraint (implicit differentiation);
#   * the loss is the sum of squares of O - O_full over all batches, heads, rows and columns,
#     and proj_q, proj_k are shared by the batch (their gradients are summed over it).

def relaxed_outputs(Q, Ks, V, M, alpha_row):
    """O_s, O_l and O of one (batch, head) slice for a block mask M [N/128, N/64] with entries
    in [0, 1] (the relaxation above). Q, Ks (the smoothed keys) and V are [N, d]."""
    Q = np.asarray(Q, np.float64)
    Ks = np.asarray(Ks, np.float64)
    V = np.asarray(V, np.float64)
    M = np.asarray(M, np.float64)
    N, d = Q.shape
    n_qb = N // BQ
    O_s = np.zeros((N, d))
    for i in range(n_qb):
        S = Q[i * BQ:(i + 1) * BQ] @ Ks.T / np.sqrt(d)
        E = np.exp(S - S.max(axis=1, keepdims=True))
        W = E * np.repeat(M[i], _f.BK)[None, :]
        l = W.sum(axis=1)
        O_s[i * BQ:(i + 1) * BQ] = np.where(l[:, None] > 0, (W @ V) / np.where(l > 0, l, 1.0)[:, None], 0.0)
    h, z = _f.linear_precompute(Ks, V)
    U = 1.0 - M
    H = np.einsum("ij,jab->iab", U, h)
    Z = U @ z
    pq = _f.phi(Q)
    O_l = np.zeros((N, d))
    for i in range(n_qb):
        if not U[i].any():
            continue
        p = pq[i * BQ:(i + 1) * BQ]
        O_l[i * BQ:(i + 1) * BQ] = (p @ H[i]) / (p @ Z[i])[:, None]
    O = _f.combine(O_s, O_l, alpha_row)
    return O_s, O_l, O


def relaxed_loss(Q, Ks, V, M, alpha_row, O_full):
    """sum of (O - O_full)^2 for the relaxed forward at mask M."""
    return float(((relaxed_outputs(Q, Ks, V, M, alpha_row)[2] - np.asarray(O_full, np.float64)) ** 2).sum())


def mask_grad(Q, Ks, V, M, alpha_row, O_full):
    """dL/dM [N/128, N/64] of L = sum (O - O_full)^2 through the relaxation, at mask M.

    With delta = 2 (O - O_full), per query row q of block i (row constants: l_q, the weighted
    sum of e^{S_qk}; den_q = phi(q) . Z_i; c_q = delta_q . O_s,q; c'_q = delta_q . O_l,q):
        sparse:  alpha_i sum_q sum_{k in j} e^{S_qk} (delta_q . V_k - c_q) / l_q
        linear: -(1 - alpha_i) sum_q [delta_q . (phi(q) h_j) - c'_q (phi(q) . z_j)] / den_q
    (the derivative of a ratio of two sums that are linear in M_ij; the linear part is zero
    for a query block with no dropped block, where O_l is defined as 0).
    """
    Q = np.asarray(Q, np.float64)
    Ks = np.asarray(Ks, np.float64)
    V = np.asarray(V, np.float64)
    M = np.asarray(M, np.float64)
    N, d = Q.shape
    n_qb, n_kb = M.shape
    O_s, O_l, O = relaxed_outputs(Q, Ks, V, M, alpha_row)
    delta = 2.0 * (O - np.asarray(O_full, np.float64))
    h, z = _f.linear_precompute(Ks, V)
    U = 1.0 - M
    Z = U @ z
    pq = _f.phi(Q)
    g = np.zeros((n_qb, n_kb))
    for i in range(n_qb):
        rows = slice(i * BQ, (i + 1) * BQ)
        dl = delta[rows]
        a = float(alpha_row[i])
        S = Q[rows] @ Ks.T / np.sqrt(d)
        E = np.exp(S - S.max(axis=1, keepdims=True))
        l = (E * np.repeat(M[i], _f.BK)[None, :]).sum(axis=1)
        if (l > 0).all():
            c = (dl * O_s[rows]).sum(axis=1)
            T = E * (dl @ V.T - c[:, None]) / l[:, None]
            g[i] += a * T.reshape(BQ, n_kb, _f.BK).sum(axis=(0, 2))
        if U[i].any():
            p = pq[rows]
            den = p @ Z[i]
            c2 = (dl * O_l[rows]).sum(axis=1)
            g[i] -= (1.0 - a) * _linear_part(p, den, dl, c2, h, z)
    return g


def mask_grad_rows(Q, Ks, V, M, alpha_row, O_full_rows):
    """Rows of mask_grad at sizes where the whole is too slow: O_full_rows maps query block i to
    the target's rows [128, d] of that block; returns {i: dL/dM[i, :]}. The same steps as
    mask_grad (relaxed forward, delta, the two parts), for those query blocks only: a row of the
    derivative depends only on its own block's outputs and mask row and on the per-key-block
    h_j, z_j."""
    Q = np.asarray(Q, np.float64)
    Ks = np.asarray(Ks, np.float64)
    V = np.asarray(V, np.float64)
    M = np.asarray(M, np.float64)
    N, d = Q.shape
    h, z = _f.linear_precompute(Ks, V)
    out = {}
    for i, target in O_full_rows.items():
        rows = slice(i * BQ, (i + 1) * BQ)
        a = float(alpha_row[i])
        S = Q[rows] @ Ks.T / np.sqrt(d)
        E = np.exp(S - S.max(axis=1, keepdims=True))
        W = E * np.repeat(M[i], _f.BK)[None, :]
        l = W.sum(axis=1)
        O_s = (W @ V) / l[:, None] if (l > 0).all() else np.zeros((BQ, d))
        U = 1.0 - M[i]
        p = _f.phi(Q[rows])
        O_l = np.zeros((BQ, d))
        if U.any():
            H = np.einsum("j,jab->ab", U, h)
            Z = U @ z
            den = p @ Z
            O_l = (p @ H) / den[:, None]
        dl = 2.0 * (a * O_s + (1.0 - a) * O_l - np.asarray(target, np.float64))
        g = np.zeros(M.shape[1])
        if (l > 0).all():
            c = (dl * O_s).sum(axis=1)
            T = E * (dl @ V.T - c[:, None]) / l[:, None]
            g += a * T.reshape(BQ, M.shape[1], _f.BK).sum(axis=(0, 2))
        if U.any():
            c2 = (dl * O_l).sum(axis=1)
            g -= (1.0 - a) * _linear_part(p, den, dl, c2, h, z)
        out[i] = g
    return out


def full_attention_rows(Q, K, V, blocks):
    """Rows of full_attention_head for the query blocks in `blocks`: {i: [128, d]}."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    out = {}
    for i in blocks:
        S = Q[i * BQ:(i + 1) * BQ] @ K.T / np.sqrt(Q.shape[1])
        out[i] = _f.softmax_rows(S) @ np.asarray(V, np.float64)
    return out


def _linear_part(p, den, dl, c2, h, z):
    """sum_q [delta_q . (phi(q) h_j) - c'_q (phi(q) . z_j)] / den_q for every block j."""
    first = np.einsum("qa,jab,qb->j", p / den[:, None], h, dl)
    second = np.einsum("q,qa,ja->j", c2 / den, p, z)
    return first - second


def soft_topk_vjp(soft, tau, g):
    """dL/dP_c from dL/dsoft for soft = sigma(P_c / tau + lambda(P_c)), lambda_i fixed by
    sum_j soft_ij = kb: with s' = soft (1 - soft),
        dL/dP_ij = s'_ij (g_ij - sum_j' s'_ij' g_ij' / sum_j' s'_ij') / tau
    (a row with sum s' = 0, e.g. every block kept, gets 0)."""
    soft = np.asarray(soft, np.float64)
    g = np.asarray(g, np.float64)
    sp = soft * (1.0 - soft)
    tot = sp.sum(axis=1, keepdims=True)
    centre = np.divide((sp * g).sum(axis=1, keepdims=True), tot, out=np.zeros_like(tot), where=tot > 0)
    return sp * (g - centre) / float(tau)


def router_vjp(Qbar, Kbar, Wq, Wk, dP):
    """dL/dWq, dL/dWk from dL/dP_c for P_c = row softmax((Qbar Wq)(Kbar Wk)^T / sqrt(d))."""
    Qbar = np.asarray(Qbar, np.float64)
    Kbar = np.asarray(Kbar, np.float64)
    d = Qbar.shape[1]
    A = Qbar @ np.asarray(Wq, np.float64)
    Bm = Kbar @ np.asarray(Wk, np.float64)
    _, P = _f.router_scores(Qbar, Kbar, Wq, Wk)
    dP = np.asarray(dP, np.float64)
    dG = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    dA = dG @ Bm / np.sqrt(d)
    dB = dG.T @ A / np.sqrt(d)
    return Qbar.T @ dA, Kbar.T @ dB


def router_grad_head(Q, K, V, Wq, Wk, alpha_row, keep_frac, tau, O_full, straight_through=True):
    """Stage-1 router gradient of one (batch, head) slice: the loss and dL/dWq, dL/dWk.

    straight_through=True is the reading above (hard mask in the forward, its gradient
    passed to the soft mask). straight_through=False evaluates the forward and dL/dM at the
    soft mask itself: the exact gradient of the smooth loss L(M_soft(Wq, Wk)), which the
    tests compare with finite differences to pin the chain of derivatives.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    N, d = Q.shape
    mu, mu32 = _f.colmean(K)
    Ks = _f.smooth_k(K, mu32)
    Qbar = _f.block_mean(Q, BQ)
    Kbar = _f.block_mean(Ks, _f.BK)
    G, P = _f.router_scores(Qbar, Kbar, Wq, Wk)
    kb = _f.kept_blocks(N // _f.BK, keep_frac)
    mask, _ = _f.topk_blocks(P, kb)
    soft, lam = _f.soft_topk(P, kb, tau)
    M = mask.astype(np.float64) if straight_through else soft
    O_s, O_l, O = relaxed_outputs(Q, Ks, V, M, alpha_row)
    loss = float(((O - np.asarray(O_full, np.float64)) ** 2).sum())
    g = mask_grad(Q, Ks, V, M, alpha_row, O_full)
    dP = soft_topk_vjp(soft, tau, g)
    dWq, dWk = router_vjp(Qbar, Kbar, Wq, Wk, dP)
    return dict(loss=loss, mask_grad=g, dP=dP, dWq=dWq, dWk=dWk, mask=mask, soft=soft,
                lam=lam, P_c=P, kb=kb, O=O, O_s=O_s, O_l=O_l, Ks=Ks, Qbar=Qbar, Kbar=Kbar)


def full_attention_head(Q, K, V):
    """The stage-1 target: dense softmax attention softmax(Q K^T / sqrt(d)) V of one slice
    (fp64; K is not smoothed here, the softmax is invariant to the column mean)."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    S = Q @ K.T / np.sqrt(Q.shape[1])
    return _f.softmax_rows(S) @ np.asarray(V, np.float64)
