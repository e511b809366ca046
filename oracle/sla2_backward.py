"""SLA2 backward — plain fp64 CPU oracle (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import, call or run
anything in this package. The GPU path shares no code with it and never calls it.

What it computes. The pages give the backward in one line each: the sparse branch is trained
with quantisation-aware training, low-bit forward and 16-bit backward, which the six-checks list
of "SLA2: Sparse-Linear Attention v2 for Diffusion Transformers" (§4, item 4) names the
straight-through estimator; and the gradient is derived by hand (§7 note 3, Appendix A
Algorithm 3, not reproduced on the pages) with the linear branch's dH_i, dZ_i computed first so
that the main loop needs one matrix addition. Readings taken here (each listed with its reason
in the design notes of the repository):

  * straight-through: the gradient is that of the unquantised forward, at the exact inputs;
    the fp32 roundings of colmean(K) and of K_s count as identities as well. So this module
    differentiates
        K_s = K - 1 mean_rows(K)^T                        (§7 note 1)
        O_s = softmax over the kept keys of Q K_s^T / sqrt(d), times V      (step 2)
        O_l = phi(Q_i) H_i / (phi(Q_i) Z_i),  H_i = sum_{j dropped} phi(K_s,j)^T V_j,
              Z_i = sum_{j dropped} column sums of phi(K_s,j)               (step 3)
        O   = alpha O_s + (1 - alpha) O_l, alpha per query block            (step 4)
    with the block mask held fixed (the hard Top-k router has no gradient; the router's
    training signal comes from SoftTop-k, a separate function);
  * an empty kept set gives O_s = 0 and an empty dropped set O_l = 0, as in the forward, and
    then no gradient flows through that branch for that query block;
  * outputs: dQ, dK, dV [N, d] and dalpha [N/128] (one value per query block of this slice).

The algorithm, written out in the order of the pages' description:
  sparse branch, per query block i with a kept set (FlashAttention-style recomputation of the
  row softmax P over the kept keys): dO_s = alpha_i dO, D = rowsum(dO_s * O_s),
  dP = dO_s V^T, dS = P * (dP - D), dQ += dS K_s / sqrt(d), dK_s += dS^T Q / sqrt(d),
  dV += P^T dO_s;
  linear branch, per query block i with a dropped set: with a = phi(Q_i), num = a H_i,
  den = a Z_i, O_l = num / den and dO_l = (1 - alpha_i) dO: dnum = dO_l / den,
  dden = -rowsum(dO_l * O_l) / den, da = dnum H_i^T + dden Z_i^T, dQ += a * (da - rowsum(da * a))
  (the Jacobian of the row softmax phi), dH_i = a^T dnum, dZ_i = a^T dden;
  then per key block j: dh_j = sum of dH_i over the query blocks that drop j, dz_j likewise,
  dV_j += phi(K_s,j) dh_j, dphi = V_j dh_j^T + 1 dz_j^T, dK_s,j += phi * (dphi - rowsum(dphi * phi));
  smoothing: dK = dK_s - 1 mean_rows(dK_s)^T;
  mixing: dalpha_i = sum over the rows of block i of dO * (O_s - O_l).

Pins (tests/test_oracle_backward.py, CPU): central finite differences of forward_exact along
random directions (every input, alpha included); torch autograd through an explicit N x N
construction of the same forward at tiny N; torch's scaled_dot_product_attention gradients when
every block is kept and alpha = 1, and with a boolean block mask for alpha = 1; the column sums
of dK vanish (the forward does not change when a constant row is added to K); alpha = 0 and
alpha = 1 switch the branches off.
"""

from __future__ import annotations

import math

import numpy as np

from .sla2 import BK, BQ, mask_to_lists, phi, softmax_rows


def _check(Q, K, V, mask, alpha_row):
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    N, d = Q.shape
    if N % BQ or N == 0:
        raise ValueError("N must be a positive multiple of 128")
    mask = (np.asarray(mask) != 0).astype(np.uint8)
    if mask.shape != (N // BQ, N // BK):
        raise ValueError("mask must be [N/128, N/64]")
    alpha_row = np.asarray(alpha_row, np.float64)
    return Q, K, V, mask, alpha_row


def _key_cols(L):
    return np.concatenate([np.arange(j * BK, (j + 1) * BK) for j in L])


def forward_exact(Q, K, V, mask, alpha_row):
    """The unquantised forward of one slice with a fixed block mask, all in fp64 and without
    fp32 roundings: the function whose gradient backward() returns. Returns (O, O_s, O_l)."""
    Q, K, V, mask, alpha_row = _check(Q, K, V, mask, alpha_row)
    N, d = Q.shape
    Ks = K - K.mean(axis=0)
    O_s = np.zeros((N, d))
    O_l = np.zeros((N, d))
    pk = phi(Ks).reshape(N // BK, BK, d)
    h = np.einsum("jra,jrb->jab", pk, V.reshape(N // BK, BK, d))
    z = pk.sum(axis=1)
    pq = phi(Q)
    for i, L in enumerate(mask_to_lists(mask)):
        rows = slice(i * BQ, (i + 1) * BQ)
        if len(L):
            cols = _key_cols(L)
            O_s[rows] = softmax_rows(Q[rows] @ Ks[cols].T / math.sqrt(d)) @ V[cols]
        drop = np.flatnonzero(mask[i] == 0)
        if len(drop):
            H, Z = h[drop].sum(axis=0), z[drop].sum(axis=0)
            O_l[rows] = (pq[rows] @ H) / (pq[rows] @ Z)[:, None]
    a = np.repeat(alpha_row, BQ)[:, None]
    return a * O_s + (1.0 - a) * O_l, O_s, O_l


def _softmax_vjp(p, dp):
    """Vector-Jacobian product of a row softmax p = softmax(x): dx = p * (dp - rowsum(dp p))."""
    return p * (dp - (dp * p).sum(axis=1, keepdims=True))


def backward(Q, K, V, mask, alpha_row, dO):
    """Gradients of sum(dO * O) for O = forward_exact(Q, K, V, mask, alpha_row).

    Returns a dict with dQ, dK, dV [N, d], dalpha [N/128] and the intermediates O_s, O_l,
    lse (row log-sum-exp of the scaled kept logits; -inf for a query block with no kept
    block), D (rowsum(dO_s * O_s)), dH [N/128, d, d], dZ [N/128, d]."""
    Q, K, V, mask, alpha_row = _check(Q, K, V, mask, alpha_row)
    dO = np.asarray(dO, np.float64)
    N, d = Q.shape
    n_qb, n_kb = N // BQ, N // BK
    c = 1.0 / math.sqrt(d)
    Ks = K - K.mean(axis=0)
    dQ = np.zeros((N, d))
    dKs = np.zeros((N, d))
    dV = np.zeros((N, d))
    O_s = np.zeros((N, d))
    O_l = np.zeros((N, d))
    lse = np.full(N, -np.inf)
    D = np.zeros(N)

    # sparse branch
    for i, L in enumerate(mask_to_lists(mask)):
        if len(L) == 0:
            continue
        rows = slice(i * BQ, (i + 1) * BQ)
        cols = _key_cols(L)
        S = Q[rows] @ Ks[cols].T * c
        m = S.max(axis=1, keepdims=True)
        lse[rows] = (m + np.log(np.exp(S - m).sum(axis=1, keepdims=True)))[:, 0]
        P = np.exp(S - lse[rows][:, None])
        O_s[rows] = P @ V[cols]
        dOs = alpha_row[i] * dO[rows]
        D[rows] = (dOs * O_s[rows]).sum(axis=1)
        dS = P * (dOs @ V[cols].T - D[rows][:, None])
        dQ[rows] += dS @ Ks[cols] * c
        dKs[cols] += dS.T @ Q[rows] * c
        dV[cols] += P.T @ dOs

    # linear branch: per query block, then per key block
    pk = phi(Ks).reshape(n_kb, BK, d)
    Vb = V.reshape(n_kb, BK, d)
    h = np.einsum("jra,jrb->jab", pk, Vb)
    z = pk.sum(axis=1)
    pq = phi(Q)
    dH = np.zeros((n_qb, d, d))
    dZ = np.zeros((n_qb, d))
    for i in range(n_qb):
        drop = np.flatnonzero(mask[i] == 0)
        if len(drop) == 0:
            continue
        rows = slice(i * BQ, (i + 1) * BQ)
        H, Z = h[drop].sum(axis=0), z[drop].sum(axis=0)
        a = pq[rows]
        num, den = a @ H, a @ Z
        O_l[rows] = num / den[:, None]
        dOl = (1.0 - alpha_row[i]) * dO[rows]
        dnum = dOl / den[:, None]
        dden = -(dOl * O_l[rows]).sum(axis=1) / den
        da = dnum @ H.T + dden[:, None] * Z[None, :]
        dQ[rows] += _softmax_vjp(a, da)
        dH[i] = a.T @ dnum
        dZ[i] = a.T @ dden
    # dh_j, dz_j: sums over the query blocks that drop key block j
    for j in range(n_kb):
        drop_j = np.flatnonzero(mask[:, j] == 0)
        dh = dH[drop_j].sum(axis=0)
        dz = dZ[drop_j].sum(axis=0)
        rk = slice(j * BK, (j + 1) * BK)
        dV[rk] += pk[j] @ dh
        dphi = Vb[j] @ dh.T + dz[None, :]
        dKs[rk] += _softmax_vjp(pk[j], dphi)

    dK = dKs - dKs.mean(axis=0)
    dalpha = (dO * (O_s - O_l)).reshape(n_qb, BQ * d).sum(axis=1)
    return dict(dQ=dQ, dK=dK, dV=dV, dalpha=dalpha, O_s=O_s, O_l=O_l, lse=lse, D=D,
                dH=dH, dZ=dZ)


def backward_spot(Q, K, V, mask, alpha_row, dO, qblocks, kblocks):
    """Some of backward()'s outputs at sizes where the full function is too slow: dQ and dalpha
    of the query blocks `qblocks`, dV of the key blocks `kblocks`. The same steps as backward(),
    restricted to what those outputs need, with the sums over a row's dropped blocks taken as the
    total minus the kept blocks (H_i = H_tot - sum_{j kept} h_j, Z_i likewise: the same sums, in
    another order). dV_j still needs dH_i of every query block that drops j, so the linear
    branch runs per query block over all of them; the sparse branch runs only for the query
    blocks in `qblocks` and those that keep a block in `kblocks`.

    Returns dict dQ {i: [128, d]}, dalpha {i: float}, dV {j: [64, d]}."""
    Q, K, V, mask, alpha_row = _check(Q, K, V, mask, alpha_row)
    dO = np.asarray(dO, np.float64)
    N, d = Q.shape
    n_qb, n_kb = N // BQ, N // BK
    c = 1.0 / math.sqrt(d)
    Ks = K - K.mean(axis=0)
    lists = mask_to_lists(mask)
    pk = phi(Ks).reshape(n_kb, BK, d)
    Vb = V.reshape(n_kb, BK, d)
    h = np.matmul(pk.transpose(0, 2, 1), Vb)            # h_j = phi(K_s,j)^T V_j
    z = pk.sum(axis=1)
    h_tot, z_tot = h.sum(axis=0), z.sum(axis=0)
    want_q = set(int(i) for i in qblocks)
    want_k = set(int(j) for j in kblocks)
    dQ = {i: np.zeros((BQ, d)) for i in want_q}
    dV = {j: np.zeros((BK, d)) for j in want_k}
    O_s, O_l = {}, {}
    # sparse branch
    for i, L in enumerate(lists):
        if len(L) == 0 or not (i in want_q or want_k.intersection(int(j) for j in L)):
            continue
        rows = slice(i * BQ, (i + 1) * BQ)
        cols = _key_cols(L)
        S = Q[rows] @ Ks[cols].T * c
        m = S.max(axis=1, keepdims=True)
        P = np.exp(S - m)
        P /= P.sum(axis=1, keepdims=True)
        Os = P @ V[cols]
        dOs = alpha_row[i] * dO[rows]
        if i in want_q:
            O_s[i] = Os
            D = (dOs * Os).sum(axis=1)
            dS = P * (dOs @ V[cols].T - D[:, None])
            dQ[i] += dS @ Ks[cols] * c
        for t, j in enumerate(L):
            if int(j) in want_k:
                dV[int(j)] += P[:, t * BK:(t + 1) * BK].T @ dOs
    # linear branch: every query block with a dropped set (dh_j needs all of them)
    pq = phi(Q)
    dH = np.zeros((n_qb, d, d))
    for i, L in enumerate(lists):
        if len(L) == n_kb:
            continue
        rows = slice(i * BQ, (i + 1) * BQ)
        H = h_tot - h[L].sum(axis=0)
        Z = z_tot - z[L].sum(axis=0)
        a = pq[rows]
        den = a @ Z
        Ol = (a @ H) / den[:, None]
        dOl = (1.0 - alpha_row[i]) * dO[rows]
        dnum = dOl / den[:, None]
        dH[i] = a.T @ dnum
        if i in want_q:
            O_l[i] = Ol
            dden = -(dOl * Ol).sum(axis=1) / den
            da = dnum @ H.T + dden[:, None] * Z[None, :]
            dQ[i] += _softmax_vjp(a, da)
    for j in want_k:
        drop_j = np.flatnonzero(mask[:, j] == 0)
        dV[j] += pk[j] @ dH[drop_j].sum(axis=0)
    dalpha = {}
    for i in want_q:
        rows = slice(i * BQ, (i + 1) * BQ)
        dalpha[i] = float((dO[rows] * (O_s.get(i, 0.0) - O_l.get(i, 0.0))).sum())
    return dict(dQ=dQ, dalpha=dalpha, dV=dV)
