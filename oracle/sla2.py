"""SLA2 inference forward — plain fp64 CPU oracle (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import,
call or run anything in this package. The GPU path (the HIP library and its
Python binding) shares no code with it and never calls it.

What it computes, per (batch, head) slice with Q, K, V in R^{N x d}, following
the summary page "SLA2: Sparse-Linear Attention with Learnable Routing and QAT"
(paper.rainbus.top, computation-flow paragraph, steps 1-4) and the page "SLA2:
Sparse-Linear Attention v2 for Diffusion Transformers" (zhaifeiyue.github.io;
§3 method flowchart, §4 symbol table and Eq. 9/11, §7 implementation notes):

  0. K smoothing: K_s = K - colmean(K) at the start of the forward (§7 note 1).
  1. Router: mean-pool Q in blocks of b_q = 128 rows and K_s in blocks of
     b_k = 64 rows; P_c = softmax(proj_q(Qbar) proj_k(Kbar)^T / sqrt(d)) per
     row; hard Top-k keeps the top k% key blocks of each row -> M_c (step 1).
  2. Sparse branch on the kept block pairs, FlashAttention style, with INT8
     Q, K and FP8 P, V (step 2).
  3. Linear branch on the dropped pairs with phi = softmax over the head dim
     (§4 symbol table): h_j = phi(K_j)^T V_j, z_j = column sums of phi(K_j),
     O_l = phi(Q_i) H_i / (phi(Q_i) Z_i) with H_i, Z_i summed over the dropped
     key blocks of query block i (step 3; §7 note 2).
  4. O = alpha * O_s + (1 - alpha) * O_l with one alpha per query block (step 4).
  Comparison workload (forward_head_sla1): the earlier SLA mix O = O_s + O_l Wo with the
     heuristic router (proj = I), §2 Q2 table of the second page.
  Training-time router (soft_topk): sigma(P_c / tau + lambda_i) with lambda_i set by
     bisection so that each row sums to kb (§4 Eq. 17 of the second page).

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * masked logits are -inf (softmax over the kept keys only), the only reading
    consistent with P_s = P_1 / alpha (§4 symbol table, Eq. 9);
  * kb = max(1, floor(k * N_kb + 1e-9)) kept blocks per row, k taken as fp32;
  * ties in P_c go to the lower key-block index; kept lists are ascending;
  * proj_q / proj_k are applied as x @ W (W[in][out]), no bias, one pair per head;
  * the router pools the smoothed K; mu = colmean over all N rows in fp64,
    rounded to fp32; K_s = fl32(K - mu32); Q is not smoothed;
  * INT8 per 128-row Q block and per 64-row K_s block; E4M3 per 64-row V block;
    P encoded as E4M3(448 * P~) with P~ = exp(S - m) against the running max m
    updated once per 64-key block in ascending order; l sums the unquantised P~;
  * empty kept set -> O_s = 0; empty dropped set -> O_l = 0;
  * alpha is used as given (no sigmoid); non-causal, padding rows are ordinary.

Pins (tests/test_oracle_*.py, all CPU): full softmax attention at k = 100%,
alpha = 1 without quantisation (against torch's scaled_dot_product_attention);
an explicit N x N masked construction at tiny N (against torch's boolean-mask
attention); rows of alpha P_s + (1 - alpha) P_l sum to 1; the linear branch
against the explicit normalised phi(Q) phi(K_s)^T (1 - M) V product; Eq. 9;
top-k against a brute-force rank count with planted ties; the proj = I special
case (the heuristic router) against torch pooling; smoothing invariance; the
online loop with identity codecs against the exact masked softmax; the codecs
(see codecs.py).

The quantised sparse branch (the codecs inside the online loop) is pinned by a
closed form of that loop, rebuilt densely in torch with its own float8_e4m3fn
and INT8 codes (tests/test_oracle_quantised.py): block b's P encoded against the
running maximum M_b, rescaled by e^(M_b - M), over 448 times the sum of the
unquantised exp(S - M); planted mistakes (the normaliser over the quantised P,
P against the final maximum, no rescale, no factor 448) each fail it. No page
prints a worked value or an error bound for the quantised result, so what the
pins fix is the composition the readings above state, not a number the pages
give.
"""

from __future__ import annotations

import math

import numpy as np

from . import codecs

BQ = 128   # query block rows (b_q)
BK = 64    # key block rows (b_k)


# ----------------------------------------------------------------------------- helpers
def kept_blocks(n_kb: int, keep_frac: float) -> int:
    """Number of kept key blocks per query block for a kept fraction k (taken as fp32)."""
    k = float(np.float32(keep_frac))
    if not (0.0 < k <= 1.0):
        raise ValueError("keep_frac must lie in (0, 1]")
    return max(1, min(n_kb, int(math.floor(k * n_kb + 1e-9))))


def softmax_rows(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def block_mean(x: np.ndarray, rows: int) -> np.ndarray:
    """Arithmetic mean of each block of `rows` consecutive rows (mean pooling, step 1)."""
    n, d = x.shape
    return np.asarray(x, dtype=np.float64).reshape(n // rows, rows, d).mean(axis=1)


# ----------------------------------------------------------------------------- step 0
def colmean(K: np.ndarray):
    """Column mean of K over all N rows, fp64, and its fp32 rounding (§7 note 1)."""
    mu = np.asarray(K, dtype=np.float64).mean(axis=0)
    return mu, mu.astype(np.float32)


def smooth_k(K: np.ndarray, mu32: np.ndarray) -> np.ndarray:
    """K_s = fl32(K - mu32), returned as float64 holding fp32 values."""
    return (np.asarray(K, dtype=np.float32) - mu32).astype(np.float64)


# ----------------------------------------------------------------------------- step 1
def router_scores(Qbar, Kbar, Wq, Wk):
    """Logits G = (Qbar Wq)(Kbar Wk)^T / sqrt(d) and P_c = row softmax(G)."""
    d = Qbar.shape[1]
    A = np.asarray(Qbar, np.float64) @ np.asarray(Wq, np.float64)
    Bm = np.asarray(Kbar, np.float64) @ np.asarray(Wk, np.float64)
    G = (A @ Bm.T) / math.sqrt(d)
    return G, softmax_rows(G)


def topk_blocks(P: np.ndarray, kb: int):
    """Hard Top-k per row: kb largest entries, ties to the lower index; lists ascending.

    Returns (mask uint8 [n_qb, n_kb], lists int32 [n_qb, kb]).
    """
    n_qb, n_kb = P.shape
    mask = np.zeros((n_qb, n_kb), dtype=np.uint8)
    lists = np.zeros((n_qb, kb), dtype=np.int32)
    for i in range(n_qb):
        row = P[i]
        order = sorted(range(n_kb), key=lambda j: (-row[j], j))
        chosen = sorted(order[:kb])
        lists[i] = chosen
        mask[i, chosen] = 1
    return mask, lists


def soft_topk(P: np.ndarray, kb: int, tau: float = 0.1, iters: int = 200):
    """SoftTop-k of the router (training time): soft mask sigma(P_ij / tau + lambda_i), with
    lambda_i the root of sum_j sigma(P_ij / tau + lambda_i) = kb found by bisection
    ("SLA2: Sparse-Linear Attention v2 for Diffusion Transformers", §4 Eq. 17 and the
    six-checks item 3; summary page, step 1).

    Reading: the row sum is kb, the kept count of the hard rule (kept_blocks), so that the
    soft mask tends to the hard Top-k mask as tau -> 0. The root lies in the bracket
    [L - max_j x_j, L - min_j x_j] with x = P / tau and L = log(kb / (n_kb - kb)): there
    every term is at most (resp. at least) kb / n_kb. Bisection halves the bracket until it
    stops shrinking in fp64 (or `iters` steps). kb = n_kb gives a mask of ones and
    lambda = +inf.

    Returns (soft mask [n_qb, n_kb] fp64, lambda [n_qb] fp64).
    """
    P = np.asarray(P, np.float64)
    n_qb, n_kb = P.shape
    if kb >= n_kb:
        return np.ones_like(P), np.full(n_qb, np.inf)
    x = P / float(tau)
    L = math.log(kb / (n_kb - kb))
    lam = np.empty(n_qb)
    for i in range(n_qb):
        lo, hi = L - x[i].max(), L - x[i].min()
        with np.errstate(over="ignore"):   # exp overflow -> a term of exactly 0
            for _ in range(iters):
                mid = 0.5 * (lo + hi)
                if mid <= lo or mid >= hi:
                    break
                if (1.0 / (1.0 + np.exp(-(x[i] + mid)))).sum() < kb:
                    lo = mid
                else:
                    hi = mid
        lam[i] = 0.5 * (lo + hi)
    with np.errstate(over="ignore"):
        soft = 1.0 / (1.0 + np.exp(-(x + lam[:, None])))
    return soft, lam


def mask_to_lists(mask: np.ndarray):
    """Ascending kept list of every row of a block mask (any 0/1 pattern)."""
    return [np.flatnonzero(np.asarray(r) != 0).astype(np.int32) for r in mask]


# ----------------------------------------------------------------------------- step 2
def sparse_exact(Q, Ks, V, lists):
    """Unquantised sparse branch: softmax over the kept keys only (masked logits = -inf)."""
    N, d = Q.shape
    out = np.zeros((N, d))
    for i, L in enumerate(lists):
        if len(L) == 0:
            continue
        cols = np.concatenate([np.arange(j * BK, (j + 1) * BK) for j in L])
        S = Q[i * BQ:(i + 1) * BQ] @ Ks[cols].T / math.sqrt(d)
        out[i * BQ:(i + 1) * BQ] = softmax_rows(S) @ V[cols]
    return out


def quantise_operands(Q, Ks, V, qk_quant=True, pv_quant=True):
    """Codes and per-block scales of Q (128 rows), K_s (64 rows) and V (64 rows).

    With a codec switched off the "codes" are the fp64 values and the scales 1.
    """
    N, d = Q.shape
    if qk_quant:
        qc, sq = codecs.int8_block_quant(Q.astype(np.float32), BQ)
        kc, sk = codecs.int8_block_quant(Ks.astype(np.float32), BK)
        qv, kv = qc.astype(np.float64), kc.astype(np.float64)
    else:
        qv, kv = np.asarray(Q, np.float64), np.asarray(Ks, np.float64)
        sq, sk = np.ones(N // BQ, np.float32), np.ones(N // BK, np.float32)
        qc = kc = None
    if pv_quant:
        vc, sv = codecs.fp8_block_quant(V.astype(np.float32), BK)
        vv = codecs.e4m3_decode(vc)
    else:
        vv = np.asarray(V, np.float64)
        sv = np.ones(N // BK, np.float32)
        vc = None
    return dict(q_codes=qc, k_codes=kc, v_codes=vc, s_q=sq, s_k=sk, s_v=sv,
                q_val=qv, k_val=kv, v_val=vv)


def sparse_online(ops, lists, d, p_quant=True):
    """FlashAttention-style loop over each query block's kept key blocks, ascending.

    Per kept block j: S = (Qhat_i Khat_j^T) s_q s_k / sqrt(d); running max m is
    raised to the block's row max; P~ = exp(S - m); l = l e^(m_old - m) + sum P~;
    Phat = E4M3(448 P~); acc = acc e^(m_old - m) + (Phat Vhat_j) s_v / 448.
    O_s = acc / l, or 0 for an empty list.
    """
    qv, kv, vv = ops["q_val"], ops["k_val"], ops["v_val"]
    sq, sk, sv = ops["s_q"], ops["s_k"], ops["s_v"]
    N = qv.shape[0]
    out = np.zeros((N, d))
    for i, L in enumerate(lists):
        if len(L) == 0:
            continue
        qi = qv[i * BQ:(i + 1) * BQ]
        m = np.full(BQ, -np.inf)
        l = np.zeros(BQ)
        acc = np.zeros((BQ, d))
        for j in L:
            kj = kv[j * BK:(j + 1) * BK]
            vj = vv[j * BK:(j + 1) * BK]
            S = (qi @ kj.T) * (float(sq[i]) * float(sk[j])) / math.sqrt(d)
            m_new = np.maximum(m, S.max(axis=1))
            corr = np.exp(m - m_new)                      # 0 on the first block (m = -inf)
            Pt = np.exp(S - m_new[:, None])
            l = l * corr + Pt.sum(axis=1)
            if p_quant:
                Ph = codecs.e4m3_round(448.0 * Pt)
            else:
                Ph = 448.0 * Pt
            acc = acc * corr[:, None] + (Ph @ vj) * (float(sv[j]) / 448.0)
            m = m_new
        out[i * BQ:(i + 1) * BQ] = acc / l[:, None]
    return out


# ----------------------------------------------------------------------------- step 3
def phi(x):
    """Linear-attention feature map: softmax over the head dimension of each row."""
    return softmax_rows(x)


def linear_precompute(Ks, V):
    """h_j = phi(K_s,j)^T V_j [n_kb, d, d] and z_j = column sums of phi(K_s,j) [n_kb, d]."""
    N, d = Ks.shape
    pk = phi(Ks).reshape(N // BK, BK, d)
    vb = np.asarray(V, np.float64).reshape(N // BK, BK, d)
    h = np.einsum("jra,jrb->jab", pk, vb)
    z = pk.sum(axis=1)
    return h, z


def linear_branch(Q, Ks, V, mask):
    """O_l from the dropped blocks: a direct sum of h_j, z_j over M_c = 0, then
    O_l = phi(q) H_i / (phi(q) . Z_i); rows of a query block with no dropped block get 0."""
    N, d = Q.shape
    n_qb = N // BQ
    h, z = linear_precompute(Ks, V)
    U = 1.0 - np.asarray(mask, np.float64)                 # dropped blocks
    H = (U @ h.reshape(h.shape[0], d * d)).reshape(n_qb, d, d)
    Z = U @ z
    pq = phi(Q)
    out = np.zeros((N, d))
    for i in range(n_qb):
        if not U[i].any():
            continue
        pqi = pq[i * BQ:(i + 1) * BQ]
        out[i * BQ:(i + 1) * BQ] = (pqi @ H[i]) / (pqi @ Z[i])[:, None]
    return out, h, z


# ----------------------------------------------------------------------------- step 4
def combine(O_s, O_l, alpha_row):
    """O = alpha O_s + (1 - alpha) O_l, alpha given per query block."""
    a = np.repeat(np.asarray(alpha_row, np.float64), BQ)[:, None]
    return a * O_s + (1.0 - a) * O_l


# ----------------------------------------------------------------------------- whole forward
def forward_head(Q, K, V, Wq, Wk, alpha_row, keep_frac, quant=True, mask=None):
    """SLA2 forward of one (batch, head) slice; returns every intermediate in a dict.

    Q, K, V: [N, d] arrays holding the exact input values. Wq, Wk: [d, d].
    alpha_row: [N/128]. With `mask` given ([N/128, N/64] 0/1) the router is skipped.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    N, d = Q.shape
    if N % BQ or N == 0:
        raise ValueError("N must be a positive multiple of 128")
    mu, mu32 = colmean(K)
    Ks = smooth_k(K, mu32)
    res = dict(mu=mu, mu32=mu32)
    if mask is None:
        Qbar = block_mean(Q, BQ)
        Kbar = block_mean(Ks, BK)
        G, P = router_scores(Qbar, Kbar, Wq, Wk)
        kb = kept_blocks(N // BK, keep_frac)
        mask, lists_arr = topk_blocks(P, kb)
        lists = list(lists_arr)
        res.update(Qbar=Qbar, Kbar=Kbar, G=G, P_c=P, kb=kb, lists=lists_arr)
    else:
        mask = (np.asarray(mask) != 0).astype(np.uint8)
        lists = mask_to_lists(mask)
    res["mask"] = mask
    ops = quantise_operands(Q, Ks, V, qk_quant=quant, pv_quant=quant)
    O_s = sparse_online(ops, lists, d, p_quant=quant)
    O_l, h, z = linear_branch(Q, Ks, V, mask)
    O = combine(O_s, O_l, alpha_row)
    res.update(ops=ops, O_s=O_s, O_l=O_l, O=O, h=h, z=z, Ks=Ks)
    return res


def forward_head_sla1(Q, K, V, Wo, keep_frac, quant=True, mask=None):
    """The earlier SLA formulation as a comparison workload, one (batch, head) slice
    ("SLA2: Sparse-Linear Attention v2 for Diffusion Transformers", §2 Q2 before/after table):
    the heuristic router softmax(Qbar Kbar^T / sqrt(d)) -> Top-k (the learnable router with
    proj_q = proj_k = I) and the mix O = O_s + Proj(O_l) with one d x d projection,
    Proj(x) = x @ Wo (no bias, no alpha). The branches are the same as in forward_head.
    """
    eye = np.eye(np.shape(Q)[1])
    res = forward_head(Q, K, V, eye, eye, np.ones(np.shape(Q)[0] // BQ), keep_frac, quant, mask)
    res["O"] = res["O_s"] + res["O_l"] @ np.asarray(Wo, np.float64)
    return res


def forward(Q, K, V, Wq, Wk, alpha, keep_frac, quant=True, mask=None, keep=("O",)):
    """Batched wrapper: Q, K, V [B, H, N, d]; Wq, Wk [H, d, d]; alpha [H, N/128];
    mask optional [B, H, N/128, N/64]. Returns a dict of stacked outputs named in `keep`."""
    B, H = Q.shape[:2]
    out = {}
    for b in range(B):
        for h in range(H):
            r = forward_head(Q[b, h], K[b, h], V[b, h], Wq[h], Wk[h], alpha[h], keep_frac,
                             quant, None if mask is None else mask[b, h])
            for name in keep:
                out.setdefault(name, []).append(r[name])
    return {k: np.stack(v).reshape((B, H) + np.shape(v[0])) for k, v in out.items()}
