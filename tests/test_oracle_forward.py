"""Pins of the oracle's forward against what the pages and the mathematics fix (CPU).

Each test checks the oracle against something other than itself: torch's own
attention kernels, dense N x N constructions of the pages' formulas (the
flowchart's masked softmax and norm(phi(Q) phi(K)^T (1-M)) V), brute force,
identities of §4 (Eq. 9, row normalisation of Eq. 11) and invariances.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_linear_pool_amd import workloads as W
from oracle import sla2

D = 128


def slice_inputs(seed=11, N=1024, bias=1.0, scale=1.0):
    q, k, v = W.random_qkv(seed, 1, 1, N, bias=bias, scale=scale)
    wq, wk, a = W.random_weights(seed, 1, N // 128)
    return q[0, 0].astype(np.float64), k[0, 0].astype(np.float64), v[0, 0].astype(np.float64), \
        wq[0], wk[0], a[0]


def token_mask(mask_c, N):
    """M[r, c] = M_c[r // 128, c // 64] (flowchart 'Expand M_c -> M')."""
    return np.repeat(np.repeat(np.asarray(mask_c, bool), 128, axis=0), 64, axis=1)[:N, :N]


def sdpa(q, k, v, mask=None):
    t = [torch.from_numpy(np.ascontiguousarray(a))[None, None] for a in (q, k, v)]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(*t, attn_mask=m)[0, 0].numpy()


def phi_dense(x):
    return torch.softmax(torch.from_numpy(x), dim=-1).numpy()


def test_full_keep_equals_textbook_attention():
    """k = 100%, alpha = 1, no quantisation -> softmax(Q K^T / sqrt d) V (Eq. 11 with alpha = 1)."""
    q, k, v, wq, wk, _ = slice_inputs(N=1024)
    r = sla2.forward_head(q, k, v, wq, wk, np.ones(8), 1.0, quant=False)
    assert r["kb"] == 16 and r["mask"].all()
    assert not r["O_l"].any()                              # no dropped block -> O_l = 0
    ref = sdpa(q, k, v)                                    # raw K: smoothing must not matter
    # K_s = fl32(K - mu32) carries fp32 rounding (~6e-8 relative), nothing more
    assert np.abs(r["O"] - ref).max() < 1e-7
    ref_s = sdpa(q, r["Ks"], v)
    assert np.abs(r["O"] - ref_s).max() < 1e-12
    assert np.isfinite(r["O"]).all()


def test_sparse_branch_equals_dense_masked_attention():
    """O_s equals attention with the expanded N x N token mask (masked logits = -inf)."""
    q, k, v, wq, wk, a = slice_inputs(N=1024)
    r = sla2.forward_head(q, k, v, wq, wk, a, 0.25, quant=False)
    M = token_mask(r["mask"], 1024)
    assert np.abs(r["O_s"] - sdpa(q, r["Ks"], v, mask=M)).max() < 1e-12
    assert np.abs(r["O_s"] - sdpa(q, k, v, mask=M)).max() < 1e-7   # raw K: fp32 K_s rounding only


def test_linear_branch_equals_dense_formula():
    """O_l equals norm(phi(Q) phi(K_s)^T * (1 - M)) V of the flowchart, built densely."""
    q, k, v, wq, wk, a = slice_inputs(N=1024)
    r = sla2.forward_head(q, k, v, wq, wk, a, 0.25, quant=False)
    M = token_mask(r["mask"], 1024)
    kt = k.astype(np.float32) - r["mu32"]
    A = phi_dense(q) @ phi_dense(kt.astype(np.float64)).T * (~M)
    ref = (A @ v) / A.sum(axis=1, keepdims=True)
    assert np.abs(r["O_l"] - ref).max() < 1e-12


def test_mixture_rows_sum_to_one_and_reproduce_output():
    """alpha P_s + (1 - alpha) P_l is row-stochastic (Eq. 11) and times V gives O."""
    q, k, v, wq, wk, a = slice_inputs(N=1024)
    r = sla2.forward_head(q, k, v, wq, wk, a, 0.25, quant=False)
    M = token_mask(r["mask"], 1024)
    S = q @ r["Ks"].T / math.sqrt(D)
    S = np.where(M, S, -np.inf)
    Ps = np.exp(S - S.max(1, keepdims=True))
    Ps /= Ps.sum(1, keepdims=True)
    L = phi_dense(q) @ phi_dense(r["Ks"]).T * (~M)
    Pl = L / L.sum(1, keepdims=True)
    al = np.repeat(a.astype(np.float64), 128)[:, None]
    mix = al * Ps + (1 - al) * Pl
    assert np.abs(mix.sum(1) - 1).max() < 1e-12
    assert np.abs(mix @ v - r["O"]).max() < 1e-10


def test_eq9_selected_mass_times_sparse_output():
    """Eq. 9: P_1 V = alpha_row * O_s with P_1 = P * M and alpha_row = P_1 1 (§4)."""
    q, k, v, wq, wk, a = slice_inputs(N=1024)
    r = sla2.forward_head(q, k, v, wq, wk, a, 0.25, quant=False)
    M = token_mask(r["mask"], 1024)
    P = torch.softmax(torch.from_numpy(q @ r["Ks"].T / math.sqrt(D)), -1).numpy()
    P1 = P * M
    mass = P1.sum(1, keepdims=True)
    assert np.abs(P1 @ v - mass * r["O_s"]).max() < 1e-12


def test_online_loop_with_identity_codecs_is_exact():
    """The block-online loop with codecs switched off equals the exact masked softmax."""
    q, k, v, wq, wk, a = slice_inputs(N=1024)
    r = sla2.forward_head(q, k, v, wq, wk, a, 0.375, quant=False)
    exact = sla2.sparse_exact(q, r["Ks"], v, list(r["lists"]))
    assert np.abs(r["O_s"] - exact).max() < 1e-12
    # order independence: the loop visits blocks in any order and gets the same result
    ops = sla2.quantise_operands(q, r["Ks"], v, False, False)
    rev = sla2.sparse_online(ops, [L[::-1] for L in r["lists"]], D, p_quant=False)
    assert np.abs(rev - exact).max() < 1e-12


def test_quantised_branch_is_close_to_exact():
    """Sanity bound: INT8 Q,K + E4M3 P,V stay within a few percent of the exact branch."""
    q, k, v, wq, wk, a = slice_inputs(N=1024)
    rq = sla2.forward_head(q, k, v, wq, wk, a, 0.25, quant=True)
    re = sla2.forward_head(q, k, v, wq, wk, a, 0.25, quant=False)
    assert np.array_equal(rq["mask"], re["mask"])
    rel = np.linalg.norm(rq["O_s"] - re["O_s"]) / np.linalg.norm(re["O_s"])
    assert 1e-3 < rel < 0.08
    # INT8-only (P, V exact) is much closer: 8-bit Q, K error only
    ops = sla2.quantise_operands(q, re["Ks"], v, True, False)
    o8 = sla2.sparse_online(ops, list(re["lists"]), D, p_quant=False)
    assert np.linalg.norm(o8 - re["O_s"]) / np.linalg.norm(re["O_s"]) < 0.02


def brute_rank_select(P, kb):
    n_qb, n_kb = P.shape
    mask = np.zeros_like(P, dtype=np.uint8)
    for i in range(n_qb):
        for j in range(n_kb):
            rank = sum(1 for t in range(n_kb)
                       if P[i, t] > P[i, j] or (P[i, t] == P[i, j] and t < j))
            mask[i, j] = rank < kb
    return mask


def test_topk_against_brute_force_with_ties():
    rng = np.random.default_rng(5)
    P = rng.random((6, 40))
    P[0, [3, 9, 17, 30]] = P[0].max() + 1                  # four-way tie at the top
    P[1, :] = 0.5                                          # whole row tied
    P[2, [1, 2]] = P[2, [5, 6]] = 2.0                      # ties straddling the cut
    for kb in (1, 3, 7, 40):
        mask, lists = sla2.topk_blocks(P, kb)
        assert np.array_equal(mask, brute_rank_select(P, kb))
        assert (mask.sum(1) == kb).all()
        for i in range(P.shape[0]):
            assert np.array_equal(lists[i], np.flatnonzero(mask[i]))
    mask, _ = sla2.topk_blocks(P, 3)
    assert list(np.flatnonzero(mask[0])) == [3, 9, 17]
    assert list(np.flatnonzero(mask[1])) == [0, 1, 2]


def test_duplicated_key_blocks_tie_to_lower_index():
    """Identical key blocks give identical scores; the lower block index wins the tie."""
    q, k, v, wq, wk, a = slice_inputs(N=1024)
    k[5 * 64:6 * 64] = k[2 * 64:3 * 64]
    r = sla2.forward_head(q, k, v, wq, wk, a, 0.25, quant=False)
    assert np.array_equal(r["P_c"][:, 5], r["P_c"][:, 2])
    for i in range(8):
        if r["mask"][i, 5]:
            assert r["mask"][i, 2]


def test_kept_block_rule():
    assert sla2.kept_blocks(512, 0.03) == 15
    assert sla2.kept_blocks(128, 0.10) == 12
    assert sla2.kept_blocks(1182, 0.05) == 59
    assert [sla2.kept_blocks(512, f) for f in (0.2, 0.1, 0.05, 0.03)] == [102, 51, 25, 15]
    assert sla2.kept_blocks(32, 0.25) == 8
    assert sla2.kept_blocks(32, 1.0) == 32 and sla2.kept_blocks(32, 1e-6) == 1
    assert sla2.kept_blocks(10, 0.3) == 3
    with pytest.raises(ValueError):
        sla2.kept_blocks(32, 0.0)


def test_identity_projection_is_heuristic_router():
    """proj_q = proj_k = I gives softmax(pool(Q) pool(K)^T / sqrt d): the earlier SLA router."""
    q, k, v, _, _, a = slice_inputs(N=1024)
    eye = np.eye(D, dtype=np.float32)
    r = sla2.forward_head(q, k, v, eye, eye, a, 0.25, quant=False)
    tq = torch.from_numpy(q.T[None])                       # [1, d, N]
    ks = torch.from_numpy(r["Ks"].T[None])
    qbar = torch.nn.functional.avg_pool1d(tq, 128)[0].T
    kbar = torch.nn.functional.avg_pool1d(ks, 64)[0].T
    ref = torch.softmax(qbar @ kbar.T / math.sqrt(D), -1).numpy()
    assert np.abs(r["P_c"] - ref).max() < 1e-14


def test_smoothing_invariance():
    """Adding a per-channel constant to K changes nothing but rounding: K is smoothed first."""
    q, k, v, wq, wk, a = slice_inputs(N=1024, bias=0.0)
    c = np.random.default_rng(9).standard_normal(D).astype(np.float32)
    k2 = (k.astype(np.float32) + c).astype(np.float64)
    r1 = sla2.forward_head(q, k, v, wq, wk, a, 0.25, quant=False)
    r2 = sla2.forward_head(q, k2, v, wq, wk, a, 0.25, quant=False)
    assert np.abs(r1["G"] - r1["G"].mean(1, keepdims=True)
                  - (r2["G"] - r2["G"].mean(1, keepdims=True))).max() < 1e-5
    assert np.array_equal(r1["mask"], r2["mask"])
    assert np.abs(r1["O"] - r2["O"]).max() < 1e-5


def test_colmean_and_pooling_closed_forms():
    N = 512
    ramp = np.tile(np.arange(N, dtype=np.float64)[:, None], (1, D))
    mu, mu32 = sla2.colmean(ramp)
    assert np.all(mu == (N - 1) / 2)
    qbar = sla2.block_mean(ramp, 128)
    assert np.array_equal(qbar[:, 0], 128 * np.arange(4) + 63.5)
    kbar = sla2.block_mean(ramp, 64)
    assert np.array_equal(kbar[:, 5], 64 * np.arange(8) + 31.5)


def test_empty_branches_give_zero():
    q, k, v, wq, wk, a = slice_inputs(N=512)
    mask = np.zeros((4, 8), np.uint8)
    mask[1] = 1                                            # full row: no dropped block
    mask[2, [0, 7]] = 1
    r = sla2.forward_head(q, k, v, wq, wk, a, 0.5, quant=True, mask=mask)
    assert not r["O_s"][0:128].any() and not r["O_s"][384:512].any()
    assert not r["O_l"][128:256].any()
    assert np.isfinite(r["O"]).all()
    al = a.astype(np.float64)
    assert np.allclose(r["O"][0:128], (1 - al[0]) * r["O_l"][0:128], rtol=0, atol=0)


def test_alpha_extremes():
    q, k, v, wq, wk, _ = slice_inputs(N=512)
    r1 = sla2.forward_head(q, k, v, wq, wk, np.ones(4), 0.25, quant=True)
    r0 = sla2.forward_head(q, k, v, wq, wk, np.zeros(4), 0.25, quant=True)
    assert np.array_equal(r1["O"], r1["O_s"]) and np.array_equal(r0["O"], r0["O_l"])


def test_total_minus_selected_identity():
    """Step 3's accumulation over dropped blocks equals the total minus the kept blocks."""
    q, k, v, wq, wk, a = slice_inputs(N=1024)
    r = sla2.forward_head(q, k, v, wq, wk, a, 0.25, quant=False)
    h, z = r["h"], r["z"]
    for i in range(8):
        sel = r["mask"][i].astype(bool)
        direct = h[~sel].sum(0)
        tms = h.sum(0) - h[sel].sum(0)
        assert np.abs(direct - tms).max() < 1e-13
        assert np.abs(z[~sel].sum(0) - (z.sum(0) - z[sel].sum(0))).max() < 1e-12


def test_projection_orientation_x_times_w():
    """proj(x) = x @ W with W[in][out]: a permutation W moves channel k to column pi(k)."""
    q, k, v, _, _, a = slice_inputs(N=512)
    pi = np.random.default_rng(4).permutation(D)
    P = np.zeros((D, D), np.float32)
    P[np.arange(D), pi] = 1.0                              # W[k][pi(k)] = 1
    eye = np.eye(D, dtype=np.float32)
    r = sla2.forward_head(q, k, v, P, eye, a, 0.5, quant=False)
    qbar = q.reshape(4, 128, D).mean(1)
    kbar = r["Ks"].reshape(8, 64, D).mean(1)
    moved = np.zeros_like(qbar)
    moved[:, pi] = qbar                                    # column pi(k) holds channel k
    assert np.abs(r["G"] - moved @ kbar.T / math.sqrt(D)).max() < 1e-12
    # the transposed reading would give a different answer on this input
    wrong = qbar[:, pi] @ kbar.T / math.sqrt(D)
    assert np.abs(r["G"] - wrong).max() > 1e-3


# ----------------------------------------------------------------------------- SLA (v1) mix
def test_sla1_relates_to_sla2_for_constant_alpha():
    """With Proj = ((1 - a) / a) I and the heuristic router, a * (O_s + O_l Proj) is the SLA2
    mix a O_s + (1 - a) O_l (second page, §2 Q2: the projection of the earlier formulation
    has to absorb the scale that alpha carries explicitly); unquantised and quantised."""
    q, k, v, _, _, _ = slice_inputs(seed=21, N=1024)
    eye = np.eye(D, dtype=np.float32)
    for a in (0.3, 0.8):
        for quant in (False, True):
            r1 = sla2.forward_head_sla1(q, k, v, ((1 - a) / a) * np.eye(D), 0.25, quant=quant)
            r2 = sla2.forward_head(q, k, v, eye, eye, np.full(1024 // 128, a), 0.25, quant=quant)
            assert np.array_equal(r1["mask"], r2["mask"])
            assert np.abs(a * r1["O"] - r2["O"]).max() < 1e-12


def test_sla1_zero_projection_is_the_sparse_branch():
    q, k, v, _, _, _ = slice_inputs(seed=22, N=1024)
    r = sla2.forward_head_sla1(q, k, v, np.zeros((D, D)), 0.25, quant=False)
    ref = sla2.sparse_exact(q, r["Ks"], v, [np.flatnonzero(m) for m in r["mask"]])
    assert np.abs(r["O"] - ref).max() < 1e-12
