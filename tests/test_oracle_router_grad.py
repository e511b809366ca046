"""Pins of the oracle's stage-1 router gradient (oracle/sla2_fit.py, router part), CPU only.

The chain has three derivatives and a relaxation; each is pinned by something other than
itself:
- the relaxation at a 0/1 mask is the method's own forward (forward_head without
  quantisation, given the same mask);
- dL/dM (mask_grad) against central finite differences of the relaxed loss, at an interior
  mask and at the hard mask;
- the SoftTop-k derivative (soft_topk_vjp, implicit lambda) against finite differences of
  soft_topk itself (its bisection is solved to fp64 precision);
- the router derivative (router_vjp) against finite differences of router_scores;
- the whole chain with the soft mask in the forward (straight_through=False, a smooth loss of
  proj_q and proj_k) against finite differences of that loss;
- planted mistakes (a dropped term, a flipped sign, no centring) fail these comparisons.
Small shapes (N = 512, d = 16: 4 query blocks, 8 key blocks) keep every difference quotient
cheap.
"""
import numpy as np
import pytest

from oracle import sla2 as F
from oracle import sla2_fit as S

N, D = 512, 16
KEEP, TAU = 0.25, 0.1


def problem(seed=0):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((N, D))
    K = rng.standard_normal((N, D)) + rng.standard_normal(D)
    V = rng.standard_normal((N, D))
    # router weights large enough that P_c is far from uniform
    Wq = rng.standard_normal((D, D)) * 2.0
    Wk = rng.standard_normal((D, D)) * 2.0
    alpha = rng.uniform(0.2, 0.8, N // 128)
    O_full = S.full_attention_head(Q, K, V)
    return Q, K, V, Wq, Wk, alpha, O_full


def smoothed(K):
    _, mu32 = F.colmean(K)
    return F.smooth_k(K, mu32)


def fd_mask(Q, Ks, V, M, alpha, O_full, eps=1e-6):
    g = np.zeros_like(M)
    for i in range(M.shape[0]):
        for j in range(M.shape[1]):
            Mp, Mm = M.copy(), M.copy()
            Mp[i, j] += eps
            Mm[i, j] -= eps
            g[i, j] = (S.relaxed_loss(Q, Ks, V, Mp, alpha, O_full)
                       - S.relaxed_loss(Q, Ks, V, Mm, alpha, O_full)) / (2 * eps)
    return g


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b)))


# ------------------------------------------------------------------ relaxation
def test_relaxation_at_a_hard_mask_is_the_forward():
    Q, K, V, Wq, Wk, alpha, _ = problem(1)
    rng = np.random.default_rng(2)
    mask = (rng.random((N // 128, N // 64)) < 0.4).astype(np.uint8)
    mask[0, :] = 0
    mask[0, 3] = 1            # one kept block
    mask[1, :] = 1
    mask[1, 5] = 0            # one dropped block
    ref = F.forward_head(Q, K, V, Wq, Wk, alpha, KEEP, quant=False, mask=mask)
    O_s, O_l, O = S.relaxed_outputs(Q, ref["Ks"], V, mask.astype(float), alpha)
    for a, b in ((O_s, ref["O_s"]), (O_l, ref["O_l"]), (O, ref["O"])):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())


def test_full_attention_target_is_softmax_attention():
    Q, K, V, *_ = problem(3)
    O = S.full_attention_head(Q, K, V)
    # every block kept in the method's unquantised forward is the same dense attention
    ones = np.ones((N // 128, N // 64), np.uint8)
    ref = F.forward_head(Q, K, V, np.eye(D), np.eye(D), np.ones(N // 128), 1.0, quant=False,
                         mask=ones)
    # (the forward's K_s is rounded to fp32: 2^-24 relative on each key value, a few 1e-8 on O)
    assert np.abs(O - ref["O_s"]).max() <= 1e-6


# ------------------------------------------------------------------ dL/dM
@pytest.mark.parametrize("where", ["interior", "hard"])
def test_mask_grad_against_differences(where):
    Q, K, V, Wq, Wk, alpha, O_full = problem(4)
    Ks = smoothed(K)
    rng = np.random.default_rng(5)
    if where == "interior":
        M = rng.uniform(0.1, 0.9, (N // 128, N // 64))
    else:
        M = (rng.random((N // 128, N // 64)) < 0.3).astype(float)
        M[:, 0] = 1.0          # every row keeps a block and drops one
        M[:, -1] = 0.0
    g = S.mask_grad(Q, Ks, V, M, alpha, O_full)
    fd = fd_mask(Q, Ks, V, M, alpha, O_full)
    assert rel(g, fd) <= 1e-6, rel(g, fd)
    assert np.abs(g).max() > 1e-3          # the comparison is not between zeros


def test_mask_grad_alpha_extremes_split_the_branches():
    """alpha = 1: only the sparse part; alpha = 0: only the linear part (each alone against
    differences, so neither part can hide behind the other)."""
    Q, K, V, Wq, Wk, _, O_full = problem(6)
    Ks = smoothed(K)
    rng = np.random.default_rng(7)
    M = rng.uniform(0.2, 0.8, (N // 128, N // 64))
    for a in (1.0, 0.0):
        alpha = np.full(N // 128, a)
        g = S.mask_grad(Q, Ks, V, M, alpha, O_full)
        assert rel(g, fd_mask(Q, Ks, V, M, alpha, O_full)) <= 1e-6


# ------------------------------------------------------------------ SoftTop-k
def test_soft_topk_vjp_against_differences():
    Q, K, V, Wq, Wk, alpha, _ = problem(8)
    Ks = smoothed(K)
    _, P = F.router_scores(F.block_mean(Q, 128), F.block_mean(Ks, 64), Wq, Wk)
    kb = F.kept_blocks(N // 64, KEEP)
    soft, _ = F.soft_topk(P, kb, TAU)
    g = np.random.default_rng(9).standard_normal(P.shape)
    dP = S.soft_topk_vjp(soft, TAU, g)
    fd = np.zeros_like(P)
    eps = 1e-7
    for i in range(P.shape[0]):
        for j in range(P.shape[1]):
            Pp, Pm = P.copy(), P.copy()
            Pp[i, j] += eps
            Pm[i, j] -= eps
            fd[i, j] = ((g * F.soft_topk(Pp, kb, TAU)[0]).sum()
                        - (g * F.soft_topk(Pm, kb, TAU)[0]).sum()) / (2 * eps)
    assert rel(dP, fd) <= 1e-5, rel(dP, fd)
    # the row-sum constraint: a gradient equal along a row changes nothing
    assert np.abs(S.soft_topk_vjp(soft, TAU, np.ones_like(g))).max() <= 1e-12


# ------------------------------------------------------------------ router
def test_router_vjp_against_differences():
    Q, K, V, Wq, Wk, *_ = problem(10)
    Ks = smoothed(K)
    Qbar, Kbar = F.block_mean(Q, 128), F.block_mean(Ks, 64)
    dP = np.random.default_rng(11).standard_normal((N // 128, N // 64))
    dWq, dWk = S.router_vjp(Qbar, Kbar, Wq, Wk, dP)
    eps = 1e-6
    for W, dW, which in ((Wq, dWq, 0), (Wk, dWk, 1)):
        fd = np.zeros_like(W)
        for a in range(D):
            for b in range(D):
                Wp, Wm = W.copy(), W.copy()
                Wp[a, b] += eps
                Wm[a, b] -= eps
                args_p = (Wp, Wk) if which == 0 else (Wq, Wp)
                args_m = (Wm, Wk) if which == 0 else (Wq, Wm)
                fd[a, b] = ((dP * F.router_scores(Qbar, Kbar, *args_p)[1]).sum()
                            - (dP * F.router_scores(Qbar, Kbar, *args_m)[1]).sum()) / (2 * eps)
        assert rel(dW, fd) <= 1e-6, (which, rel(dW, fd))


# ------------------------------------------------------------------ whole chain
def soft_loss(Q, K, V, Wq, Wk, alpha, O_full):
    Ks = smoothed(K)
    _, P = F.router_scores(F.block_mean(Q, 128), F.block_mean(Ks, 64), Wq, Wk)
    soft, _ = F.soft_topk(P, F.kept_blocks(N // 64, KEEP), TAU)
    return S.relaxed_loss(Q, Ks, V, soft, alpha, O_full)


def test_chain_with_the_soft_mask_against_differences():
    Q, K, V, Wq, Wk, alpha, O_full = problem(12)
    r = S.router_grad_head(Q, K, V, Wq, Wk, alpha, KEEP, TAU, O_full, straight_through=False)
    assert abs(r["loss"] - soft_loss(Q, K, V, Wq, Wk, alpha, O_full)) <= 1e-12 * r["loss"]
    rng = np.random.default_rng(13)
    eps = 1e-6
    for which in (0, 1):
        dW = r["dWq"] if which == 0 else r["dWk"]
        W = Wq if which == 0 else Wk
        for a, b in rng.integers(0, D, (12, 2)):
            Wp, Wm = W.copy(), W.copy()
            Wp[a, b] += eps
            Wm[a, b] -= eps
            lp = soft_loss(Q, K, V, *((Wp, Wk) if which == 0 else (Wq, Wp)), alpha, O_full)
            lm = soft_loss(Q, K, V, *((Wm, Wk) if which == 0 else (Wq, Wm)), alpha, O_full)
            fd = (lp - lm) / (2 * eps)
            assert abs(dW[a, b] - fd) <= 1e-5 * np.abs(dW).max(), (which, a, b, dW[a, b], fd)


def test_straight_through_forward_is_the_hard_forward():
    Q, K, V, Wq, Wk, alpha, O_full = problem(14)
    r = S.router_grad_head(Q, K, V, Wq, Wk, alpha, KEEP, TAU, O_full)
    ref = F.forward_head(Q, K, V, Wq, Wk, alpha, KEEP, quant=False)
    assert (r["mask"] == ref["mask"]).all()
    assert np.abs(r["O"] - ref["O"]).max() <= 1e-12
    assert abs(r["loss"] - ((ref["O"] - O_full) ** 2).sum()) <= 1e-12 * r["loss"]
    # dL/dM at the hard mask is what the soft mask receives
    Ks = ref["Ks"]
    g = S.mask_grad(Q, Ks, V, ref["mask"].astype(float), alpha, O_full)
    assert np.abs(r["mask_grad"] - g).max() == 0.0
    assert np.abs(r["dWq"]).max() > 0 and np.abs(r["dWk"]).max() > 0


# ------------------------------------------------------------------ planted mistakes
def test_planted_mistakes_fail_the_pins(monkeypatch):
    Q, K, V, Wq, Wk, alpha, O_full = problem(15)
    Ks = smoothed(K)
    M = np.random.default_rng(16).uniform(0.2, 0.8, (N // 128, N // 64))
    fd = fd_mask(Q, Ks, V, M, alpha, O_full)
    base = S.mask_grad(Q, Ks, V, M, alpha, O_full)
    assert rel(base, fd) <= 1e-6

    # (1) the c_q term of the sparse part dropped: O_s taken as zero inside the derivative
    real_outputs = S.relaxed_outputs

    def no_c(*a):
        O_s, O_l, O = real_outputs(*a)
        return O_s * 0.0, O_l, O
    monkeypatch.setattr(S, "relaxed_outputs", no_c)
    assert rel(S.mask_grad(Q, Ks, V, M, alpha, O_full), fd) > 1e-2
    monkeypatch.setattr(S, "relaxed_outputs", real_outputs)

    # (2) the linear part with the wrong sign
    real_linear = S._linear_part
    monkeypatch.setattr(S, "_linear_part", lambda *a: -real_linear(*a))
    assert rel(S.mask_grad(Q, Ks, V, M, alpha, O_full), fd) > 1e-2
    monkeypatch.setattr(S, "_linear_part", real_linear)

    # (3) SoftTop-k derivative without the centring term (lambda held fixed)
    _, P = F.router_scores(F.block_mean(Q, 128), F.block_mean(Ks, 64), Wq, Wk)
    kb = F.kept_blocks(N // 64, KEEP)
    soft, _ = F.soft_topk(P, kb, TAU)
    g = np.random.default_rng(17).standard_normal(P.shape)
    wrong = soft * (1 - soft) * g / TAU
    eps = 1e-7
    i, j = 1, 2
    Pp, Pm = P.copy(), P.copy()
    Pp[i, j] += eps
    Pm[i, j] -= eps
    fd_ij = ((g * F.soft_topk(Pp, kb, TAU)[0]).sum() - (g * F.soft_topk(Pm, kb, TAU)[0]).sum()) / (2 * eps)
    right = S.soft_topk_vjp(soft, TAU, g)[i, j]
    assert abs(right - fd_ij) <= 1e-5 * abs(fd_ij) + 1e-9
    assert abs(wrong[i, j] - fd_ij) > 1e-3 * abs(fd_ij)


def test_mask_grad_rows_equals_mask_grad():
    """The row-restricted derivative (for sampled rows at large sizes) against the whole one,
    and the row-restricted full-attention target against the whole target."""
    Q, K, V, Wq, Wk, alpha, O_full = problem(18)
    Ks = smoothed(K)
    M = (np.random.default_rng(19).random((N // 128, N // 64)) < 0.3).astype(float)
    M[0, :] = 1.0                                   # a row with no dropped block
    M[1, :] = 0.0
    M[1, 2] = 1.0
    whole = S.mask_grad(Q, Ks, V, M, alpha, O_full)
    rows = S.full_attention_rows(Q, K, V, [0, 1, 3])
    for i, r in rows.items():
        assert np.abs(r - O_full[128 * i:128 * (i + 1)]).max() <= 1e-12
    part = S.mask_grad_rows(Q, Ks, V, M, alpha, rows)
    for i, g in part.items():
        assert np.abs(g - whole[i]).max() <= 1e-10 * np.abs(whole[i]).max()
