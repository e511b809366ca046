"""Pins of the oracle's backward (oracle/sla2_backward.py) on the CPU.

The backward is the gradient of the unquantised forward with the block mask held fixed (the
straight-through reading of "INT8/FP8 forward, FP16 backward", "SLA2: Sparse-Linear Attention v2
for Diffusion Transformers" §4 six checks item 4; §7 note 3). The pages print no worked
gradient, so the oracle is pinned against things it does not share code with:
  * central finite differences of forward_exact along random directions, for Q, K, V and alpha;
  * torch autograd (fp64) through an explicit N x N construction of the forward: masked softmax
    with -inf logits, normalised phi(Q) phi(K_s)^T (1 - M) V, K_s = K - colmean(K), the mix;
  * torch's scaled_dot_product_attention gradients for alpha = 1 (all blocks kept, and with a
    boolean block mask);
  * the column sums of dK vanish (adding one row vector to every row of K changes nothing).
"""
import math

import numpy as np
import pytest
import torch

from oracle import sla2_backward as bw

D = 128


def rand_case(seed, n_qb=3, special_rows=True, alpha="random"):
    """A slice with n_qb query blocks, a random block mask (row 1 all kept and row 2 none kept
    when special_rows), alpha per query block, and dO."""
    rng = np.random.default_rng(seed)
    N = 128 * n_qb
    Q = rng.standard_normal((N, D))
    K = rng.standard_normal((N, D)) + 0.5          # a non-zero column mean to smooth away
    V = rng.standard_normal((N, D))
    mask = (rng.random((n_qb, 2 * n_qb)) < 0.4).astype(np.uint8)
    mask[0, 0], mask[0, 1] = 1, 0
    if special_rows and n_qb >= 3:
        mask[1, :] = 1
        mask[2, :] = 0
    if alpha == "random":
        a = rng.uniform(0.1, 0.9, n_qb)
    else:
        a = np.full(n_qb, float(alpha))
    dO = rng.standard_normal((N, D))
    return Q, K, V, mask, a, dO


def loss(Q, K, V, mask, a, dO):
    O, _, _ = bw.forward_exact(Q, K, V, mask, a)
    return float((dO * O).sum())


@pytest.mark.parametrize("seed", [1, 2])
def test_finite_differences(seed):
    Q, K, V, mask, a, dO = rand_case(seed)
    g = bw.backward(Q, K, V, mask, a, dO)
    rng = np.random.default_rng(100 + seed)
    eps = 1e-5
    args = dict(Q=Q, K=K, V=V)
    for name, grad in (("Q", g["dQ"]), ("K", g["dK"]), ("V", g["dV"])):
        E = rng.standard_normal(args[name].shape)
        plus = dict(args, **{name: args[name] + eps * E})
        minus = dict(args, **{name: args[name] - eps * E})
        fd = (loss(plus["Q"], plus["K"], plus["V"], mask, a, dO)
              - loss(minus["Q"], minus["K"], minus["V"], mask, a, dO)) / (2 * eps)
        an = float((grad * E).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)
    E = rng.standard_normal(a.shape)
    fd = (loss(Q, K, V, mask, a + eps * E, dO) - loss(Q, K, V, mask, a - eps * E, dO)) / (2 * eps)
    assert abs(fd - float((g["dalpha"] * E).sum())) <= 1e-7 * max(1.0, abs(fd))


def dense_forward_torch(Q, K, V, mask, a):
    """The forward built from N x N matrices (no blocks in the arithmetic)."""
    N = Q.shape[0]
    M = torch.from_numpy(np.kron(mask, np.ones((128, 64))).astype(bool))
    Ks = K - K.mean(dim=0, keepdim=True)
    S = (Q @ Ks.T) / math.sqrt(D)
    S = S.masked_fill(~M, float("-inf"))
    any_kept = M.any(dim=1, keepdim=True)
    P = torch.softmax(torch.where(any_kept, S, torch.zeros_like(S)), dim=1)
    O_s = torch.where(any_kept, P @ V, torch.zeros_like(V))
    W = (torch.softmax(Q, dim=1) @ torch.softmax(Ks, dim=1).T) * (~M).to(Q.dtype)
    any_drop = (~M).any(dim=1, keepdim=True)
    den = torch.where(any_drop, W.sum(dim=1, keepdim=True), torch.ones_like(W[:, :1]))
    O_l = torch.where(any_drop, (W @ V) / den, torch.zeros_like(V))
    ar = a.repeat_interleave(128)[:, None]
    return ar * O_s + (1 - ar) * O_l


@pytest.mark.parametrize("seed,alpha", [(3, "random"), (4, 0.0), (5, 1.0)])
def test_torch_autograd_dense(seed, alpha):
    Q, K, V, mask, a, dO = rand_case(seed, alpha=alpha)
    g = bw.backward(Q, K, V, mask, a, dO)
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V, a)]
    O = dense_forward_torch(t[0], t[1], t[2], mask, t[3])
    O.backward(torch.from_numpy(dO))
    for name, tt in zip(("dQ", "dK", "dV", "dalpha"), t):
        ref = tt.grad.numpy()
        assert np.abs(g[name] - ref).max() <= 1e-10 * max(1.0, np.abs(ref).max()), name


def test_all_kept_alpha_one_is_sdpa():
    rng = np.random.default_rng(6)
    N = 256
    Q, K, V, dO = (rng.standard_normal((N, D)) for _ in range(4))
    mask = np.ones((N // 128, N // 64), np.uint8)
    g = bw.backward(Q, K, V, mask, np.ones(N // 128), dO)
    t = [torch.tensor(x, requires_grad=True) for x in (Q, K, V)]
    O = torch.nn.functional.scaled_dot_product_attention(*(x[None, None] for x in t))
    O[0, 0].backward(torch.from_numpy(dO))
    for name, tt in zip(("dQ", "dK", "dV"), t):
        assert np.abs(g[name] - tt.grad.numpy()).max() <= 1e-11, name


def test_block_mask_alpha_one_is_masked_sdpa():
    Q, K, V, mask, _, dO = rand_case(7, n_qb=2, special_rows=False)
    mask[:, 2] = 1                                 # every query block keeps something
    g = bw.backward(Q, K, V, mask, np.ones(2), dO)
    M = torch.from_numpy(np.kron(mask, np.ones((128, 64))).astype(bool))
    t = [torch.tensor(x, requires_grad=True) for x in (Q, K, V)]
    O = torch.nn.functional.scaled_dot_product_attention(*(x[None, None] for x in t),
                                                         attn_mask=M[None, None])
    O[0, 0].backward(torch.from_numpy(dO))
    for name, tt in zip(("dQ", "dK", "dV"), t):
        assert np.abs(g[name] - tt.grad.numpy()).max() <= 1e-11, name


def test_dk_column_sums_vanish():
    Q, K, V, mask, a, dO = rand_case(8)
    g = bw.backward(Q, K, V, mask, a, dO)
    assert np.abs(g["dK"].sum(axis=0)).max() <= 1e-11 * np.abs(g["dK"]).sum(axis=0).max()
    # and the sparse branch alone already has zero column sums before the centring
    g1 = bw.backward(Q, K, V, mask, np.ones_like(a), dO)
    assert np.abs(g1["dK"].sum(axis=0)).max() <= 1e-9


def test_branch_switches():
    """alpha = 1 leaves no gradient through O_l (rows of a block with nothing kept get none);
    alpha = 0 none through O_s (a block with nothing dropped gets none)."""
    Q, K, V, mask, _, dO = rand_case(9)
    g1 = bw.backward(Q, K, V, mask, np.ones(3), dO)
    assert np.all(g1["dQ"][256:384] == 0)           # block 2 keeps nothing
    g0 = bw.backward(Q, K, V, mask, np.zeros(3), dO)
    assert np.all(g0["dQ"][128:256] == 0)           # block 1 drops nothing
    assert np.all(np.isneginf(g0["lse"][256:384]))


def test_backward_spot_equals_the_full_backward():
    """backward_spot (selected query and key blocks, dropped sums as total minus kept) against
    backward() at a size where both run: a random mask with an all-kept and an all-dropped
    query block and a key block kept by every query block."""
    rng = np.random.default_rng(61)
    N, d = 1024, 16
    Q = rng.standard_normal((N, d))
    K = rng.standard_normal((N, d)) + rng.standard_normal(d)
    V = rng.standard_normal((N, d))
    dO = rng.standard_normal((N, d))
    mask = (rng.random((N // 128, N // 64)) < 0.3).astype(np.uint8)
    mask[2, :] = 1
    mask[3, :] = 0
    mask[:, 5] = 1
    mask[3, 5] = 0
    alpha = rng.uniform(0.1, 0.9, N // 128)
    full = bw.backward(Q, K, V, mask, alpha, dO)
    qb, kb = [0, 2, 3, 7], [0, 5, 9, 15]
    spot = bw.backward_spot(Q, K, V, mask, alpha, dO, qb, kb)
    for i in qb:
        ref = full["dQ"][i * 128:(i + 1) * 128]
        assert np.abs(spot["dQ"][i] - ref).max() <= 1e-10 * np.abs(ref).max()
        assert abs(spot["dalpha"][i] - full["dalpha"][i]) <= 1e-10 * abs(full["dalpha"]).max()
    for j in kb:
        ref = full["dV"][j * 64:(j + 1) * 64]
        assert np.abs(spot["dV"][j] - ref).max() <= 1e-10 * np.abs(ref).max()
