"""SoftTop-k router on the GPU (sla2_router_soft) against the oracle's soft_topk.

Both sides compute the logits and P_c in fp64; the GPU rounds x = P_c / tau to fp32 and
bisects lambda in fp32 (row sums of 512 fp32 terms, about 3e-5 absolute noise, so lambda is
off by about 3e-5 / sum sigma'(.) and each mask entry by about 1e-6). Tolerances: mask
max-abs 2e-5, lambda 1e-4 absolute, every GPU row sum within 1e-3 of kb.
"""
import sys

import numpy as np
import pytest
import torch

from block_sparse_linear_pool_amd import sla2
from block_sparse_linear_pool_amd import workloads as W
from oracle import sla2 as oracle
from tests.gpu_helpers import dev, host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TDT = {"fp32": torch.float32, "bf16": torch.bfloat16}
MASK_TOL, LAM_TOL, SUM_TOL = 2e-5, 1e-4, 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_pc(q, k, wq, wk):
    """P_c of one (b, h) slice, the oracle's step 1 up to the softmax."""
    mu, mu32 = oracle.colmean(k)
    ks = oracle.smooth_k(k, mu32)
    _, P = oracle.router_scores(oracle.block_mean(np.asarray(q, np.float64), 128),
                                oracle.block_mean(ks, 64), wq, wk)
    return P


def check(q, k, wq, wk, keep, tau, dtype, heads):
    B, H, N, _ = q.shape
    kb = oracle.kept_blocks(N // 64, keep)
    soft, lam = sla2.sla2_router_soft(dev(q, TDT[dtype]), dev(k, TDT[dtype]), dev(wq), dev(wk),
                                      keep, tau)
    torch.cuda.synchronize()
    soft, lam = host(soft), host(lam)
    assert np.isfinite(soft).all()
    for b, h in heads:
        P = oracle_pc(q[b, h], k[b, h], wq[h], wk[h])
        ref, lref = oracle.soft_topk(P, kb, tau)
        e_m = np.abs(soft[b, h] - ref).max()
        rows = soft[b, h].astype(np.float64).sum(1)
        say(f"  b{b} h{h} kb {kb} tau {tau}: mask maxabs {e_m:.2e}, "
            f"row sums {rows.min():.5f}..{rows.max():.5f}")
        assert e_m <= MASK_TOL
        assert np.abs(rows - kb).max() <= SUM_TOL
        if kb < N // 64:
            assert np.abs(lam[b, h] - lref).max() <= LAM_TOL
        else:
            assert np.isinf(lam[b, h]).all() and (soft[b, h] == 1.0).all()


@pytest.mark.parametrize("name,heads,tau", [("tiny_iid_N2048", None, 0.1),
                                            ("grid_8x32x32_N8192", [0, 5], 0.1),
                                            ("grid_8x32x32_N8192", [3], 0.02),
                                            ("grid_8x32x32_N8192", [4], 1.0)])
def test_soft_router_matches_oracle(name, heads, tau):
    w = W.WORKLOADS[name]
    q, k, v = W.generate(w, heads=heads)
    wq, wk, alpha = W.weights(w)
    if heads is not None:
        wq, wk = wq[heads], wk[heads]
    keep = w.keep_frac[0]
    say("soft router", name, q.shape, keep, tau)
    B, H = q.shape[:2]
    check(q, k, wq, wk, keep, tau, w.dtype, [(b, h) for b in range(B) for h in range(H)])


@pytest.mark.parametrize("N,keep", [(128, 0.5), (128, 1.0), (640, 0.1), (1024, 1e-3),
                                    (262144, 0.002)])
def test_soft_router_small_and_edge_keeps(N, keep):
    """Smallest shape, every block kept (ones, lambda = inf), a ragged grid, kb = 1, and the
    largest length (4096 key blocks a row, kb = 8)."""
    q, k, _ = W.random_qkv(61 + N, 1, 2, N)
    wq, wk, _ = W.random_weights(61 + N, 2, N // 128)
    say("soft router edge", N, keep)
    check(q, k, wq, wk, keep, 0.1, "fp32", [(0, 0), (0, 1)])


def test_soft_router_constant_rows():
    """Equal key blocks give equal logits: every row of P_c is uniform, so every mask entry
    is kb / N_kb."""
    N = 2048
    q, k, _ = W.random_qkv(71, 1, 1, N)
    k[0, 0] = np.tile(k[0, 0, :64], (N // 64, 1))
    wq, wk, _ = W.random_weights(71, 1, N // 128)
    soft, _ = sla2.sla2_router_soft(dev(q), dev(k), dev(wq), dev(wk), 0.25, 0.1)
    kb = oracle.kept_blocks(N // 64, 0.25)
    assert np.abs(host(soft) - kb / (N // 64)).max() <= MASK_TOL


def test_soft_router_benchmark_size_and_determinism():
    """The Wan2.1-1.3B 480P-shaped workload (12 heads, N = 32768, 3% kept): two heads checked
    against the oracle; a second call gives identical bits."""
    w = W.WORKLOADS["wan13b_480p_N32768"]
    q, k, _ = W.generate(w)
    wq, wk, _ = W.weights(w)
    keep = w.keep_frac[-1]
    say("soft router bench size", keep)
    check(q, k, wq, wk, keep, 0.1, w.dtype, [(0, 0), (0, 9)])
    g = [dev(q, TDT[w.dtype]), dev(k, TDT[w.dtype]), dev(wq), dev(wk)]
    a, la = sla2.sla2_router_soft(*g, keep, 0.1)
    b, lb = sla2.sla2_router_soft(*g, keep, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
