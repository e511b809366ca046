"""GPU parity of sla2_router_grad (the stage-1 router gradient) against the oracle's
straight-through chain (oracle/sla2_fit.py router_grad_head), through the C ABI.

Cases: the i.i.d. workload's shape (fp32, 2 heads, N = 2048, keep 25 %); a batch of two (the
gradients are summed over it); two heads of the 8x32x32 grid workload (bf16, N = 8192, keep
10 %); keep 100 % (every block kept: the soft mask is 1 and the gradient 0, with no NaN); and
the bench's 12-head N = 32768 workload in one call, sampled rows of the mask gradient. The
router weights are the generators' N(0, 1/d) draws scaled up so that P_c is not flat: every
row's kb-th and (kb + 1)-th largest P_c then differ by far more than the router's 1e-5 band, a
precondition checked on the oracle's P_c, so the GPU's hard mask is the oracle's (checked
through sla2_router).

Tolerances. The dense pass takes Q, K_s, V, phi(Q), phi(K_s) and the scaled delta as f16
(each element rounded with relative error at most 2^-12 = 2.4e-4) with fp32 accumulation; a
block pair's number sums 8192 products whose rounding errors are independent, so its relative
error is of order 2^-12 times the ratio of the terms' magnitudes to the sum's, a few 1e-4
where delta V^T - c cancels; the router part is fp32 with fp64 sums and adds little. Bound:
2e-3 relative L2 on the mask gradient and on dproj_q, dproj_k (measured 3e-5 to 3e-4). The
loss follows from the forward's own tolerance: with |dO| <= 3e-3 |O| (the forward's relative
L2 bound, set by the linear branch's bf16 operands), |L_gpu - L| <= 2 |O - O_full| |dO| +
|dO|^2 per head (measured up to 2.4e-4 relative where alpha = 0 makes O the linear branch
alone, 1.6e-5 elsewhere).
"""
import sys

import numpy as np
import pytest
import torch

from block_sparse_linear_pool_amd import sla2
from block_sparse_linear_pool_amd import workloads as W
from oracle import sla2 as F
from oracle import sla2_fit as S
from tests.gpu_helpers import check_mask_band, dev, host, rel_l2, rows_agreeing

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TAU = 0.1
GRAD_TOL = 2e-3
O_TOL = 3e-3     # the forward's relative L2 bound on O
GAP = 1e-4     # smallest relative gap between the kb-th and (kb + 1)-th largest P_c


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_case(q, k, v, wq, wk, alpha, keep):
    B, H, N, _ = q.shape
    O_full = np.zeros(q.shape)
    refs = {}
    for b in range(B):
        for h in range(H):
            O_full[b, h] = S.full_attention_head(q[b, h], k[b, h], v[b, h])
            r = S.router_grad_head(q[b, h], k[b, h], v[b, h], wq[h], wk[h], alpha[h], keep, TAU,
                                   O_full[b, h])
            kb = r["kb"]
            if kb < N // 64:
                s = -np.sort(-r["P_c"], axis=1)
                gap = ((s[:, kb - 1] - s[:, kb]) / s[:, kb - 1]).min()
                assert gap > GAP, f"near tie in the router of b{b} h{h}: {gap:.2e}"
            refs[(b, h)] = r
    return O_full, refs


def run_and_compare(q, k, v, wq, wk, alpha, keep, tdt):
    B, H = q.shape[:2]
    O_full, refs = oracle_case(q, k, v, wq, wk, alpha, keep)
    g = [dev(q, tdt), dev(k, tdt), dev(v, tdt), dev(wq), dev(wk), dev(alpha)]
    loss, dwq, dwk, mg = sla2.sla2_router_grad(*g, keep, dev(O_full.astype(np.float32)), tau=TAU,
                                               want_mask_grad=True)
    _, mask, _ = sla2.sla2_router(g[0], g[1], g[3], g[4], keep)
    torch.cuda.synchronize()
    loss, dwq, dwk, mg, mask = host(loss), host(dwq), host(dwk), host(mg), host(mask)
    for (b, h), r in refs.items():
        assert (mask[b, h] == r["mask"]).all(), (b, h)
        e = rel_l2(mg[b, h], r["mask_grad"])
        say(f"  b{b} h{h}: mask grad relL2 {e:.2e} (|g| max {np.abs(r['mask_grad']).max():.2e})")
        assert e <= GRAD_TOL
    for h in range(H):
        ref_loss = sum(refs[(b, h)]["loss"] for b in range(B))
        ref_q = sum(refs[(b, h)]["dWq"] for b in range(B))
        ref_k = sum(refs[(b, h)]["dWk"] for b in range(B))
        el = abs(loss[h] - ref_loss) / ref_loss
        dO = sum(O_TOL ** 2 * float((refs[(b, h)]["O"] ** 2).sum()) for b in range(B)) ** 0.5
        loss_tol = (2.0 * ref_loss ** 0.5 * dO + dO ** 2) / ref_loss
        eq, ek = rel_l2(dwq[h], ref_q), rel_l2(dwk[h], ref_k)
        say(f"  h{h}: loss {loss[h]:.6e} rel {el:.2e}; dproj_q relL2 {eq:.2e}; dproj_k relL2 {ek:.2e}")
        assert el <= loss_tol, (el, loss_tol)
        assert np.isfinite(dwq[h]).all() and np.isfinite(dwk[h]).all()
        if np.abs(ref_q).max() > 0:
            assert eq <= GRAD_TOL and ek <= GRAD_TOL
        else:
            assert not dwq[h].any() and not dwk[h].any()
    return refs


def test_router_grad_iid_fp32():
    q, k, v = W.random_qkv(21, 1, 2, 2048)
    wq, wk, alpha = W.random_weights(21, 2, 16, alpha_lo=0.2)
    say("router grad: i.i.d. fp32, 2 heads, N 2048, keep 0.25")
    run_and_compare(q, k, v, wq * 10, wk * 10, alpha, 0.25, torch.float32)


def test_router_grad_batch_of_two():
    q, k, v = W.random_qkv(23, 2, 2, 1024)
    wq, wk, alpha = W.random_weights(23, 2, 8, alpha_lo=0.2)
    say("router grad: batch of two, fp32, N 1024, keep 0.25")
    run_and_compare(q, k, v, wq * 10, wk * 10, alpha, 0.25, torch.float32)


@pytest.mark.timeout(600)
def test_router_grad_grid_bf16():
    w = W.WORKLOADS["grid_8x32x32_N8192"]
    heads = [4, 10]
    q, k, v = W.generate(w, heads=heads)
    wq, wk, alpha = W.weights(w)
    say("router grad: grid workload bf16, heads", heads, "N 8192, keep 0.1")
    run_and_compare(q, k, v, wq[heads] * 8, wk[heads] * 8, alpha[heads], 0.1, torch.bfloat16)


def test_router_grad_everything_kept():
    q, k, v = W.random_qkv(25, 1, 2, 1024)
    wq, wk, alpha = W.random_weights(25, 2, 8, alpha_lo=0.2)
    say("router grad: keep 1.0")
    refs = run_and_compare(q, k, v, wq * 10, wk * 10, alpha, 1.0, torch.float32)
    for r in refs.values():
        assert not r["dWq"].any() and not r["dWk"].any()


@pytest.mark.timeout(600)
def test_router_grad_bench_size_sampled_rows():
    """The 12-head N = 32768 workload as bench.py runs it (all heads in one call, 3 % kept, the
    target from the library's unquantised forward at keep 1): rows of the mask gradient of
    heads 0 and 7 against the oracle's row-restricted derivative (its own router, its own
    full-attention rows), on query blocks whose GPU kept set is the oracle's."""
    w = W.WORKLOADS["wan13b_480p_N32768"]
    keep = w.keep_frac[-1]
    q, k, v = W.generate(w)
    wq, wk, alpha = W.weights(w)
    t = torch.bfloat16
    g = [dev(q, t), dev(k, t), dev(v, t), dev(wq), dev(wk), dev(alpha)]
    eye = dev(np.broadcast_to(np.eye(128, dtype=np.float32), (w.H, 128, 128)).copy())
    ones = dev(np.ones((w.H, w.n_qb), np.float32))
    say("router grad at the bench size: GPU")
    o_full = sla2.sla2_forward(g[0], g[1], g[2], eye, eye, ones, 1.0, quant="none")
    loss, dwq, dwk, mg = sla2.sla2_router_grad(*g, keep, o_full, tau=TAU, want_mask_grad=True)
    _, mask, _ = sla2.sla2_router(g[0], g[1], g[3], g[4], keep)
    torch.cuda.synchronize()
    mg, mask, loss = host(mg), host(mask), host(loss)
    assert np.isfinite(mg).all() and np.isfinite(host(dwq)).all() and np.isfinite(host(dwk)).all()
    assert (loss > 0).all()
    checked = 0
    for h in (0, 7):
        r = F.forward_head(q[0, h], k[0, h], v[0, h], wq[h], wk[h], alpha[h], keep, quant=False)
        check_mask_band(r["P_c"], r["kb"], mask[0, h])
        agree = rows_agreeing(mask[0, h], r["mask"])
        rows = [i for i in (0, 100, 255) if agree[i]]
        targets = S.full_attention_rows(q[0, h], k[0, h], v[0, h], rows)
        ref = S.mask_grad_rows(q[0, h], r["Ks"], v[0, h], r["mask"].astype(np.float64), alpha[h],
                               targets)
        for i in rows:
            e = rel_l2(mg[0, h, i], ref[i])
            say(f"  h{h} query block {i}: mask grad relL2 {e:.2e} (|g| max {np.abs(ref[i]).max():.2e})")
            assert e <= GRAD_TOL
            checked += 1
    assert checked >= 3


@pytest.mark.parametrize("N,keep", [(128, 0.5), (384, 0.2), (640, 0.5)])
def test_router_grad_small_shapes_and_alpha_extremes(N, keep):
    """The smallest shapes (one query block, two key blocks; a ragged 5 x 10 grid), kb = 1 and
    kb = half the row, alpha at 0 and at 1 in some query blocks (each part of the derivative
    alone there)."""
    q, k, v = W.random_qkv(29 + N, 1, 2, N)
    wq, wk, alpha = W.random_weights(29 + N, 2, N // 128, alpha_lo=0.2)
    alpha[0, 0] = 0.0
    alpha[1, -1] = 1.0
    say(f"router grad: N {N}, keep {keep}")
    run_and_compare(q, k, v, wq * 10, wk * 10, alpha, keep, torch.float32)


def test_router_grad_zero_residual():
    """O_full equal to the forward's own output: delta = 0, so the loss, the mask gradient and
    both projection gradients are exactly zero."""
    q, k, v = W.random_qkv(31, 1, 2, 1024)
    wq, wk, alpha = W.random_weights(31, 2, 8, alpha_lo=0.2)
    g = [dev(q), dev(k), dev(v), dev(wq * 10), dev(wk * 10), dev(alpha)]
    O = sla2.sla2_forward(*g, 0.25, quant="none")
    loss, dwq, dwk, mg = sla2.sla2_router_grad(*g, 0.25, O, tau=TAU, want_mask_grad=True)
    torch.cuda.synchronize()
    assert not host(loss).any() and not host(mg).any()
    assert not host(dwq).any() and not host(dwk).any()
