"""The backward pass on the GPU (sla2_backward, through the C ABI) against the oracle's
backward (oracle/sla2_backward.py), element by element per (batch, head) slice.

Tolerance. The GPU rounds every matrix-product operand to bf16 (unit roundoff 2^-9) and
accumulates in fp32. The longest chain (Q, K_s -> S -> P -> dS -> dK, and its twin through
dO_s, V -> dP) rounds about four operands, each to at most 2^-9 relative, and dS = P (dP - D)
can lose up to about a factor 2 to cancellation (D is the P-weighted mean of dP): 4 * 2 * 2^-9
= 1.6e-2. So every gradient must be within relative L2 2e-2 of the oracle, per slice.
"""
import sys

import numpy as np
import pytest
import torch

from block_sparse_linear_pool_amd import sla2
from block_sparse_linear_pool_amd import workloads as W
from oracle import sla2_backward as bw
from tests.gpu_helpers import dev, host, oracle_router_masks, rel_l2

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TDT = {"fp32": torch.float32, "bf16": torch.bfloat16}
TOL = 2e-2
NAMES = ("dQ", "dK", "dV", "dalpha")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_backward(q, k, v, mask, alpha, dO, dtype):
    t = TDT[dtype]
    out = sla2.sla2_backward(dev(q, t), dev(k, t), dev(v, t), dev(mask, torch.uint8), dev(alpha),
                             dev(dO))
    torch.cuda.synchronize()
    return [host(x) for x in out]


def check(q, k, v, mask, alpha, dO, dtype, heads):
    got = gpu_backward(q, k, v, mask, alpha, dO, dtype)
    for x in got:
        assert np.isfinite(x).all()
    for b, h in heads:
        r = bw.backward(q[b, h], k[b, h], v[b, h], mask[b, h], alpha[h], dO[b, h])
        errs = [rel_l2(g[b, h], r[n]) for g, n in zip(got, NAMES)]
        say(f"  b{b} h{h}: " + ", ".join(f"{n} {e:.2e}" for n, e in zip(NAMES, errs)))
        assert max(errs) <= TOL
    return got


def test_backward_random_masks_with_empty_and_full_rows():
    """N = 512 (4 query blocks, 8 key blocks), fp32 inputs; per head a random mask in which
    query block 1 keeps every key block (no linear branch) and block 2 keeps none (no sparse
    branch)."""
    B, H, N = 1, 2, 512
    q, k, v = W.random_qkv(91, B, H, N)
    mask = W.random_mask(91, B, H, N // 128, N // 64, 0.4)
    mask[:, :, 1, :] = 1
    mask[:, :, 2, :] = 0
    _, _, alpha = W.random_weights(91, H, N // 128, alpha_lo=0.1)
    dO = W.grad_out(91, q.shape)
    say("backward small", q.shape)
    check(q, k, v, mask, alpha, dO, "fp32", [(0, 0), (0, 1)])


@pytest.mark.parametrize("B,H,N,dtype,frac", [(1, 3, 640, "bf16", 0.3), (3, 1, 1152, "fp32", 0.15),
                                              (1, 1, 2176, "bf16", 0.6)])
def test_backward_ragged_block_counts(B, H, N, dtype, frac):
    """Odd numbers of query blocks (5, 9, 17) and key blocks (10, 18, 34), odd head and batch
    counts, sparse to dense masks (key lists of 5 to 16 of the 17 query blocks at 60 %)."""
    q, k, v = W.random_qkv(N + B, B, H, N, dtype=dtype)
    mask = W.random_mask(N + B, B, H, N // 128, N // 64, frac)
    _, _, alpha = W.random_weights(N + B, H, N // 128, alpha_lo=0.05)
    dO = W.grad_out(N + B, q.shape)
    say("backward ragged", q.shape, dtype)
    check(q, k, v, mask, alpha, dO, dtype, [(b, h) for b in range(B) for h in range(H)])


def test_backward_two_batches_fp32():
    """B = 2 (alpha shared by the batches, dalpha per batch), fp32 inputs, N = 1024."""
    B, H, N = 2, 2, 1024
    q, k, v = W.random_qkv(96, B, H, N)
    mask = W.random_mask(96, B, H, N // 128, N // 64, 0.25)
    _, _, alpha = W.random_weights(96, H, N // 128, alpha_lo=0.1)
    dO = W.grad_out(96, q.shape)
    say("backward two batches")
    check(q, k, v, mask, alpha, dO, "fp32", [(0, 1), (1, 0), (1, 1)])


def test_backward_long_key_lists():
    """Key blocks kept by every query block (64 of them at N = 8192): their lists are cut into
    work items of 16 query blocks whose partial sums are added back in a fixed order."""
    B, H, N = 1, 1, 8192
    q, k, v = W.random_qkv(95, B, H, N, dtype="bf16")
    mask = W.random_mask(95, B, H, N // 128, N // 64, 0.05)
    mask[:, :, :, 3] = 1
    mask[:, :, :, 77] = 1
    mask[:, :, 5, :] = 1
    _, _, alpha = W.random_weights(95, H, N // 128, alpha_lo=0.1)
    dO = W.grad_out(95, q.shape)
    say("backward long key lists")
    check(q, k, v, mask, alpha, dO, "bf16", [(0, 0)])


@pytest.mark.parametrize("fill", [0, 1])
def test_backward_uniform_masks(fill):
    """Every block dropped (pure linear attention) or every block kept (full attention)."""
    B, H, N = 1, 2, 1024
    q, k, v = W.random_qkv(92 + fill, B, H, N, dtype="bf16")
    mask = np.full((B, H, N // 128, N // 64), fill, np.uint8)
    _, _, alpha = W.random_weights(92, H, N // 128, alpha_lo=0.1)
    dO = W.grad_out(92, q.shape)
    say("backward uniform mask", fill)
    check(q, k, v, mask, alpha, dO, "bf16", [(0, 0), (0, 1)])


@pytest.mark.parametrize("a", [0.0, 1.0])
def test_backward_alpha_extremes(a):
    """alpha = 0 (linear branch only) and alpha = 1 (sparse branch only)."""
    B, H, N = 1, 1, 1024
    q, k, v = W.random_qkv(94, B, H, N, dtype="bf16")
    mask = W.random_mask(94, B, H, N // 128, N // 64, 0.3)
    alpha = np.full((H, N // 128), a, np.float32)
    dO = W.grad_out(94, q.shape)
    say("backward alpha", a)
    check(q, k, v, mask, alpha, dO, "bf16", [(0, 0)])


@pytest.mark.parametrize("name,heads", [("tiny_iid_N2048", None), ("grid_8x32x32_N8192", [1, 8])])
def test_backward_router_masks(name, heads):
    """The masks the router gives on the synthetic workloads (ragged kept lists per key block)."""
    w = W.WORKLOADS[name]
    q, k, v = W.generate(w, heads=heads)
    wq, wk, alpha = W.weights(w)
    if heads is not None:
        wq, wk, alpha = wq[heads], wk[heads], alpha[heads]
    mask = oracle_router_masks(q, k, wq, wk, w.keep_frac[0])
    dO = W.grad_out(w.seed, q.shape)
    say("backward router mask", name, q.shape)
    B, H = q.shape[:2]
    check(q, k, v, mask, alpha, dO, w.dtype, [(b, h) for b in range(B) for h in range(H)])


@pytest.mark.timeout(600)
def test_backward_benchmark_size_and_determinism():
    """The Wan2.1-1.3B 480P-shaped workload (12 heads, N = 32768, 3 % kept, the router's mask):
    two heads against the oracle; a second call gives identical bits."""
    w = W.WORKLOADS["wan13b_480p_N32768"]
    q, k, v = W.generate(w)
    wq, wk, alpha = W.weights(w)
    t = TDT[w.dtype]
    g = [dev(q, t), dev(k, t), dev(v, t)]
    mask = oracle_router_masks(q, k, wq, wk, w.keep_frac[-1])
    dO = W.grad_out(w.seed, q.shape)
    ga, gd, gm = dev(alpha), dev(dO), dev(mask, torch.uint8)
    first = sla2.sla2_backward(*g, gm, ga, gd)
    second = sla2.sla2_backward(*g, gm, ga, gd)
    torch.cuda.synchronize()
    for x, y in zip(first, second):
        assert torch.equal(x, y)
    got = [host(x) for x in first]
    say("backward bench size")
    for b, h in [(0, 3), (0, 10)]:
        r = bw.backward(q[b, h], k[b, h], v[b, h], mask[b, h], alpha[h], dO[b, h])
        errs = [rel_l2(x[b, h], r[n]) for x, n in zip(got, NAMES)]
        say(f"  b{b} h{h}: " + ", ".join(f"{n} {e:.2e}" for n, e in zip(NAMES, errs)))
        assert max(errs) <= TOL


@pytest.mark.timeout(900)
def test_backward_wan14b_full_size():
    """The largest shape: B = 1, H = 40, N = 75648 (591 query blocks, 1182 key blocks), 5 %
    kept, the (oracle) router's mask; every head in one call, one head against the oracle."""
    w = W.WORKLOADS["wan14b_720p_N75648"]
    q, k, v = W.generate(w)
    wq, wk, alpha = W.weights(w)
    t = TDT[w.dtype]
    g = [dev(q, t), dev(k, t), dev(v, t)]
    mask = oracle_router_masks(q, k, wq, wk, w.keep_frac[0])
    dO = W.grad_out(w.seed, q.shape)
    got = [host(x) for x in sla2.sla2_backward(*g, dev(mask, torch.uint8), dev(alpha), dev(dO))]
    for x in got:
        assert np.isfinite(x).all()
    b, h = 0, 27
    say("backward wan14b: oracle on one head")
    r = bw.backward(q[b, h], k[b, h], v[b, h], mask[b, h], alpha[h], dO[b, h])
    errs = [rel_l2(x[b, h], r[n]) for x, n in zip(got, NAMES)]
    say(f"  b{b} h{h}: " + ", ".join(f"{n} {e:.2e}" for n, e in zip(NAMES, errs)))
    assert max(errs) <= TOL


@pytest.mark.parametrize("row", [(1, 0), (0, 1), (1, 1), (0, 0)])
def test_backward_smallest_shape(row):
    """N = 128: one query block, two key blocks, every mask row (one kept, the other kept,
    both kept: no linear branch, none kept: no sparse branch); bf16 inputs."""
    B, H, N = 1, 1, 128
    q, k, v = W.random_qkv(97, B, H, N, dtype="bf16")
    mask = np.array(row, np.uint8).reshape(1, 1, 1, 2)
    alpha = np.full((H, 1), 0.6, np.float32)
    dO = W.grad_out(97, q.shape)
    say("backward N=128, mask row", row)
    check(q, k, v, mask, alpha, dO, "bf16", [(0, 0)])
