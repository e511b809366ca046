"""The library's largest sequence length, N = 262144 (2048 query blocks, 4096 key blocks), one
head: the full forward (router, codecs, both branches) and the backward against the oracle.

A key block index then needs 12 bits and a query block index 11, the router selects from 4096
candidates per row, and the backward's key lists reach 2048 entries (one key block kept by
every query block). Tolerances are the ones of the other parity tests: forward O within
relative L2 3e-3 and max-abs 2e-2 of the oracle's own forward on the query blocks whose kept
sets agree, masks within the 1e-5 near-tie band; gradients within relative L2 2e-2 (the bf16
backward's bound).
"""
import sys

import numpy as np
import pytest
import torch

from block_sparse_linear_pool_amd import sla2
from block_sparse_linear_pool_amd import workloads as W
from oracle import sla2 as oracle
from oracle import sla2_backward as oracle_bwd
from tests.gpu_helpers import (MAX_ABS_TOL, REL_L2_TOL, check_mask_band, dev, host, rel_l2,
                               row_errors, rows_agreeing)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

N = 262144
NQB, NKB = N // 128, N // 64
SEED = 211


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def inputs():
    q, k, v = W.random_qkv(SEED, 1, 1, N, dtype="bf16")
    wq, wk, alpha = W.random_weights(SEED, 1, NQB)
    return q, k, v, wq, wk, alpha


@pytest.mark.timeout(600)
def test_forward_max_n():
    """sla2_forward at N = 262144 with 0.2 % kept (9 of 4096 key blocks per row)."""
    q, k, v, wq, wk, alpha = inputs()
    keep = 0.002
    kb = oracle.kept_blocks(NKB, keep)
    g = [dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16)]
    say("forward N=262144: GPU")
    O = sla2.sla2_forward(*g, dev(wq), dev(wk), dev(alpha), keep)
    _, mask, _ = sla2.sla2_router(g[0], g[1], dev(wq), dev(wk), keep)
    torch.cuda.synchronize()
    O, mask = host(O), host(mask)
    assert np.isfinite(O).all()
    say("forward N=262144: oracle")
    r = oracle.forward_head(q[0, 0], k[0, 0], v[0, 0], wq[0], wk[0], alpha[0], keep, quant=True)
    differ = check_mask_band(r["P_c"], kb, mask[0, 0])
    rows = rows_agreeing(mask[0, 0], r["mask"])
    say(f"  rows whose kept set differs inside the tie band: {differ} of {NQB}")
    e, m = row_errors(O[0, 0], r["O"], rows)
    say(f"  O relL2 {e:.2e} maxabs {m:.2e} on {int(rows.sum())} query blocks")
    assert rows.mean() >= 0.9
    assert e <= REL_L2_TOL and m <= MAX_ABS_TOL


def test_backward_max_n():
    """sla2_backward at N = 262144: a random mask (about two kept blocks per row) plus an
    all-kept query block, an all-dropped one and a key block kept by every query block.

    The oracle's plain sums over the dropped blocks of every row and column make a full head at
    this size take hours on a host, so the oracle checks samples (backward_spot: the same steps
    restricted to some blocks, dropped sums taken as total minus kept): dQ and dalpha of query
    blocks 0, 5 (all kept), 6 (all dropped), 1000 and 2047, dV of key blocks 0, 777 (kept by
    every query block but 6), 2000 and 4095. Properties that hold at any size cover the rest:
    the gradients are linear in dO for a fixed mask (two calls add up to the call on the sum,
    within the bf16 rounding of the operands), the key gradient of the mean-centred keys sums
    to zero over the keys, and everything is finite."""
    q, k, v, _, _, alpha = inputs()
    mask = W.random_mask(SEED, 1, 1, NQB, NKB, 2.0 / NKB)
    mask[0, 0, 5, :] = 1
    mask[0, 0, 6, :] = 0
    mask[0, 0, :, 777] = 1
    mask[0, 0, 6, 777] = 0
    d1 = W.grad_out(SEED, q.shape)
    d2 = W.grad_out(SEED + 1, q.shape)
    g = [dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16),
         dev(mask, torch.uint8), dev(alpha)]
    say("backward N=262144: three calls")
    r1 = [host(x) for x in sla2.sla2_backward(*g, dev(d1))]
    r2 = [host(x) for x in sla2.sla2_backward(*g, dev(d2))]
    r12 = [host(x) for x in sla2.sla2_backward(*g, dev(d1 + d2))]
    torch.cuda.synchronize()
    for x in r1 + r2 + r12:
        assert np.isfinite(x).all()
    names = ("dQ", "dK", "dV", "dalpha")
    errs = [rel_l2(c, a + b) for a, b, c in zip(r1, r2, r12)]
    say("  linearity: " + ", ".join(f"{n} {e:.2e}" for n, e in zip(names, errs)))
    assert max(errs) <= 2e-2
    say("backward N=262144: oracle samples")
    qb, kb = [0, 5, 6, 1000, 2047], [0, 777, 2000, 4095]
    spot = oracle_bwd.backward_spot(q[0, 0], k[0, 0], v[0, 0], mask[0, 0], alpha[0], d1[0, 0],
                                    qb, kb)
    da_scale = max(abs(x) for x in spot["dalpha"].values())
    for i in qb:
        e = rel_l2(r1[0][0, 0, 128 * i:128 * (i + 1)], spot["dQ"][i])
        ea = abs(float(r1[3][0, 0, i]) - spot["dalpha"][i]) / da_scale
        say(f"  query block {i}: dQ relL2 {e:.2e}, dalpha err {ea:.2e} (of the largest)")
        assert e <= 2e-2 and ea <= 2e-2
    for j in kb:
        e = rel_l2(r1[2][0, 0, 64 * j:64 * (j + 1)], spot["dV"][j])
        say(f"  key block {j}: dV relL2 {e:.2e}")
        assert e <= 2e-2
    for dK in (r1[1], r12[1]):
        col = np.abs(dK[0, 0].astype(np.float64).sum(axis=0)).max()
        scale = np.abs(dK[0, 0]).astype(np.float64).sum(axis=0).max()
        say(f"  dK column sums: max {col:.2e} (sum of magnitudes {scale:.2e})")
        assert col <= 1e-4 * scale
