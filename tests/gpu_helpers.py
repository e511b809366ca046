"""Shared helpers of the GPU parity tests: device copies, the oracle per head, comparisons."""
from __future__ import annotations

import numpy as np
import torch

from oracle import sla2 as oracle

REL_L2_TOL = 3e-3      # O against the oracle (relative L2)
MAX_ABS_TOL = 2e-2     # O against the oracle (max abs)
BAND = 1e-5            # router near-tie band (relative, in P_c)


def dev(arr, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device="cuda:0", dtype=dtype)


def host(t):
    return t.detach().to("cpu").numpy()


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def oracle_heads(q, k, v, wq, wk, alpha, keep, heads=None, mask=None, quant=True):
    """Oracle forward for each (b, h) in `heads` (default all); returns {(b, h): result dict}."""
    B, H = q.shape[:2]
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    out = {}
    for b, h in heads:
        m = None if mask is None else mask[b, h]
        out[(b, h)] = oracle.forward_head(q[b, h], k[b, h], v[b, h], wq[h], wk[h], alpha[h],
                                          keep, quant=quant, mask=m)
    return out


def oracle_router_masks(q, k, wq, wk, keep):
    """The oracle router's hard Top-k masks [B, H, N/128, N/64] (uint8): the input mask of the
    backward tests, given to the GPU and to the oracle alike."""
    B, H, N, _ = q.shape
    kb = oracle.kept_blocks(N // 64, keep)
    out = np.zeros((B, H, N // 128, N // 64), np.uint8)
    for b in range(B):
        for h in range(H):
            _, mu32 = oracle.colmean(k[b, h])
            ks = oracle.smooth_k(k[b, h], mu32)
            _, P = oracle.router_scores(oracle.block_mean(np.asarray(q[b, h], np.float64), 128),
                                        oracle.block_mean(ks, 64), wq[h], wk[h])
            out[b, h] = oracle.topk_blocks(P, kb)[0]
    return out


def rows_agreeing(gpu_mask, oracle_mask):
    """Query blocks whose GPU kept set is the oracle's own. A row block of O depends only on its
    own mask row (its kept list in the sparse branch, its dropped set in the linear one), so
    there the oracle's rows, computed with its own router, are the expected values. Rows whose
    sets differ are held to the near-tie band (check_mask_band); their outputs are not compared,
    since the oracle takes no input from the GPU."""
    return ((np.asarray(gpu_mask) != 0) == (np.asarray(oracle_mask) != 0)).all(axis=-1)


def row_errors(got, ref, rows):
    """rel L2 and max-abs of got against ref over the 128-row blocks selected by `rows`."""
    sel = np.repeat(np.asarray(rows, bool), 128)
    return rel_l2(np.asarray(got)[sel], np.asarray(ref)[sel]), max_abs(np.asarray(got)[sel],
                                                                        np.asarray(ref)[sel])


def check_mask_band(P, kb, gpu_mask):
    """Router contract: the GPU kept set has kb members per row, holds every block whose
    P_c exceeds the oracle's kb-th largest T by more than 1e-5 relative and no block below
    T by more than that. Returns the number of rows that differ from the oracle's set."""
    n_qb, n_kb = P.shape
    gm = np.asarray(gpu_mask) != 0
    assert (gm.sum(1) == kb).all(), "kept count per row differs from kb"
    differ = 0
    for i in range(n_qb):
        T = np.sort(P[i])[::-1][kb - 1]
        must = P[i] > T * (1 + BAND)
        never = P[i] < T * (1 - BAND)
        assert gm[i][must].all(), f"row {i}: a block above the band was dropped"
        assert not gm[i][never].any(), f"row {i}: a block below the band was kept"
        ref = np.zeros(n_kb, bool)
        ref[sorted(range(n_kb), key=lambda j: (-P[i, j], j))[:kb]] = True
        differ += int((ref != gm[i]).any())
    return differ
