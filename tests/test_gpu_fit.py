"""Stage-1 alpha fit on the GPU (sla2_fit_alpha, through the C ABI) against the oracle's fit
(oracle/sla2_fit.py), and its consistency with the backward.

Tolerances. On the same fp32 taps both sides sum in fp64, so the GPU's alpha (rounded to fp32)
is within 1e-6 of the oracle's. End to end, the taps come from each side's own forward (parity
3e-3 relative L2), so alpha, a ratio of inner products of those taps, is held to 2e-2 absolute.
At the fitted alpha the loss is at its minimum, so the backward's dalpha for dO = 2 (O - O_full)
must be small next to its change over a step of 0.1 in alpha (the loss's curvature), up to the
straight-through gap between the quantised taps and the unquantised gradient.
"""
import sys

import numpy as np
import pytest
import torch

from block_sparse_linear_pool_amd import sla2
from block_sparse_linear_pool_amd import workloads as W
from oracle import sla2 as oracle
from oracle import sla2_fit as fit
from tests.gpu_helpers import check_mask_band, dev, host, rows_agreeing

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_fit_matches_oracle_on_given_taps():
    B, H, N, D = 2, 3, 512, 128
    rng = np.random.default_rng(101)
    O_s = rng.standard_normal((B, H, N, D)).astype(np.float32)
    O_l = rng.standard_normal((B, H, N, D)).astype(np.float32)
    O_full = (0.6 * O_s + 0.4 * O_l + 0.5 * rng.standard_normal((B, H, N, D))).astype(np.float32)
    O_full[:, 0, :128] = 1.5 * O_s[:, 0, :128] - 0.5 * O_l[:, 0, :128]        # clipped to 1
    O_full[:, 1, 128:256] = -0.3 * O_s[:, 1, 128:256] + 1.3 * O_l[:, 1, 128:256]   # clipped to 0
    O_l[:, 2, 384:] = O_s[:, 2, 384:]                                         # branches agree: 1
    got = host(sla2.sla2_fit_alpha(dev(O_full), dev(O_s), dev(O_l)))
    ref = fit.fit_alpha(O_full, O_s, O_l)
    say("alpha", np.round(got, 4).tolist())
    assert np.abs(got - ref).max() <= 1e-6
    assert got[0, 0] == 1.0 and got[1, 1] == 0.0 and got[2, 3] == 1.0


def test_fit_end_to_end_and_backward_at_the_minimum():
    w = W.WORKLOADS["tiny_iid_N2048"]
    q, k, v = W.generate(w)
    wq, wk, _ = W.weights(w)
    keep = w.keep_frac[0]
    B, H, N, D = q.shape
    g = [dev(q), dev(k), dev(v)]
    eye = dev(np.broadcast_to(np.eye(D, dtype=np.float32), (H, D, D)).copy())
    ones = dev(np.ones((H, N // 128), np.float32))
    O_full = sla2.sla2_forward(*g, eye, eye, ones, 1.0)          # every block kept: full attention
    _, taps = sla2.sla2_forward(*g, dev(wq), dev(wk), ones, keep, taps=("O_s", "O_l"))
    a_gpu = sla2.sla2_fit_alpha(O_full, taps["O_s"], taps["O_l"])
    _, mask, _ = sla2.sla2_router(g[0], g[1], dev(wq), dev(wk), keep)
    torch.cuda.synchronize()
    mask_h = host(mask)
    # the oracle's own pipeline; alpha of a query block depends only on that block's mask row,
    # so it is compared where the GPU's kept set is the oracle's (near-tie rows aside)
    Of, Os, Ol = (np.empty((B, H, N, D)) for _ in range(3))
    agree = np.zeros((H, N // 128), bool)
    for h in range(H):
        r1 = oracle.forward_head(q[0, h], k[0, h], v[0, h], np.eye(D), np.eye(D), np.ones(N // 128),
                                 1.0)
        r = oracle.forward_head(q[0, h], k[0, h], v[0, h], wq[h], wk[h], np.ones(N // 128), keep)
        check_mask_band(r["P_c"], r["kb"], mask_h[0, h])
        agree[h] = rows_agreeing(mask_h[0, h], r["mask"])
        Of[0, h], Os[0, h], Ol[0, h] = r1["O"], r["O_s"], r["O_l"]
    a_ref = fit.fit_alpha(Of, Os, Ol)
    a = host(a_gpu)
    say("alpha gpu", np.round(a, 3).tolist())
    say("alpha ref", np.round(a_ref, 3).tolist())
    assert agree.mean() >= 0.9
    assert np.abs(a - a_ref)[agree].max() <= 2e-2
    # reported, not asserted (the pages only say "close to"): the kept row mass P_1 1 per
    # query block, from the oracle's exact softmax over all keys
    mass = np.zeros((H, N // 128))
    for h in range(H):
        Ks = oracle.smooth_k(k[0, h], oracle.colmean(k[0, h])[1])
        P = oracle.softmax_rows(np.asarray(q[0, h], np.float64) @ Ks.T / np.sqrt(D))
        M = np.kron(mask_h[0, h], np.ones((128, 64)))
        mass[h] = (P * M).sum(axis=1).reshape(N // 128, 128).mean(axis=1)
    say("kept row mass", np.round(mass, 3).tolist())
    # backward at alpha* and alpha* + 0.1 with dO = 2 (O - O_full)
    def dalpha(alpha):
        O = sla2.sla2_forward_with_mask(*g, mask, dev(alpha))
        dO = 2.0 * (O - O_full)
        _, _, _, da = sla2.sla2_backward(*g, mask, dev(alpha), dO.contiguous())
        torch.cuda.synchronize()
        return host(da).sum(axis=0)
    g0 = dalpha(a)
    g1 = dalpha(np.minimum(a + 0.1, 1.0).astype(np.float32))
    inner = (a > 0.05) & (a < 0.85)
    say("interior blocks", int(inner.sum()), "max |g0| / |g1 - g0|",
        float(np.max(np.abs(g0[inner]) / np.abs(g1[inner] - g0[inner]))))
    assert inner.any()
    assert np.all(np.abs(g0[inner]) <= 0.25 * np.abs(g1[inner] - g0[inner]))


@pytest.mark.timeout(300)
def test_fit_full_size_two_batches():
    """The bench's shape with two batches (B = 2, H = 12, N = 32768: 256 query blocks a head),
    per-block mixing weights drawn from [-0.3, 1.3] so that about three in eight are clipped."""
    B, H, N, D = 2, 12, 32768, 128
    nqb = N // 128
    rng = np.random.default_rng(103)
    O_s = rng.standard_normal((B, H, N, D), dtype=np.float32)
    O_l = rng.standard_normal((B, H, N, D), dtype=np.float32)
    a = np.repeat(rng.uniform(-0.3, 1.3, (1, H, nqb)), 128, axis=2)[..., None].astype(np.float32)
    O_full = a * O_s + (1 - a) * O_l + 0.3 * rng.standard_normal((B, H, N, D), dtype=np.float32)
    got = host(sla2.sla2_fit_alpha(dev(O_full), dev(O_s), dev(O_l)))
    ref = fit.fit_alpha(O_full, O_s, O_l)
    clipped = int(((ref == 0.0) | (ref == 1.0)).sum())
    say(f"full size: max |alpha - oracle| {np.abs(got - ref).max():.2e}, {clipped} of {H * nqb} clipped")
    assert np.abs(got - ref).max() <= 1e-6
    assert clipped > 0
