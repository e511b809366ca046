"""GPU parity of the paths the headline workload does not reach (through the C ABI).

- The unquantised sparse branch (SLA2_QUANT_NONE) against the oracle with quant=False: the tiny
  i.i.d. workload (fp32 inputs; the configuration that runs both variants) through the router
  and with the oracle's mask, and two heads of the 8x32x32 grid workload (bf16 inputs).
- Dense block masks through sla2_forward_with_mask at N = 16384 (256 key blocks a row): rows
  with 129, 200 and 255 kept blocks (past the 128 the attention kernel stages per row, so
  block indices and scales come from memory), rows 60-90 % kept (the linear branch then sums
  the dropped blocks directly instead of total minus kept), a full and an empty row.
- sla2_forward at keep 0.75 (the router's kept count above half of the row).
- The unquantised forward at the 12-head N = 32768 workload, all heads in one call.
- The workspace's error word: clear after every forward, reported when set.
"""
import sys

import numpy as np
import pytest
import torch

from block_sparse_linear_pool_amd import sla2
from block_sparse_linear_pool_amd import workloads as W
from oracle import sla2 as oracle
from tests.gpu_helpers import (MAX_ABS_TOL, REL_L2_TOL, check_mask_band, dev, host, max_abs,
                               oracle_heads, rel_l2, row_errors, rows_agreeing)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TDT = {"fp32": torch.float32, "bf16": torch.bfloat16}
# O_s of the unquantised branch: fp32 products and sums over 128-term dot products and up to
# 64 kb terms per output; each rounding is 2^-24 relative, so the relative L2 error stays
# around 1e-6. The bound leaves a factor 10.
EXACT_OS_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def load(name, heads=None):
    w = W.WORKLOADS[name]
    q, k, v = W.generate(w, heads=heads)
    wq, wk, alpha = W.weights(w)
    if heads is not None:
        wq, wk, alpha = wq[heads], wk[heads], alpha[heads]
    t = TDT[w.dtype]
    g = (dev(q, t), dev(k, t), dev(v, t), dev(wq), dev(wk), dev(alpha))
    return w, (q, k, v, wq, wk, alpha), g


# ------------------------------------------------------------------ SLA2_QUANT_NONE
@pytest.mark.parametrize("name,heads", [("tiny_iid_N2048", None), ("grid_8x32x32_N8192", [4, 10])])
def test_unquantised_forward_with_oracle_mask(name, heads):
    w, (q, k, v, wq, wk, alpha), g = load(name, heads)
    keep = w.keep_frac[0]
    say("unquantised with mask", name, q.shape, keep)
    ref = oracle_heads(q, k, v, wq, wk, alpha, keep, quant=False)
    B, H = q.shape[:2]
    mask = np.zeros((B, H, w.n_qb, w.n_kb), np.uint8)
    for (b, h), r in ref.items():
        mask[b, h] = r["mask"]
    O, taps = sla2.sla2_forward_with_mask(g[0], g[1], g[2], dev(mask, torch.uint8), g[5],
                                          taps=("O_s", "O_l"), quant="none")
    torch.cuda.synchronize()
    O, Os, Ol = host(O), host(taps["O_s"]), host(taps["O_l"])
    for (b, h), r in ref.items():
        e_s, e_l, e_o = rel_l2(Os[b, h], r["O_s"]), rel_l2(Ol[b, h], r["O_l"]), rel_l2(O[b, h], r["O"])
        m_o = max_abs(O[b, h], r["O"])
        say(f"  b{b} h{h}: O_s {e_s:.2e} O_l {e_l:.2e} O relL2 {e_o:.2e} maxabs {m_o:.2e}")
        assert e_s <= EXACT_OS_TOL
        assert e_l <= 5e-3
        assert e_o <= REL_L2_TOL and m_o <= MAX_ABS_TOL


def test_unquantised_full_path_tiny():
    """sla2_forward with quant = none on the tiny workload: the router's mask (within the band),
    then O against the unquantised oracle's own forward on the query blocks whose kept sets
    agree; the quantised call on the same inputs differs from it by the codecs' error only."""
    w, (q, k, v, wq, wk, alpha), g = load("tiny_iid_N2048")
    keep = w.keep_frac[0]
    O = host(sla2.sla2_forward(*g, keep, quant="none"))
    Oq = host(sla2.sla2_forward(*g, keep))
    _, mask, _ = sla2.sla2_router(g[0], g[1], g[3], g[4], keep)
    mask = host(mask)
    ref = oracle_heads(q, k, v, wq, wk, alpha, keep, quant=False)
    for (b, h), r in ref.items():
        check_mask_band(r["P_c"], r["kb"], mask[b, h])
        rows = rows_agreeing(mask[b, h], r["mask"])
        assert rows.mean() >= 0.9
        e, m = row_errors(O[b, h], r["O"], rows)
        eq, _ = row_errors(Oq[b, h], r["O"], rows)
        say(f"  h{h}: unquantised O relL2 {e:.2e} maxabs {m:.2e}; quantised vs it {eq:.2e}")
        assert e <= REL_L2_TOL and m <= MAX_ABS_TOL
        assert e < eq < 0.08          # the low-bit call is further from the exact result


def test_unquantised_edge_rows():
    """Empty and full rows, a single kept block, alpha at 0 and 1, without quantisation."""
    N = 1024
    q, k, v = W.random_qkv(77, 1, 2, N)
    wq, wk, alpha = W.random_weights(77, 2, N // 128)
    alpha[0, 2], alpha[1, 3] = 0.0, 1.0
    rng = np.random.default_rng(7)
    mask = (rng.random((1, 2, 8, 16)) < 0.4).astype(np.uint8)
    mask[0, 0, 0] = 0
    mask[0, 0, 1] = 1
    mask[0, 1, 4] = 0
    mask[0, 1, 4, 9] = 1
    ref = oracle_heads(q, k, v, wq, wk, alpha, 0.5, mask=mask, quant=False)
    O, taps = sla2.sla2_forward_with_mask(dev(q), dev(k), dev(v), dev(mask, torch.uint8),
                                          dev(alpha), taps=("O_s",), quant="none")
    O, Os = host(O), host(taps["O_s"])
    assert not Os[0, 0, 0:128].any()
    for (b, h), r in ref.items():
        assert rel_l2(Os[b, h], r["O_s"]) <= EXACT_OS_TOL
        assert rel_l2(O[b, h], r["O"]) <= REL_L2_TOL and max_abs(O[b, h], r["O"]) <= MAX_ABS_TOL


# ------------------------------------------------------------------ dense masks
@pytest.mark.timeout(400)
def test_dense_masks_many_kept_blocks():
    """N = 16384, 256 key blocks a row: rows with 129, 200, 255 and 256 kept blocks, rows with
    60-90 % kept, an empty row; low-bit and unquantised."""
    N, H = 16384, 2
    q, k, v = W.random_qkv(91, 1, H, N, dtype="bf16")
    wq, wk, alpha = W.random_weights(91, H, N // 128, alpha_lo=0.2)
    nqb, nkb = N // 128, N // 64
    rng = np.random.default_rng(92)
    mask = np.zeros((1, H, nqb, nkb), np.uint8)
    for h in range(H):
        for i in range(nqb):
            frac = rng.uniform(0.6, 0.9)
            mask[0, h, i, rng.choice(nkb, int(frac * nkb), replace=False)] = 1
        for i, cnt in zip(range(0, 10, 2), (129, 200, 255, 256, 0)):
            mask[0, h, i] = 0
            mask[0, h, i, np.sort(rng.choice(nkb, cnt, replace=False))] = 1
    counts = mask.sum(-1)
    say("dense masks: kept per row", counts.min(), counts.max(), "rows > 128:", int((counts > 128).sum()))
    gq, gk, gv = (dev(a, torch.bfloat16) for a in (q, k, v))
    gm, ga = dev(mask, torch.uint8), dev(alpha)
    ws = sla2.workspace_for(gq, "forward_with_mask")
    for quant in ("i8_fp8", "none"):
        O = host(sla2.sla2_forward_with_mask(gq, gk, gv, gm, ga, workspace=ws, quant=quant))
        assert sla2.sla2_workspace_status(ws) == 0
        for h in range(H):
            r = oracle.forward_head(q[0, h], k[0, h], v[0, h], wq[h], wk[h], alpha[h], 0.5,
                                    quant=quant == "i8_fp8", mask=mask[0, h])
            e, m = rel_l2(O[0, h], r["O"]), max_abs(O[0, h], r["O"])
            say(f"  {quant} h{h}: O relL2 {e:.2e} maxabs {m:.2e}")
            assert e <= REL_L2_TOL and m <= MAX_ABS_TOL
            for i, cnt in zip(range(0, 10, 2), (129, 200, 255, 256, 0)):
                rows = slice(128 * i, 128 * (i + 1))
                er = rel_l2(O[0, h, rows], r["O"][rows])
                assert er <= REL_L2_TOL, (quant, h, cnt, er)


def test_forward_keep_three_quarters():
    """sla2_forward at keep 0.75 (24 of 32 key blocks kept): the linear branch sums the dropped
    blocks directly."""
    w, (q, k, v, wq, wk, alpha), g = load("tiny_iid_N2048")
    keep = 0.75
    O = host(sla2.sla2_forward(*g, keep))
    _, mask, _ = sla2.sla2_router(g[0], g[1], g[3], g[4], keep)
    mask = host(mask)
    assert (mask.sum(-1) == 24).all()
    ref = oracle_heads(q, k, v, wq, wk, alpha, keep, quant=True)
    for (b, h), r in ref.items():
        check_mask_band(r["P_c"], r["kb"], mask[b, h])
        rows = rows_agreeing(mask[b, h], r["mask"])
        assert rows.mean() >= 0.9
        e, m = row_errors(O[b, h], r["O"], rows)
        say(f"  keep 0.75 h{h}: O relL2 {e:.2e} maxabs {m:.2e}")
        assert e <= REL_L2_TOL and m <= MAX_ABS_TOL


# ------------------------------------------------------------------ error word
def test_workspace_error_word():
    """A forward clears the word and its bounded waits leave it clear; a word set by hand (the
    host's view of a wait that gave up) is reported, and the next forward clears it again."""
    w, _, g = load("tiny_iid_N2048")
    keep = w.keep_frac[0]
    ws = sla2.workspace_for(g[0], "forward", keep)
    sla2.sla2_forward(*g, keep, workspace=ws)
    assert sla2.sla2_workspace_status(ws) == 0
    ws[:4].view(torch.int32).fill_(1)
    assert sla2.sla2_workspace_status(ws) == 9
    sla2.sla2_forward(*g, keep, workspace=ws)
    assert sla2.sla2_workspace_status(ws) == 0


@pytest.mark.timeout(600)
def test_unquantised_bench_size():
    """sla2_forward with quant = none on the 12-head N = 32768 workload in one call: heads 2
    and 11 against the unquantised oracle's own forward (rows whose kept sets agree)."""
    w = W.WORKLOADS["wan13b_480p_N32768"]
    keep = w.keep_frac[-1]
    q, k, v = W.generate(w)
    wq, wk, alpha = W.weights(w)
    t = torch.bfloat16
    g = [dev(q, t), dev(k, t), dev(v, t), dev(wq), dev(wk), dev(alpha)]
    say("unquantised at the bench size")
    O, taps = sla2.sla2_forward(*g, keep, taps=("O_s",), quant="none")
    _, mask, _ = sla2.sla2_router(g[0], g[1], g[3], g[4], keep)
    torch.cuda.synchronize()
    O, Os, mask = host(O), host(taps["O_s"]), host(mask)
    for h in (2, 11):
        r = oracle.forward_head(q[0, h], k[0, h], v[0, h], wq[h], wk[h], alpha[h], keep,
                                quant=False)
        check_mask_band(r["P_c"], r["kb"], mask[0, h])
        rows = rows_agreeing(mask[0, h], r["mask"])
        assert rows.mean() >= 0.9
        e_s, _ = row_errors(Os[0, h], r["O_s"], rows)
        e, m = row_errors(O[0, h], r["O"], rows)
        say(f"  h{h}: O_s relL2 {e_s:.2e}; O relL2 {e:.2e} maxabs {m:.2e}")
        assert e_s <= EXACT_OS_TOL
        assert e <= REL_L2_TOL and m <= MAX_ABS_TOL
