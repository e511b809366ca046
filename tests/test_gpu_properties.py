"""Properties the forward and backward must have exactly, checked on every row of the 12-head
N = 32768 workload through the C ABI (the oracle's per-head cost limits its own checks there to
sampled heads and rows).

- Scaling V by 2 scales O by 2 bit for bit: every step that touches V commutes with an exact
  power-of-two scale (bf16 inputs; the E4M3 codes of V are unchanged because the block scale
  doubles with the block's absolute maximum; h_j, H_tot, the accumulator's units and N_l
  double; the softmax weights, phi and the normaliser do not depend on V), quantised and
  unquantised.
- The backward is linear in the upstream gradient: 2 dO gives twice every gradient, bit for bit.
- Relabelling the heads (Q, K, V, the projections and alpha together) relabels the outputs bit
  for bit: every (batch, head) slice is computed on its own, whatever workgroup takes it.
"""
import numpy as np
import pytest
import torch

from block_sparse_linear_pool_amd import sla2
from block_sparse_linear_pool_amd import workloads as W
from tests.gpu_helpers import dev, host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def inputs():
    w = W.WORKLOADS["wan13b_480p_N32768"]
    q, k, v = W.generate(w)
    wq, wk, alpha = W.weights(w)
    return w, q, k, v, wq, wk, alpha


@pytest.mark.timeout(600)
@pytest.mark.parametrize("quant", ["i8_fp8", "none"])
def test_scaling_v_scales_o_exactly(quant):
    w, q, k, v, wq, wk, alpha = inputs()
    keep = w.keep_frac[-1]
    t = torch.bfloat16
    g = [dev(q, t), dev(k, t)]
    gv = dev(v, t)
    rest = [dev(wq), dev(wk), dev(alpha)]
    o1 = sla2.sla2_forward(g[0], g[1], gv, *rest, keep, quant=quant)
    o2 = sla2.sla2_forward(g[0], g[1], gv * 2, *rest, keep, quant=quant)
    torch.cuda.synchronize()
    o1, o2 = host(o1), host(o2)
    assert np.isfinite(o1).all() and np.abs(o1).max() > 0
    assert np.array_equal(o2, 2 * o1)


@pytest.mark.timeout(600)
def test_head_relabelling_relabels_outputs_exactly():
    w, q, k, v, wq, wk, alpha = inputs()
    keep = w.keep_frac[-1]
    perm = np.random.default_rng(5).permutation(w.H)
    t = torch.bfloat16
    o1 = sla2.sla2_forward(dev(q, t), dev(k, t), dev(v, t), dev(wq), dev(wk), dev(alpha), keep)
    o2 = sla2.sla2_forward(dev(q[:, perm], t), dev(k[:, perm], t), dev(v[:, perm], t),
                           dev(wq[perm]), dev(wk[perm]), dev(alpha[perm]), keep)
    _, m1, _ = sla2.sla2_router(dev(q, t), dev(k, t), dev(wq), dev(wk), keep)
    _, m2, _ = sla2.sla2_router(dev(q[:, perm], t), dev(k[:, perm], t), dev(wq[perm]),
                                dev(wk[perm]), keep)
    torch.cuda.synchronize()
    assert np.array_equal(host(m2), host(m1)[:, perm])
    assert np.array_equal(host(o2), host(o1)[:, perm])


@pytest.mark.timeout(600)
def test_backward_is_linear_in_the_upstream_gradient_exactly():
    """dQ, dK, dV and dalpha of 2 dO are twice those of dO bit for bit (the bf16 copy of
    alpha dO, every product, D, the centring of dK and the linear branch's terms all commute
    with the exact scale), for the router's own mask on the full workload."""
    w, q, k, v, wq, wk, alpha = inputs()
    keep = w.keep_frac[-1]
    t = torch.bfloat16
    g = [dev(q, t), dev(k, t), dev(v, t)]
    _, mask, _ = sla2.sla2_router(g[0], g[1], dev(wq), dev(wk), keep)
    do = dev(W.grad_out(w.seed, q.shape))
    a = dev(alpha)
    r1 = [host(x) for x in sla2.sla2_backward(*g, mask, a, do)]
    r2 = [host(x) for x in sla2.sla2_backward(*g, mask, a, do * 2)]
    for x1, x2 in zip(r1, r2):
        assert np.isfinite(x1).all() and np.abs(x1).max() > 0
        assert np.array_equal(x2, 2 * x1)
