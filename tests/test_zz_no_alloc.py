"""The allocation-free router entry point, sla2_router_noalloc, against sla2_router (GPU,
through the C ABI). Both run the same kernels on the same inputs, so block lists, masks and
scores must be identical (index work: bit for bit). Two calls in a row share the GPU's static
scratch: the first at the 12-head N = 32768 workload (14 MB of the 32 MiB scratch), the second
smaller (the 2-head N = 2048 workload), which must not see the first call's leftovers."""
import sys

import numpy as np
import pytest
import torch

from block_sparse_linear_pool_amd import sla2
from block_sparse_linear_pool_amd import workloads as W
from tests.gpu_helpers import dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def inputs(name):
    w = W.WORKLOADS[name]
    q, k, v = W.generate(w)
    wq, wk, alpha = W.weights(w)
    t = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return w, dev(q, t), dev(k, t), dev(wq), dev(wk)


def test_noalloc_router_equals_router_on_two_calls():
    sla2.sla2_init_device()
    for name in ("wan13b_480p_N32768", "tiny_iid_N2048"):
        w, q, k, wq, wk = inputs(name)
        keep = w.keep_frac[-1]
        need = sla2.sla2_workspace_bytes(w.B, w.H, w.N, q.dtype, "router")
        say(name, "router workspace bytes", need, "of", sla2.NOALLOC_SCRATCH_BYTES)
        assert need <= sla2.NOALLOC_SCRATCH_BYTES
        ref_b, ref_m, ref_s = sla2.sla2_router(q, k, wq, wk, keep, want_scores=True)
        blocks = torch.full_like(ref_b, -7)
        mask = torch.full_like(ref_m, 9)
        scores = torch.full_like(ref_s, float("nan"))
        sla2.sla2_router_noalloc(q, k, wq, wk, keep, blocks, mask, scores)
        torch.cuda.synchronize()
        assert torch.equal(blocks, ref_b)
        assert torch.equal(mask, ref_m)
        assert torch.equal(scores, ref_s)
        # the lists only (mask and scores not requested)
        b2 = torch.full_like(ref_b, -7)
        sla2.sla2_router_noalloc(q, k, wq, wk, keep, b2)
        torch.cuda.synchronize()
        assert torch.equal(b2, ref_b)
        say(name, "identical;", int((ref_m.sum(-1) == ref_b.shape[-1]).all()))


def test_noalloc_router_rejects_a_shape_beyond_the_scratch():
    q = torch.zeros((1, 40, 75648, 128), dtype=torch.bfloat16, device="cuda:0")
    w = torch.zeros((40, 128, 128), device="cuda:0")
    blocks = torch.zeros((1, 40, 591, 59), dtype=torch.int32, device="cuda:0")
    with pytest.raises(sla2.SLA2Error) as e:
        sla2.sla2_router_noalloc(q, q, w, w, 0.05, blocks)
    assert e.value.status == 6
