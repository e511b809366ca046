"""The C ABI on the host, no GPU: the library loads, exports what include/sla2.h declares,
and rejects every bad argument with its status code before anything is enqueued."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from block_sparse_linear_pool_amd import sla2
from oracle import sla2 as oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, DTYPE, MISAL, ARG, WS, DEV, HIP, TIMEOUT = range(10)
E = sla2.ENTRY

A = 0x10000          # fake 16-byte-aligned "device" addresses: never dereferenced
MIS = 0x10008


def declared_functions():
    text = open(os.path.join(ROOT, "include", "sla2.h")).read()
    return sorted(set(re.findall(r"\b(sla2_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = sla2.lib()
    names = declared_functions()
    assert set(names) == {"sla2_blocks_kept", "sla2_workspace_bytes", "sla2_workspace_status",
                          "sla2_init_device", "sla2_router_noalloc",
                          "sla2_status_string", "sla2_router", "sla2_router_soft",
                          "sla2_linear_precompute", "sla2_forward", "sla2_forward_sla1",
                          "sla2_forward_with_mask", "sla2_backward", "sla2_fit_alpha",
                          "sla2_router_grad"}
    for n in names:
        assert hasattr(L, n), n


def test_blocks_kept_matches_oracle_rule():
    rng = np.random.default_rng(0)
    for n_kb in (1, 2, 16, 32, 128, 512, 1182, 4096):
        for k in list(rng.random(50)) + [0.03, 0.05, 0.1, 0.2, 0.25, 0.3, 1.0, 1e-7]:
            k = float(np.float32(k))
            if k <= 0:
                continue
            assert sla2.sla2_blocks_kept(n_kb, k) == oracle.kept_blocks(n_kb, k), (n_kb, k)
    for bad in (0.0, -0.1, 1.0001, float("nan"), float("inf")):
        assert sla2.sla2_blocks_kept(512, bad) == -1
    assert sla2.sla2_blocks_kept(0, 0.5) == -1


def test_workspace_bytes():
    a = sla2.sla2_workspace_bytes(1, 12, 32768, keep_frac=0.03)
    b = sla2.sla2_workspace_bytes(2, 12, 32768, keep_frac=0.03)
    assert 0 < a < b
    assert sla2.sla2_workspace_bytes(1, 1, 100) == 0
    assert sla2.sla2_workspace_bytes(1, 1, 128, d=64) == 0
    assert sla2.sla2_workspace_bytes(1, 1, 262144 + 128) == 0
    assert sla2.sla2_workspace_bytes(256, 256, 128) == 0        # B*H > 65535
    assert sla2.sla2_workspace_bytes(1, 1, 1024, entry=8) == 0  # no such entry
    assert sla2.sla2_workspace_bytes(1, 1, 1024, entry=-1) == 0
    for bad in (0.0, 1.5, float("nan")):                          # keep_frac matters for these
        assert sla2.sla2_workspace_bytes(1, 1, 1024, entry="forward", keep_frac=bad) == 0
        assert sla2.sla2_workspace_bytes(1, 1, 1024, entry="forward_sla1", keep_frac=bad) == 0
        assert sla2.sla2_workspace_bytes(1, 1, 1024, entry="router_grad", keep_frac=bad) == 0
        assert sla2.sla2_workspace_bytes(1, 1, 1024, entry="router", keep_frac=bad) > 0
    for s in range(10):
        assert isinstance(sla2.sla2_status_string(s), str) and sla2.sla2_status_string(s)


def expected_forward_bytes(B, H, N, kb):
    """The forward's regions, from what its kernels keep (each rounded up to 256 bytes)."""
    up = lambda x: -(-x // 256) * 256
    BH, nqb, nkb, d = B * H, N // 128, N // 64, 128
    np_ = -(-nkb // 8)
    regions = [4, BH * nqb * d * 8, BH * nkb * d * 8, BH * d * 8, BH * d * 4,   # err, sums, mu
               BH * nkb * d * 4, BH * nqb * d * 4,                             # B, A (fp32)
               BH * nqb * nkb, BH * nqb * kb * 4, BH * nqb * 4,                # mask, lists, counts
               BH * N * d, BH * N * d, BH * nkb * 4, BH * nkb * 4,             # K, V codes, scales
               BH * nkb * d * d * 2, BH * d * d * 4, BH * d * 4,               # h_j^T bf16, totals
               BH * N * d, BH * nqb * 4,                                       # Q codes, scales
               BH * nkb * d * 4, BH * np_ * d * d * 4, BH * np_ * d * 4]       # z_j, partials
    return sum(up(r) for r in regions)


def test_workspace_bytes_per_entry_point():
    """Each entry point asks only for what its kernels use: at the 12-head N = 32768 shape with
    3 % kept the forward needs 0.42 GB, the backward 1.29 GB (its bf16 operand copies, dH_i^T and
    the work-item partials), the router 14 MB."""
    B, H, N = 1, 12, 32768
    kb = sla2.sla2_blocks_kept(N // 64, 0.03)
    size = {e: sla2.sla2_workspace_bytes(B, H, N, entry=e, keep_frac=0.03) for e in E}
    assert size["forward"] == expected_forward_bytes(B, H, N, kb)
    assert 0.41e9 < size["forward"] < 0.43e9
    assert size["router"] == size["router_soft"] < 15e6
    assert size["linear_precompute"] < size["forward"]
    assert size["forward_with_mask"] < size["forward"] + 4 * B * H * (N // 128) * (N // 64)
    assert size["forward_sla1"] > size["forward"]               # plus the alpha = 1 row
    assert size["backward"] > 3 * size["forward"]
    # the list stride of the forward is kb: more kept blocks, more bytes
    assert sla2.sla2_workspace_bytes(B, H, N, entry="forward", keep_frac=0.2) > size["forward"]
    # Wan-14B 720P shape: the forward needs 3.4 GB, not the backward's 10.5 GB
    f5 = sla2.sla2_workspace_bytes(1, 40, 75648, entry="forward", keep_frac=0.05)
    assert 3.2e9 < f5 < 3.6e9
    assert sla2.sla2_workspace_bytes(1, 40, 75648, entry="backward") > 2.5 * f5
    # the router gradient: the forward's regions, the soft mask, O, O_s, O_l (fp32), f16 copies
    # of K_s, V, phi(K_s), the mask gradient and the router part
    up = lambda x: -(-x // 256) * 256
    BH, nqb, nkb, d, E_ = B * H, N // 128, N // 64, 128, B * H * N * 128
    extra = [BH * nqb * nkb * 4, BH * nqb * 4, E_ * 4, E_ * 4, E_ * 4, E_ * 2, E_ * 2, E_ * 2,
             BH * nqb * nkb * 4, BH * nqb * 4, BH * nqb * d * 4, BH * nqb * d * 4,
             BH * nqb * nkb * 4, BH * nkb * d * 4]
    assert size["router_grad"] == size["forward"] + sum(up(r) for r in extra)


def shape(B=1, H=2, N=1024, d=128, dtype=1):
    return sla2.Shape(B, H, N, d, dtype)


def need(shp, entry, keep=0.25):
    return sla2.lib().sla2_workspace_bytes(ctypes.byref(shp), E[entry], keep)


def fwd(shp, q=A, k=A, v=A, wq=A, wk=A, alpha=A, keep=0.25, quant=1, O=A, taps=None, ws=A,
        wsb=None):
    if wsb is None:
        wsb = need(shp, "forward", keep if 0 < keep <= 1 else 1.0) if shp else 0
    return sla2.lib().sla2_forward(ctypes.byref(shp) if shp else None, q, k, v, wq, wk, alpha,
                                   keep, quant, O, ctypes.byref(taps) if taps else None, ws, wsb,
                                   None)


def test_forward_validation_codes():
    assert fwd(None) == NULL
    assert fwd(shape(d=64)) == SHAPE
    assert fwd(shape(N=1000)) == SHAPE
    assert fwd(shape(N=0)) == SHAPE
    assert fwd(shape(B=0)) == SHAPE
    assert fwd(shape(B=300, H=300)) == SHAPE
    assert fwd(shape(dtype=7)) == DTYPE
    assert fwd(shape(), q=None) == NULL
    assert fwd(shape(), alpha=None) == NULL
    assert fwd(shape(), O=None) == NULL
    assert fwd(shape(), v=MIS) == MISAL
    assert fwd(shape(), wk=MIS) == MISAL
    taps = sla2.Taps(O_s=MIS)
    assert fwd(shape(), taps=taps) == MISAL
    for bad in (0.0, 1.5, float("nan"), -1.0):
        assert fwd(shape(), keep=bad) == ARG
    assert fwd(shape(), quant=2) == ARG
    assert fwd(shape(), quant=-1) == ARG
    s = shape()
    assert fwd(s, wsb=need(s, "forward") - 1) == WS
    assert fwd(s, wsb=need(s, "router")) == WS                  # sized for another entry
    assert fwd(s, ws=None) == NULL
    assert fwd(s, ws=MIS) == MISAL


def test_other_entry_points_validate():
    L = sla2.lib()
    s = shape()
    big = need(s, "backward")   # the largest plan: serves every entry point's size check
    r = L.sla2_router(ctypes.byref(s), A, A, A, A, 0.25, None, None, None, A, big, None)
    assert r == NULL                                            # blocks is required
    r = L.sla2_router(ctypes.byref(s), A, A, A, A, 2.0, None, A, None, A, big, None)
    assert r == ARG
    r = L.sla2_router(ctypes.byref(s), A, A, A, A, 0.25, MIS, A, None, A, big, None)
    assert r == MISAL
    soft = L.sla2_router_soft
    assert soft(ctypes.byref(s), A, A, A, A, 0.25, 0.1, None, None, None, A, big, None) == NULL
    assert soft(ctypes.byref(s), A, A, A, A, 0.25, 0.0, A, None, None, A, big, None) == ARG   # tau > 0
    assert soft(ctypes.byref(s), A, A, A, A, 0.25, float("nan"), A, None, None, A, big, None) == ARG
    assert soft(ctypes.byref(s), A, A, A, A, 0.25, 1e-45, A, None, None, A, big, None) == ARG  # 1/tau inf
    assert soft(ctypes.byref(s), A, A, A, A, 1.5, 0.1, A, None, None, A, big, None) == ARG
    assert soft(ctypes.byref(s), A, A, A, A, 0.25, 0.1, A, MIS, None, A, big, None) == MISAL
    assert soft(ctypes.byref(s), A, A, A, A, 0.25, 0.1, A, None, None, A, need(s, 'router_soft') - 1, None) == WS
    sla1 = L.sla2_forward_sla1
    assert sla1(ctypes.byref(s), A, A, A, A, 0.25, 1, A, None, None, A, big, None) == NULL   # O_l required
    assert sla1(ctypes.byref(s), A, A, A, None, 0.25, 1, A, A, None, A, big, None) == NULL  # proj_o required
    assert sla1(ctypes.byref(s), A, A, A, A, 0.25, 2, A, A, None, A, big, None) == ARG      # no such mode
    assert sla1(ctypes.byref(s), A, A, A, A, 0.0, 1, A, A, None, A, big, None) == ARG
    assert sla1(ctypes.byref(s), A, A, A, A, 0.25, 1, A, MIS, None, A, big, None) == MISAL
    assert sla1(ctypes.byref(s), A, A, A, A, 0.25, 1, A, A, None, A, need(s, 'forward_sla1') - 1, None) == WS
    r = L.sla2_linear_precompute(ctypes.byref(s), A, A, None, None, None, A, A, A, big, None)
    assert r == NULL                                            # k_colmean required
    r = L.sla2_linear_precompute(ctypes.byref(s), A, A, A, MIS, None, A, A, A, big, None)
    assert r == MISAL
    r = L.sla2_forward_with_mask(ctypes.byref(s), A, A, A, None, A, 1, A, None, A, big, None)
    assert r == NULL                                            # mask required
    r = L.sla2_forward_with_mask(ctypes.byref(s), A, A, A, A, A, 3, A, None, A, big, None)
    assert r == ARG
    r = L.sla2_forward_with_mask(ctypes.byref(shape(N=64)), A, A, A, A, A, 1, A, None, A, big, None)
    assert r == SHAPE
    bwd = L.sla2_backward
    assert bwd(ctypes.byref(s), A, A, A, None, A, A, A, A, A, A, None, A, big, None) == NULL  # mask
    assert bwd(ctypes.byref(s), A, A, A, A, A, None, A, A, A, A, None, A, big, None) == NULL  # dO
    assert bwd(ctypes.byref(s), A, A, A, A, A, A, A, A, A, None, None, A, big, None) == NULL  # dalpha
    assert bwd(ctypes.byref(s), A, A, A, A, A, A, A, MIS, A, A, None, A, big, None) == MISAL
    assert bwd(ctypes.byref(s), A, A, A, A, A, A, A, A, A, A, None, A, need(s, 'backward') - 1, None) == WS
    assert bwd(ctypes.byref(s), A, A, A, A, A, A, A, A, A, A, None, A, need(s, 'forward'), None) == WS
    assert bwd(ctypes.byref(shape(N=200)), A, A, A, A, A, A, A, A, A, A, None, A, big,
               None) == SHAPE
    fa = L.sla2_fit_alpha
    assert fa(ctypes.byref(s), A, A, None, A, None) == NULL
    assert fa(ctypes.byref(s), A, MIS, A, A, None) == MISAL
    assert fa(ctypes.byref(shape(N=100)), A, A, A, A, None) == SHAPE


def test_valid_arguments_reach_the_device_check_without_a_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert fwd(shape()) in (HIP, DEV)


def test_workspace_status_validates_before_touching_the_device():
    L = sla2.lib()
    assert L.sla2_workspace_status(None, 1024, None) == NULL
    assert L.sla2_workspace_status(MIS, 1024, None) == MISAL
    assert L.sla2_workspace_status(A, 255, None) == WS
    assert "bounded wait" in sla2.sla2_status_string(TIMEOUT)


def test_noalloc_router_validates_on_the_host():
    L = sla2.lib()
    s = shape()
    f = L.sla2_router_noalloc
    assert f(ctypes.byref(s), A, A, A, A, 0.25, None, None, None, None) == NULL   # blocks required
    assert f(ctypes.byref(s), A, A, A, A, 0.0, None, A, None, None) == ARG
    assert f(ctypes.byref(s), A, A, A, MIS, 0.25, None, A, None, None) == MISAL
    assert f(ctypes.byref(shape(N=100)), A, A, A, A, 0.25, None, A, None, None) == SHAPE
    # the router at B*H = 12, N = 32768 fits the static scratch; at H = 40, N = 75648 it does not
    assert need(shape(1, 12, 32768), "router") <= sla2.NOALLOC_SCRATCH_BYTES
    big = shape(1, 40, 75648)
    assert need(big, "router") > sla2.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), A, A, A, A, 0.05, None, A, None, None) == WS


def test_router_grad_validates_on_the_host():
    L = sla2.lib()
    s = shape()
    n = need(s, "router_grad")
    f = L.sla2_router_grad

    def call(q=A, k=A, v=A, wq=A, wk=A, al=A, keep=0.25, tau=0.1, of=A, dq=A, dk=A, loss=A,
             mg=None, ws=A, wsb=n, shp=s):
        return f(ctypes.byref(shp), q, k, v, wq, wk, al, keep, tau, of, dq, dk, loss, mg, ws, wsb,
                 None)
    assert call(of=None) == NULL                     # the target is required
    assert call(dq=None) == NULL
    assert call(loss=None) == NULL
    assert call(v=None) == NULL
    assert call(mg=MIS) == MISAL                     # optional, but aligned when given
    assert call(dk=MIS) == MISAL
    assert call(tau=0.0) == ARG
    assert call(tau=float("inf")) == ARG
    assert call(keep=0.0) == ARG
    assert call(keep=1.5) == ARG
    assert call(wsb=n - 1) == WS
    assert call(wsb=need(s, "forward")) == WS        # sized for another entry
    assert call(ws=None) == NULL
    assert call(shp=shape(N=100)) == SHAPE
    import torch
    if not torch.cuda.is_available():
        assert call() in (HIP, DEV)                  # valid arguments reach the device check
