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
OK, NULL, SHAPE, DTYPE, MISAL, ARG, WS, DEV, HIP = range(9)

A = 0x10000          # fake 16-byte-aligned "device" addresses: never dereferenced
MIS = 0x10008


def declared_functions():
    text = open(os.path.join(ROOT, "include", "sla2.h")).read()
    return sorted(set(re.findall(r"\b(sla2_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = sla2.lib()
    names = declared_functions()
    assert set(names) == {"sla2_blocks_kept", "sla2_workspace_bytes", "sla2_status_string",
                          "sla2_router", "sla2_router_soft", "sla2_linear_precompute",
                          "sla2_forward", "sla2_forward_sla1", "sla2_forward_with_mask",
                          "sla2_backward", "sla2_fit_alpha"}
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
    a = sla2.sla2_workspace_bytes(1, 12, 32768)
    b = sla2.sla2_workspace_bytes(2, 12, 32768)
    assert 0 < a < b
    assert sla2.sla2_workspace_bytes(1, 1, 100) == 0
    assert sla2.sla2_workspace_bytes(1, 1, 128, d=64) == 0
    assert sla2.sla2_workspace_bytes(1, 1, 262144 + 128) == 0
    assert sla2.sla2_workspace_bytes(256, 256, 128) == 0        # B*H > 65535
    for s in range(9):
        assert isinstance(sla2.sla2_status_string(s), str) and sla2.sla2_status_string(s)


def shape(B=1, H=2, N=1024, d=128, dtype=1):
    return sla2.Shape(B, H, N, d, dtype)


def fwd(shp, q=A, k=A, v=A, wq=A, wk=A, alpha=A, keep=0.25, quant=1, O=A, taps=None, ws=A,
        wsb=None):
    if wsb is None:
        wsb = sla2.lib().sla2_workspace_bytes(ctypes.byref(shp)) if shp else 0
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
    assert fwd(shape(), quant=0) == ARG
    s = shape()
    need = sla2.lib().sla2_workspace_bytes(ctypes.byref(s))
    assert fwd(s, wsb=need - 1) == WS
    assert fwd(s, ws=None) == NULL
    assert fwd(s, ws=MIS) == MISAL


def test_other_entry_points_validate():
    L = sla2.lib()
    s = shape()
    need = L.sla2_workspace_bytes(ctypes.byref(s))
    r = L.sla2_router(ctypes.byref(s), A, A, A, A, 0.25, None, None, None, A, need, None)
    assert r == NULL                                            # blocks is required
    r = L.sla2_router(ctypes.byref(s), A, A, A, A, 2.0, None, A, None, A, need, None)
    assert r == ARG
    r = L.sla2_router(ctypes.byref(s), A, A, A, A, 0.25, MIS, A, None, A, need, None)
    assert r == MISAL
    soft = L.sla2_router_soft
    assert soft(ctypes.byref(s), A, A, A, A, 0.25, 0.1, None, None, None, A, need, None) == NULL
    assert soft(ctypes.byref(s), A, A, A, A, 0.25, 0.0, A, None, None, A, need, None) == ARG   # tau > 0
    assert soft(ctypes.byref(s), A, A, A, A, 0.25, float("nan"), A, None, None, A, need, None) == ARG
    assert soft(ctypes.byref(s), A, A, A, A, 0.25, 1e-45, A, None, None, A, need, None) == ARG  # 1/tau inf
    assert soft(ctypes.byref(s), A, A, A, A, 1.5, 0.1, A, None, None, A, need, None) == ARG
    assert soft(ctypes.byref(s), A, A, A, A, 0.25, 0.1, A, MIS, None, A, need, None) == MISAL
    assert soft(ctypes.byref(s), A, A, A, A, 0.25, 0.1, A, None, None, A, need - 1, None) == WS
    sla1 = L.sla2_forward_sla1
    assert sla1(ctypes.byref(s), A, A, A, A, 0.25, 1, A, None, None, A, need, None) == NULL   # O_l required
    assert sla1(ctypes.byref(s), A, A, A, None, 0.25, 1, A, A, None, A, need, None) == NULL  # proj_o required
    assert sla1(ctypes.byref(s), A, A, A, A, 0.25, 0, A, A, None, A, need, None) == ARG      # quantised only
    assert sla1(ctypes.byref(s), A, A, A, A, 0.0, 1, A, A, None, A, need, None) == ARG
    assert sla1(ctypes.byref(s), A, A, A, A, 0.25, 1, A, MIS, None, A, need, None) == MISAL
    assert sla1(ctypes.byref(s), A, A, A, A, 0.25, 1, A, A, None, A, need - 1, None) == WS
    r = L.sla2_linear_precompute(ctypes.byref(s), A, A, None, None, None, A, A, A, need, None)
    assert r == NULL                                            # k_colmean required
    r = L.sla2_linear_precompute(ctypes.byref(s), A, A, A, MIS, None, A, A, A, need, None)
    assert r == MISAL
    r = L.sla2_forward_with_mask(ctypes.byref(s), A, A, A, None, A, 1, A, None, A, need, None)
    assert r == NULL                                            # mask required
    r = L.sla2_forward_with_mask(ctypes.byref(s), A, A, A, A, A, 3, A, None, A, need, None)
    assert r == ARG
    r = L.sla2_forward_with_mask(ctypes.byref(shape(N=64)), A, A, A, A, A, 1, A, None, A, need, None)
    assert r == SHAPE
    bwd = L.sla2_backward
    assert bwd(ctypes.byref(s), A, A, A, None, A, A, A, A, A, A, None, A, need, None) == NULL  # mask
    assert bwd(ctypes.byref(s), A, A, A, A, A, None, A, A, A, A, None, A, need, None) == NULL  # dO
    assert bwd(ctypes.byref(s), A, A, A, A, A, A, A, A, A, None, None, A, need, None) == NULL  # dalpha
    assert bwd(ctypes.byref(s), A, A, A, A, A, A, A, MIS, A, A, None, A, need, None) == MISAL
    assert bwd(ctypes.byref(s), A, A, A, A, A, A, A, A, A, A, None, A, need - 1, None) == WS
    assert bwd(ctypes.byref(shape(N=200)), A, A, A, A, A, A, A, A, A, A, None, A, need,
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
