"""Thin Python binding of libsla2.so (ctypes). Argument marshalling only.

Every step of the SLA2 forward runs in the HIP kernels behind the C ABI
declared in include/sla2.h; PyTorch only provides device memory and the
stream. Importing works without a GPU (the host-only functions and the
argument checks run on the CPU); the library must have been built
(python -m block_sparse_linear_pool_amd.build), otherwise loading fails loudly.

Function names match the C entry points.
"""

from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsla2.so")

SLA2_FP32, SLA2_BF16 = 0, 1
SLA2_QUANT_NONE, SLA2_QUANT_I8_FP8 = 0, 1
QUANT = {"none": SLA2_QUANT_NONE, "i8_fp8": SLA2_QUANT_I8_FP8}
# sla2_entry: the entry point a workspace is sized for
ENTRY = {"router": 0, "router_soft": 1, "linear_precompute": 2, "forward": 3,
         "forward_with_mask": 4, "forward_sla1": 5, "backward": 6, "router_grad": 7}
D = 128

STATUS = {
    0: "SLA2_OK", 1: "SLA2_ERR_NULL_POINTER", 2: "SLA2_ERR_BAD_SHAPE", 3: "SLA2_ERR_BAD_DTYPE",
    4: "SLA2_ERR_MISALIGNED", 5: "SLA2_ERR_BAD_ARGUMENT", 6: "SLA2_ERR_WORKSPACE_TOO_SMALL",
    7: "SLA2_ERR_UNSUPPORTED_DEVICE", 8: "SLA2_ERR_HIP", 9: "SLA2_ERR_WAIT_TIMEOUT",
}


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32)]


TAP_NAMES = ("O_s", "O_l", "q_codes", "k_codes", "v_codes", "s_q", "s_k", "s_v", "k_colmean")
MAX_STAGES = 9   # SLA2_MAX_STAGES


class Taps(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in TAP_NAMES] + [("stage_events", ctypes.c_void_p)]


def event_array(events, count=MAX_STAGES + 1):
    """ctypes array of raw hipEvent_t handles of torch.cuda.Event objects (created if needed)."""
    if len(events) != count:
        raise ValueError(f"need {count} events")
    for e in events:
        if e.cuda_event == 0:
            e.record()                         # torch creates the event on first record
    return (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])


class SLA2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}: {sla2_status_string(status)}")


_lib = None


def lib():
    """The loaded libsla2.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_linear_pool_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, f32, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float, ctypes.c_int32
        L.sla2_blocks_kept.argtypes = [i32, f32]
        L.sla2_blocks_kept.restype = i32
        L.sla2_workspace_bytes.argtypes = [ctypes.POINTER(Shape), ctypes.c_int, f32]
        L.sla2_workspace_bytes.restype = sz
        L.sla2_workspace_status.argtypes = [vp, sz, vp]
        L.sla2_workspace_status.restype = ctypes.c_int
        L.sla2_status_string.argtypes = [ctypes.c_int]
        L.sla2_status_string.restype = ctypes.c_char_p
        L.sla2_router.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, f32, vp, vp, vp, vp, sz, vp]
        L.sla2_router_soft.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, f32, f32, vp, vp,
                                       ctypes.POINTER(vp), vp, sz, vp]
        L.sla2_linear_precompute.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp, vp, vp,
                                             vp, sz, vp]
        L.sla2_forward.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp, vp, f32, ctypes.c_int,
                                   vp, ctypes.POINTER(Taps), vp, sz, vp]
        L.sla2_forward_sla1.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, f32, ctypes.c_int,
                                        vp, vp, ctypes.POINTER(vp), vp, sz, vp]
        L.sla2_forward_with_mask.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp, ctypes.c_int,
                                             vp, ctypes.POINTER(Taps), vp, sz, vp]
        L.sla2_backward.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                    ctypes.POINTER(vp), vp, sz, vp]
        L.sla2_fit_alpha.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp]
        L.sla2_router_grad.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp, vp, f32, f32,
                                       vp, vp, vp, vp, vp, vp, sz, vp]
        L.sla2_init_device.argtypes = []
        L.sla2_router_noalloc.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, f32, vp, vp, vp,
                                          vp]
        for name in ("sla2_router", "sla2_router_soft", "sla2_linear_precompute", "sla2_forward",
                     "sla2_forward_sla1", "sla2_forward_with_mask", "sla2_backward",
                     "sla2_fit_alpha", "sla2_init_device", "sla2_router_noalloc",
                     "sla2_router_grad"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(status: int, where: str):
    if status != 0:
        raise SLA2Error(status, where)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def shape_of(q: torch.Tensor) -> Shape:
    if q.dim() != 4:
        raise ValueError("Q, K, V must be [B, H, N, d]")
    dt = {torch.float32: SLA2_FP32, torch.bfloat16: SLA2_BF16}.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, N, d = q.shape
    return Shape(B, H, N, d, dt)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


# ------------------------------------------------------------------ host-only helpers
def sla2_blocks_kept(n_key_blocks: int, keep_frac: float) -> int:
    return int(lib().sla2_blocks_kept(int(n_key_blocks), float(keep_frac)))


def sla2_workspace_bytes(B: int, H: int, N: int, dtype=torch.bfloat16, entry: str = "forward",
                         keep_frac: float = 1.0, d: int = D) -> int:
    """Workspace bytes of one entry point (ENTRY names) for this shape; keep_frac matters for
    "forward" and "forward_sla1" only (0 for an invalid shape, entry or keep_frac)."""
    dt = SLA2_FP32 if dtype == torch.float32 else SLA2_BF16
    e = ENTRY.get(entry, -1) if isinstance(entry, str) else int(entry)
    return int(lib().sla2_workspace_bytes(ctypes.byref(Shape(B, H, N, d, dt)), e,
                                          float(keep_frac)))


def sla2_workspace_status(workspace: torch.Tensor) -> int:
    """Status of the workspace's error word after the work enqueued so far (synchronises the
    current stream): 0, or 9 (SLA2_ERR_WAIT_TIMEOUT) if a bounded wait in the attention kernel
    of the last forward on this workspace gave up."""
    return int(lib().sla2_workspace_status(_ptr(workspace), workspace.numel(),
                                           _stream(workspace.device)))


def sla2_status_string(status: int) -> str:
    return lib().sla2_status_string(int(status)).decode()


def workspace_for(q: torch.Tensor, entry: str = "forward", keep_frac: float = 1.0) -> torch.Tensor:
    """A device workspace for `entry` on q's shape (keep_frac: see sla2_workspace_bytes)."""
    B, H, N, _ = q.shape
    n = sla2_workspace_bytes(B, H, N, q.dtype, entry, keep_frac)
    if n == 0:
        raise SLA2Error(2, "sla2_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=q.device)


# ------------------------------------------------------------------ entry points
def sla2_router(q, k, proj_q, proj_k, keep_frac, want_mask=True, want_scores=False,
                workspace=None):
    """Returns (blocks [B,H,N/128,kb] int32, mask uint8 or None, scores fp32 or None)."""
    _contig(q, k, proj_q, proj_k)
    shp = shape_of(q)
    B, H, N, _ = q.shape
    nqb, nkb = N // 128, N // 64
    kb = sla2_blocks_kept(nkb, keep_frac)
    if kb < 1:
        raise SLA2Error(5, "sla2_router")
    dev = q.device
    blocks = torch.empty((B, H, nqb, kb), dtype=torch.int32, device=dev)
    mask = torch.empty((B, H, nqb, nkb), dtype=torch.uint8, device=dev) if want_mask else None
    scores = torch.empty((B, H, nqb, nkb), dtype=torch.float32, device=dev) if want_scores else None
    ws = workspace if workspace is not None else workspace_for(q, "router")
    st = lib().sla2_router(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(proj_q), _ptr(proj_k),
                           float(keep_frac), _ptr(mask), _ptr(blocks), _ptr(scores), _ptr(ws),
                           ws.numel(), _stream(dev))
    _check(st, "sla2_router")
    return blocks, mask, scores


NOALLOC_SCRATCH_BYTES = 32 << 20   # SLA2_NOALLOC_SCRATCH_BYTES


def sla2_init_device():
    """One-time set-up of the current device (done by the first call of any entry point)."""
    _check(lib().sla2_init_device(), "sla2_init_device")


def sla2_router_noalloc(q, k, proj_q, proj_k, keep_frac, blocks, mask=None, scores=None):
    """sla2_router without a workspace (the library's static per-GPU scratch); the caller
    passes every output: blocks [B,H,N/128,kb] int32, mask and scores optional. Returns blocks."""
    _contig(q, k, proj_q, proj_k, blocks, mask, scores)
    shp = shape_of(q)
    st = lib().sla2_router_noalloc(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(proj_q),
                                   _ptr(proj_k), float(keep_frac), _ptr(mask), _ptr(blocks),
                                   _ptr(scores), _stream(q.device))
    _check(st, "sla2_router_noalloc")
    return blocks


def sla2_router_soft(q, k, proj_q, proj_k, keep_frac, tau=0.1, want_lambda=True,
                     workspace=None, out=None, events=None):
    """SoftTop-k router: returns (soft mask [B,H,N/128,N/64] fp32, lambda [B,H,N/128] fp32 or None).

    `events`: optional list of 5 torch.cuda.Event(enable_timing=True), recorded before the
    first and after each of the four kernels on the current stream."""
    _contig(q, k, proj_q, proj_k, out)
    shp = shape_of(q)
    B, H, N, _ = q.shape
    nqb, nkb = N // 128, N // 64
    dev = q.device
    soft = out if out is not None else torch.empty((B, H, nqb, nkb), dtype=torch.float32, device=dev)
    lam = torch.empty((B, H, nqb), dtype=torch.float32, device=dev) if want_lambda else None
    ws = workspace if workspace is not None else workspace_for(q, "router_soft")
    evs = None
    if events is not None:
        if len(events) < 5:
            raise ValueError("sla2_router_soft needs 5 events")
        for e in events[:5]:
            if e.cuda_event == 0:
                e.record()                     # torch creates the event on first record
        evs = (ctypes.c_void_p * 5)(*[e.cuda_event for e in events[:5]])
    st = lib().sla2_router_soft(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(proj_q), _ptr(proj_k),
                                float(keep_frac), float(tau), _ptr(soft), _ptr(lam), evs, _ptr(ws),
                                ws.numel(), _stream(dev))
    _check(st, "sla2_router_soft")
    return soft, lam


def sla2_linear_precompute(k, v, want_h=True, want_z=True, workspace=None):
    """Returns dict k_colmean, h (or None), z (or None), h_total, z_total (fp32)."""
    _contig(k, v)
    shp = shape_of(k)
    B, H, N, d = k.shape
    nkb = N // 64
    dev = k.device
    out = {
        "k_colmean": torch.empty((B, H, d), dtype=torch.float32, device=dev),
        "h": torch.empty((B, H, nkb, d, d), dtype=torch.float32, device=dev) if want_h else None,
        "z": torch.empty((B, H, nkb, d), dtype=torch.float32, device=dev) if want_z else None,
        "h_total": torch.empty((B, H, d, d), dtype=torch.float32, device=dev),
        "z_total": torch.empty((B, H, d), dtype=torch.float32, device=dev),
    }
    ws = workspace if workspace is not None else workspace_for(k, "linear_precompute")
    st = lib().sla2_linear_precompute(ctypes.byref(shp), _ptr(k), _ptr(v), _ptr(out["k_colmean"]),
                                      _ptr(out["h"]), _ptr(out["z"]), _ptr(out["h_total"]),
                                      _ptr(out["z_total"]), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "sla2_linear_precompute")
    return out


def _make_taps(q, want, events=None):
    if not want:
        if events is None:
            return None, None
        taps = Taps()
        taps._events = event_array(events)
        taps.stage_events = ctypes.cast(taps._events, ctypes.c_void_p)
        return taps, None
    B, H, N, d = q.shape
    dev = q.device
    t = {
        "O_s": torch.empty((B, H, N, d), dtype=torch.float32, device=dev),
        "O_l": torch.empty((B, H, N, d), dtype=torch.float32, device=dev),
        "q_codes": torch.empty((B, H, N, d), dtype=torch.int8, device=dev),
        "k_codes": torch.empty((B, H, N, d), dtype=torch.int8, device=dev),
        "v_codes": torch.empty((B, H, N, d), dtype=torch.uint8, device=dev),
        "s_q": torch.empty((B, H, N // 128), dtype=torch.float32, device=dev),
        "s_k": torch.empty((B, H, N // 64), dtype=torch.float32, device=dev),
        "s_v": torch.empty((B, H, N // 64), dtype=torch.float32, device=dev),
        "k_colmean": torch.empty((B, H, d), dtype=torch.float32, device=dev),
    }
    if want is not True:
        t = {k: v for k, v in t.items() if k in want}
    taps = Taps(**{k: (v.data_ptr() if v is not None else None) for k, v in t.items()})
    if events is not None:
        taps._events = event_array(events)
        taps.stage_events = ctypes.cast(taps._events, ctypes.c_void_p)
    return taps, t


def sla2_forward(q, k, v, proj_q, proj_k, alpha, keep_frac, taps=False, out=None,
                 workspace=None, events=None, quant="i8_fp8"):
    """O [B,H,N,d] fp32; with taps=True (or a collection of tap names) also a dict of taps.

    quant: "i8_fp8" (the low-bit sparse branch) or "none" (fp32 operands).
    `events`: optional list of 10 torch.cuda.Event(enable_timing=True); the library records
    them before the first and after every kernel on the current stream."""
    _contig(q, k, v, proj_q, proj_k, alpha, out)
    shp = shape_of(q)
    dev = q.device
    o = out if out is not None else torch.empty(q.shape, dtype=torch.float32, device=dev)
    ctaps, tdict = _make_taps(q, taps, events)
    ws = workspace if workspace is not None else workspace_for(q, "forward", keep_frac)
    st = lib().sla2_forward(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(proj_q),
                            _ptr(proj_k), _ptr(alpha), float(keep_frac), QUANT[quant],
                            _ptr(o), ctypes.byref(ctaps) if ctaps else None, _ptr(ws),
                            ws.numel(), _stream(dev))
    _check(st, "sla2_forward")
    return (o, tdict) if taps else o


def sla2_forward_sla1(q, k, v, proj_o, keep_frac, out=None, o_l=None, workspace=None,
                      events=None, quant="i8_fp8"):
    """The earlier SLA mix (comparison workload): returns (O, O_l) fp32 [B,H,N,d].

    `events`: optional list of 10 torch.cuda.Event(enable_timing=True), recorded before the
    first and after each of the nine kernels on the current stream."""
    _contig(q, k, v, proj_o, out, o_l)
    shp = shape_of(q)
    dev = q.device
    o = out if out is not None else torch.empty(q.shape, dtype=torch.float32, device=dev)
    ol = o_l if o_l is not None else torch.empty(q.shape, dtype=torch.float32, device=dev)
    ws = workspace if workspace is not None else workspace_for(q, "forward_sla1", keep_frac)
    evs = event_array(events) if events is not None else None
    st = lib().sla2_forward_sla1(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(proj_o),
                                 float(keep_frac), QUANT[quant], _ptr(o), _ptr(ol), evs,
                                 _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "sla2_forward_sla1")
    return o, ol


def sla2_forward_with_mask(q, k, v, mask, alpha, taps=False, out=None, workspace=None,
                           events=None, quant="i8_fp8"):
    """O [B,H,N,d] fp32 from a caller block mask [B,H,N/128,N/64] uint8."""
    _contig(q, k, v, mask, alpha, out)
    shp = shape_of(q)
    dev = q.device
    o = out if out is not None else torch.empty(q.shape, dtype=torch.float32, device=dev)
    ctaps, tdict = _make_taps(q, taps, events)
    ws = workspace if workspace is not None else workspace_for(q, "forward_with_mask")
    st = lib().sla2_forward_with_mask(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(mask),
                                      _ptr(alpha), QUANT[quant], _ptr(o),
                                      ctypes.byref(ctaps) if ctaps else None, _ptr(ws),
                                      ws.numel(), _stream(dev))
    _check(st, "sla2_forward_with_mask")
    return (o, tdict) if taps else o


BACKWARD_STAGES = 14   # kernels (stage events: one more)


def sla2_backward(q, k, v, mask, alpha, grad_out, out=None, workspace=None, events=None):
    """Gradients of sum(grad_out * O) for the unquantised SLA2 forward with a fixed block mask:
    returns (dQ, dK, dV, dalpha), fp32 [B,H,N,d] x 3 and [B,H,N/128].

    mask [B,H,N/128,N/64] uint8 (the forward's block mask); alpha [H,N/128] fp32; grad_out
    [B,H,N,d] fp32. `out`: optional tuple of the four output tensors. `events`: optional list
    of 15 torch.cuda.Event(enable_timing=True) recorded before the first and after each of the
    fourteen stages on the current stream."""
    _contig(q, k, v, mask, alpha, grad_out)
    shp = shape_of(q)
    dev = q.device
    B, H, N, _ = q.shape
    if out is None:
        out = (torch.empty(q.shape, dtype=torch.float32, device=dev),
               torch.empty(q.shape, dtype=torch.float32, device=dev),
               torch.empty(q.shape, dtype=torch.float32, device=dev),
               torch.empty((B, H, N // 128), dtype=torch.float32, device=dev))
    _contig(*out)
    ws = workspace if workspace is not None else workspace_for(q, "backward")
    evs = event_array(events, BACKWARD_STAGES + 1) if events is not None else None
    st = lib().sla2_backward(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(mask),
                             _ptr(alpha), _ptr(grad_out), _ptr(out[0]), _ptr(out[1]),
                             _ptr(out[2]), _ptr(out[3]), evs, _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "sla2_backward")
    return out


def sla2_fit_alpha(o_full, o_s, o_l, out=None):
    """Stage-1 alpha fit: [H, N/128] fp32 alpha minimising the MSE of alpha O_s + (1 - alpha) O_l
    against O_full (all [B,H,N,d] fp32), clipped to [0, 1]."""
    _contig(o_full, o_s, o_l, out)
    B, H, N, d = o_s.shape
    shp = Shape(B, H, N, d, SLA2_FP32)
    a = out if out is not None else torch.empty((H, N // 128), dtype=torch.float32,
                                                device=o_s.device)
    st = lib().sla2_fit_alpha(ctypes.byref(shp), _ptr(o_full), _ptr(o_s), _ptr(o_l), _ptr(a),
                              _stream(o_s.device))
    _check(st, "sla2_fit_alpha")
    return a


def sla2_router_grad(q, k, v, proj_q, proj_k, alpha, keep_frac, o_full, tau=0.1,
                     want_mask_grad=False, workspace=None):
    """Stage-1 router gradient: returns (loss [H] fp64, dproj_q [H,d,d], dproj_k [H,d,d],
    mask_grad [B,H,N/128,N/64] fp32 or None) for L = sum (O - O_full)^2 with the hard mask in
    the unquantised forward and its gradient passed straight through to SoftTop-k."""
    _contig(q, k, v, proj_q, proj_k, alpha, o_full)
    shp = shape_of(q)
    B, H, N, d = q.shape
    dev = q.device
    loss = torch.empty(H, dtype=torch.float64, device=dev)
    dwq = torch.empty((H, d, d), dtype=torch.float32, device=dev)
    dwk = torch.empty((H, d, d), dtype=torch.float32, device=dev)
    mg = (torch.empty((B, H, N // 128, N // 64), dtype=torch.float32, device=dev)
          if want_mask_grad else None)
    ws = workspace if workspace is not None else workspace_for(q, "router_grad", keep_frac)
    st = lib().sla2_router_grad(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(proj_q),
                                _ptr(proj_k), _ptr(alpha), float(keep_frac), float(tau),
                                _ptr(o_full), _ptr(dwq), _ptr(dwk), _ptr(loss), _ptr(mg), _ptr(ws),
                                ws.numel(), _stream(dev))
    _check(st, "sla2_router_grad")
    return loss, dwq, dwk, mg
