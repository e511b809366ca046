"""Number codecs of the SLA2 oracle (test infrastructure; fp64 numpy, CPU only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this module. The GPU path shares no code with it.

The pages name the formats but not their details: the summary page "SLA2: Sparse-
Linear Attention with Learnable Routing and QAT" (paper.rainbus.top, computation
flow, step 2) quantises Q and K to low bit and P and V to low bit; the method
table of "SLA2: Sparse-Linear Attention v2 for Diffusion Transformers" (§2 Q2,
row "Acceleration") says INT8/FP8 forward. The readings used here:

* INT8: symmetric, one scale per block of rows (the whole block x d), amax taken
  exactly, inv = fl32(127/amax), code = clamp(rne(fl32(x*inv)), -127, 127),
  scale = fl32(amax/127); an all-zero block has scale 0 and codes 0. All steps
  are IEEE fp32 so that a GPU doing the same fp32 steps gets the same codes.
* FP8: OCP E4M3 ("FN" variant): bias 7, no infinities, 0x7F/0xFF are NaN,
  largest finite 448, smallest normal 2^-6, subnormal step 2^-9. Encoding
  rounds to the nearest finite value, ties to the even code, and saturates
  magnitudes above 448 to 448.

Pins (tests/test_oracle_codecs.py): every one of the 256 codes is decoded and
compared with torch's float8_e4m3fn; the encoder equals a brute-force nearest
search over the finite codes with ties to the even code; the INT8 codec obeys
|x - q*s| <= s/2, maps amax to +-127 and a zero block to zero.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each OCP E4M3 code (uint8) as float64; NaN for 0x7F and 0xFF."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m / 8.0, -6)
    val = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_round(x) -> np.ndarray:
    """Nearest finite E4M3 value (ties to even mantissa), saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # exponent of the binade [2^e, 2^(e+1)); values below 2^-6 use the subnormal step
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # guard log2 rounding at exact powers of two
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > a, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= a, e + 1, e)
    e = np.maximum(e, -6.0)
    step = np.ldexp(1.0, (e - 3).astype(np.int64))   # 3 mantissa bits
    r = np.rint(a / step) * step                      # np.rint: half to even
    r = np.minimum(r, E4M3_MAX)
    r = np.where(a > 0, r, 0.0)
    return np.copysign(r, x)


def e4m3_encode(x) -> np.ndarray:
    """uint8 OCP E4M3 codes of x (rounded as e4m3_round)."""
    r = e4m3_round(x)
    a = np.abs(r)
    neg = np.signbit(r)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > a, e - 1, e)
    normal = a >= 2.0 ** -6
    e_field = np.where(normal, e + 7, 0).astype(np.int64)
    m_field = np.where(normal, np.rint((a / np.ldexp(1.0, e.astype(np.int64)) - 1.0) * 8.0),
                       np.rint(a / 2.0 ** -9)).astype(np.int64)
    code = (e_field << 3) | m_field
    code = np.where(a == 0, 0, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def int8_block_quant(x32: np.ndarray, rows: int):
    """Symmetric INT8 codes of an fp32 matrix [N, d] with one scale per `rows` rows.

    Returns (codes int8 [N, d], scales float32 [N/rows]).
    """
    x32 = np.asarray(x32, dtype=np.float32)
    n, d = x32.shape
    blocks = x32.reshape(n // rows, rows, d)
    amax = np.abs(blocks).max(axis=(1, 2)).astype(np.float32)
    codes = np.zeros_like(blocks, dtype=np.int8)
    scales = np.zeros(n // rows, dtype=np.float32)
    for i in range(n // rows):
        if amax[i] == 0:
            continue
        inv = np.float32(127.0) / amax[i]                     # IEEE fp32 division
        y = blocks[i] * inv                                   # fp32 product
        codes[i] = np.clip(np.rint(y), -127, 127).astype(np.int8)
        scales[i] = amax[i] / np.float32(127.0)
    return codes.reshape(n, d), scales


def fp8_block_quant(x32: np.ndarray, rows: int):
    """OCP E4M3 codes of an fp32 matrix [N, d] with one scale per `rows` rows (amax -> 448).

    Returns (codes uint8 [N, d], scales float32 [N/rows]).
    """
    x32 = np.asarray(x32, dtype=np.float32)
    n, d = x32.shape
    blocks = x32.reshape(n // rows, rows, d)
    amax = np.abs(blocks).max(axis=(1, 2)).astype(np.float32)
    codes = np.zeros_like(blocks, dtype=np.uint8)
    scales = np.zeros(n // rows, dtype=np.float32)
    for i in range(n // rows):
        if amax[i] == 0:
            continue
        inv = np.float32(E4M3_MAX) / amax[i]
        y = (blocks[i] * inv).astype(np.float64)              # fp32 product, exact in fp64
        codes[i] = e4m3_encode(y)
        scales[i] = amax[i] / np.float32(E4M3_MAX)
    return codes.reshape(n, d), scales
