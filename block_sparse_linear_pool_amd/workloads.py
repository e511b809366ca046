"""Seeded synthetic inputs for the SLA2 forward (shared by the oracle tests and the GPU path).

This module only draws and lays out data. It holds none of the method's
arithmetic: no pooling, scoring, quantisation, softmax or mixing happens here.

The pages measure SLA2 on video latents of Wan2.1-1.3B (480P) and Wan2.1-14B
(720P) ("SLA2: Sparse-Linear Attention v2 for Diffusion Transformers", §5
Table 1). Those Q/K/V tensors are not available, so a smooth space-time field on
the same (t, y, x) token grids stands in for them: Q and K share one field per
(batch, head), which gives local, block-structured attention like a video DiT.

Recipe per (batch b, head h), rng = numpy default_rng([seed, b, h]), draws in
this order: 16 frequency triples f ~ U(0, 2) cycles per axis extent, 16 phases
~ U(0, 2*pi), 16 x d amplitudes ~ N(0, 1), Q noise, K noise, K channel bias, V.

  field[n, c] = sum_s a[s, c] * sin(2*pi*(f_t t/T + f_y y/Y + f_x x/X) + phase_s)
  with n = (t*Y + y)*X + x, each channel scaled to unit std over the real tokens;
  Q = 0.6 field + 0.4 N(0,1);  K = 0.6 field + 0.4 N(0,1) + bias_c;  V = N(0,1).

Rows past the real token count (padding up to a multiple of 128) are zero.
Values are rounded to bf16 (round to nearest even); those bf16 values are the
inputs of both the oracle and the GPU path.

The tiny case draws Q, K, V i.i.d. N(0,1) in fp32, plus a per-channel N(0,1)
bias on K. Router weights come from default_rng([seed, 10**6]): proj_q and
proj_k per head ~ N(0, 1/d) in fp32, then alpha per (head, query block) ~ U(lo, 1).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

HEAD_DIM = 128
Q_BLOCK = 128
K_BLOCK = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int                      # padded token count, multiple of 128
    keep_frac: tuple            # one or more kept key-block fractions
    seed: int
    dtype: str                  # "fp32" or "bf16"
    grid: tuple | None = None   # (T, Y, X) token grid; None = i.i.d. inputs
    alpha_lo: float = 0.5
    d: int = HEAD_DIM

    @property
    def n_real(self) -> int:
        return self.N if self.grid is None else int(np.prod(self.grid))

    @property
    def n_qb(self) -> int:
        return self.N // Q_BLOCK

    @property
    def n_kb(self) -> int:
        return self.N // K_BLOCK


WORKLOADS = {
    # tiny i.i.d. case the oracle finishes in well under a second
    "tiny_iid_N2048": Workload("tiny_iid_N2048", 1, 2, 2048, (0.25,), 1, "fp32",
                               None, alpha_lo=0.0),
    # small structured case on an 8x32x32 grid, keep 10%
    "grid_8x32x32_N8192": Workload("grid_8x32x32_N8192", 1, 12, 8192, (0.10,), 2,
                                   "bf16", (8, 32, 32)),
    # Wan2.1-1.3B-480P-shaped latents: 21x30x52 tokens padded to 32768, keep 3%
    "wan13b_480p_N32768": Workload("wan13b_480p_N32768", 1, 12, 32768, (0.03,), 3,
                                   "bf16", (21, 30, 52)),
    # sparsity sweep, paired cond/uncond batch: keep 20/10/5/3%
    "sweep_B2_N32768": Workload("sweep_B2_N32768", 2, 12, 32768,
                                (0.20, 0.10, 0.05, 0.03), 4, "bf16", (21, 30, 52)),
    # Wan2.1-14B-720P-shaped latents: 21x45x80 tokens padded to 75648, keep 5%
    "wan14b_720p_N75648": Workload("wan14b_720p_N75648", 1, 40, 75648, (0.05,), 5,
                                   "bf16", (21, 45, 80)),
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _field(rng: np.random.Generator, grid, n_real: int, d: int) -> np.ndarray:
    T, Y, X = grid
    freqs = rng.uniform(0.0, 2.0, size=(16, 3))
    phases = rng.uniform(0.0, 2.0 * math.pi, size=16)
    amps = rng.standard_normal((16, d))
    n = np.arange(n_real)
    x = n % X
    y = (n // X) % Y
    t = n // (X * Y)
    arg = 2.0 * math.pi * (np.outer(t / T, freqs[:, 0]) + np.outer(y / Y, freqs[:, 1])
                           + np.outer(x / X, freqs[:, 2])) + phases[None, :]
    field = np.sin(arg) @ amps
    field /= field.std(axis=0, keepdims=True)
    return field


def head_qkv(w: Workload, b: int, h: int):
    """Q, K, V of one (batch, head) as float32 arrays [N, d] holding the exact input values."""
    rng = np.random.default_rng([w.seed, b, h])
    N, d, nr = w.N, w.d, w.n_real
    if w.grid is None:
        q = rng.standard_normal((N, d))
        k = rng.standard_normal((N, d)) + rng.standard_normal(d)[None, :]
        v = rng.standard_normal((N, d))
        out = [a.astype(np.float32) for a in (q, k, v)]
    else:
        f = _field(rng, w.grid, nr, d)
        qn = rng.standard_normal((nr, d))
        kn = rng.standard_normal((nr, d))
        kbias = rng.standard_normal(d)
        vv = rng.standard_normal((nr, d))
        out = []
        for a in (0.6 * f + 0.4 * qn, 0.6 * f + 0.4 * kn + kbias[None, :], vv):
            full = np.zeros((N, d), dtype=np.float32)
            full[:nr] = a
            out.append(full)
    if w.dtype == "bf16":
        out = [bf16_bits_to_f32(to_bf16_bits(a)) for a in out]
    return out


def weights(w: Workload):
    """proj_q, proj_k [H, d, d] float32 (applied as x @ W) and alpha [H, N/128] float32."""
    rng = np.random.default_rng([w.seed, 10 ** 6])
    d = w.d
    wq = np.empty((w.H, d, d), dtype=np.float32)
    wk = np.empty((w.H, d, d), dtype=np.float32)
    for h in range(w.H):
        wq[h] = rng.normal(0.0, 1.0 / math.sqrt(d), (d, d))
        wk[h] = rng.normal(0.0, 1.0 / math.sqrt(d), (d, d))
    alpha = rng.uniform(w.alpha_lo, 1.0, (w.H, w.n_qb)).astype(np.float32)
    return wq, wk, alpha


def generate(w: Workload, heads=None, batches=None):
    """Q, K, V as float32 [B', H', N, d] for the selected batches/heads (all by default)."""
    batches = list(range(w.B)) if batches is None else list(batches)
    heads = list(range(w.H)) if heads is None else list(heads)
    shape = (len(batches), len(heads), w.N, w.d)
    q = np.empty(shape, np.float32)
    k = np.empty(shape, np.float32)
    v = np.empty(shape, np.float32)
    for bi, b in enumerate(batches):
        for hi, h in enumerate(heads):
            q[bi, hi], k[bi, hi], v[bi, hi] = head_qkv(w, b, h)
    return q, k, v


def random_qkv(seed: int, B: int, H: int, N: int, d: int = HEAD_DIM, bias: float = 1.0,
               scale: float = 1.0, dtype: str = "fp32"):
    """Plain i.i.d. inputs for edge-case tests: Q,K,V ~ scale*N(0,1), K plus a channel bias."""
    rng = np.random.default_rng([seed, 7])
    q = scale * rng.standard_normal((B, H, N, d))
    k = scale * rng.standard_normal((B, H, N, d)) + bias * rng.standard_normal((B, H, 1, d))
    v = rng.standard_normal((B, H, N, d))
    out = [a.astype(np.float32) for a in (q, k, v)]
    if dtype == "bf16":
        out = [bf16_bits_to_f32(to_bf16_bits(a)) for a in out]
    return out


def random_weights(seed: int, H: int, n_qb: int, d: int = HEAD_DIM, alpha_lo: float = 0.0):
    rng = np.random.default_rng([seed, 10 ** 6])
    wq = rng.normal(0.0, 1.0 / math.sqrt(d), (H, d, d)).astype(np.float32)
    wk = rng.normal(0.0, 1.0 / math.sqrt(d), (H, d, d)).astype(np.float32)
    alpha = rng.uniform(alpha_lo, 1.0, (H, n_qb)).astype(np.float32)
    return wq, wk, alpha


def grad_out(seed: int, shape) -> np.ndarray:
    """The upstream gradient dO of a backward test or bench: i.i.d. N(0, 1), fp32."""
    rng = np.random.default_rng([seed, 11])
    return rng.standard_normal(shape, dtype=np.float32)


def random_mask(seed: int, B: int, H: int, n_qb: int, n_kb: int, frac: float) -> np.ndarray:
    """A block mask [B, H, n_qb, n_kb] uint8 with each entry kept with probability frac."""
    rng = np.random.default_rng([seed, 13])
    return (rng.random((B, H, n_qb, n_kb)) < frac).astype(np.uint8)
