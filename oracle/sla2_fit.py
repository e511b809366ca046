"""Stage-1 alpha fitting — plain fp64 CPU oracle (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import, call or run
anything in this package. The GPU path shares no code with it and never calls it.

"SLA2: Sparse-Linear Attention v2 for Diffusion Transformers" fits the router and alpha in a
first stage with an MSE loss against full attention on Q/K/V tensors, and notes that alpha then
lands close to the kept row mass P_1 1 (§4 six checks item 5; §5 training table; §3 mixing
O = alpha O_s + (1 - alpha) O_l). Readings taken here (listed with their reasons in the design
notes of the repository):

  * the alpha part only, with the router held fixed: O is affine in alpha, so the MSE
    sum over the block's rows and all batches of |alpha O_s + (1 - alpha) O_l - O_full|^2 is a
    quadratic in each query block's alpha, minimised by
        alpha* = <O_full - O_l, O_s - O_l> / |O_s - O_l|^2
    (inner products over the 128 rows x d of the block, summed over the batch, since alpha is
    one value per head and query block);
  * alpha is kept in [0, 1] (the convex combination of §4 check 2): alpha* is clipped;
  * a block whose branches agree (|O_s - O_l| = 0) gets alpha = 1.
"""

from __future__ import annotations

import numpy as np

BQ = 128


def fit_alpha(O_full, O_s, O_l):
    """alpha* per (head, query block) for [B, H, N, d] arrays; returns [H, N/128] (fp64)."""
    O_full = np.asarray(O_full, np.float64)
    O_s = np.asarray(O_s, np.float64)
    O_l = np.asarray(O_l, np.float64)
    B, H, N, d = O_s.shape
    diff = (O_s - O_l).reshape(B, H, N // BQ, BQ * d)
    res = (O_full - O_l).reshape(B, H, N // BQ, BQ * d)
    num = (res * diff).sum(axis=(0, 3))
    den = (diff * diff).sum(axis=(0, 3))
    alpha = np.ones((H, N // BQ))
    ok = den > 0
    alpha[ok] = num[ok] / den[ok]
    return np.clip(alpha, 0.0, 1.0)


def mse(alpha, O_full, O_s, O_l):
    """The stage-1 loss for a given alpha [H, N/128] (sum of squares over everything)."""
    a = np.repeat(np.asarray(alpha, np.float64), BQ, axis=1)[None, :, :, None]
    O = a * np.asarray(O_s, np.float64) + (1.0 - a) * np.asarray(O_l, np.float64)
    return float(((O - np.asarray(O_full, np.float64)) ** 2).sum())
