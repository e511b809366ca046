"""Pins of the oracle's stage-1 alpha fit (oracle/sla2_fit.py) on the CPU.

alpha* minimises the MSE of alpha O_s + (1 - alpha) O_l against O_full per (head, query block)
("SLA2: Sparse-Linear Attention v2 for Diffusion Transformers", §4 six checks item 5). Pins: a
target that is itself such a mix gives back its alpha; scipy's bounded scalar minimiser of the
loss agrees; the clipping to [0, 1]; alpha shared by the batches; the degenerate block.
"""
import numpy as np
import pytest
from scipy.optimize import minimize_scalar

from oracle import sla2_fit as fit

D = 16


def taps(seed, B=1, H=2, N=256):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, H, N, D)), rng.standard_normal((B, H, N, D))


def test_recovers_the_mixing_weight():
    O_s, O_l = taps(1, B=2)
    a0 = np.array([[0.3, 0.9], [0.0, 1.0]])
    a = np.repeat(a0, 128, axis=1)[None, :, :, None]
    O_full = a * O_s + (1 - a) * O_l
    assert np.allclose(fit.fit_alpha(O_full, O_s, O_l), a0, atol=1e-12)


def test_matches_a_scalar_minimiser():
    O_s, O_l = taps(2)
    rng = np.random.default_rng(3)
    O_full = 0.6 * O_s + 0.4 * O_l + 0.5 * rng.standard_normal(O_s.shape)
    got = fit.fit_alpha(O_full, O_s, O_l)
    for h in range(2):
        for i in range(2):
            def loss(x):
                al = got.copy()
                al[h, i] = x
                return fit.mse(al, O_full, O_s, O_l)
            ref = minimize_scalar(loss, bounds=(0.0, 1.0), method="bounded",
                                  options={"xatol": 1e-10}).x
            assert abs(got[h, i] - ref) < 1e-6


@pytest.mark.parametrize("beyond,expect", [(1.7, 1.0), (-0.4, 0.0)])
def test_clipped_to_unit_interval(beyond, expect):
    O_s, O_l = taps(4)
    O_full = beyond * O_s + (1 - beyond) * O_l
    assert np.allclose(fit.fit_alpha(O_full, O_s, O_l), expect)


def test_batches_share_alpha():
    """Two batches pulling towards 0.2 and 0.8 with equal weight meet at their weighted mean."""
    O_s, O_l = taps(5, B=1)
    O_s2 = np.concatenate([O_s, O_s])
    O_l2 = np.concatenate([O_l, O_l])
    a = np.array([0.2, 0.8])[:, None, None, None]
    O_full = a * O_s2 + (1 - a) * O_l2
    assert np.allclose(fit.fit_alpha(O_full, O_s2, O_l2), 0.5, atol=1e-12)


def test_equal_branches_give_one():
    O_s, _ = taps(6)
    assert np.all(fit.fit_alpha(O_s + 1.0, O_s, O_s) == 1.0)
