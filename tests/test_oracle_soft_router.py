"""Pins of the oracle's SoftTop-k router (training-time step 1) on the CPU.

The soft mask is sigma(P_ij / tau + lambda_i) with lambda_i chosen so each row sums to kb
("SLA2: Sparse-Linear Attention v2 for Diffusion Transformers", §4 Eq. 17; six-checks item 3).
The oracle finds lambda_i by bisection; these tests check it against a closed form (rows with
two distinct values make the row-sum equation a quadratic in e^lambda), a library root
finder (scipy's brentq), the uniform row, monotonicity, symmetry of ties and the tau -> 0
limit, which must give the hard Top-k mask (built here by a plain argsort).
"""
import math

import numpy as np
import pytest
from scipy.optimize import brentq

from oracle import sla2


def random_rows(seed, n_qb=6, n_kb=512, spread=2.0):
    rng = np.random.default_rng(seed)
    return sla2.softmax_rows(spread * rng.standard_normal((n_qb, n_kb)))


def sig(x):
    return 1.0 / (1.0 + np.exp(-x))


@pytest.mark.parametrize("kb", [1, 15, 100, 511])
def test_rows_sum_to_kb(kb):
    P = random_rows(1)
    soft, lam = sla2.soft_topk(P, kb, 0.1)
    assert np.allclose(soft.sum(1), kb, rtol=0, atol=1e-9)
    assert ((soft > 0) & (soft < 1)).all()


@pytest.mark.parametrize("n1,kb,tau", [(3, 15, 0.1), (40, 15, 0.1), (100, 200, 0.05), (7, 5, 1.0)])
def test_two_level_rows_closed_form(n1, kb, tau):
    """n1 entries of value a and n2 of value b: with u = e^lambda, A = e^(a/tau), B = e^(b/tau),
    n1 uA/(1+uA) + n2 uB/(1+uB) = kb is u^2 AB (n1+n2-kb) + u (n1 A + n2 B - kb (A+B)) - kb = 0."""
    n_kb = 512
    n2 = n_kb - n1
    a = 3.0 / n_kb                       # the n1 large entries
    b = (1.0 - n1 * a) / n2              # the rest, so the row sums to 1 like P_c
    P = np.full((1, n_kb), b)
    P[0, :n1] = a
    A, B = math.exp(a / tau), math.exp(b / tau)
    qa, qb, qc = A * B * (n1 + n2 - kb), n1 * A + n2 * B - kb * (A + B), -kb
    u = (-qb + math.sqrt(qb * qb - 4 * qa * qc)) / (2 * qa)
    soft, lam = sla2.soft_topk(P, kb, tau)
    assert abs(lam[0] - math.log(u)) < 1e-9
    assert abs(soft[0, 0] - u * A / (1 + u * A)) < 1e-12
    assert abs(soft[0, -1] - u * B / (1 + u * B)) < 1e-12


def test_uniform_row():
    n_kb, kb, tau = 512, 15, 0.1
    P = np.full((2, n_kb), 1.0 / n_kb)
    soft, lam = sla2.soft_topk(P, kb, tau)
    assert np.allclose(soft, kb / n_kb, atol=1e-12)
    assert np.allclose(lam, math.log(kb / (n_kb - kb)) - 1.0 / (n_kb * tau), atol=1e-9)


@pytest.mark.parametrize("seed,kb,tau", [(2, 15, 0.1), (3, 60, 0.1), (4, 15, 0.02), (5, 300, 0.5)])
def test_lambda_matches_brentq(seed, kb, tau):
    P = random_rows(seed, spread=3.0)
    soft, lam = sla2.soft_topk(P, kb, tau)
    for i in range(P.shape[0]):
        x = P[i] / tau
        ref = brentq(lambda l: sig(x + l).sum() - kb, -x.max() - 50, -x.min() + 50, xtol=1e-14,
                     rtol=1e-15, maxiter=500)
        assert abs(lam[i] - ref) < 1e-9


def test_monotone_and_ties_symmetric():
    P = random_rows(6, n_qb=3)
    P[:, 10] = P[:, 20]                  # planted ties: equal scores, equal soft values
    soft, _ = sla2.soft_topk(P, 15, 0.1)
    assert np.array_equal(soft[:, 10], soft[:, 20])
    for i in range(P.shape[0]):
        o = np.argsort(P[i], kind="stable")
        assert np.all(np.diff(soft[i][o]) >= 0)


def test_small_tau_gives_hard_topk():
    """tau -> 0: the soft mask tends to the kb largest entries (a plain argsort here; the
    rows have no ties near the boundary)."""
    P = random_rows(7, n_qb=5, spread=3.0)
    kb = 15
    for i in range(P.shape[0]):
        s = np.sort(P[i])[::-1]
        assert s[kb - 1] - s[kb] > 1e-9   # a gap at the boundary
    soft, _ = sla2.soft_topk(P, kb, 1e-9)
    hard = np.zeros_like(P)
    for i in range(P.shape[0]):
        hard[i, np.argsort(-P[i], kind="stable")[:kb]] = 1.0
    assert np.abs(soft - hard).max() < 1e-6


def test_all_kept_is_ones():
    P = random_rows(8, n_qb=2, n_kb=64)
    soft, lam = sla2.soft_topk(P, 64, 0.1)
    assert (soft == 1.0).all() and np.isinf(lam).all()
