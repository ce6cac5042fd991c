"""Pins of the oracle's T_tau and optimal projection (CPU only).

Each test ties oracle.ternarize / oracle.optimal_projection to something the
pages or mathematics fix independently of the code: hand-worked vectors,
a Gaussian closed form, brute force over all ternary vectors, invariances.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy import optimize, special, stats

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _cases():
    with open(os.path.join(HERE, "golden", "ternarize_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["why"][:40])
def test_hand_worked_vectors(case):
    t = oracle.ternarize(np.array(case["x"], dtype=np.float64), case["tau"])
    assert t.tolist() == case["t"]


def test_threshold_is_mean_times_tau():
    # The fixed-point sum truncates each |x_j| at 2**-s with
    # s = 52 - e(M) - ceil(log2 N), so thr lies in (tau*mean - tau*2**-s, tau*mean]
    # up to the final roundings; compare against math.fsum's exact sum.
    rng = np.random.default_rng(5)
    for n in (1, 2, 3, 17, 1000, 4097):
        x = rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 6)
        for tau in (1.0, 0.7):
            thr, big = oracle.mean_abs_threshold(x, tau)
            t64 = float(np.float32(tau))
            exact = t64 * math.fsum(np.abs(x)) / n
            s = 52 - math.frexp(big)[1] - (n - 1).bit_length()
            assert big == np.abs(x).max()
            assert exact - t64 * 2.0 ** -s - 4e-16 * exact <= thr <= exact * (1 + 4e-16)


def test_sign_and_scale_invariance():
    rng = np.random.default_rng(1)
    for n in (5, 64, 1001):
        x = rng.standard_normal(n)
        for tau in (0.3, 0.7, 1.0, 2.0, 4.0):
            t = oracle.ternarize(x, tau)
            assert np.array_equal(oracle.ternarize(-x, tau), -t)
            for p in (-40, -3, 5, 60):
                assert np.array_equal(oracle.ternarize(np.ldexp(x, p), tau), t)


def test_order_free():
    # A permutation of the input permutes the output (the mean does not
    # depend on summation order).
    rng = np.random.default_rng(2)
    x = rng.standard_normal(3000) * np.exp(rng.standard_normal(3000) * 3)
    perm = rng.permutation(x.size)
    for tau in (0.7, 1.0, 2.0):
        assert np.array_equal(oracle.ternarize(x[perm], tau), oracle.ternarize(x, tau)[perm])


def test_output_is_ternary_and_nonzero():
    rng = np.random.default_rng(3)
    for n in (1, 2, 7, 100):
        for tau in (0.7, 2.0, 50.0):
            t = oracle.ternarize(rng.standard_normal(n), tau)
            assert set(np.unique(t)).issubset({-1, 0, 1})
            assert np.count_nonzero(t) >= 1


@pytest.mark.parametrize("tau", [0.7, 1.0, 2.0])
def test_gaussian_zero_fraction_closed_form(tau):
    # For iid N(0,1), mean|x| -> sqrt(2/pi); the zero fraction tends to
    # P(|x| <= tau*sqrt(2/pi)) = erf(tau/sqrt(pi)).  The pages report
    # ~41/57/87% zeros at tau = 0.7/1.0/2.0 on real matrices (§1, §3.2).
    rng = np.random.default_rng(10)
    x = rng.standard_normal(1_000_000)
    zf = float(np.mean(oracle.ternarize(x, tau) == 0))
    closed = special.erf(tau / math.sqrt(math.pi))
    assert abs(zf - closed) < 0.003
    pages = {0.7: 0.41, 1.0: 0.57, 2.0: 0.87}[tau]
    assert abs(zf - pages) < 0.03


def _captured(x, t):
    """Fraction of ||x||^2 captured by the best multiple of ternary t."""
    t = t.astype(np.float64)
    return float((x @ t) ** 2 / (t @ t) / (x @ x))


def test_optimal_projection_vs_brute_force():
    rng = np.random.default_rng(4)
    for n in range(1, 8):
        for _ in range(6):
            x = rng.standard_normal(n)
            if n > 2:
                x[rng.integers(n)] = 0.0
            best = 0.0
            for tt in itertools.product((-1, 0, 1), repeat=n):
                tt = np.array(tt, dtype=np.float64)
                if not tt.any():
                    continue
                best = max(best, (x @ tt) ** 2 / (tt @ tt))
            t, alpha = oracle.optimal_projection(x)
            got = (x @ t) ** 2 / (t.astype(np.float64) @ t)
            assert got == pytest.approx(best, rel=1e-12, abs=1e-300)
            # alpha is the least-squares scale for t
            assert alpha == pytest.approx((x @ t) / np.count_nonzero(t), rel=1e-12)


def test_project_columns_is_brute_force_per_column():
    # every column of a 5 x 4 matrix separately: the ternary t that captures
    # the most energy (x.t)^2 / ||t||^2 over all 3^5 - 1 candidates, in the
    # column's own position (a transposed or shuffled result fails)
    rng = np.random.default_rng(9)
    X = rng.standard_normal((5, 4))
    X[2, 1] = 0.0
    P = oracle.project_columns(X)
    assert P.shape == X.shape and P.dtype == np.int8
    cands = [np.array(tt, dtype=np.float64) for tt in itertools.product((-1, 0, 1), repeat=5) if any(tt)]
    for j in range(X.shape[1]):
        x = X[:, j]
        best = max((x @ tt) ** 2 / (tt @ tt) for tt in cands)
        t = P[:, j].astype(np.float64)
        assert (x @ t) ** 2 / (t @ t) == pytest.approx(best, rel=1e-12)
        assert np.all(np.sign(t[t != 0]) == np.sign(x[t != 0]))


def test_threshold_ties_optimal_projection_on_gaussians():
    # Continuum: a threshold at t sigma captures 2 phi(t)^2 / Q(t) of the
    # energy.  The optimum solves phi(t) = 2 t Q(t).  The pages say T_0.7
    # empirically ties the optimal projection (§2.2).
    phi, Q = stats.norm.pdf, stats.norm.sf
    cap = lambda t: 2 * phi(t) ** 2 / Q(t)
    t_opt = optimize.brentq(lambda t: phi(t) - 2 * t * Q(t), 0.1, 2.0)
    t07 = 0.7 * math.sqrt(2 / math.pi)
    rng = np.random.default_rng(11)
    x = rng.standard_normal(1_000_000)
    c07 = _captured(x, oracle.ternarize(x, 0.7))
    copt = _captured(x, oracle.optimal_projection(x)[0])
    assert c07 == pytest.approx(cap(t07), abs=0.003)
    assert copt == pytest.approx(cap(t_opt), abs=0.003)
    assert copt >= c07
    assert c07 / copt > 0.995


def test_optimal_projection_is_global_not_first_peak():
    # the prefix score S_s / sqrt(s) is not unimodal: with one large entry and
    # many equal smaller ones it dips at s = 2 and then rises past s = 1
    x = np.array([1.0] + [0.3] * 40)
    score = np.cumsum(np.abs(x)) / np.sqrt(np.arange(1, x.size + 1))
    assert score[1] < score[0] < score[-1]
    t, alpha = oracle.optimal_projection(x)
    assert np.count_nonzero(t) == x.size
    assert alpha == pytest.approx(np.mean(np.abs(x)))


def test_optimal_projection_ties_and_degenerate_inputs():
    t, a = oracle.optimal_projection(np.zeros(5))
    assert list(t) == [1, 0, 0, 0, 0] and a == 0.0
    # within a run of equal magnitudes the score is quasi-convex in s, so a
    # run is kept whole or not at all: here the run wins (1, 1.34, 1.62,
    # 1.85, 1.65), there the single large entry does (2, 1.77, 1.73, 1.75)
    t, _ = oracle.optimal_projection(np.array([-0.9, 1.0, 0.9, -0.9, 0.0]))
    assert list(t) == [-1, 1, 1, -1, 0]
    t, _ = oracle.optimal_projection(np.array([-0.5, 2.0, 0.5, -0.5]))
    assert list(t) == [0, 1, 0, 0]
    # among entries of equal magnitude the order is by index
    t, _ = oracle.optimal_projection(np.array([0.1, 0.1, 3.0, 0.1]))
    assert list(t) == [0, 0, 1, 0]
    t, _ = oracle.optimal_projection(np.array([-2.0]))
    assert list(t) == [-1]


def test_projection_decompositions_match_the_threshold_form():
    # §2.2: the optimal projection empirically ties T_0.7, and each greedy
    # step still never raises ||R||^2
    rng = np.random.default_rng(3)
    A = (0.02 * rng.standard_normal((48, 40))).astype(np.float32)
    for block in (0, 5):
        if block:
            rp = oracle.decompose_block(A, 1.0, 0.7, block=block, seed=1, projection=True)
            rt = oracle.decompose_block(A, 1.0, 0.7, block=block, seed=1)
        else:
            rp = oracle.decompose_seq(A, 1.0, 0.7, seed=1, projection=True)
            rt = oracle.decompose_seq(A, 1.0, 0.7, seed=1)
        assert np.all(np.diff(rp.trace) <= 1e-12 * rp.norm_a2)
        assert abs(rp.E - rt.E) < 0.02
        assert rp.E == pytest.approx(oracle.energy_from_factors(A, rp.B, rp.C, rp.D), abs=1e-12)
