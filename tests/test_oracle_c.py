"""Pins of the plain C fp64 oracle (oracle/c/externd_oracle.c), CPU only.

The C oracle is a second, independent transcription of T_tau (§2.2) and the
greedy sequential decomposition (§2.3) in plain loops.  Each test ties it to
something the pages or mathematics fix: hand-worked T_tau vectors, the
Gaussian zero-fraction closed form, a SplitMix64 known answer, exact
recovery of ternary rank-1 matrices, the exact residual decrease
d^2 nnz(u) nnz(v), brute force over all ternary rank-1 fits, sign symmetry,
and the special cases E = 1 (zero matrix, single entry).  Last, it is
compared with the numpy oracle on the same seeded inputs.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import oracle.c_oracle as coracle
import synthetic

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(coracle.LIB):
        coracle.build_c()


def _cases():
    with open(os.path.join(HERE, "golden", "ternarize_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["why"][:40])
def test_hand_worked_vectors(case):
    t = coracle.ternarize(np.array(case["x"], dtype=np.float64), case["tau"])
    assert t.tolist() == case["t"]


def test_gaussian_zero_fraction_closed_form():
    # For x ~ N(0, 1), mean|x| = sqrt(2/pi), so T_tau keeps |x| > tau sqrt(2/pi)
    # and the kept fraction is 1 - erf(tau / sqrt(pi)).
    rng = np.random.default_rng(11)
    x = rng.standard_normal(400000)
    for tau in (0.7, 1.0, 2.0):
        zero = float(np.mean(coracle.ternarize(x, tau) == 0))
        assert abs(zero - math.erf(tau / math.sqrt(math.pi))) < 3e-3


def test_threshold_within_the_fixed_point_window():
    rng = np.random.default_rng(12)
    for n in (1, 3, 1000, 4097):
        x = rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 6)
        thr, big = coracle.threshold(x, 0.7)
        exact = float(np.float32(0.7)) * math.fsum(np.abs(x)) / n
        _, e = math.frexp(big)
        s = 52 - e - (n - 1).bit_length()
        assert exact - float(np.float32(0.7)) * 2.0 ** -s * 1.0001 <= thr <= exact * (1 + 4e-16)


def test_splitmix64_known_answer():
    assert coracle.splitmix64_mix(0) == 0xE220A8397B1DCDAF
    u = coracle.start_vector(3, 5, 4096)
    assert set(np.unique(u).tolist()) == {-1.0, 1.0}
    assert abs(float(u.mean())) < 0.05


def test_exact_recovery_of_ternary_rank1():
    rng = np.random.default_rng(9)
    for trial in range(3):
        m, n = 24, 17
        us = rng.choice([-1, 0, 1], size=m, p=[0.3, 0.4, 0.3])
        vs = rng.choice([-1, 0, 1], size=n, p=[0.3, 0.4, 0.3])
        us[0], vs[0] = 1, -1
        A = (0.375 * np.outer(us, vs)).astype(np.float32)
        B, C, D, trace, E = coracle.decompose_seq(A, 4, 0.7, seed=trial)
        assert trace[0] == 0.0 and E == 1.0
        assert abs(D[0]) == 0.375 and np.all(D[1:] == 0.0)
        assert np.array_equal(np.outer(B[:, 0], C[0]) * D[0], A.astype(np.float64))


def test_zero_and_single_entry_matrices():
    _, _, D, _, E = coracle.decompose_seq(np.zeros((7, 5), np.float32), 5, 0.7)
    assert E == 1.0 and np.all(D == 0.0)
    A = np.zeros((9, 13), dtype=np.float32)
    A[4, 7] = -2.5
    B, C, D, trace, E = coracle.decompose_seq(A, 3, 0.7)
    assert E == 1.0 and trace[0] == 0.0
    assert B[4, 0] * C[0, 7] * D[0] == -2.5


def test_decrease_is_exact_and_residual_never_grows():
    # Each component lowers ||R||^2 by exactly (u^T R v)^2 / (nnz(u) nnz(v)),
    # which is d^2 nnz(u) nnz(v) with the least-squares d.
    A = synthetic.gaussian(40, 33, 4)
    B, C, D, trace, E = coracle.decompose_seq(A, 40, 0.7, seed=2)
    prev = float(np.sum(A.astype(np.float64) ** 2))
    for i in range(40):
        dec = D[i] ** 2 * np.count_nonzero(B[:, i]) * np.count_nonzero(C[i])
        assert trace[i] <= prev
        assert abs((prev - trace[i]) - dec) <= 1e-12 * prev
        prev = trace[i]
    assert abs(E - (1.0 - trace[-1] / float(np.sum(A.astype(np.float64) ** 2)))) < 1e-15


def test_first_component_never_beats_brute_force():
    rng = np.random.default_rng(7)
    tern = [np.array(t, dtype=float) for t in itertools.product((-1, 0, 1), repeat=4) if any(t)]
    for trial in range(5):
        A = rng.standard_normal((4, 4)).astype(np.float32)
        R = A.astype(np.float64)
        best = max((u @ R @ v) ** 2 / ((u @ u) * (v @ v)) for u in tern for v in tern)
        B, C, D, trace, E = coracle.decompose_seq(A, 1, 0.7, seed=trial)
        got = float(np.sum(R ** 2)) - trace[0]
        assert 0 < got <= best * (1 + 1e-12)


def test_sign_symmetry():
    A = synthetic.gaussian(30, 26, 8)
    B, C, D, trace, E = coracle.decompose_seq(A, 20, 0.7, seed=1)
    Bn, Cn, Dn, tn, En = coracle.decompose_seq(-A, 20, 0.7, seed=1)
    assert np.array_equal(Bn, B) and np.array_equal(Cn, -C)
    assert np.array_equal(Dn, D) and np.array_equal(tn, trace) and En == E


def test_agrees_with_the_numpy_oracle():
    # Two transcriptions that share no code: the same ternarization bits on
    # random vectors, and the same decomposition on a seeded matrix.
    rng = np.random.default_rng(21)
    for n in (1, 2, 5, 64, 1000, 2560):
        x = rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 3)
        for tau in (0.7, 1.0, 2.0):
            assert np.array_equal(coracle.ternarize(x, tau), oracle.ternarize(x, tau))
    for r in range(6):
        assert np.array_equal(coracle.start_vector(7, r, 300), oracle.init_signs(7, r, 300).astype(np.float64))
    A = synthetic.gaussian(48, 40, 3)
    B, C, D, trace, E = coracle.decompose_seq(A, 40, 0.7, seed=5)
    ref = oracle.decompose_seq(A, 40 / 40, 0.7, seed=5)
    assert np.array_equal(B, ref.B) and np.array_equal(C, ref.C)
    np.testing.assert_allclose(D, ref.D, rtol=1e-12, atol=0)
    np.testing.assert_allclose(trace, ref.trace, rtol=1e-10)
    assert abs(E - ref.E) < 1e-12


def test_block_width_one_equals_sequential():
    # With b = 1 the decorrelated targets are positive multiples of R^T u
    # and R v, T_tau is scale invariant and the joint solve is the single
    # scale: the block iteration reproduces the sequential one (§2.3, §2.4).
    A = synthetic.gaussian(40, 28, 4)
    Bs, Cs, Ds, ts, Es = coracle.decompose_seq(A, 28, 0.7, seed=5)
    Bb, Cb, Db, tb, Eb, retries = coracle.decompose_block(A, 28, 1, 0.7, seed=5)
    assert np.array_equal(Bb, Bs) and np.array_equal(Cb, Cs)
    np.testing.assert_allclose(Db, Ds, rtol=1e-10)
    np.testing.assert_allclose(tb, ts, rtol=1e-9)
    assert retries == 0


def test_block_energy_and_residual_bookkeeping():
    # E = 1 - ||A - B diag(D) C||^2 / ||A||^2 (§2.1) recomputed from the C
    # oracle's own factors, a residual that never grows block to block, and
    # ternary factors with a trailing partial block (k = 150, b = 8).
    A = synthetic.gaussian(96, 80, 6)
    B, C, D, trace, E, retries = coracle.decompose_block(A, 150, 8, 0.7, seed=0)
    assert trace.size == 19 and set(np.unique(B)).issubset({-1, 0, 1}) and set(np.unique(C)).issubset({-1, 0, 1})
    A64 = A.astype(np.float64)
    a2 = float(np.sum(A64 ** 2))
    resid = A64 - (B.astype(np.float64) * D) @ C.astype(np.float64)
    assert abs((1.0 - float(np.sum(resid ** 2)) / a2) - E) < 1e-12
    prev = np.concatenate([[a2], trace[:-1]])
    assert np.all(trace <= prev * (1 + 1e-14))


def test_block_agrees_with_the_numpy_oracle():
    A = synthetic.gaussian(96, 80, 6)
    B, C, D, trace, E, retries = coracle.decompose_block(A, 160, 8, 0.7, seed=0)
    ref = oracle.decompose_block(A, 2.0, 0.7, block=8, seed=0)
    assert ref.extra["b"] == 8 and ref.B.shape[1] == 160
    assert np.array_equal(B, ref.B) and np.array_equal(C, ref.C)
    np.testing.assert_allclose(D, ref.D, rtol=1e-9)
    np.testing.assert_allclose(trace, ref.trace, rtol=1e-9)
    assert abs(E - ref.E) < 1e-12
    assert retries == ref.extra["ridge_retries"]
