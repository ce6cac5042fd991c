"""Pins of the oracle's codec, energy, storage formula and starting-vector rule."""
import math

import numpy as np
import pytest

import oracle


def test_pack2_known_words():
    # hand-packed: +1 -> 01, -1 -> 11, 0 -> 00, element j at bits 2j..2j+1
    T = np.array([[1, -1, 0, 1]], dtype=np.int8)
    assert oracle.pack2(T).tolist() == [[1 + (3 << 2) + (1 << 6)]]
    T = np.zeros((1, 17), dtype=np.int8)
    T[0, 15] = -1
    T[0, 16] = 1
    assert oracle.pack2(T).tolist() == [[3 << 30, 1]]


def test_pack2_roundtrip_and_invalid():
    rng = np.random.default_rng(0)
    for L in (1, 15, 16, 17, 100):
        T = rng.integers(-1, 2, size=(5, L)).astype(np.int8)
        assert np.array_equal(oracle.unpack2(oracle.pack2(T), L), T)
    with pytest.raises(ValueError):
        oracle.unpack2(np.array([[2]], dtype=np.uint32), 1)
    with pytest.raises(ValueError):
        oracle.unpack2(np.array([[1 << 2]], dtype=np.uint32), 1)


def test_energy_of_exact_factors():
    rng = np.random.default_rng(1)
    B = rng.integers(-1, 2, size=(20, 7))
    C = rng.integers(-1, 2, size=(7, 11))
    D = rng.standard_normal(7)
    A = (B * D) @ C
    assert oracle.energy_from_factors(A, B, C, D) == pytest.approx(1.0, abs=1e-14)
    assert oracle.energy_from_factors(A, B, C, np.zeros(7)) == 0.0


def test_bpw_eq1():
    # Eq. 1 (§2.6) for a square matrix at mu=2 with 43% zeros: 2*2*(2-0.43)
    assert oracle.bpw_eff(2.0, 100, 100, 0.43) == pytest.approx(6.28)
    # mask entropy quoted on the pages for 43% zeros, H(0.43) ~ 0.99 bits
    h = -(0.43 * math.log2(0.43) + 0.57 * math.log2(0.57))
    assert round(h, 2) == 0.99
    # fixed 2-bit codes, counted by hand: each of 512 components stores
    # 256 + 256 codes of 2 bits (1024 bits) and one 32-bit scale, 1056 bits;
    # 512 * 1056 = 540,672 bits over 256 * 256 = 65,536 weights = 8.25
    assert oracle.bpw_packed2(512, 256, 256) == 8.25
    # a tall matrix: 3 * (2 * (40 + 10) + 32) = 396 bits over 400 weights
    assert oracle.bpw_packed2(3, 40, 10) == pytest.approx(0.99)


def test_zero_fraction_hand_counted():
    # B has 2 zeros of 6 entries, C has 3 of 6: 5 of 12 over both factors
    B = np.array([[1, 0], [0, -1], [1, 1]], dtype=np.int8)
    C = np.array([[0, 0, 1], [-1, 0, 1]], dtype=np.int8)
    assert oracle.zero_fraction(B, C) == pytest.approx(5 / 12, abs=1e-15)
    assert oracle.zero_fraction(np.zeros((4, 2)), np.zeros((2, 3))) == 1.0
    assert oracle.zero_fraction(np.ones((4, 2)), -np.ones((2, 3))) == 0.0


def test_splitmix64_known_answer():
    # First SplitMix64 output from state 0, as published with the generator.
    assert oracle.splitmix64_mix(0) == 0xE220A8397B1DCDAF


def test_init_signs_matches_scalar_hash_and_is_balanced():
    u = oracle.init_signs(7, 3, 1000)
    for r in (0, 1, 500, 999):
        assert u[r] == (-1.0 if oracle.init_hash(7, 3, r) >> 63 else 1.0)
    big = oracle.init_signs(0, 0, 200_000)
    assert abs(big.mean()) < 0.01
    # different components and seeds give uncorrelated starts
    a, b, c = oracle.init_signs(0, 0, 50_000), oracle.init_signs(0, 1, 50_000), oracle.init_signs(1, 0, 50_000)
    assert abs(a @ b) / 50_000 < 0.02 and abs(a @ c) / 50_000 < 0.02
    Ub = oracle.init_block(0, 4, 3, 64)
    assert np.array_equal(Ub[:, 1], oracle.init_signs(0, 5, 64))


def test_apply_factors_pins():
    # y = B (diag(D) (C x)) must equal the dense product (B diag(D) C) x, and on
    # one-hot inputs it returns the columns of the reconstruction.
    rng = np.random.default_rng(12)
    for (m, n, k) in [(5, 7, 3), (37, 53, 20), (1, 9, 4), (8, 1, 2)]:
        B = rng.integers(-1, 2, size=(m, k)).astype(np.int8)
        C = rng.integers(-1, 2, size=(k, n)).astype(np.int8)
        D = rng.standard_normal(k)
        x = rng.standard_normal(n)
        dense = oracle.reconstruct(B, C, D)
        np.testing.assert_allclose(oracle.apply_factors(B, C, D, x), dense @ x, rtol=1e-12, atol=1e-12)
        for j in range(n):
            e = np.zeros(n)
            e[j] = 1.0
            np.testing.assert_allclose(oracle.apply_factors(B, C, D, e), dense[:, j], rtol=0, atol=1e-12)
    # a single component: y = d u (v . x)
    u = np.array([1, 0, -1], dtype=np.int8)
    v = np.array([[0, 1, 1, -1]], dtype=np.int8)
    x = np.array([0.5, 2.0, -1.0, 3.0])
    assert oracle.apply_factors(u[:, None], v, np.array([0.25]), x).tolist() == [-0.5, 0.0, 0.5]
