"""Pins of the oracle's sequential and block ALS (CPU only).

Each check is fixed by the pages or by mathematics rather than by retyping
the oracle: the exact least-squares decrease of a rank-1 deflation, a
brute-force optimum on tiny matrices, exact recovery of ternary rank-1
matrices, symmetries, the prefix property, block b=1 against sequential,
and the residual-monotone property the pages prove.
"""
import itertools

import numpy as np
import pytest

import oracle
import synthetic


def _small(m, n, seed, scale=1.0):
    return synthetic.gaussian(m, n, seed, std=scale)


def test_rank_rule():
    assert oracle.rank_for(256, 256, 2.0) == 512
    assert oracle.rank_for(2560, 2560, 2.0) == 5120
    assert oracle.rank_for(9728, 2560, 3.0) == 7680
    assert oracle.rank_for(1024, 2560, 2.5) == 2560
    assert oracle.rank_for(4096, 4096, 3.5) == 14336
    assert oracle.rank_for(10, 3, 0.5) == 2          # 1.5 rounds up
    assert oracle.rank_for(7, 7, 0.0) == 0


def test_block_width_rule():
    assert oracle.block_width(2560, 2560, 64) == 64
    assert oracle.block_width(1024, 2560, 256) == 128   # cap floor(1024/8)
    assert oracle.block_width(15, 100, 64) == 1         # cap 1 -> sequential
    assert oracle.block_width(100, 100, 1) == 1


def test_sequential_invariants():
    A = _small(48, 40, 0)
    r = oracle.decompose_seq(A, 1.5, 0.7, iters=15, seed=3)
    k = oracle.rank_for(48, 40, 1.5)
    assert r.B.shape == (48, k) and r.C.shape == (k, 40) and r.D.shape == (k,)
    assert set(np.unique(r.B)).issubset({-1, 0, 1})
    assert set(np.unique(r.C)).issubset({-1, 0, 1})
    # every component has a nonzero u and v (the fallback guarantees it)
    assert np.all(np.count_nonzero(r.B, axis=0) > 0)
    assert np.all(np.count_nonzero(r.C, axis=1) > 0)
    # ||R||^2 never increases (Appendix), and each step removes exactly
    # (u^T R v)^2 / (||u||^2 ||v||^2), the least-squares optimum for that u, v
    prev = np.concatenate([[r.norm_a2], r.trace[:-1]])
    assert np.all(r.trace <= prev * (1 + 1e-12))
    np.testing.assert_allclose(prev - r.trace, r.extra["decrease"], rtol=1e-9,
                               atol=1e-12 * r.norm_a2)
    # the energy of the factors alone matches the trace
    assert oracle.energy_from_factors(A, r.B, r.C, r.D) == pytest.approx(r.E, abs=1e-12)


def test_scale_is_least_squares():
    # For the fitted u, v, no other scale lowers ||R - d u v^T||.
    A = _small(30, 20, 1)
    R = A.astype(np.float64)
    fit = oracle.rank1_fit(R, oracle.init_signs(0, 0, 30), 0.7, 15)
    u, v = fit["u"].astype(float), fit["v"].astype(float)
    f = lambda d: float(np.sum((R - d * np.outer(u, v)) ** 2))
    d = fit["d"]
    for eps in (1e-3, -1e-3, 1e-6, -1e-6):
        assert f(d) <= f(d * (1 + eps))


def test_brute_force_rank1_bound():
    # The ALS decrease can never beat the best ternary rank-1 fit.
    rng = np.random.default_rng(7)
    tern = [np.array(t, dtype=float) for t in itertools.product((-1, 0, 1), repeat=4) if any(t)]
    for trial in range(5):
        R = rng.standard_normal((4, 4))
        best = max((u @ R @ v) ** 2 / ((u @ u) * (v @ v)) for u in tern for v in tern)
        fit = oracle.rank1_fit(R, oracle.init_signs(trial, 0, 4), 0.7, 15)
        got = fit["c"] ** 2 / (fit["nnz_u"] * fit["nnz_v"])
        assert got <= best * (1 + 1e-12)
        assert got > 0


def test_exact_recovery_of_ternary_rank1():
    rng = np.random.default_rng(9)
    for trial in range(4):
        m, n = 24, 17
        us = rng.choice([-1, 0, 1], size=m, p=[0.3, 0.4, 0.3])
        vs = rng.choice([-1, 0, 1], size=n, p=[0.3, 0.4, 0.3])
        us[0], vs[0] = 1, -1
        A = (0.375 * np.outer(us, vs)).astype(np.float32)
        r = oracle.decompose_seq(A, 0.25, 0.7, seed=trial)
        assert r.trace[0] == 0.0
        assert r.E == 1.0
        assert np.all(r.D[1:] == 0.0)
        assert abs(r.D[0]) == 0.375


def test_single_entry_matrix():
    A = np.zeros((9, 13), dtype=np.float32)
    A[4, 7] = -2.5
    r = oracle.decompose_seq(A, 0.5, 1.0, seed=0)
    assert r.E == 1.0
    assert r.B[:, 0].tolist() == [0] * 4 + [int(np.sign(r.B[4, 0]))] + [0] * 4
    assert np.count_nonzero(r.C[0]) == 1 and r.C[0, 7] != 0
    assert r.D[0] * r.B[4, 0] * r.C[0, 7] == -2.5


def test_zero_matrix():
    r = oracle.decompose_seq(np.zeros((8, 8), np.float32), 1.0, 0.7)
    assert r.E == 1.0 and np.all(r.D == 0.0)


def test_symmetries():
    A = _small(40, 32, 2)
    r = oracle.decompose_seq(A, 1.0, 0.7, seed=1)
    rn = oracle.decompose_seq(-A, 1.0, 0.7, seed=1)
    assert np.array_equal(rn.B, r.B) and np.array_equal(rn.C, -r.C)
    assert np.array_equal(rn.D, r.D)
    for p in (-7, 9):
        rs = oracle.decompose_seq(np.ldexp(A, p), 1.0, 0.7, seed=1)
        assert np.array_equal(rs.B, r.B) and np.array_equal(rs.C, r.C)
        assert np.array_equal(rs.D, np.ldexp(r.D, p))
        assert rs.E == r.E


def test_prefix_property():
    A = _small(36, 36, 3)
    r_small = oracle.decompose_seq(A, 0.5, 1.0, seed=2)
    r_big = oracle.decompose_seq(A, 1.5, 1.0, seed=2)
    k1 = r_small.D.size
    assert np.array_equal(r_big.B[:, :k1], r_small.B)
    assert np.array_equal(r_big.C[:k1], r_small.C)
    assert np.array_equal(r_big.D[:k1], r_small.D)
    assert r_big.E >= r_small.E


def test_block_width_one_equals_sequential():
    # With b = 1 the decorrelated targets are positive multiples of R^T u and
    # R v, T_tau is scale invariant and the joint solve reduces to the single
    # scale, so the block iteration reproduces the sequential one (§2.3, §2.4).
    A = _small(40, 28, 4)
    rs = oracle.decompose_seq(A, 1.0, 0.7, seed=5)
    rb = oracle.decompose_block(A, 1.0, 0.7, block=1, seed=5, force_width=1)
    assert np.array_equal(rb.B, rs.B) and np.array_equal(rb.C, rs.C)
    np.testing.assert_allclose(rb.D, rs.D, rtol=1e-10)
    np.testing.assert_allclose(rb.trace, rs.trace, rtol=1e-9)


def test_block_invariants():
    A = _small(96, 80, 6)
    r = oracle.decompose_block(A, 2.0, 0.7, block=8, seed=0)
    assert r.extra["b"] == 8
    prev = np.concatenate([[r.norm_a2], r.trace[:-1]])
    # per-block decrease is rhs^T M^-1 rhs >= 0 and equals the drop of ||R||^2
    assert np.all(r.extra["decrease"] >= 0)
    np.testing.assert_allclose(prev - r.trace, r.extra["decrease"], rtol=1e-8,
                               atol=1e-12 * r.norm_a2)
    assert oracle.energy_from_factors(A, r.B, r.C, r.D) == pytest.approx(r.E, abs=1e-12)
    assert set(np.unique(r.B)).issubset({-1, 0, 1})


def test_block_close_to_sequential():
    # Pages (§3.1 table caption): block within about 0.2 points of sequential.
    A = synthetic.gaussian(256, 256, 0)
    rs = oracle.decompose_seq(A, 1.0, 0.7, seed=0)
    rb = oracle.decompose_block(A, 1.0, 0.7, block=32, seed=0)
    assert abs(rb.E - rs.E) < 0.005


def test_block_trailing_partial_block():
    A = _small(64, 64, 8)
    r = oracle.decompose_block(A, 0.7, 0.7, block=8, seed=0)   # k = 45 -> 5 full + 5
    assert r.D.size == 45 and r.trace.size == 6
    assert oracle.energy_from_factors(A, r.B, r.C, r.D) == pytest.approx(r.E, abs=1e-12)


@pytest.mark.parametrize("tau,lo,hi", [(0.7, 0.36, 0.47), (1.0, 0.52, 0.62), (2.0, 0.82, 0.92)])
def test_factor_sparsity_tracks_tau(tau, lo, hi):
    # Pages (§1): tau = 0.7 / 1.0 / 2.0 give about 41 / 57 / 87 % zeros.
    A = synthetic.gaussian(128, 128, 1)
    r = oracle.decompose_seq(A, 1.0, tau, seed=0)
    zf = oracle.zero_fraction(r.B, r.C)
    assert lo < zf < hi


def test_energy_grows_with_mu():
    A = synthetic.gaussian(64, 64, 2)
    es = [oracle.decompose_seq(A, mu, 0.7, seed=0).E for mu in (0.5, 1.0, 2.0, 3.0)]
    assert all(b >= a for a, b in zip(es, es[1:]))
    assert es[-1] > 0.99


def test_rank_for_energy_matches_separate_runs():
    # Choosing mu per matrix (§3.3): the rank the trace scan picks must be the
    # smallest rank whose own, separate decomposition reaches the target --
    # found here by brute force over every rank.
    A = _small(24, 20, 11)
    a2 = float(np.sum(A.astype(np.float64) ** 2))
    big = oracle.decompose_seq(A, 1.5, 0.7, seed=4)
    energies = [oracle.decompose_seq(A, 0.0, 0.7, seed=4, k=c).E for c in range(1, big.D.size + 1)]
    for target in (0.0, 0.3, 0.6, 0.9, 0.99, energies[-1], 1.0 + 1e-9):
        want = next((c for c, e in zip(range(1, len(energies) + 1), energies) if e >= target), -1)
        assert oracle.rank_for_energy(big.trace, a2, target) == want


def test_rank_for_energy_block_steps():
    A = _small(64, 48, 12)
    a2 = float(np.sum(A.astype(np.float64) ** 2))
    big = oracle.decompose_block(A, 1.0, 0.7, block=6, seed=2)   # k = 48: 8 blocks of 6
    b = big.extra["b"]
    assert b == 6
    for nb in range(1, big.trace.size + 1):
        small = oracle.decompose_block(A, 0.0, 0.7, block=6, seed=2, k=nb * b)
        assert small.E == 1.0 - big.trace[nb - 1] / a2
        target = small.E
        got = oracle.rank_for_energy(big.trace, a2, target, step=b, total=big.D.size)
        assert got <= nb * b and got % b == 0
    assert oracle.rank_for_energy(big.trace, a2, 2.0, step=b) == -1
    assert oracle.rank_for_energy([], 0.0, 0.5) == 0
    # a trailing partial block is capped at the decomposition's rank
    assert oracle.rank_for_energy([5.0, 1.0], 10.0, 0.85, step=4, total=7) == 7


def test_sweep_on_a_single_block_continues_the_iterations():
    # With one block, adding it back restores R = A, and the refit starts
    # from the stored U, so it is the same run continued: one sweep of 15
    # iterations equals extraction with 30 when the refit is kept, and keeps
    # the 15-iteration block otherwise (whichever leaves less residual).
    # seeds 2 and 9 keep the stored block, 8 and 16 take the refit; with
    # 3 iterations every case takes it
    for seed, it in ((2, 15), (8, 15), (9, 15), (16, 15), (1, 3), (4, 3)):
        A = _small(48, 40, 20 + seed)
        r15 = oracle.decompose_block(A, 0.0, 0.7, iters=it, block=5, seed=seed, k=5)
        r30 = oracle.decompose_block(A, 0.0, 0.7, iters=2 * it, block=5, seed=seed, k=5)
        assert not np.array_equal(r15.B, r30.B)
        sw = oracle.decompose_block(A, 0.0, 0.7, iters=it, block=5, seed=seed, k=5, sweeps=1)
        want = r30 if r30.E >= r15.E else r15
        assert np.array_equal(sw.B, want.B) and np.array_equal(sw.C, want.C)
        np.testing.assert_allclose(sw.D, want.D, rtol=1e-12, atol=0)
        assert abs(sw.E - max(r15.E, r30.E)) <= 1e-12
        assert sw.extra["sweep_kept_old"] == (0 if r30.E >= r15.E else 1)


def test_sweeps_are_monotone_and_consistent():
    A = _small(96, 80, 31)
    base = oracle.decompose_block(A, 1.0, 0.7, block=10, seed=5)
    sw = oracle.decompose_block(A, 1.0, 0.7, block=10, seed=5, sweeps=4)
    tr = sw.extra["sweep_trace"]
    a2 = sw.norm_a2
    # never above the extraction's residual, never rising from sweep to sweep
    assert tr[0] <= base.trace[-1] and np.all(np.diff(tr) <= 0)
    # the recorded residual is the residual of the returned factors
    R = A.astype(np.float64) - oracle.reconstruct(sw.B, sw.C, sw.D)
    np.testing.assert_allclose(np.sum(R * R), tr[-1], rtol=1e-10)
    assert sw.E == 1.0 - tr[-1] / a2
    # the pages report a clear gain on Gaussian-like matrices
    assert sw.E > base.E + 1e-3
    # zero sweeps is the plain extraction
    z = oracle.decompose_block(A, 1.0, 0.7, block=10, seed=5, sweeps=0)
    assert np.array_equal(z.B, base.B) and np.array_equal(z.D, base.D) and z.E == base.E
    with pytest.raises(ValueError):
        oracle.decompose_block(_small(12, 12, 1), 1.0, 0.7, block=10, sweeps=1)


# ---- importance-weighted ALS (§2.5) ----------------------------------------

def _skewed_h(n, seed, sigma=1.5):
    rng = np.random.default_rng(seed)
    return np.exp(sigma * rng.standard_normal(n))


def test_importance_weights_rule():
    h = np.array([0.5, 2.0, 1.0, 0.0])
    np.testing.assert_array_equal(oracle.importance_weights(h, 0.0), [0.25, 1.0, 0.5, 0.0])
    np.testing.assert_array_equal(oracle.importance_weights(h, 0.5), [0.75, 1.5, 1.0, 0.5])
    np.testing.assert_array_equal(oracle.importance_weights(np.zeros(3), 2.0), [2.0, 2.0, 2.0])
    for bad in ((np.zeros(3), 0.0), (np.array([1.0, -1.0]), 0.0), (np.array([1.0, np.nan]), 0.0),
                (np.ones(2), -1.0)):
        with pytest.raises(ValueError):
            oracle.importance_weights(*bad)


@pytest.mark.parametrize("lam", [0.0, 3.0])
def test_uniform_weights_reduce_to_the_plain_algorithm(lam):
    # a flat importance vector gives h~ = 1 + lambda; for 1 and 4 (powers of
    # two) every step scales exactly, T_tau is scale free and d cancels the
    # factor, so the weighted run is the plain run bit for bit
    A = _small(40, 32, 9)
    w = oracle.importance_weights(np.full(32, 0.37), lam)
    s0 = oracle.decompose_seq(A, 1.0, 0.7, seed=3)
    s1 = oracle.decompose_seq(A, 1.0, 0.7, seed=3, weights=w)
    assert np.array_equal(s0.B, s1.B) and np.array_equal(s0.C, s1.C)
    np.testing.assert_array_equal(s0.D, s1.D)
    assert s1.E == s0.E
    b0 = oracle.decompose_block(A, 1.0, 0.7, block=4, seed=3)
    b1 = oracle.decompose_block(A, 1.0, 0.7, block=4, seed=3, weights=w)
    assert np.array_equal(b0.B, b1.B) and np.array_equal(b0.C, b1.C)
    np.testing.assert_allclose(b1.D, b0.D, rtol=1e-12)
    assert abs(b1.E - b0.E) <= 1e-12


def test_large_lambda_approaches_the_plain_algorithm():
    A = _small(40, 32, 10)
    w = oracle.importance_weights(_skewed_h(32, 1), 1e9)
    s0 = oracle.decompose_seq(A, 1.0, 0.7, seed=1)
    s1 = oracle.decompose_seq(A, 1.0, 0.7, seed=1, weights=w)
    assert abs(s1.E - s0.E) <= 1e-6


def test_weighted_scale_is_weighted_least_squares():
    A = _small(30, 24, 11)
    w = oracle.importance_weights(_skewed_h(24, 2), 0.0)
    res = oracle.decompose_seq(A, 0.5, 0.7, seed=2, record={0, 5}, weights=w)
    for i, rec in res.extra["records"].items():
        R = rec["R"]
        u = res.B[:, i].astype(np.float64)
        v = res.C[i].astype(np.float64)
        sw = np.sqrt(w)
        X = (np.outer(u, v) * sw).reshape(-1, 1)
        y = (R * sw).reshape(-1)
        d_ls = np.linalg.lstsq(X, y, rcond=None)[0][0]
        assert abs(res.D[i] - d_ls) <= 1e-12 * max(1.0, abs(d_ls))
        # each half-step's target is, up to a positive factor (T_tau is scale
        # free), the weighted least-squares fit of the free vector: for v the
        # weights cancel column by column, for u they do not
        hist = res.extra["records"][i]["fit"]["hist"]
        for t in range(1, len(hist)):
            up = hist[t - 1][3]
            y, vt, x, _ = hist[t]
            v_ls = np.array([np.linalg.lstsq((up * sw[j])[:, None], R[:, j] * sw[j], rcond=None)[0][0]
                             for j in range(R.shape[1])])
            np.testing.assert_allclose(y / np.sum(up * up), v_ls, rtol=1e-10, atol=1e-14)
            u_ls = np.array([np.linalg.lstsq((vt * sw)[:, None], R[r] * sw, rcond=None)[0][0]
                             for r in range(R.shape[0])])
            np.testing.assert_allclose(x / np.sum(w * vt * vt), u_ls, rtol=1e-10, atol=1e-14)


def test_block_targets_are_weighted_least_squares():
    # U target: rows of min_U ||(R - U V^T) diag(sqrt w)||^2; V target: the
    # weights cancel column by column, so it is the plain least-squares fit
    rng = np.random.default_rng(5)
    R = rng.standard_normal((20, 18))
    V = rng.choice([-1.0, 0.0, 1.0], size=(18, 4))
    U = rng.choice([-1.0, 0.0, 1.0], size=(20, 4))
    w = oracle.importance_weights(_skewed_h(18, 3), 0.1)
    T, Q = oracle.block_u_target(R, V, w)
    sw = np.sqrt(w)
    for i in range(20):
        x = np.linalg.lstsq(V * sw[:, None], R[i] * sw, rcond=None)[0]
        np.testing.assert_allclose(T[i], x, rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(Q, R @ (V * w[:, None]), rtol=1e-13)
    TV = oracle.block_v_target(R, U)
    for j in range(18):
        x_w = np.linalg.lstsq(U * sw[j], R[:, j] * sw[j], rcond=None)[0]
        np.testing.assert_allclose(TV[j], x_w, rtol=1e-4, atol=1e-6)


@pytest.mark.parametrize("block", [0, 6])
def test_weighted_runs_are_monotone_and_consistent(block):
    A = _small(64, 48, 12)
    w = oracle.importance_weights(_skewed_h(48, 4), 0.0)
    dec = oracle.decompose_block if block else (lambda *a, **k: oracle.decompose_seq(*a[:3], **k))
    kw = dict(seed=1, weights=w)
    if block:
        kw["block"] = block
    r = dec(A, 1.0, 0.7, **kw)
    assert np.all(np.diff(r.trace) <= 1e-12 * r.norm_a2)
    assert abs(r.E - oracle.energy_from_factors(A, r.B, r.C, r.D, weights=w)) <= 1e-12
    assert r.norm_a2 == pytest.approx(float(np.sum((A.astype(np.float64) ** 2) @ w)), rel=1e-14)


@pytest.mark.parametrize("block", [0, 6])
def test_weighting_raises_the_weighted_energy(block):
    # §2.5: on a skewed importance vector the weighted algorithm preserves
    # more weighted energy than the plain one
    A = _small(64, 48, 13)
    w = oracle.importance_weights(_skewed_h(48, 5, sigma=2.0), 0.0)
    if block:
        r0 = oracle.decompose_block(A, 1.0, 0.7, block=block, seed=2)
        r1 = oracle.decompose_block(A, 1.0, 0.7, block=block, seed=2, weights=w)
    else:
        r0 = oracle.decompose_seq(A, 1.0, 0.7, seed=2)
        r1 = oracle.decompose_seq(A, 1.0, 0.7, seed=2, weights=w)
    e0 = oracle.energy_from_factors(A, r0.B, r0.C, r0.D, weights=w)
    assert r1.E > e0 + 0.01, (r1.E, e0)


# ---- the single-entry safeguard (appendix §7) ----

def test_single_entry_bound_is_the_best_single_entry_fit():
    # brute force over every one-entry ternary component +-e_r e_c^T with its
    # least-squares scale: the decrease is w_c R_rc^2, the best one the bound
    rng = np.random.default_rng(5)
    R = rng.normal(size=(5, 4))
    R[2, 1] = R[0, 3] = 3.0   # a tie: the first in row-major order wins
    w = rng.uniform(0.5, 2.0, 4)
    for weights in (None, w):
        best, pos = -1.0, None
        for r in range(5):
            for c in range(4):
                u = np.zeros(5); u[r] = 1.0
                v = np.zeros(4); v[c] = 1.0
                wc = 1.0 if weights is None else weights[c]
                d = R[r, c]
                after = R - d * np.outer(u, v)
                dec = oracle.weighted_norm2(R, weights) - oracle.weighted_norm2(after, weights)
                if dec > best + 1e-12:
                    best, pos = dec, (r, c)
        bound, r, c = oracle.single_entry_bound(R, weights)
        assert abs(bound - best) <= 1e-12 * best and (r, c) == pos
    assert oracle.single_entry_bound(R)[1:] == (0, 3)


def test_safeguard_never_activates_on_gaussian_matrices():
    # the pages: the ALS decrease is far larger than the single-entry bound
    A = _small(64, 48, 3)
    assert oracle.decompose_seq(A, 1.0, 0.7, 15, 0).extra["safeguard_would"] == 0
    assert oracle.decompose_block(A, 1.0, 0.7, 15, 8, 0).extra["safeguard_would"] == 0


def test_safeguard_replaces_a_dense_fit_by_the_dominant_entry():
    # tau = 0 keeps every nonzero entry, so one iteration gives dense +-1
    # vectors whose decrease c^2 / (m n) falls far below a dominant entry's
    A = _small(12, 10, 1, 0.01)
    A[3, 7] = 5.0
    plain = oracle.decompose_seq(A, 0.2, 0.0, 1, 0)
    assert plain.extra["safeguard_would"] >= 1
    assert np.count_nonzero(plain.B[:, 0]) == 12 and np.count_nonzero(plain.C[0]) == 10
    safe = oracle.decompose_seq(A, 0.2, 0.0, 1, 0, safeguard=True)
    assert safe.extra["safeguard_would"] >= 1
    assert np.array_equal(np.nonzero(safe.B[:, 0])[0], [3]) and np.array_equal(np.nonzero(safe.C[0])[0], [7])
    assert safe.B[3, 0] == 1 and safe.C[0, 7] == 1 and safe.D[0] == float(A[3, 7])
    assert safe.trace[0] < plain.trace[0]


@pytest.mark.parametrize("tau,iters", [(0.0, 1), (0.7, 2), (2.0, 1)])
def test_safeguard_gives_the_geometric_rate(tau, iters):
    # with the safeguard every component lowers ||R||^2 by at least
    # max R_ij^2 >= ||R||^2 / (m n), the geometric rate in m n of §7
    m, n = 8, 6
    A = _small(m, n, 9)
    res = oracle.decompose_seq(A, 3.0, tau, iters, 0, safeguard=True)
    prev = res.norm_a2
    for t in res.trace:
        assert t <= (1.0 - 1.0 / (m * n)) * prev * (1 + 1e-12) + 1e-300
        prev = t
