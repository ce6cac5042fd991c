"""GPU parity of the sequential path against the fp64 oracle.

Bars (from the method's precision requirements): ternarization of identical
inputs is bit-exact; each GEMV output and each scale d is within 1e-5
(norm-wise relative) of the fp64 oracle applied to the same fp32 inputs;
the fp32 deflation is bit-exact against a float32 CPU emulation; end-to-end
energy is within 2e-3 of the oracle's on the same seeded input, and the
energy the GPU reports agrees with an fp64 recomputation from its own factors
to 1e-5.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def _goldens():
    p = os.path.join(HERE, "golden", "oracle_energies.json")
    if not os.path.exists(p):
        return {}
    return json.load(open(p))["entries"]


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _codes_to_host(t):
    return t.cpu().numpy().view(np.uint32)


def _relnorm(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def _factors(res):
    B = oracle.unpack2(_codes_to_host(res.B2), res.m).T
    C = oracle.unpack2(_codes_to_host(res.C2), res.n)
    D = res.D.cpu().numpy().astype(np.float64)
    return B, C, D


# ---------------------------------------------------------------------------
# single-step kernels
# ---------------------------------------------------------------------------

def _ternarize_cases():
    rng = np.random.default_rng(0)
    cases = [np.array(c["x"], np.float32) for c in
             json.load(open(os.path.join(HERE, "golden", "ternarize_cases.json")))["cases"]]
    for n in (1, 2, 15, 16, 17, 255, 1000, 2560, 9728, 100_003):
        cases.append(rng.standard_normal(n).astype(np.float32))
    cases.append((rng.standard_normal(5000) * np.exp(3 * rng.standard_normal(5000))).astype(np.float32))
    cases.append(np.full(77, -0.125, np.float32))                       # all ties
    z = np.zeros(300, np.float32); z[123] = -1e-30; cases.append(z)     # one tiny entry
    cases.append(np.zeros(40, np.float32))                              # all zero
    d = np.zeros(64, np.float32); d[[5, 40]] = 3.0; d[7] = -3.0; cases.append(d)   # tie at max
    cases.append(np.float32(1e-40) * np.ones(33, np.float32))           # subnormals
    return cases


def test_ternarize_bit_exact(lib):
    for x in _ternarize_cases():
        for tau in (0.0, 0.7, 1.0, 2.0, 5.0):
            codes, nnz = lib.ternarize(_dev(x), tau)
            ref = oracle.ternarize(x.astype(np.float64), tau)
            assert np.array_equal(_codes_to_host(codes), oracle.pack2(ref[None, :])[0]), (x.size, tau)
            assert int(nnz.item()) == int(np.count_nonzero(ref))


@pytest.mark.parametrize("m,n", [(1, 1), (1, 300), (300, 1), (257, 517), (2560, 2560), (9728, 2560)])
def test_gemv_parity(lib, m, n):
    rng = np.random.default_rng(m * 7 + n)
    R = rng.standard_normal((m, n)).astype(np.float32)
    u = rng.choice([-1, 0, 1], size=m, p=[0.3, 0.4, 0.3]).astype(np.int8)
    v = rng.choice([-1, 0, 1], size=n, p=[0.3, 0.4, 0.3]).astype(np.int8)
    Rd = _dev(R)
    uc = _dev(oracle.pack2(u[None, :])[0].view(np.int32))
    vc = _dev(oracle.pack2(v[None, :])[0].view(np.int32))
    y = lib.gemv_t(Rd, uc).cpu().numpy()
    x = lib.gemv_n(Rd, vc).cpu().numpy()
    R64 = R.astype(np.float64)
    assert _relnorm(y, R64.T @ u) <= 1e-5
    assert _relnorm(x, R64 @ v) <= 1e-5


def test_deflate_bit_exact(lib):
    rng = np.random.default_rng(3)
    m, n = 333, 517
    R = rng.standard_normal((m, n)).astype(np.float32)
    u = rng.choice([-1, 0, 1], size=m).astype(np.int8)
    v = rng.choice([-1, 0, 1], size=n).astype(np.int8)
    d = np.float32(0.3712)
    Rd = _dev(R)
    lib.deflate(Rd, _dev(oracle.pack2(u[None])[0].view(np.int32)),
                _dev(oracle.pack2(v[None])[0].view(np.int32)), float(d))
    expect = (R - (d * np.outer(u, v).astype(np.float32))).astype(np.float32)
    assert np.array_equal(Rd.cpu().numpy(), expect)


# ---------------------------------------------------------------------------
# per-step parity of the full decomposition (captured component)
# ---------------------------------------------------------------------------

# stats[mode] of each requested sequential mode (persistent streaming reports 3)
_MODE_STAT = {0: 0, 1: 1, 2: 3}


def _check_component(res, A, comp, tau, iters, seed):
    cap = {k: v.cpu().numpy() for k, v in res.capture.items()}
    R = cap["R"]
    assert np.array_equal(cap["Rcol"], R), "row and column copies of R differ"
    R64 = R.astype(np.float64)
    m, n = R.shape
    u = oracle.init_signs(seed, comp, m)
    for t in range(iters):
        y = cap["y"][t]
        assert _relnorm(y, R64.T @ u) <= 1e-5, ("y", t)
        v = cap["v"][t].astype(np.float64)
        assert np.array_equal(oracle.ternarize(y.astype(np.float64), tau), cap["v"][t]), ("v", t)
        x = cap["x"][t]
        assert _relnorm(x, R64 @ v) <= 1e-5, ("x", t)
        assert np.array_equal(oracle.ternarize(x.astype(np.float64), tau), cap["u"][t]), ("u", t)
        u = cap["u"][t].astype(np.float64)
    d_ref = (u @ R64 @ v) / (np.count_nonzero(u) * np.count_nonzero(v))
    d = float(cap["d"][0])
    assert abs(d - d_ref) <= 1e-5 * abs(d_ref) + 1e-30
    # stored factors of this component are the captured final u, v, d
    B, C, D = _factors(res)
    assert np.array_equal(B[:, comp], cap["u"][iters - 1])
    assert np.array_equal(C[comp], cap["v"][iters - 1])
    assert D[comp] == np.float64(np.float32(d))
    # the deflation is one fp32 rounding per entry
    expect = (R - np.float32(d) * np.outer(cap["u"][iters - 1], cap["v"][iters - 1]).astype(np.float32))
    assert np.array_equal(cap["R_next"], expect.astype(np.float32))
    if comp == 0:
        assert np.array_equal(R, A)


@pytest.mark.parametrize("mode", [1, 0, 2])
@pytest.mark.parametrize("comp", [0, 5, 511])
def test_capture_parity_gauss256(lib, mode, comp):
    c = synthetic.WORKLOADS["gauss256"]
    A = synthetic.workload_matrix("gauss256")
    Ad = _dev(A)
    res = lib.decompose(Ad, c["mu"], c["tau"], c["iters"], 0, c["seed"], mode=mode, capture=comp,
                        stats=True)
    torch.cuda.synchronize()
    assert res.stat("mode") == _MODE_STAT[mode]
    _check_component(res, A, comp, c["tau"], c["iters"], c["seed"])
    # the capture build computes exactly what the production build computes
    plain = lib.decompose(Ad, c["mu"], c["tau"], c["iters"], 0, c["seed"], mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(plain.B2, res.B2) and torch.equal(plain.C2, res.C2)
    assert torch.equal(plain.D, res.D) and torch.equal(plain.energy, res.energy)


@pytest.mark.parametrize("m,n,comp", [(37, 53, 3), (300, 1, 0), (2, 129, 1), (700, 450, 9)])
def test_capture_parity_ragged(lib, m, n, comp):
    A = synthetic.gaussian(m, n, 11)
    res = lib.decompose(_dev(A), 1.0, 1.0, 6, 0, 3, capture=comp)
    torch.cuda.synchronize()
    _check_component(res, A, comp, 1.0, 6, 3)


def test_capture_parity_llm2560_full_size(lib):
    c = synthetic.WORKLOADS["llm2560"]
    A = synthetic.workload_matrix("llm2560")
    res = lib.decompose(_dev(A), c["mu"], c["tau"], c["iters"], 0, c["seed"], capture=2, stats=True)
    torch.cuda.synchronize()
    assert res.stat("mode") == 1 and res.stat("grid") == 256
    _check_component(res, A, 2, c["tau"], c["iters"], c["seed"])


# ---------------------------------------------------------------------------
# end to end
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [1, 0])
def test_end_to_end_gauss256(lib, mode):
    c = synthetic.WORKLOADS["gauss256"]
    A = synthetic.workload_matrix("gauss256")
    Ad = _dev(A)
    res = lib.decompose(Ad, c["mu"], c["tau"], c["iters"], 0, c["seed"], mode=mode, trace=True,
                        stats=True)
    E = float(res.energy.item())
    ref = oracle.decompose_seq(A, c["mu"], c["tau"], c["iters"], c["seed"])
    assert abs(E - ref.E) <= 2e-3
    B, C, D = _factors(res)
    assert abs(E - oracle.energy_from_factors(A, B, C, D)) <= 1e-5
    assert abs(float(lib.energy(Ad, res.B2, res.C2, res.D).item()) - E) <= 1e-5
    tr = res.trace.cpu().numpy()
    assert np.all(np.diff(tr) <= 1e-9 * ref.norm_a2)
    assert abs(1 - tr[-1] / ref.norm_a2 - E) <= 1e-5
    assert res.stat("nnz_b") == np.count_nonzero(B) and res.stat("nnz_c") == np.count_nonzero(C)
    assert res.stat("timeouts") == 0
    # run-to-run determinism
    again = lib.decompose(Ad, c["mu"], c["tau"], c["iters"], 0, c["seed"], mode=mode)
    assert torch.equal(again.B2, res.B2) and torch.equal(again.D, res.D)
    assert torch.equal(again.energy, res.energy)


def test_end_to_end_llm2560_sequential(lib):
    g = _goldens().get("llm2560_seq")
    if g is None:
        pytest.skip("oracle golden for the 2560x2560 sequential run not generated")
    c = synthetic.WORKLOADS["llm2560"]
    A = synthetic.workload_matrix("llm2560")
    Ad = _dev(A)
    res = lib.decompose(Ad, c["mu"], c["tau"], c["iters"], 0, c["seed"], stats=True)
    E = float(res.energy.item())
    assert abs(E - g["E"]) <= 2e-3
    B, C, D = _factors(res)
    assert abs(E - oracle.energy_from_factors(A, B, C, D)) <= 1e-5
    assert abs(oracle.zero_fraction(B, C) - g["zero_fraction"]) < 0.01
    assert res.stat("timeouts") == 0


def test_symmetries_bit_exact(lib):
    A = synthetic.gaussian(200, 150, 5)
    base = lib.decompose(_dev(A), 1.0, 0.7, 15, 0, 0)
    neg = lib.decompose(_dev(-A), 1.0, 0.7, 15, 0, 0)
    sc = lib.decompose(_dev(np.ldexp(A, 7)), 1.0, 0.7, 15, 0, 0)
    torch.cuda.synchronize()
    Bb, Cb, Db = _factors(base)
    Bn, Cn, Dn = _factors(neg)
    Bs, Cs, Ds = _factors(sc)
    assert np.array_equal(Bn, Bb) and np.array_equal(Cn, -Cb) and np.array_equal(Dn, Db)
    assert np.array_equal(Bs, Bb) and np.array_equal(Cs, Cb) and np.array_equal(Ds, np.ldexp(Db, 7))
    assert torch.equal(sc.energy, base.energy)


def test_prefix_property(lib):
    A = synthetic.gaussian(256, 256, 1)
    small = lib.decompose(_dev(A), 0.5, 0.7, 15, 0, 2)
    big = lib.decompose(_dev(A), 1.5, 0.7, 15, 0, 2)
    torch.cuda.synchronize()
    k1 = small.k
    assert torch.equal(big.B2[:k1], small.B2) and torch.equal(big.C2[:k1], small.C2)
    assert torch.equal(big.D[:k1], small.D)
    assert float(big.energy.item()) >= float(small.energy.item())


def test_degenerate_inputs(lib):
    # all-zero matrix: every component is inert, E := 1
    z = lib.decompose(_dev(np.zeros((64, 48), np.float32)), 1.0, 0.7, 15, 0, 0, stats=True)
    assert float(z.energy.item()) == 1.0 and float(z.D.abs().max().item()) == 0.0
    # exact ternary rank-1 matrix is recovered by the first component
    rng = np.random.default_rng(9)
    us = rng.choice([-1, 0, 1], size=96); vs = rng.choice([-1, 0, 1], size=80)
    us[0] = 1; vs[0] = -1
    A = (0.375 * np.outer(us, vs)).astype(np.float32)
    r = lib.decompose(_dev(A), 0.05, 0.7, 15, 0, 0)
    assert float(r.energy.item()) == 1.0
    assert abs(float(r.D[0].item())) == 0.375
    # single nonzero entry
    A = np.zeros((40, 30), np.float32); A[17, 3] = -2.5
    r = lib.decompose(_dev(A), 0.1, 1.0, 15, 0, 0)
    assert float(r.energy.item()) == 1.0
    # non-finite input -> NaN energy, zeroed factors
    A = synthetic.gaussian(32, 32, 0); A[3, 4] = np.inf
    r = lib.decompose(_dev(A), 1.0, 0.7, 15, 0, 0, stats=True)
    assert np.isnan(float(r.energy.item())) and r.stat("nonfinite") == 1
    assert float(r.D.abs().max().item()) == 0.0


def test_shape_limits_and_modes(lib):
    assert lib.resident_fits(2560, 2560)
    assert not lib.resident_fits(4096, 4096)
    A = synthetic.gaussian(600, 40, 2)   # fits; streaming forced
    a = lib.decompose(_dev(A), 1.0, 0.7, 15, 0, 0, mode=lib.MODE_STREAMING, stats=True)
    b = lib.decompose(_dev(A), 1.0, 0.7, 15, 0, 0, mode=lib.MODE_RESIDENT, stats=True)
    p = lib.decompose(_dev(A), 1.0, 0.7, 15, 0, 0, mode=lib.MODE_PERSISTENT, stats=True)
    assert a.stat("mode") == 0 and b.stat("mode") == 1 and p.stat("mode") == 3
    ref = oracle.decompose_seq(A, 1.0, 0.7, 15, 0)
    assert abs(float(a.energy.item()) - ref.E) <= 2e-3
    assert abs(float(b.energy.item()) - ref.E) <= 2e-3
    assert abs(float(p.energy.item()) - ref.E) <= 2e-3
    with pytest.raises(lib.ExterndError):   # n % 4 != 0: not for the persistent kernel
        lib.decompose(_dev(synthetic.gaussian(64, 30, 0)), 0.5, 0.7, 1, 0, 0, mode=lib.MODE_PERSISTENT)
    with pytest.raises(lib.ExterndError):
        lib.decompose(_dev(synthetic.gaussian(4096, 4096, 0)), 0.01, 0.7, 1, 0, 0,
                      mode=lib.MODE_RESIDENT)


def test_reconstruct_matches_oracle(lib):
    A = synthetic.gaussian(130, 70, 4)
    res = lib.decompose(_dev(A), 1.0, 0.7, 15, 0, 0)
    Ah = lib.reconstruct(res.B2, res.C2, res.D, 130, 70).cpu().numpy()
    B, C, D = _factors(res)
    ref = oracle.reconstruct(B, C, D)
    assert np.max(np.abs(Ah - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_streaming_beyond_resident_limit(lib):
    # The 9728 x 2560 matrix does not fit on chip: AUTO runs the persistent
    # streaming kernel, and the streaming kernel chain is run too.  The first
    # 32 components against the oracle's, with the per-component trace.
    c = synthetic.WORKLOADS["mlp9728"]
    A = synthetic.workload_matrix("mlp9728")
    m, n = A.shape
    assert not lib.resident_fits(m, n)
    mu = 32.25 / min(m, n)
    Ad = _dev(A)
    ref = oracle.decompose_seq(A, mu, c["tau"], c["iters"], c["seed"])
    for mode, stat in ((lib.MODE_AUTO, 3), (lib.MODE_STREAMING, 0)):
        res = lib.decompose(Ad, mu, c["tau"], c["iters"], 0, c["seed"], mode=mode, trace=True, stats=True)
        E = float(res.energy.item())
        assert res.k == 32 and res.stat("mode") == stat
        assert abs(E - ref.E) <= 2e-3, (E, ref.E)
        B, C, D = _factors(res)
        assert abs(E - oracle.energy_from_factors(A, B, C, D)) <= 1e-5
        tr = res.trace.cpu().numpy()
        assert np.all(np.diff(tr) <= 1e-9 * ref.norm_a2)
        assert np.max(np.abs(tr - np.asarray(ref.trace))) <= 2e-3 * ref.norm_a2
        assert res.stat("nnz_b") == np.count_nonzero(B) and res.stat("nnz_c") == np.count_nonzero(C)


@pytest.mark.parametrize("m,n,comp", [(37, 52, 3), (2, 128, 1), (700, 452, 9), (5000, 300, 4),
                                      (1100, 5000, 2), (4096, 4096, 1), (2000, 8000, 2),
                                      (10240, 10240, 1)])
def test_capture_parity_streaming_persistent(lib, m, n, comp):
    # The persistent streaming kernel (R in device memory, one cooperative
    # launch) on every kind of shape it covers: ragged slabs, workgroups with
    # no rows or no columns, each of its (KR, KC) tilings (5,5), (5,10),
    # (10,5), (8,8), (5,20) through the 9728 x 2560 tests, (20,5) and (20,20),
    # and its largest shape, 10240 x 10240 (40 rows per workgroup, column
    # blocks of 64 words; R is 419 MB, past the 256 MB last-level cache).
    A = synthetic.gaussian(m, n, 12)
    mu = (comp + 3.25) / min(m, n)
    res = lib.decompose(_dev(A), mu, 1.0, 6, 0, 3, mode=lib.MODE_PERSISTENT, capture=comp, stats=True)
    torch.cuda.synchronize()
    assert res.stat("mode") == 3 and res.stat("grid") > 0
    _check_component(res, A, comp, 1.0, 6, 3)
    plain = lib.decompose(_dev(A), mu, 1.0, 6, 0, 3, mode=lib.MODE_PERSISTENT)
    torch.cuda.synchronize()
    assert torch.equal(plain.B2, res.B2) and torch.equal(plain.C2, res.C2) and torch.equal(plain.D, res.D)


def test_streaming_persistent_256_components(lib):
    # 256 components of the 9728 x 2560 LLM-shaped matrix in persistent
    # streaming mode against the oracle's: energy, the energy from the
    # factors, the trace.
    c = synthetic.WORKLOADS["mlp9728"]
    A = synthetic.workload_matrix("mlp9728")
    mu = 256.25 / min(A.shape)
    res = lib.decompose(_dev(A), mu, 0.7, c["iters"], 0, c["seed"], mode=lib.MODE_PERSISTENT, trace=True,
                        stats=True)
    E = float(res.energy.item())
    assert res.k == 256 and res.stat("mode") == 3 and res.stat("timeouts") == 0
    ref = oracle.decompose_seq(A, mu, 0.7, c["iters"], c["seed"])
    assert abs(E - ref.E) <= 2e-3, (E, ref.E)
    B, C, D = _factors(res)
    assert abs(E - oracle.energy_from_factors(A, B, C, D)) <= 1e-5
    tr = res.trace.cpu().numpy()
    assert np.all(np.diff(tr) <= 1e-9 * ref.norm_a2)
    assert np.max(np.abs(tr - np.asarray(ref.trace))) <= 2e-3 * ref.norm_a2
    # the safeguard decisions follow each trajectory (fp32 here, fp64 in the
    # oracle); they are compared exactly where the margins are wide
    # (test_gpu_safeguard.py), here within 2 % of the components
    assert abs(res.stat("safeguard") - ref.extra["safeguard_would"]) <= 0.02 * res.k
