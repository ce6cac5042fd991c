"""Full-size GPU runs of the block-ALS workloads against the fp64 oracle's goldens.

The goldens (tests/golden/oracle_energies.json) are written by
tests/golden/make_oracle_goldens.py, which calls only oracle/.  Each run is
checked to the same bar as the 2560 x 2560 case: energy within 2e-3 of the
oracle's, the reported energy within 1e-5 of an fp64 CPU recomputation from
the GPU's own unpacked factors, zero fraction close to the oracle's, and
valid 2-bit ternary codes (no 0b10 code, zero padding).
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


def _golden(name):
    p = os.path.join(HERE, "golden", "oracle_energies.json")
    entries = json.load(open(p))["entries"] if os.path.exists(p) else {}
    if name not in entries:
        pytest.skip(f"oracle golden {name} not generated")
    return entries[name]


def _factors(res, k=None):
    k = res.k if k is None else k
    B = oracle.unpack2(res.B2[:k].cpu().numpy().view(np.uint32), res.m).T
    C = oracle.unpack2(res.C2[:k].cpu().numpy().view(np.uint32), res.n)
    D = res.D[:k].cpu().numpy().astype(np.float64)
    return B, C, D


def _check_full(A, res, g, zf_tol=0.01):
    E = float(res.energy.item())
    print(f"  {g['name']}: E gpu {E:.6f} oracle {g['E']:.6f}", flush=True)
    assert res.k == g["k"]
    assert abs(E - g["E"]) <= 2e-3, (E, g["E"])
    B, C, D = _factors(res)
    assert abs(E - oracle.energy_from_factors(A, B, C, D)) <= 1e-5
    assert abs(oracle.zero_fraction(B, C) - g["zero_fraction"]) < zf_tol
    assert res.stat("mode") == 2
    assert res.stat("nnz_b") == np.count_nonzero(B) and res.stat("nnz_c") == np.count_nonzero(C)
    assert res.stat("nonfinite") == 0
    return E


def test_mlp9728_block128(lib):
    g = _golden("mlp9728_block128")
    c = synthetic.WORKLOADS["mlp9728"]
    A = synthetic.workload_matrix("mlp9728")
    res = lib.decompose(torch.from_numpy(A).cuda(), c["mu"], c["tau"], c["iters"], c["block"],
                        c["seed"], stats=True)
    torch.cuda.synchronize()
    _check_full(A, res, g)
    # packed 2-bit output: (k, ceil(m/16)) and (k, ceil(n/16)) int32 words
    assert tuple(res.B2.shape) == (7680, 9728 // 16) and tuple(res.C2.shape) == (7680, 2560 // 16)


def test_layer_back_to_back(lib):
    c = synthetic.WORKLOADS["layer"]
    shapes = synthetic.layer_shapes()
    mats = {name: synthetic.workload_matrix("layer", name) for name, _, _ in shapes}
    dev = {name: torch.from_numpy(A).cuda() for name, A in mats.items()}
    # all seven decompositions queued on one stream before any check
    outs = {name: lib.decompose(dev[name], c["mu"], c["tau"], c["iters"], c["block"], c["seed"],
                                stats=True)
            for name, _, _ in shapes}
    torch.cuda.synchronize()
    for name, m, n in shapes:
        assert mats[name].shape == (m, n)
        _check_full(mats[name], outs[name], _golden(f"layer_{name}_block128"))


def test_lowrank4096_mu_tau_sweep(lib):
    c = synthetic.WORKLOADS["lowrank4096"]
    A = synthetic.workload_matrix("lowrank4096")
    Ad = torch.from_numpy(A).cuda()
    na2 = float(np.sum(A.astype(np.float64) ** 2))
    b = c["block"]
    zf_by_tau = {}
    for tau in c["taus"]:
        mu_max = max(c["mus"])
        res = lib.decompose(Ad, mu_max, tau, c["iters"], b, c["seed"], trace=True, stats=True)
        torch.cuda.synchronize()
        tr = res.trace.cpu().numpy()
        B, C, D = _factors(res)
        E_full = float(res.energy.item())
        assert abs(E_full - oracle.energy_from_factors(A, B, C, D)) <= 1e-5
        es = []
        for mu in c["mus"]:
            g = _golden(f"lowrank4096_tau{tau}_mu{mu}")
            k = oracle.rank_for(4096, 4096, mu)
            assert k % b == 0 and k == g["k"]
            E = 1.0 - tr[k // b - 1] / na2
            print(f"  tau {tau} mu {mu}: E gpu {E:.6f} oracle {g['E']:.6f}", flush=True)
            assert abs(E - g["E"]) <= 2e-3, (tau, mu, E, g["E"])
            assert abs(oracle.zero_fraction(B[:, :k], C[:k]) - g["zero_fraction"]) < 0.01
            es.append(E)
        assert all(e1 <= e2 + 1e-12 for e1, e2 in zip(es, es[1:])), es   # E grows with mu
        zf_by_tau[tau] = oracle.zero_fraction(B, C)
    taus = sorted(zf_by_tau)
    assert all(zf_by_tau[t1] < zf_by_tau[t2] for t1, t2 in zip(taus, taus[1:])), zf_by_tau


@pytest.mark.parametrize("block", [0, 16])
def test_gauss256_against_the_c_oracle(lib, block):
    # The 256 x 256 Gaussian workload in both modes against the plain C fp64
    # oracle run on the same seeded input: energy within 2e-3, and the GPU's
    # energy within 1e-5 of the one recomputed from its own factors.
    import oracle.c_oracle as coracle
    if not os.path.exists(coracle.LIB):
        coracle.build_c()
    c = synthetic.WORKLOADS["gauss256"]
    A = synthetic.workload_matrix("gauss256")
    k = lib.rank(256, 256, c["mu"])
    res = lib.decompose(torch.from_numpy(A).cuda(), c["mu"], c["tau"], c["iters"], block, c["seed"],
                        stats=True)
    torch.cuda.synchronize()
    if block:
        b = lib.block_width(256, 256, block)
        *_, E_ref, _ = coracle.decompose_block(A, k, b, c["tau"], c["iters"], c["seed"])
    else:
        *_, E_ref = coracle.decompose_seq(A, k, c["tau"], c["iters"], c["seed"])
    E = float(res.energy.item())
    print(f"  gauss256 block={block}: E gpu {E:.6f} C oracle {E_ref:.6f}", flush=True)
    assert abs(E - E_ref) <= 2e-3
    B, C, D = _factors(res)
    assert abs(E - oracle.energy_from_factors(A, B, C, D)) <= 1e-5
