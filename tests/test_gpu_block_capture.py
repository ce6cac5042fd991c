"""Per-step parity of the block-ALS path (ExTernD §2.4) on identical inputs.

One iteration of one block is captured from the GPU run: the residual R
the block is fitted to, the U entering the iteration, the contraction
P = U^T R, the decorrelation inverse (U^T U + eps I)^-1, the V target, the
V codes, Q = R V, (V^T V + eps I)^-1, the U target and the U codes, plus
the joint solve's right side of the final iteration.  Each step is then
recomputed by the fp64 oracle from the GPU's own inputs to that step:

* P, Q, both inverses, both targets and the right side within 1e-5
  relative, per component (row) for the vectors;
* every code row bit-exact against the oracle's T_tau of the GPU's target;
* the block's scales d within 1e-5 of the oracle's joint solve on the
  block's final U and V and the captured R;
* no decorrelation inverse left unconverged in the whole run.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _codes(t, L):
    return oracle.unpack2(t.cpu().numpy().view(np.uint32), L).astype(np.float64)   # rows x L


def _rel_rows(got, ref):
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return float(np.max(num / np.where(den > 0, den, 1.0)))


def _rel(got, ref):
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def _check_block(lib, A, mu, tau, b, blk, it, iters=15, seed=0, h=None, lam=0.0):
    m, n = A.shape
    Ad = _dev(A)
    imp = _dev(h) if h is not None else None
    res = lib.decompose(Ad, mu, tau, iters, b, seed, stats=True, importance=imp, lam=lam,
                        block_capture=(blk, it))
    torch.cuda.synchronize()
    cap = res.block_capture
    bb = cap["P"].shape[0]
    w = None if h is None else oracle.importance_weights(h.astype(np.float64), lam)
    R = cap["R"].cpu().numpy().astype(np.float64)
    U = _codes(cap["U_in"], m).T                        # m x bb
    # V half-step
    P_ref = (R.T @ U).T                                 # bb x n
    assert _rel_rows(cap["P"].cpu().numpy(), P_ref) <= TOL
    Gi_ref = oracle.decorrelation_inverse(U.T @ U)
    assert _rel(cap["GinvU"].cpu().numpy(), Gi_ref) <= TOL
    Vt_ref = oracle.block_v_target(R, U).T              # bb x n
    Vt = cap["Vt"].cpu().numpy()
    assert _rel_rows(Vt, Vt_ref) <= TOL
    V = _codes(cap["V"], n)                             # bb x n
    assert np.array_equal(V.T, oracle.ternarize_columns(Vt.T.astype(np.float64), tau))
    # U half-step
    Vw = V.T if w is None else V.T * w[:, None]
    Q_ref = (R @ Vw).T                                  # bb x m
    assert _rel_rows(cap["Q"].cpu().numpy(), Q_ref) <= TOL
    Gv = V @ Vw
    assert _rel(cap["GinvV"].cpu().numpy(), oracle.decorrelation_inverse(Gv)) <= TOL
    Ut_ref = oracle.block_u_target(R, V.T, w)[0].T      # bb x m
    Ut = cap["Ut"].cpu().numpy()
    assert _rel_rows(Ut, Ut_ref) <= TOL
    Uo = _codes(cap["U_out"], m)
    assert np.array_equal(Uo.T, oracle.ternarize_columns(Ut.T.astype(np.float64), tau))
    # joint scale solve on the block's final factors
    c0 = blk * b
    Uf = _codes(res.B2[c0:c0 + bb], m).T
    Vf = _codes(res.C2[c0:c0 + bb], n).T
    if it == iters - 1:
        assert np.array_equal(Uf, Uo.T)
    Qf = R @ (Vf if w is None else Vf * w[:, None])
    d_ref, rhs_ref = oracle.joint_scales(Uf, Vf, Qf, w)
    assert _rel(cap["rhs"].cpu().numpy(), rhs_ref) <= TOL
    d = res.D[c0:c0 + bb].cpu().numpy().astype(np.float64)
    assert _rel(d, d_ref) <= TOL, (_rel(d, d_ref), bb)
    assert res.stat("inverse_unconverged") == 0
    assert res.stat("timeouts") == 0
    assert res.stat("safeguard") == 0    # appendix §7: it never activates
    return res


@pytest.mark.parametrize("blk,it", [(0, 0), (0, 14), (37, 6), (79, 14)])
def test_block_capture_llm2560_b64(lib, blk, it):
    c = synthetic.WORKLOADS["llm2560"]
    A = synthetic.workload_matrix("llm2560")
    _check_block(lib, A, c["mu"], c["tau"], c["block"], blk, it, c["iters"], c["seed"])


def test_block_capture_mlp9728_b128(lib):
    c = synthetic.WORKLOADS["mlp9728"]
    A = synthetic.workload_matrix("mlp9728")
    _check_block(lib, A, c["mu"], c["tau"], c["block"], 23, 9, c["iters"], c["seed"])


@pytest.mark.parametrize("m,n,mu,b,blk,it", [
    (900, 1000, 0.3, 100, 2, 3),     # k = 270: a trailing block of 70 (partial pivot tiles)
    (320, 400, 0.5, 40, 3, 14),      # k = 160: b = 40, partial 16-component tiles on the b <= 64 path
    (256, 300, 0.25, 16, 1, 0),      # one 16-component tile
    (517, 389, 1.0, 48, 8, 7),       # ragged shape, k = 389: last block of 5
])
def test_block_capture_ragged(lib, m, n, mu, b, blk, it):
    A = synthetic.gaussian(m, n, 13)
    _check_block(lib, A, mu, 0.7, b, blk, it, 15, 2)


@pytest.mark.parametrize("b", [32, 128])
def test_block_capture_importance_weighted(lib, b):
    A = synthetic.llm_like(1100, 1024, 6)
    h = synthetic.importance(1024, 6)
    _check_block(lib, A, 0.5, 0.7, b, 2, 5, 15, 1, h=h, lam=0.01)


def test_block_capture_tall_three_digit_gram(lib):
    # m = 33001 > 32639: the U-side Gram's entries need three base-256 digits
    # in the exact-residual inverse (b <= 64), and 2063 code words per row
    # (not a multiple of four) take the Gram's word loads; the V side (n = 256)
    # has two digits.
    A = synthetic.gaussian(33001, 256, 21)
    _check_block(lib, A, 0.3, 0.7, 32, 1, 3, 15, 4)


def test_block_capture_contraction_of_2_23_rows(lib):
    # m = 2^23: the U-side Gram's entries could need a fourth base-256 digit,
    # so that side takes the Gram workgroups and the fp32 Newton-Schulz with
    # the fp64 refinement; the V side (n = 16) the exact-residual form.
    A = synthetic.gaussian(1 << 23, 16, 22)
    _check_block(lib, A, 0.5, 0.7, 2, 1, 3, 15, 5)
