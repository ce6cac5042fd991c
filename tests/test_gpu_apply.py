"""GPU checks of inference with the 2-bit factors (§2.6): y = B (diag(D) (C x))
against the fp64 oracle (oracle.apply_factors, pinned to the dense
reconstruction), on decomposed and on random factors, ragged shapes, k = 0,
and bit-identical repeated calls."""
import numpy as np
import pytest
import torch

import oracle
import synthetic

pytestmark = pytest.mark.gpu


def _relnorm(a, b):
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(np.asarray(a, dtype=np.float64) - b) / max(np.linalg.norm(b), 1e-300))


def _random_factors(m, n, k, seed):
    rng = np.random.default_rng(seed)
    B = rng.choice([-1, 0, 1], size=(m, k), p=[0.3, 0.4, 0.3]).astype(np.int8)
    C = rng.choice([-1, 0, 1], size=(k, n), p=[0.3, 0.4, 0.3]).astype(np.int8)
    D = (rng.standard_normal(k) * 0.01).astype(np.float32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    B2 = dev(oracle.pack2(B.T).view(np.int32))
    C2 = dev(oracle.pack2(C).view(np.int32))
    return B, C, D, B2, C2, dev(D)


def test_apply_decomposed_factors(lib):
    c = synthetic.WORKLOADS["gauss256"]
    A = synthetic.workload_matrix("gauss256")
    res = lib.decompose(torch.from_numpy(A).cuda(), c["mu"], c["tau"], c["iters"], 0, c["seed"])
    B = oracle.unpack2(res.B2.cpu().numpy().view(np.uint32), 256).T
    C = oracle.unpack2(res.C2.cpu().numpy().view(np.uint32), 256)
    D = res.D.cpu().numpy().astype(np.float64)
    x = np.random.default_rng(3).standard_normal(256).astype(np.float32)
    y = lib.apply(res.B2, res.C2, res.D, 256, 256, torch.from_numpy(x).cuda()).cpu().numpy()
    assert _relnorm(y, oracle.apply_factors(B, C, D, x)) <= 1e-5
    # the factors approximate A: y is close to A x (E ~ 0.996)
    assert _relnorm(y, A.astype(np.float64) @ x) < 0.1


@pytest.mark.parametrize("m,n,k", [(37, 53, 20), (1, 300, 70), (300, 1, 70), (129, 16, 65), (2560, 2560, 5120)])
def test_apply_random_factors(lib, m, n, k):
    B, C, D, B2, C2, Dd = _random_factors(m, n, k, m + n + k)
    x = np.random.default_rng(k).standard_normal(n).astype(np.float32)
    xd = torch.from_numpy(x).cuda()
    y1 = lib.apply(B2, C2, Dd, m, n, xd)
    y2 = lib.apply(B2, C2, Dd, m, n, xd)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert _relnorm(y1.cpu().numpy(), oracle.apply_factors(B, C, D.astype(np.float64), x)) <= 1e-5


def test_apply_zero_rank(lib):
    x = torch.ones(8, dtype=torch.float32, device="cuda")
    e = torch.empty((0, 1), dtype=torch.int32, device="cuda")
    y = lib.apply(e, e, torch.empty(0, dtype=torch.float32, device="cuda"), 5, 8, x)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0 and y.numel() == 5
