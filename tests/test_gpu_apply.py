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


# ---- B row by row: the code transpose and the int8-MFMA apply (apply_rows) ----

@pytest.mark.parametrize("rows,cols", [(1, 1), (37, 53), (16, 16), (129, 300), (2048, 1000), (5, 4097)])
def test_transpose_codes(lib, rows, cols):
    rng = np.random.default_rng(rows * 7 + cols)
    T = rng.choice([-1, 0, 1], size=(rows, cols)).astype(np.int8)
    src = torch.from_numpy(oracle.pack2(T).view(np.int32)).cuda()
    dst = lib.transpose_codes(src, rows, cols)
    back = lib.transpose_codes(dst, cols, rows)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy().view(np.uint32), oracle.pack2(T.T))
    assert torch.equal(back, src)


def _apply_rows_case(lib, m, n, k, seed, x=None):
    B, C, D, B2, C2, Dd = _random_factors(m, n, k, seed)
    BT2 = lib.transpose_codes(B2, k, m)
    if x is None:
        x = np.random.default_rng(seed + 1).standard_normal(n).astype(np.float32)
    xd = torch.from_numpy(x).cuda()
    y1 = lib.apply_rows(BT2, C2, Dd, m, n, xd)
    y2 = lib.apply_rows(BT2, C2, Dd, m, n, xd)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert np.array_equal(BT2.cpu().numpy().view(np.uint32), oracle.pack2(B))
    return y1.cpu().numpy(), oracle.apply_factors(B, C, D.astype(np.float64), x)


@pytest.mark.parametrize("m,n,k", [(37, 53, 20), (1, 300, 70), (300, 1, 70), (129, 16, 65), (200, 4097, 33),
                                   (2560, 2560, 5120), (300, 20000, 40), (1000, 1024, 1024), (1000, 2048, 999),
                                   (70, 40960, 48)])
def test_apply_rows_random_factors(lib, m, n, k):
    # ragged rows (n % 64 != 0: the unaligned load path), one-row and one-column
    # factors, a vector longer than one LDS chunk (20000 > 16384, 40960 > 32768),
    # and whole-stretch rows (the unmasked path) with a ragged number of rows
    y, ref = _apply_rows_case(lib, m, n, k, m + 2 * n + 3 * k)
    assert _relnorm(y, ref) <= 1e-5


def test_apply_rows_wide_range_vector(lib):
    # entries spanning 2^-40 .. 2^10: the small ones are rounded to the fixed-point
    # grid (2^-30 of the largest), which the norm-wise bar absorbs
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(700) * np.exp2(rng.uniform(-40, 10, 700))).astype(np.float32)
    y, ref = _apply_rows_case(lib, 90, 700, 150, 5, x=x)
    assert _relnorm(y, ref) <= 1e-5


def test_apply_rows_matches_apply_and_decomposed(lib):
    # on decomposed factors: the same y as the component-major path, to 1e-5
    c = synthetic.WORKLOADS["gauss256"]
    A = synthetic.workload_matrix("gauss256")
    res = lib.decompose(torch.from_numpy(A).cuda(), c["mu"], c["tau"], c["iters"], 0, c["seed"])
    x = torch.from_numpy(np.random.default_rng(3).standard_normal(256).astype(np.float32)).cuda()
    BT2 = lib.transpose_codes(res.B2, res.k, 256)
    y_rows = lib.apply_rows(BT2, res.C2, res.D, 256, 256, x).cpu().numpy()
    y_comp = lib.apply(res.B2, res.C2, res.D, 256, 256, x).cpu().numpy()
    B = oracle.unpack2(res.B2.cpu().numpy().view(np.uint32), 256).T
    C = oracle.unpack2(res.C2.cpu().numpy().view(np.uint32), 256)
    ref = oracle.apply_factors(B, C, res.D.cpu().numpy().astype(np.float64), x.cpu().numpy())
    assert _relnorm(y_rows, ref) <= 1e-5
    assert _relnorm(y_rows, y_comp) <= 1e-5


def test_apply_rows_full_size(lib):
    # 16384 x 16384, k = 32768 (the bench's inference shape): against the
    # component-major path on the whole vector, and against the oracle on 48
    # sampled rows, each computed exactly from w = D (C x) in fp64
    m = n = 16384
    k = 32768
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)

    def codes(rows, L):
        w = torch.randint(-2**31, 2**31 - 1, (rows, (L + 15) // 16), dtype=torch.int64, device="cuda",
                          generator=gen).to(torch.int32)
        return (w | ((w >> 1) & 0x55555555)).contiguous()   # no invalid code 10
    B2, C2 = codes(k, m), codes(k, n)
    D = (torch.randn(k, device="cuda", generator=gen) * 0.01).contiguous()
    x = torch.randn(n, device="cuda", generator=gen)
    BT2 = lib.transpose_codes(B2, k, m)
    y_rows = lib.apply_rows(BT2, C2, D, m, n, x)
    y_comp = lib.apply(B2, C2, D, m, n, x)
    torch.cuda.synchronize()
    yr = y_rows.cpu().numpy()
    assert _relnorm(yr, y_comp.cpu().numpy()) <= 1e-5
    xh = x.cpu().numpy().astype(np.float64)
    Ch = C2.cpu().numpy().view(np.uint32)
    w = np.empty(k)
    for i0 in range(0, k, 2048):
        w[i0:i0 + 2048] = oracle.unpack2(Ch[i0:i0 + 2048], n).astype(np.float64) @ xh
    w *= D.cpu().numpy().astype(np.float64)
    rows = np.random.default_rng(1).choice(m, 48, replace=False)
    Bt = oracle.unpack2(BT2.cpu().numpy().view(np.uint32)[rows], k).astype(np.float64)
    ref = Bt @ w
    assert _relnorm(yr[rows], ref) <= 1e-5


def test_apply_rows_workspace_and_out(lib):
    # a caller workspace and output: the same bits as the allocating call, twice
    # in a row (the second on other factors of a smaller shape), and a
    # workspace that is too small is refused
    B, C, D, B2, C2, Dd = _random_factors(300, 2048, 512, 9)
    BT2 = lib.transpose_codes(B2, 512, 300)
    x = torch.from_numpy(np.random.default_rng(4).standard_normal(2048).astype(np.float32)).cuda()
    ref = lib.apply_rows(BT2, C2, Dd, 300, 2048, x)
    need = lib.apply_rows_workspace_bytes(300, 2048, 512)
    assert need > 4 * 512
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.empty(300, dtype=torch.float32, device="cuda")
    y = lib.apply_rows(BT2, C2, Dd, 300, 2048, x, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert y.data_ptr() == out.data_ptr() and torch.equal(y, ref)
    B3, C3, D3, B23, C23, Dd3 = _random_factors(100, 1024, 64, 10)
    x3 = torch.from_numpy(np.random.default_rng(5).standard_normal(1024).astype(np.float32)).cuda()
    y3 = lib.apply_rows(lib.transpose_codes(B23, 64, 100), C23, Dd3, 100, 1024, x3, workspace=ws)
    torch.cuda.synchronize()
    assert _relnorm(y3.cpu().numpy(), oracle.apply_factors(B3, C3, D3.astype(np.float64), x3.cpu().numpy())) <= 1e-5
    with pytest.raises(lib.ExterndError):
        lib.apply_rows(BT2, C2, Dd, 300, 2048, x, workspace=ws[:need // 2])


def test_apply_rows_edge_cases(lib):
    x = torch.ones(8, dtype=torch.float32, device="cuda")
    e = torch.empty((0, 1), dtype=torch.int32, device="cuda")
    y = lib.apply_rows(e, e, torch.empty(0, dtype=torch.float32, device="cuda"), 5, 8, x)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0 and y.numel() == 5
    B, C, D, B2, C2, Dd = _random_factors(40, 30, 20, 2)
    BT2 = lib.transpose_codes(B2, 20, 40)
    xz = torch.zeros(30, dtype=torch.float32, device="cuda")
    assert torch.count_nonzero(lib.apply_rows(BT2, C2, Dd, 40, 30, xz)).item() == 0
    xn = torch.ones(30, dtype=torch.float32, device="cuda")
    xn[7] = float("nan")
    assert torch.isnan(lib.apply_rows(BT2, C2, Dd, 40, 30, xn)).all()
    with pytest.raises(ValueError):
        lib.apply_rows(BT2, C2, Dd, 40, 30, torch.ones(29, dtype=torch.float32, device="cuda"))
