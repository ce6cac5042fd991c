"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/externd.h, and rejects bad arguments on the host before
any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "externd.h")
LIB = os.path.join(ROOT, "ternary_rank_weight_amd", "libexternd.so")


@pytest.fixture(scope="module")
def clib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()
    return ctypes.CDLL(LIB)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(externd_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("externd_decompose", "externd_energy", "externd_reconstruct"):
        assert must in names


def test_every_declared_symbol_is_exported(clib):
    for name in declared_functions():
        assert hasattr(clib, name), name


def test_binding_lists_every_symbol():
    import ternary_rank_weight_amd as trw
    assert set(trw.ABI_SYMBOLS) == set(declared_functions())


def test_rank_and_block_width(clib):
    import ternary_rank_weight_amd as trw
    assert trw.rank(2560, 2560, 2.0) == 5120
    assert trw.rank(9728, 2560, 3.0) == 7680
    assert trw.rank(4096, 4096, 3.5) == 14336
    assert trw.rank(10, 3, 0.5) == 2
    assert trw.rank(0, 3, 1.0) == -1
    assert trw.block_width(2560, 2560, 64) == 64
    assert trw.block_width(1024, 2560, 256) == 128
    assert trw.block_width(15, 100, 64) == 1
    assert trw.block_width(100, 100, 0) == 1


def test_rank_matches_oracle():
    import oracle
    import ternary_rank_weight_amd as trw
    for (m, n, mu) in [(256, 256, 2.0), (100, 37, 1.3), (7, 9, 0.5), (4096, 2560, 2.5), (3, 3, 0.1667)]:
        assert trw.rank(m, n, mu) == oracle.rank_for(m, n, mu)
    for (m, n, b) in [(2560, 2560, 64), (1024, 2560, 256), (15, 100, 64), (64, 64, 1), (64, 64, 9)]:
        assert trw.block_width(m, n, b) == oracle.block_width(m, n, b)


def _decompose_args(clib):
    f = clib.externd_decompose
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                  ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return f


@pytest.mark.parametrize("case", [
    dict(A=0), dict(energy=0), dict(m=0), dict(n=-3), dict(mu=0.0), dict(mu=float("nan")),
    dict(mu=float("inf")), dict(tau=-0.1), dict(tau=float("nan")), dict(iters=0),
    dict(B2=0), dict(D=0),
])
def test_decompose_rejects_bad_arguments(clib, case):
    f = _decompose_args(clib)
    fake = 0x1000  # never dereferenced: validation fails first
    a = dict(A=fake, m=16, n=16, mu=1.0, tau=0.7, iters=15, block=0, B2=fake, C2=fake, D=fake,
             energy=fake)
    a.update(case)
    st = f(a["A"] or None, a["m"], a["n"], a["mu"], a["tau"], a["iters"], a["block"], None,
           a["B2"] or None, a["C2"] or None, a["D"] or None, a["energy"] or None, None)
    assert st == 1  # EXTERND_EINVAL
    clib.externd_last_error.restype = ctypes.c_char_p
    assert clib.externd_last_error()


def test_status_strings(clib):
    clib.externd_status_string.restype = ctypes.c_char_p
    assert clib.externd_status_string(0) == b"ok"
    assert clib.externd_status_string(1) == b"invalid argument"
    assert clib.externd_status_string(99) == b"unknown status"


def test_single_step_entry_points_validate(clib):
    fake = ctypes.c_void_p(0x1000)
    clib.externd_ternarize.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert clib.externd_ternarize(fake, 0, ctypes.c_float(0.7), None, fake, None) == 1
    assert clib.externd_ternarize(None, 10, ctypes.c_float(0.7), None, fake, None) == 1
    clib.externd_deflate.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p]
    assert clib.externd_deflate(fake, 4, 4, fake, fake, ctypes.c_float(float("nan")), None) == 1
    clib.externd_energy.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                    ctypes.c_void_p]
    assert clib.externd_energy(fake, 4, 4, None, None, None, 3, None, fake) == 1


def test_workspace_bytes_without_device():
    import ternary_rank_weight_amd as trw
    # block and streaming sizes depend on the shape only
    blk = trw.workspace_bytes(2560, 2560, 2.0, 64)
    assert blk > 0 and blk == trw.workspace_bytes(2560, 2560, 3.0, 64)
    assert trw.workspace_bytes(9728, 2560, 3.0, 128) > blk
    st = trw.workspace_bytes(2560, 2560, 2.0, 0, trw.MODE_STREAMING)
    assert st > 0
    assert trw.workspace_bytes(0, 5, 1.0, 0, trw.MODE_STREAMING) == 0
    assert trw.workspace_bytes(5, 5, float("nan"), 0, trw.MODE_STREAMING) == 0
    assert trw.workspace_bytes(5, 5, 1.0, 0, 7) == 0


def test_decompose_rejects_misaligned_workspace(clib):
    import ternary_rank_weight_amd as trw
    f = _decompose_args(clib)
    f.argtypes = f.argtypes[:-1] + [ctypes.POINTER(trw._Opts)]
    o = trw._Opts()
    o.struct_size = ctypes.sizeof(trw._Opts)
    o.mode = trw.MODE_AUTO
    o.capture_component = -1
    o.workspace = ctypes.c_void_p(0x1000 + 8)
    o.workspace_bytes = 1 << 30
    fake = 0x1000
    st = f(fake, 16, 16, 1.0, 0.7, 15, 0, None, fake, fake, fake, fake, ctypes.byref(o))
    assert st == 1
    clib.externd_last_error.restype = ctypes.c_char_p
    assert b"aligned" in clib.externd_last_error()


def test_rank_for_energy_matches_oracle(clib):
    import numpy as np
    import oracle
    import ternary_rank_weight_amd as trw
    rng = np.random.default_rng(3)
    for step, total in ((1, 40), (8, 37), (64, 5120)):
        n = (total + step - 1) // step
        tr = np.sort(rng.uniform(0.0, 10.0, n))[::-1].copy()
        for target in (-1.0, 0.0, 0.1, 0.5, 0.9, 1.0 - tr[-1] / 10.0, 0.999999, 2.0):
            want = oracle.rank_for_energy(tr, 10.0, target, step=step, total=total)
            assert trw.rank_for_energy(tr, total, step, 10.0, target) == want
    assert trw.rank_for_energy([], 0, 1, 0.0, 0.5) == 0
    # the prefix energy comes back from the C side with the rank
    tr = np.array([8.0, 5.0, 2.0, 1.0])
    c, e = trw.rank_for_energy(tr, 40, 10, 10.0, 0.75, with_energy=True)
    assert c == 30 and e == 1.0 - 2.0 / 10.0
    c, e = trw.rank_for_energy(tr, 35, 10, 10.0, 0.85, with_energy=True)
    assert c == 35 and e == 0.9
    c, e = trw.rank_for_energy(tr, 40, 10, 10.0, 0.95, with_energy=True)
    assert c == -1 and np.isnan(e)
    assert trw.rank_for_energy([], 0, 1, 0.0, 0.5, with_energy=True) == (0, 1.0)
    with pytest.raises(trw.ExterndError):
        trw.rank_for_energy([1.0], 1, 0, 1.0, 0.5)
    with pytest.raises(trw.ExterndError):
        trw.rank_for_energy([1.0], 1, 1, -1.0, 0.5)
    with pytest.raises(trw.ExterndError):
        trw.rank_for_energy([1.0], 1, 1, 1.0, float("nan"))


def test_decompose_rejects_bad_sweeps_and_lambda(clib):
    import ternary_rank_weight_amd as trw
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    for sweeps, block, lam in ((1, 0, 0.0), (1, 1, 0.0), (-1, 8, 0.0), (0, 8, -1.0), (0, 0, float("nan")),
                               (0, 0, float("inf"))):
        o = trw._Opts()
        o.struct_size = ctypes.sizeof(trw._Opts)
        o.mode = -1
        o.capture_component = -1
        o.sweeps = sweeps
        o.importance_lambda = lam
        st = trw._decompose(fake, 64, 64, 1.0, 0.7, 15, block, None, fake, fake, fake, fake, ctypes.byref(o))
        assert st == 1, (sweeps, block, lam)


def test_projection_option_limits(clib):
    import ternary_rank_weight_amd as trw
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    for m, n, tern, mode, want in ((16385, 16, 1, -1, 4), (16, 16385, 1, -1, 4), (64, 64, 1, 1, 4),
                                   (64, 64, 2, -1, 1), (64, 64, -1, -1, 1)):
        o = trw._Opts()
        o.struct_size = ctypes.sizeof(trw._Opts)
        o.mode = mode
        o.capture_component = -1
        o.ternarizer = tern
        st = trw._decompose(fake, m, n, 0.01, 0.7, 15, 0, None, fake, fake, fake, fake, ctypes.byref(o))
        assert st == want, (m, n, tern, mode)
    clib.externd_project.restype = ctypes.c_int
    clib.externd_project.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
    assert clib.externd_project(fake, 0, None, fake, None) == 1
    assert clib.externd_project(fake, 16385, None, fake, None) == 4


def _opts(trw, **kw):
    o = trw._Opts()
    o.struct_size = ctypes.sizeof(trw._Opts)
    o.mode = -1
    o.capture_component = -1
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def test_block_wider_than_the_kernels_is_refused(clib):
    # the pages' default b = 256 on a 4096 x 4096 matrix: the width rule gives
    # 256, above the widest block the kernels take, so the call is refused
    # (EXTERND_EUNSUPPORTED) before any device work instead of narrowing b
    import ternary_rank_weight_amd as trw
    assert trw.block_width(4096, 4096, 256) == 256
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    st = trw._decompose(fake, 4096, 4096, 1.0, 0.7, 15, 256, None, fake, fake, fake, fake,
                        ctypes.byref(_opts(trw)))
    assert st == 4
    clib.externd_last_error.restype = ctypes.c_char_p
    assert b"128" in clib.externd_last_error()


def test_safeguard_option_limits(clib):
    import ternary_rank_weight_amd as trw
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    for kw, block, want in ((dict(safeguard=2), 0, 1), (dict(safeguard=-1), 0, 1),
                            (dict(safeguard=1), 8, 4), (dict(safeguard=1, mode=1), 0, 4),
                            (dict(safeguard=1, ternarizer=1), 0, 4)):
        st = trw._decompose(fake, 64, 64, 1.0, 0.7, 15, block, None, fake, fake, fake, fake,
                            ctypes.byref(_opts(trw, **kw)))
        assert st == want, (kw, block)


def test_block_capture_range_is_checked(clib):
    import ternary_rank_weight_amd as trw
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    for blk, it in ((-1, 0), (8, 0), (0, -1), (0, 15)):   # 64 x 64, mu 1, b 8: 8 blocks, 15 iterations
        bc = trw._BlockCapture()
        bc.block, bc.iteration = blk, it
        o = _opts(trw, block_capture=ctypes.pointer(bc))
        st = trw._decompose(fake, 64, 64, 1.0, 0.7, 15, 8, None, fake, fake, fake, fake, ctypes.byref(o))
        assert st == 1, (blk, it)
