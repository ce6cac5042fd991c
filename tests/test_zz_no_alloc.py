"""externd_decompose_noalloc, the entry point for callers that cannot
allocate: its results must equal externd_decompose's on the resident path
bit for bit (the same kernels on the same inputs), on two calls in a row
whose second input is smaller than the first (the static scratch keeps the
first call's contents, so whatever must start at zero has to be cleared),
and requests it cannot serve must be refused before any device work."""
import ctypes

import numpy as np
import pytest
import torch

import synthetic

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _same(got, ref):
    assert torch.equal(got.B2, ref.B2) and torch.equal(got.C2, ref.C2)
    assert torch.equal(got.D, ref.D) and torch.equal(got.energy, ref.energy)
    assert torch.equal(got.trace, ref.trace) and torch.equal(got.stats, ref.stats)
    assert torch.equal(got.norm_a2, ref.norm_a2)


def test_noalloc_matches_decompose_on_two_calls(lib):
    c = synthetic.WORKLOADS["llm2560"]
    big = _dev(synthetic.workload_matrix("llm2560"))
    small = _dev(synthetic.gaussian(300, 200, 5))
    h = _dev(synthetic.importance(200, 5))
    ref_big = lib.decompose(big, c["mu"], c["tau"], c["iters"], 0, c["seed"], mode=lib.MODE_RESIDENT,
                            trace=True, stats=True)
    ref_small = lib.decompose(small, 1.0, 0.7, 15, 0, 3, mode=lib.MODE_RESIDENT, trace=True, stats=True,
                              importance=h, lam=0.1)
    got_big = lib.decompose_noalloc(big, c["mu"], c["tau"], c["iters"], 0, c["seed"], trace=True, stats=True)
    got_small = lib.decompose_noalloc(small, 1.0, 0.7, 15, 0, 3, trace=True, stats=True, importance=h, lam=0.1)
    torch.cuda.synchronize()
    assert ref_big.stat("mode") == 1 and got_big.stat("mode") == 1
    _same(got_big, ref_big)
    _same(got_small, ref_small)
    # and once more at the large size after the small call
    again = lib.decompose_noalloc(big, c["mu"], c["tau"], c["iters"], 0, c["seed"], trace=True, stats=True)
    torch.cuda.synchronize()
    _same(again, ref_big)


def test_noalloc_refuses_what_it_cannot_serve(lib):
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: every case is refused first

    def opts(**kw):
        o = lib._Opts()
        o.struct_size = ctypes.sizeof(lib._Opts)
        o.mode = -1
        o.capture_component = -1
        for k, v in kw.items():
            setattr(o, k, v)
        return o

    f = lib._decompose_noalloc
    # block mode, streaming mode, a caller workspace
    assert f(fake, 512, 512, 1.0, 0.7, 15, 16, None, fake, fake, fake, fake, ctypes.byref(opts())) == 4
    assert f(fake, 512, 512, 1.0, 0.7, 15, 0, None, fake, fake, fake, fake, ctypes.byref(opts(mode=0))) == 4
    assert f(fake, 512, 512, 1.0, 0.7, 15, 0, None, fake, fake, fake, fake,
             ctypes.byref(opts(workspace=fake, workspace_bytes=1 << 30))) == 1
    # a rank whose safeguard bitmap alone exceeds the static scratch
    assert f(fake, 2560, 2560, 800.0, 0.7, 15, 0, None, fake, fake, fake, fake, ctypes.byref(opts())) == 2
    lib._last_error.restype = ctypes.c_char_p
    assert b"scratch" in lib._last_error()
    # a shape that does not fit on chip
    assert f(fake, 9728, 2560, 1.0, 0.7, 15, 0, None, fake, fake, fake, fake, ctypes.byref(opts())) == 4
