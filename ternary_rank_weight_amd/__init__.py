"""Python binding of libexternd.so, the MI355X ExTernD library.

ExTernD ("ExTernD: Expanded-Rank Ternary Decomposition Ternary LLM PTQ with
Accuracy Approaching Any Quantization Level", §2) factors a weight matrix as
A ~ B diag(D) C with ternary B, C.  Every step runs in the HIP kernels behind
the C ABI declared in include/externd.h; this module only marshals torch
tensors (device memory) and the current HIP stream into those calls.  It
raises ImportError when the shared library has not been built; there is no
fallback implementation.
"""
import ctypes
import os

import torch

__all__ = [
    "decompose", "decompose_noalloc", "energy", "reconstruct", "apply", "rank", "block_width", "resident_fits",
    "workspace_bytes",
    "rank_for_energy", "mu_for_energy", "project",
    "ternarize", "gemv_t", "gemv_n", "deflate", "Decomposition", "ExterndError",
    "STAT", "MODE_AUTO", "MODE_STREAMING", "MODE_RESIDENT", "MODE_PERSISTENT", "library_path",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libexternd.so")

MODE_AUTO, MODE_STREAMING, MODE_RESIDENT, MODE_PERSISTENT = -1, 0, 1, 2
STATS_LEN = 16
STAT = {"sum_nnz_u": 0, "sum_nnz_v": 1, "nnz_b": 2, "nnz_c": 3, "fallbacks": 4,
        "nonfinite": 5, "mode": 6, "grid": 7, "ridge_retries": 8, "timeouts": 9,
        "inverse_unconverged": 10, "sweep_kept_old": 11, "ns_iterations": 12, "ns_restarts": 13,
        "iterations": 14, "safeguard": 15}

if not os.path.exists(library_path):
    raise ImportError(f"{library_path} is missing; build it with "
                      "`python ternary_rank_weight_amd/build.py`")
_lib = ctypes.CDLL(library_path)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float


class _BlockCapture(ctypes.Structure):
    _fields_ = [
        ("block", ctypes.c_int64), ("iteration", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("R", _p), ("U_in", _p), ("P", _p), ("GinvU", _p), ("Vt", _p), ("V", _p),
        ("Q", _p), ("GinvV", _p), ("Ut", _p), ("U_out", _p), ("rhs", _p),
    ]


class _Opts(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("reserved0", ctypes.c_uint32),
        ("seed", ctypes.c_uint64), ("mode", ctypes.c_int32), ("reserved1", ctypes.c_int32),
        ("trace", _p), ("stats", _p),
        ("capture_component", ctypes.c_int64),
        ("capture_R", _p), ("capture_Rcol", _p), ("capture_R_next", _p),
        ("capture_y", _p), ("capture_x", _p), ("capture_v", _p), ("capture_u", _p),
        ("capture_d", _p),
        ("workspace", _p), ("workspace_bytes", ctypes.c_uint64),
        ("norm_a2", _p),
        ("sweeps", _i32), ("ternarizer", _i32), ("sweep_trace", _p),
        ("importance", _p), ("importance_lambda", ctypes.c_float), ("safeguard", _i32),
        ("block_capture", ctypes.POINTER(_BlockCapture)),
    ]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_decompose = _sig("externd_decompose", ctypes.c_int,
                  [_p, _i64, _i64, _f32, _f32, _i32, _i32, _p, _p, _p, _p, _p, ctypes.POINTER(_Opts)])
_decompose_noalloc = _sig("externd_decompose_noalloc", ctypes.c_int,
                          [_p, _i64, _i64, _f32, _f32, _i32, _i32, _p, _p, _p, _p, _p, ctypes.POINTER(_Opts)])
_energy = _sig("externd_energy", ctypes.c_int, [_p, _i64, _i64, _p, _p, _p, _i64, _p, _p])
_reconstruct = _sig("externd_reconstruct", ctypes.c_int, [_p, _p, _p, _i64, _i64, _i64, _p, _p])
_apply = _sig("externd_apply", ctypes.c_int, [_p, _p, _p, _i64, _i64, _i64, _p, _p, _p])
_apply_rows = _sig("externd_apply_rows", ctypes.c_int, [_p, _p, _p, _i64, _i64, _i64, _p, _p, _p, _p, ctypes.c_size_t])
_apply_rows_ws = _sig("externd_apply_rows_workspace_bytes", ctypes.c_size_t, [_i64, _i64, _i64])
_transpose_codes = _sig("externd_transpose_codes", ctypes.c_int, [_p, _i64, _i64, _p, _p])
_rank = _sig("externd_rank", ctypes.c_int64, [_i64, _i64, _f32])
_block_width = _sig("externd_block_width", ctypes.c_int32, [_i64, _i64, _i32])
_resident_fits = _sig("externd_resident_fits", ctypes.c_int32, [_i64, _i64])
_workspace_bytes = _sig("externd_workspace_bytes", ctypes.c_uint64, [_i64, _i64, _f32, _i32, _i32])
_rank_for_energy = _sig("externd_rank_for_energy", ctypes.c_int64,
                        [ctypes.POINTER(ctypes.c_double), _i64, _i64, _i32, ctypes.c_double, ctypes.c_double,
                         ctypes.POINTER(ctypes.c_double)])
_ternarize = _sig("externd_ternarize", ctypes.c_int, [_p, _i64, _f32, _p, _p, _p])
_project = _sig("externd_project", ctypes.c_int, [_p, _i64, _p, _p, _p])
_gemv_t = _sig("externd_gemv_t", ctypes.c_int, [_p, _i64, _i64, _p, _p, _p])
_gemv_n = _sig("externd_gemv_n", ctypes.c_int, [_p, _i64, _i64, _p, _p, _p])
_deflate = _sig("externd_deflate", ctypes.c_int, [_p, _i64, _i64, _p, _p, _f32, _p])
_status_string = _sig("externd_status_string", ctypes.c_char_p, [ctypes.c_int])
_last_error = _sig("externd_last_error", ctypes.c_char_p, [])

# Every exported symbol of the C ABI, for load checks.
ABI_SYMBOLS = ("externd_decompose", "externd_decompose_noalloc", "externd_energy", "externd_reconstruct", "externd_apply",
               "externd_apply_rows", "externd_apply_rows_workspace_bytes", "externd_transpose_codes", "externd_rank",
               "externd_block_width", "externd_resident_fits", "externd_workspace_bytes",
               "externd_rank_for_energy",
               "externd_ternarize", "externd_project",
               "externd_gemv_t", "externd_gemv_n", "externd_deflate",
               "externd_status_string", "externd_last_error")


class ExterndError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(f"{_status_string(status).decode()}: {_last_error().decode()}")


def _check(status):
    if status != 0:
        raise ExterndError(status)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def rank(m, n, mu):
    """k = mu * min(m, n) rounded half away from zero (§2.1)."""
    return int(_rank(m, n, mu))


def block_width(m, n, block):
    """Block width used for a request (§2.4); 1 means sequential."""
    return int(_block_width(m, n, block))


def resident_fits(m, n):
    return bool(_resident_fits(m, n))


def workspace_bytes(m, n, mu, block=0, mode=MODE_AUTO):
    """Device workspace externd_decompose needs for these arguments (0: invalid)."""
    return int(_workspace_bytes(m, n, mu, block, mode))


class Decomposition:
    """Device outputs of one decomposition.

    B2: (k, ceil(m/16)) int32 words of 2-bit codes (component-major B),
    C2: (k, ceil(n/16)) int32 words (rows of C), D: (k,) float32,
    energy: (1,) float64, trace / stats: optional device tensors,
    capture: dict of captured tensors when requested.
    """

    def __init__(self, m, n, k, B2, C2, D, energy, trace, stats, capture, norm_a2=None, block=1):
        self.m, self.n, self.k = m, n, k
        self.B2, self.C2, self.D, self.energy = B2, C2, D, energy
        self.trace, self.stats, self.capture = trace, stats, capture
        self.norm_a2, self.block = norm_a2, block

    def stat(self, name):
        return int(self.stats[STAT[name]].item())


def decompose(A, mu, tau, iters=15, block=0, seed=0, mode=MODE_AUTO, trace=False, stats=False,
              capture=None, out=None, workspace=None, sweeps=0, importance=None, lam=0.0,
              projection=False, safeguard=False, block_capture=None, _entry=None):
    """Run externd_decompose on the current stream.

    A: (m, n) float32 CUDA tensor.  capture: component index whose
    intermediate vectors and residuals are recorded (sequential path only).
    out: optional Decomposition whose B2/C2/D/energy buffers are reused.
    workspace: optional contiguous CUDA tensor used as the library's scratch
    memory (at least workspace_bytes(...) bytes, 256-byte aligned); the
    library then allocates nothing.
    sweeps: refinement sweeps after extraction (block mode only); with
    trace=True their predicted ||R||^2 values land in .sweep_trace.
    importance: optional (n,) float32 CUDA tensor of per-input-channel second
    moments h; the column weights are h / max(h) + lam (importance-weighted
    ALS), and energy / trace / norm_a2 become weighted.
    projection: use the optimal ternary projection instead of T_tau
    (streaming or block mode; AUTO picks streaming).
    safeguard: apply the single-entry safeguard (sequential path, streaming
    mode); stats["safeguard"] counts the would-be replacements either way.
    block_capture: (block index, iteration) of the block path to record; the
    tensors land in .block_capture (R, U_in, P, GinvU, Vt, V, Q, GinvV, Ut,
    U_out, rhs; rows are components, codes as int32 words).
    """
    _need(A, torch.float32, "A")
    if A.dim() != 2:
        raise ValueError("A must be 2-D")
    m, n = A.shape
    k = rank(m, n, mu)
    if k < 0:
        raise ValueError("bad mu")
    dev = A.device
    if out is not None and (out.m, out.n, out.k) == (m, n, k):
        B2, C2, D, E = out.B2, out.C2, out.D, out.energy
    else:
        B2 = torch.empty((k, (m + 15) // 16), dtype=torch.int32, device=dev)
        C2 = torch.empty((k, (n + 15) // 16), dtype=torch.int32, device=dev)
        D = torch.empty((k,), dtype=torch.float32, device=dev)
        E = torch.empty((1,), dtype=torch.float64, device=dev)
    b = block_width(m, n, block)
    ntrace = ((k + b - 1) // b) if b > 1 else k
    tr = torch.empty((max(ntrace, 1),), dtype=torch.float64, device=dev) if trace else None
    st = torch.zeros((STATS_LEN,), dtype=torch.int64, device=dev) if stats else None
    na2 = torch.empty((1,), dtype=torch.float64, device=dev) if trace else None
    swt = torch.empty((sweeps,), dtype=torch.float64, device=dev) if trace and sweeps > 0 else None
    opts = _Opts()
    opts.struct_size = ctypes.sizeof(_Opts)
    opts.seed = seed
    opts.mode = mode
    opts.trace = _ptr(tr)
    opts.stats = _ptr(st)
    opts.norm_a2 = _ptr(na2)
    opts.sweeps = int(sweeps)
    opts.sweep_trace = _ptr(swt)
    if importance is not None:
        _need(importance, torch.float32, "importance")
        if importance.dim() != 1 or importance.numel() != n:
            raise ValueError("importance must have n entries")
        opts.importance = _ptr(importance)
    opts.importance_lambda = float(lam)
    opts.ternarizer = 1 if projection else 0
    opts.safeguard = 1 if safeguard else 0
    opts.capture_component = -1
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" \
                or not workspace.is_contiguous():
            raise TypeError("workspace must be a contiguous CUDA tensor")
        opts.workspace = _ptr(workspace)
        opts.workspace_bytes = workspace.numel() * workspace.element_size()
    cap = None
    if capture is not None:
        cap = {
            "R": torch.empty((m, n), dtype=torch.float32, device=dev),
            "Rcol": torch.empty((m, n), dtype=torch.float32, device=dev),
            "R_next": torch.empty((m, n), dtype=torch.float32, device=dev),
            "y": torch.empty((iters, n), dtype=torch.float32, device=dev),
            "x": torch.empty((iters, m), dtype=torch.float32, device=dev),
            "v": torch.empty((iters, n), dtype=torch.int8, device=dev),
            "u": torch.empty((iters, m), dtype=torch.int8, device=dev),
            "d": torch.empty((1,), dtype=torch.float32, device=dev),
        }
        opts.capture_component = int(capture)
        opts.capture_R = _ptr(cap["R"])
        opts.capture_Rcol = _ptr(cap["Rcol"])
        opts.capture_R_next = _ptr(cap["R_next"])
        opts.capture_y = _ptr(cap["y"])
        opts.capture_x = _ptr(cap["x"])
        opts.capture_v = _ptr(cap["v"])
        opts.capture_u = _ptr(cap["u"])
        opts.capture_d = _ptr(cap["d"])
    bcap = None
    if block_capture is not None:
        blk, it = block_capture
        bb = min(b, k - blk * b) if b > 1 else 0
        if b <= 1 or not 0 <= blk * b < k:
            raise ValueError("block_capture needs block mode and a block index below ceil(k/b)")
        wm, wn = (m + 15) // 16, (n + 15) // 16
        f32 = dict(dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        bcap = {"R": torch.empty((m, n), **f32), "U_in": torch.empty((bb, wm), **i32),
                "P": torch.empty((bb, n), **f32), "GinvU": torch.empty((bb, bb), **f32),
                "Vt": torch.empty((bb, n), **f32), "V": torch.empty((bb, wn), **i32),
                "Q": torch.empty((bb, m), **f32), "GinvV": torch.empty((bb, bb), **f32),
                "Ut": torch.empty((bb, m), **f32), "U_out": torch.empty((bb, wm), **i32),
                "rhs": torch.empty((bb,), dtype=torch.float64, device=dev)}
        bc = _BlockCapture()
        bc.block, bc.iteration = int(blk), int(it)
        for name, tensor in bcap.items():
            setattr(bc, name, _ptr(tensor))
        opts.block_capture = ctypes.pointer(bc)
    _check((_entry or _decompose)(_ptr(A), m, n, mu, tau, iters, block, _stream(), _ptr(B2), _ptr(C2),
                                  _ptr(D), _ptr(E), ctypes.byref(opts)))
    res = Decomposition(m, n, k, B2, C2, D, E, tr, st, cap, na2, b)
    res.sweep_trace = swt
    res.block_capture = bcap
    return res


def decompose_noalloc(A, mu, tau, iters=15, block=0, seed=0, **kw):
    """Run externd_decompose_noalloc: decompose() on the resident sequential
    path with the library's static scratch, for callers that cannot
    allocate (the outputs here are still allocated by torch).  Takes the
    keyword arguments of decompose() except workspace."""
    if kw.get("workspace") is not None:
        raise ValueError("decompose_noalloc brings its own scratch")
    return decompose(A, mu, tau, iters, block, seed, _entry=_decompose_noalloc, **kw)


def rank_for_energy(trace, total, step, norm_a2, target, with_energy=False):
    """Smallest prefix rank whose energy reaches target (host-side scan of a
    trace; see externd_rank_for_energy).  -1 if none does.  with_energy:
    return (rank, energy of that prefix) instead, the energy NaN for -1."""
    import numpy as np
    tr = np.ascontiguousarray(np.asarray(trace, dtype=np.float64))
    e = ctypes.c_double(0.0)
    r = int(_rank_for_energy(tr.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), tr.size, int(total),
                             int(step), float(norm_a2), float(target), ctypes.byref(e)))
    if r == -2:
        raise ExterndError(1)
    return (r, e.value) if with_energy else r


def mu_for_energy(A, target, mu_max, tau, iters=15, block=0, seed=0):
    """Smallest mu (a multiple of 1/min(m, n), and of b/min(m, n) in block
    mode) whose decomposition reaches energy >= target, from one run at
    mu_max (§3.3).  Returns (mu, k, energy_at_k) or None if mu_max is short."""
    res = decompose(A, mu_max, tau, iters, block, seed, trace=True)
    torch.cuda.synchronize()
    tr = res.trace.cpu().numpy()
    a2 = float(res.norm_a2.item())
    c, e = rank_for_energy(tr, res.k, res.block, a2, target, with_energy=True)
    if c < 0:
        return None
    m, n = A.shape
    return c / min(m, n), c, e


def energy(A, B2, C2, D):
    """E = 1 - ||A - B diag(D) C||^2 / ||A||^2 from 2-bit factors, fp64 (§2.1)."""
    _need(A, torch.float32, "A")
    m, n = A.shape
    k = D.numel()
    E = torch.empty((1,), dtype=torch.float64, device=A.device)
    _check(_energy(_ptr(A), m, n, _ptr(B2), _ptr(C2), _ptr(D), k, _stream(), _ptr(E)))
    return E


def reconstruct(B2, C2, D, m, n):
    """A_hat = B diag(D) C as an (m, n) float32 tensor (§2.1)."""
    k = D.numel()
    out = torch.empty((m, n), dtype=torch.float32, device=D.device)
    _check(_reconstruct(_ptr(B2), _ptr(C2), _ptr(D), m, n, k, _stream(), _ptr(out)))
    return out


def apply(B2, C2, D, m, n, x):
    """y = B (diag(D) (C x)) from the 2-bit factors (§2.6); x: float32 (n,)."""
    _need(x, torch.float32, "x")
    if x.numel() != n:
        raise ValueError("x must have n entries")
    k = D.numel()
    y = torch.empty((m,), dtype=torch.float32, device=x.device)
    _check(_apply(_ptr(B2), _ptr(C2), _ptr(D), m, n, k, _ptr(x), _stream(), _ptr(y)))
    return y


def transpose_codes(src, rows, cols):
    """Transpose a 2-bit code matrix: src holds `rows` rows of `cols` codes
    (ceil(cols/16) int32 words per row); returns `cols` rows of `rows` codes.
    transpose_codes(B2, k, m) gives B row by row, the form apply_rows reads."""
    _need(src, torch.int32, "src")
    if src.numel() != rows * ((cols + 15) // 16):
        raise ValueError("src must hold rows * ceil(cols/16) words")
    dst = torch.empty((cols, (rows + 15) // 16), dtype=torch.int32, device=src.device)
    _check(_transpose_codes(_ptr(src), rows, cols, _stream(), _ptr(dst)))
    return dst


def apply_rows_workspace_bytes(m, n, k):
    """Device workspace apply_rows needs for this shape (0: invalid)."""
    return int(_apply_rows_ws(m, n, k))


def apply_rows(BT2, C2, D, m, n, x, out=None, workspace=None):
    """y = B (diag(D) (C x)) (§2.6) with B row by row (BT2 = transpose_codes(B2,
    k, m)), on int8 MFMA with the vectors in exact fixed point; x: float32 (n,).
    out: optional float32 (m,) CUDA tensor written and returned; workspace:
    optional contiguous CUDA tensor of at least apply_rows_workspace_bytes(m,
    n, k) bytes (256-byte aligned), so that the call allocates nothing."""
    _need(x, torch.float32, "x")
    if x.numel() != n:
        raise ValueError("x must have n entries")
    k = D.numel()
    if out is None:
        out = torch.empty((m,), dtype=torch.float32, device=x.device)
    else:
        _need(out, torch.float32, "out")
        if out.numel() != m:
            raise ValueError("out must have m entries")
    wsb = 0
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" \
                or not workspace.is_contiguous():
            raise TypeError("workspace must be a contiguous CUDA tensor")
        wsb = workspace.numel() * workspace.element_size()
    _check(_apply_rows(_ptr(BT2), _ptr(C2), _ptr(D), m, n, k, _ptr(x), _stream(), _ptr(out), _ptr(workspace), wsb))
    return out


def ternarize(x, tau):
    """T_tau of a float32 vector (§2.2) -> (2-bit code words, nnz)."""
    _need(x, torch.float32, "x")
    N = x.numel()
    codes = torch.empty(((N + 15) // 16,), dtype=torch.int32, device=x.device)
    nnz = torch.empty((1,), dtype=torch.int32, device=x.device)
    _check(_ternarize(_ptr(x), N, tau, _stream(), _ptr(codes), _ptr(nnz)))
    return codes, nnz


def project(x):
    """Optimal ternary projection of a float32 vector (§2.2) -> (codes, nnz)."""
    _need(x, torch.float32, "x")
    N = x.numel()
    codes = torch.empty(((N + 15) // 16,), dtype=torch.int32, device=x.device)
    nnz = torch.empty((1,), dtype=torch.int32, device=x.device)
    _check(_project(_ptr(x), N, _stream(), _ptr(codes), _ptr(nnz)))
    return codes, nnz


def gemv_t(R, u_codes):
    """y = R^T u with u as 2-bit codes (§2.3)."""
    _need(R, torch.float32, "R")
    m, n = R.shape
    y = torch.empty((n,), dtype=torch.float32, device=R.device)
    _check(_gemv_t(_ptr(R), m, n, _ptr(u_codes), _stream(), _ptr(y)))
    return y


def gemv_n(R, v_codes):
    """x = R v with v as 2-bit codes (§2.3)."""
    _need(R, torch.float32, "R")
    m, n = R.shape
    x = torch.empty((m,), dtype=torch.float32, device=R.device)
    _check(_gemv_n(_ptr(R), m, n, _ptr(v_codes), _stream(), _ptr(x)))
    return x


def deflate(R, u_codes, v_codes, d):
    """R <- R - d u v^T in place (§2.3 step 3)."""
    _need(R, torch.float32, "R")
    m, n = R.shape
    _check(_deflate(_ptr(R), m, n, _ptr(u_codes), _ptr(v_codes), float(d), _stream()))
    return R
