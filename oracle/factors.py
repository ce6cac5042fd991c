"""Energy, reconstruction, 2-bit codes and the storage cost formula (fp64).

Test infrastructure: only tests, the smoke check and the benchmark's CPU
baseline may use this module.  Written independently of the GPU path's codec.

Sources (ExTernD: Expanded-Rank Ternary Decomposition Ternary LLM PTQ with
Accuracy Approaching Any Quantization Level):
  §2.1  A_hat = B diag(D) C and energy E = 1 - ||A - A_hat||_F^2 / ||A||_F^2
  §2.6  Eq. 1: bpw_eff = mu * (m + n) / max(m, n) * (2 - sparsity)

2-bit code (an exchange format of this library, not of the pages): a ternary
row of length L is stored as ceil(L/16) little-endian uint32 words; element j
sits in bits 2*(j % 16) and 2*(j % 16) + 1 of word j // 16, with
00 -> 0, 01 -> +1, 11 -> -1; 10 is invalid.  Unused trailing bits are 00.
B is stored component-major (row i holds column i of B), C row-major.
"""
import numpy as np

__all__ = ["reconstruct", "energy_from_factors", "pack2", "unpack2",
           "zero_fraction", "bpw_eff", "bpw_packed2"]


def reconstruct(B, C, D):
    """A_hat = B diag(D) C in fp64 (§2.1)."""
    Bf = np.asarray(B, dtype=np.float64)
    Cf = np.asarray(C, dtype=np.float64)
    Df = np.asarray(D, dtype=np.float64)
    return (Bf * Df[None, :]) @ Cf


def apply_factors(B, C, D, x):
    """Inference with the factors (§2.6): y = B (diag(D) (C x)) in fp64."""
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    return B @ (D * (C @ x))


def energy_from_factors(A, B, C, D, weights=None):
    """E = 1 - ||A - B diag(D) C||^2 / ||A||^2 in fp64, from the factors alone
    (§2.1).  weights: optional column weights h~; both norms are then the
    weighted sums sum_ij h~_j X_ij^2 (§2.5)."""
    A64 = np.asarray(A, dtype=np.float64)
    diff = A64 - reconstruct(B, C, D)
    if weights is None:
        na2 = float(np.sum(A64 * A64))
        r2 = float(np.sum(diff * diff))
    else:
        w = np.asarray(weights, dtype=np.float64)
        na2 = float(np.sum((A64 * A64) @ w))
        r2 = float(np.sum((diff * diff) @ w))
    if na2 == 0.0:
        return 1.0
    return 1.0 - r2 / na2


def pack2(T):
    """Pack a 2-D ternary array (rows x L, values in {-1,0,1}) into uint32 words."""
    T = np.asarray(T)
    rows, L = T.shape
    words = (L + 15) // 16
    codes = np.zeros((rows, words * 16), dtype=np.uint32)
    codes[:, :L][T == 1] = 1
    codes[:, :L][T == -1] = 3
    if np.any((T != 0) & (T != 1) & (T != -1)):
        raise ValueError("non-ternary entry")
    shifts = (2 * np.arange(16, dtype=np.uint32))[None, None, :]
    out = (codes.reshape(rows, words, 16) << shifts).sum(axis=2, dtype=np.uint64)
    return out.astype(np.uint32)


def unpack2(W, L):
    """Inverse of pack2: uint32 words (rows x ceil(L/16)) -> int8 rows x L.

    Raises ValueError on the invalid code 10 or on nonzero padding bits.
    """
    W = np.asarray(W, dtype=np.uint32)
    rows, words = W.shape
    if words != (L + 15) // 16:
        raise ValueError("word count does not match length")
    shifts = (2 * np.arange(16, dtype=np.uint32))[None, None, :]
    codes = (W[:, :, None] >> shifts) & np.uint32(3)
    codes = codes.reshape(rows, words * 16)
    if np.any(codes == 2):
        raise ValueError("invalid 2-bit code 10")
    if np.any(codes[:, L:] != 0):
        raise ValueError("nonzero padding")
    out = np.zeros((rows, L), dtype=np.int8)
    c = codes[:, :L]
    out[c == 1] = 1
    out[c == 3] = -1
    return out


def zero_fraction(B, C):
    """Fraction of zeros over both ternary factors together."""
    B = np.asarray(B)
    C = np.asarray(C)
    zeros = int(np.count_nonzero(B == 0)) + int(np.count_nonzero(C == 0))
    return zeros / float(B.size + C.size)


def bpw_eff(mu, m, n, sparsity):
    """Eq. 1 (§2.6): storage per original weight under mask+sign packing."""
    return mu * (m + n) / max(m, n) * (2.0 - sparsity)


def bpw_packed2(k, m, n):
    """Bits per original weight of the fixed 2-bit codes plus fp32 scales."""
    return (2.0 * k * (m + n) + 32.0 * k) / (m * n)
