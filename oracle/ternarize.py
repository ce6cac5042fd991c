"""Mean-threshold ternarizer T_tau and the optimal ternary projection (fp64).

Test infrastructure: only tests, the smoke check and the benchmark's CPU
baseline may use this module. The product path never calls it.

Source: "ExTernD: Expanded-Rank Ternary Decomposition Ternary LLM PTQ with
Accuracy Approaching Any Quantization Level", §2.2 (definition of T_tau and of
the closed-form optimal ternary projection).

Definition on the page: entry i of T_tau(x) is sign(x_i) when |x_i| exceeds tau
times the mean of |x| over the whole vector, else 0; when nothing would be
kept, the single largest entry is kept instead.

Readings where the page leaves a step open:

* The mean is taken over the vector's own length N (m for u, n for v).
* The mean is computed in a fixed, order-free way so that two
  implementations fed identical inputs agree bit for bit:
    M = max |x_j|; e = frexp exponent of M (M < 2**e);
    L = ceil(log2 N); s = 52 - e - L;
    q_j = floor(|x_j| * 2**s) as an exact integer (each < 2**(52-L));
    S = (sum_j q_j) * 2**-s, the sum being < 2**52 and hence exact in float64;
    thr = (tau * S) / N in float64, tau being the float32 value widened.
  Every q_j and their sum are exact, so S is below the exact sum of |x| by
  less than N * 2**-s and thr below tau * mean|x| by less than tau * 2**-s
  (a relative 2**-37 or so for a typical vector).
* The comparison is strict (|x_i| > thr); sign(0) = 0.
* Fallback when nothing passes: the smallest index i with |x_i| = M keeps
  its sign. When x is identically zero the result is +1 at index 0.
"""
import math

import numpy as np

__all__ = ["mean_abs_threshold", "ternarize", "ternarize_columns", "optimal_projection",
           "project_columns"]


def _ceil_log2(n):
    """ceil(log2(n)) for a positive integer n, exactly (0 for n = 1)."""
    return (int(n) - 1).bit_length()


def mean_abs_threshold(x, tau):
    """Return (thr, M) for T_tau on the 1-D vector x.

    thr is tau times the fixed-point mean of |x| (see the module docstring);
    M is max |x|.  When M == 0 the threshold is returned as 0.0.
    """
    a = np.abs(np.asarray(x, dtype=np.float64))
    n = a.size
    if n == 0:
        raise ValueError("empty vector")
    big = float(a.max())
    if big == 0.0:
        return 0.0, 0.0
    _, e = math.frexp(big)          # big = f * 2**e with 0.5 <= f < 1
    s = 52 - e - _ceil_log2(n)
    q = np.floor(np.ldexp(a, s)).astype(np.int64)
    total = int(q.sum(dtype=np.int64))
    assert 0 <= total < (1 << 52)
    S = math.ldexp(float(total), -s)  # exact: total < 2**52
    tau64 = float(np.float32(tau))
    thr = (tau64 * S) / float(n)
    return thr, big


def ternarize(x, tau):
    """T_tau(x) as an int8 vector in {-1, 0, +1} (page §2.2)."""
    xv = np.asarray(x, dtype=np.float64)
    if xv.ndim != 1:
        raise ValueError("ternarize takes a 1-D vector")
    thr, big = mean_abs_threshold(xv, tau)
    t = np.zeros(xv.size, dtype=np.int8)
    if big == 0.0:
        t[0] = 1
        return t
    keep = np.abs(xv) > thr
    t[keep & (xv > 0)] = 1
    t[keep & (xv < 0)] = -1
    if not keep.any():
        i = int(np.flatnonzero(np.abs(xv) == big)[0])
        t[i] = 1 if xv[i] > 0 else -1
    return t


def ternarize_columns(X, tau):
    """Apply T_tau to every column of the 2-D array X (block ALS, page §2.4)."""
    X = np.asarray(X, dtype=np.float64)
    out = np.empty(X.shape, dtype=np.int8)
    for j in range(X.shape[1]):
        out[:, j] = ternarize(X[:, j], tau)
    return out


def _fixed_point_magnitudes(a):
    """q_j = floor(|x_j| * 2**s) with the shift of mean_abs_threshold (exact
    integers, every partial sum below 2**52)."""
    big = float(a.max())
    _, e = math.frexp(big)
    s = 52 - e - _ceil_log2(a.size)
    return np.floor(np.ldexp(a, s)).astype(np.int64)


def optimal_projection(x):
    """Closed-form argmin over ternary t and real alpha of ||x - alpha t||_2.

    Page §2.2: sort |x| in decreasing order and keep the prefix of length s
    that maximises (1/sqrt(s)) * (sum of the s largest |x|).  Returns
    (t, alpha) with t in {-1,0,1}^N and alpha the least-squares scale (the
    mean of the kept |x|).

    Readings (so that two implementations agree bit for bit): the order is
    that of |x| with equal values taken in index order; the prefix sums are
    those of the fixed-point magnitudes q_j of mean_abs_threshold (exact
    integers), and prefixes s and r are compared exactly as Q_s^2 r against
    Q_r^2 s, the shortest prefix winning a tie.  This chooses the optimum of
    the magnitudes truncated to about 2**-37 relative.  x identically zero
    gives +1 at index 0 (as for T_tau).
    """
    xv = np.asarray(x, dtype=np.float64)
    a = np.abs(xv)
    t = np.zeros(a.size, dtype=np.int8)
    if a.size == 0:
        raise ValueError("empty vector")
    if float(a.max()) == 0.0:
        t[0] = 1
        return t, 0.0
    order = np.argsort(-a, kind="stable")
    q = _fixed_point_magnitudes(a)[order]
    best, best_q, run = 1, int(q[0]), int(q[0])
    for size in range(2, a.size + 1):
        run += int(q[size - 1])
        if run * run * best > best_q * best_q * size:
            best, best_q = size, run
    sel = order[:best]
    t[sel] = np.where(xv[sel] > 0, 1, np.where(xv[sel] < 0, -1, 0)).astype(np.int8)
    alpha = float(np.sum(a[sel]) / best)
    return t, alpha


def project_columns(X):
    """Optimal ternary projection of every column of X (block ALS variant)."""
    X = np.asarray(X, dtype=np.float64)
    out = np.empty(X.shape, dtype=np.int8)
    for j in range(X.shape[1]):
        out[:, j] = optimal_projection(X[:, j])[0]
    return out
