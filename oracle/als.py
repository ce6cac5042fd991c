"""Greedy expanded-rank ternary decomposition A ~ B diag(D) C, in fp64.

Test infrastructure: only tests, the smoke check and the benchmark's CPU
baseline may use this module.  It is a plain, slow transcription of the
method as the pages describe it; matrix products come from numpy (a library
primitive), nothing is fused or reordered.

Sources (ExTernD: Expanded-Rank Ternary Decomposition Ternary LLM PTQ with
Accuracy Approaching Any Quantization Level):
  §2.1  representation, k = mu * min(m, n), energy E
  §2.3  greedy sequential ALS: alternating ternary fit, optimal scale, deflation
  §2.4  batched block ALS with decorrelated targets and a joint scale solve,
        and refinement sweeps over the extracted blocks
  §2.5  importance-weighted ALS (column weights h~ = h / max(h) + lambda)
  Appendix (monotone residual): the residual norm never increases.

Readings where the pages leave a step open:
  * k = round-half-away(mu * min(m, n)) computed in fp64, mu widened from fp32.
  * One iteration is the V update followed by the U update; there are `iters`
    of them and no early stop.  The scale uses the final u and v, and u.x with
    x = R v from the last iteration equals u^T R v.
  * u0 / U0 come from oracle.init_rule (dense +-1, keyed on the component index).
  * Block mode: b_eff = min(block, floor(min(m, n) / 8)); a trailing partial
    block takes the remaining components.  The ridge is
    eps = 1e-6 * trace(G) / b for each Gram matrix G.  The joint scale system
    [(U^T U) o (V^T V)] d = diag(U^T R V) is solved by Cholesky; if that fails
    it is retried with the same kind of ridge and the event is counted.
  * ||A|| = 0 gives E = 1.
  * Refinement sweeps restart each block's iterations from its stored U and
    keep the refit only if ||R||^2 does not grow, so the energy never falls
    (the pages report a monotone rise).
  * Safeguard (appendix §7, which only names it): the single-entry bound is
    max_ij w_j R_ij^2, the decrease of the one-entry component e_r e_c^T with
    d = R_rc.  A fit whose decrease falls below it "would activate" the
    safeguard and is counted; with safeguard=True (sequential mode) it is
    replaced by that entry, the first in row-major order on a tie.  Block
    mode counts blocks whose joint decrease d . rhs falls below the bound.
"""
import math

import numpy as np

from .init_rule import init_signs, init_block
from .ternarize import ternarize, ternarize_columns, optimal_projection, project_columns


def _tern(x, tau, projection):
    """The ternarizer of one vector: T_tau, or the optimal projection (§2.2)."""
    return optimal_projection(x)[0] if projection else ternarize(x, tau)


def _tern_cols(X, tau, projection):
    return project_columns(X) if projection else ternarize_columns(X, tau)

__all__ = ["rank_for", "block_width", "ridge", "decompose_seq", "decompose_block",
           "rank1_fit", "SeqResult", "rank_for_energy", "importance_weights", "weighted_norm2",
           "block_u_target", "block_v_target", "decorrelation_inverse", "joint_scales",
           "single_entry_bound"]


def rank_for(m, n, mu):
    """k = mu * min(m, n), rounded half away from zero (§2.1)."""
    mu64 = float(np.float32(mu))
    v = mu64 * float(min(m, n))
    whole = math.floor(v)
    return int(whole) + (1 if v - whole >= 0.5 else 0)


def block_width(m, n, block):
    """Effective block width: requested b capped at floor(min(m,n)/8) (§2.4).

    Returns 1 (sequential) when the request or the cap is below 2.
    """
    if block <= 1:
        return 1
    b = min(int(block), min(m, n) // 8)
    return b if b >= 2 else 1


def ridge(G):
    """eps for (G + eps I): 1e-6 times the mean diagonal of G (§2.4 names eps only)."""
    b = G.shape[0]
    return 1e-6 * float(np.trace(G)) / b


class SeqResult:
    """Factors and diagnostics of one decomposition.

    B: m x k int8, C: k x n int8, D: k float64, trace: ||R||^2 after each
    component (sequential) or block (block mode), E: energy preserved,
    norm_a2: ||A||^2, extra: mode-specific diagnostics.
    """

    def __init__(self, B, C, D, trace, E, norm_a2, extra=None):
        self.B, self.C, self.D = B, C, D
        self.trace, self.E, self.norm_a2 = trace, E, norm_a2
        self.extra = extra or {}


def importance_weights(h, lam):
    """Column weights of the importance-weighted objective (§2.5):
    h~ = h / max(h) + lambda, for per-input-channel second moments h >= 0."""
    h = np.asarray(h, dtype=np.float64)
    if h.ndim != 1 or not np.all(np.isfinite(h)) or np.any(h < 0) or not np.isfinite(lam) or lam < 0:
        raise ValueError("h must be finite and >= 0, lambda finite and >= 0")
    mx = float(h.max()) if h.size else 0.0
    if mx == 0.0 and lam == 0.0:
        raise ValueError("all weights would be zero")
    return (h / mx if mx > 0 else np.zeros_like(h)) + float(lam)


def weighted_norm2(R, w):
    """sum_ij w_j R_ij^2 (w = None: the plain squared Frobenius norm)."""
    R = np.asarray(R, dtype=np.float64)
    return float(np.sum(R * R)) if w is None else float(np.sum((R * R) @ w))


def single_entry_bound(R, w=None):
    """The single-entry bound of appendix §7: the largest decrease of the
    weighted residual norm one ternary entry can give, max_ij w_j R_ij^2
    (the component e_r e_c^T with d = R_rc), and its position (r, c), the
    first in row-major order on a tie."""
    R = np.asarray(R, dtype=np.float64)
    ent = R * R if w is None else (R * R) * np.asarray(w, dtype=np.float64)[None, :]
    idx = int(np.argmax(ent))
    r, c = divmod(idx, R.shape[1])
    return float(ent[r, c]), r, c


def rank1_fit(R, u0, tau, iters, w=None, projection=False):
    """Alternating ternary fit of one component against residual R (§2.3 steps 1-2).

    w: optional column weights h~ (§2.5).  The v update keeps the plain
    target R^T u (the weights cancel column by column); the u update targets
    x = R diag(w) v, and d is the weighted least-squares scale
    u^T R diag(w) v / (||u||^2 v^T diag(w) v).

    Returns dict with u, v (int8), d, c = u^T R diag(w) v, the history of the
    intermediate vectors (y_t = R^T u, v_t, x_t = R diag(w) v, u_t), nnz counts
    and sv = v^T diag(w) v.  R is not modified.
    """
    u = np.asarray(u0, dtype=np.float64)
    hist = []
    x = None
    v = None
    for _ in range(iters):
        y = R.T @ u
        v = _tern(y, tau, projection).astype(np.float64)
        x = R @ v if w is None else R @ (w * v)
        u_new = _tern(x, tau, projection).astype(np.float64)
        hist.append((y, v.copy(), x, u_new.copy()))
        u = u_new
    nu = float(np.count_nonzero(u))
    nv = float(np.count_nonzero(v))
    sv = nv if w is None else float(w @ (v * v))
    c = float(u @ x)
    d = c / (nu * sv)
    return {"u": u.astype(np.int8), "v": v.astype(np.int8), "d": d, "c": c,
            "nnz_u": int(nu), "nnz_v": int(nv), "sv": sv, "hist": hist}


def decompose_seq(A, mu, tau, iters=15, seed=0, k=None, record=None, weights=None, projection=False,
                  safeguard=False):
    """Greedy sequential ALS (§2.3).  Returns SeqResult.

    record: optional set of component indices whose rank1_fit history and
    pre-deflation residual are kept in result.extra["records"].
    weights: optional column weights h~ (importance_weights, §2.5); the
    trace, norm_a2 and E are then the weighted ones.
    projection: ternarize with the optimal ternary projection instead of
    T_tau (§2.2; tau is then unused).
    safeguard: replace a fit whose decrease of ||R||^2 falls below the
    single-entry bound by that single entry (appendix §7).  Either way
    extra["safeguard_would"] counts the components where it would.
    """
    w = None if weights is None else np.asarray(weights, dtype=np.float64)
    A = np.asarray(A)
    m, n = A.shape
    if k is None:
        k = rank_for(m, n, mu)
    would = 0
    R = A.astype(np.float64, copy=True)
    norm_a2 = weighted_norm2(R, w)
    B = np.zeros((m, k), dtype=np.int8)
    C = np.zeros((k, n), dtype=np.int8)
    D = np.zeros(k, dtype=np.float64)
    trace = np.zeros(k, dtype=np.float64)
    decrease = np.zeros(k, dtype=np.float64)
    sum_nnz_u = 0
    records = {}
    for i in range(k):
        u0 = init_signs(seed, i, m)
        if record is not None and i in record:
            records[i] = {"R": R.copy()}
        fit = rank1_fit(R, u0, tau, iters, w, projection)
        u = fit["u"].astype(np.float64)
        v = fit["v"].astype(np.float64)
        d = fit["d"]
        den = fit["nnz_u"] * fit["sv"]
        dec = fit["c"] ** 2 / den if den > 0 else 0.0
        bound, br, bc = single_entry_bound(R, w)
        if dec < bound:
            would += 1
            if safeguard:
                u = np.zeros(m)
                v = np.zeros(n)
                u[br] = 1.0
                v[bc] = 1.0
                d = float(R[br, bc])
                dec = bound
        R -= d * np.outer(u, v)
        B[:, i] = u.astype(np.int8)
        C[i, :] = v.astype(np.int8)
        D[i] = d
        trace[i] = weighted_norm2(R, w)
        decrease[i] = dec
        sum_nnz_u += sum(int(np.count_nonzero(h[3])) for h in fit["hist"])
        if record is not None and i in record:
            records[i]["fit"] = fit
    last = trace[k - 1] if k > 0 else norm_a2
    E = 1.0 - last / norm_a2 if norm_a2 > 0 else 1.0
    return SeqResult(B, C, D, trace, E, norm_a2,
                     {"decrease": decrease, "records": records, "sum_nnz_u": sum_nnz_u,
                      "safeguard_would": would})


def _cholesky_solve(G, rhs, eps):
    """Solve (G + eps I) X = rhs by Cholesky (rhs may be a matrix)."""
    Gr = G + eps * np.eye(G.shape[0])
    Lc = np.linalg.cholesky(Gr)
    z = np.linalg.solve(Lc, rhs)
    return np.linalg.solve(Lc.T, z)


def decorrelation_inverse(G):
    """(G + eps I)^-1 with the ridge eps of the decorrelated targets (§2.4),
    by Cholesky in fp64."""
    G = np.asarray(G, dtype=np.float64)
    return _cholesky_solve(G, np.eye(G.shape[0]), ridge(G))


def block_v_target(R, U):
    """Decorrelated V target [(U^T U + eps I)^-1 U^T R]^T (§2.4).  With column
    weights it is unchanged: each column's weight cancels (§2.5)."""
    GU = U.T @ U
    return _cholesky_solve(GU, (R.T @ U).T, ridge(GU)).T


def block_u_target(R, V, w=None):
    """Decorrelated U target Q (V^T diag(w) V + eps I)^-1 with Q = R diag(w) V
    (§2.4; §2.5 for the weights, w = None meaning all ones).  Returns
    (target, Q)."""
    Vw = V if w is None else V * w[:, None]
    Q = R @ Vw
    GV = V.T @ Vw
    return _cholesky_solve(GV, Q.T, ridge(GV)).T, Q


def _fit_block(R, U, tau, iters, w=None, projection=False):
    """The alternating block iterations of §2.4 from the starting block U.
    Returns (U, V, Q) with Q = R diag(w) V from the last iteration."""
    V = None
    Q = None
    for _ in range(iters):
        V = _tern_cols(block_v_target(R, U), tau, projection).astype(np.float64)
        T, Q = block_u_target(R, V, w)
        U = _tern_cols(T, tau, projection).astype(np.float64)
    return U, V, Q


def joint_scales(U, V, Q, w=None):
    """The joint scale solve of §2.4 (see _joint_scales): returns (d, rhs)."""
    d, rhs, _ = _joint_scales(U, V, Q, w)
    return d, rhs


def _joint_scales(U, V, Q, w=None):
    """Solve [(U^T U) o (V^T diag(w) V)] d = diag(U^T R diag(w) V) (§2.4,
    §2.5); the right side is read off Q = R diag(w) V.  Returns (d, rhs,
    retried)."""
    rhs = np.sum(U * Q, axis=0)
    Mjs = (U.T @ U) * (V.T @ (V if w is None else V * w[:, None]))
    try:
        return _cholesky_solve(Mjs, rhs, 0.0), rhs, False
    except np.linalg.LinAlgError:
        return _cholesky_solve(Mjs, rhs, ridge(Mjs)), rhs, True


def decompose_block(A, mu, tau, iters=15, block=256, seed=0, k=None, force_width=None, sweeps=0,
                    weights=None, projection=False):
    """Batched block ALS with decorrelated targets (§2.4).  Returns SeqResult.

    Each iteration:  P = R^T U;  V <- T_col( P (U^T U + eps I)^-1 );
                     Q = R V;    U <- T_col( Q (V^T V + eps I)^-1 ).
    Then diag(U^T R V) is read off the last Q, the b scales solve
    [(U^T U) o (V^T V)] d = diag(U^T R V), and R <- R - U diag(d) V^T.

    sweeps: refinement sweeps after extraction (§2.4, refinement).  Each sweep
    visits the blocks in order: the block's contribution is added back to R,
    the block iterations run again starting from its stored U, the scales are
    solved jointly, and the refitted block replaces the stored one when it
    leaves ||R||^2 no larger than before the visit; otherwise the stored block
    is deflated again.  extra["sweep_trace"][s] is ||R||^2 after sweep s and
    extra["sweep_kept_old"] counts the visits that kept the stored block.

    force_width: run the block iteration with exactly this width, bypassing
    the cap and the fall-back to sequential mode (used to pin b = 1 against
    the sequential algorithm).

    weights: optional column weights h~ (importance_weights, §2.5): the U
    update and the joint solve use R diag(w) and V^T diag(w) V, the V update
    keeps the plain R; trace, norm_a2 and E are the weighted ones.

    projection: ternarize with the optimal ternary projection (§2.2).
    """
    w = None if weights is None else np.asarray(weights, dtype=np.float64)
    A = np.asarray(A)
    m, n = A.shape
    if k is None:
        k = rank_for(m, n, mu)
    b = block_width(m, n, block) if force_width is None else int(force_width)
    if b == 1 and force_width is None:
        if sweeps:
            raise ValueError("refinement sweeps need block mode (b >= 2)")
        res = decompose_seq(A, mu, tau, iters, seed, k, weights=w, projection=projection)
        res.extra["b"] = 1
        return res
    R = A.astype(np.float64, copy=True)
    norm_a2 = weighted_norm2(R, w)
    B = np.zeros((m, k), dtype=np.int8)
    C = np.zeros((k, n), dtype=np.int8)
    D = np.zeros(k, dtype=np.float64)
    nblocks = (k + b - 1) // b
    trace = np.zeros(nblocks, dtype=np.float64)
    decrease = np.zeros(nblocks, dtype=np.float64)
    ridge_retries = 0
    would = 0
    for blk in range(nblocks):
        c0 = blk * b
        bb = min(b, k - c0)
        bound = single_entry_bound(R, w)[0]
        U, V, Q = _fit_block(R, init_block(seed, c0, bb, m), tau, iters, w, projection)
        d, rhs, retried = _joint_scales(U, V, Q, w)
        ridge_retries += int(retried)
        would += int(float(d @ rhs) < bound)
        R -= (U * d) @ V.T
        B[:, c0:c0 + bb] = U.astype(np.int8)
        C[c0:c0 + bb, :] = V.T.astype(np.int8)
        D[c0:c0 + bb] = d
        trace[blk] = weighted_norm2(R, w)
        decrease[blk] = float(d @ rhs)
    sweep_trace = np.zeros(sweeps, dtype=np.float64)
    kept_old = 0
    r2 = trace[-1] if nblocks > 0 else norm_a2
    for sw in range(sweeps):
        for blk in range(nblocks):
            c0 = blk * b
            bb = min(b, k - c0)
            Uo = B[:, c0:c0 + bb].astype(np.float64)
            Vo = C[c0:c0 + bb, :].T.astype(np.float64)
            Rp = R + (Uo * D[c0:c0 + bb]) @ Vo.T
            U, V, Q = _fit_block(Rp, Uo, tau, iters, w, projection)
            d, _, retried = _joint_scales(U, V, Q, w)
            ridge_retries += int(retried)
            Rn = Rp - (U * d) @ V.T
            r2n = weighted_norm2(Rn, w)
            if r2n <= r2:
                R, r2 = Rn, r2n
                B[:, c0:c0 + bb] = U.astype(np.int8)
                C[c0:c0 + bb, :] = V.T.astype(np.int8)
                D[c0:c0 + bb] = d
            else:
                kept_old += 1
        sweep_trace[sw] = r2
    last = r2
    E = 1.0 - last / norm_a2 if norm_a2 > 0 else 1.0
    return SeqResult(B, C, D, trace, E, norm_a2,
                     {"decrease": decrease, "b": b, "ridge_retries": ridge_retries,
                      "sweep_trace": sweep_trace, "sweep_kept_old": kept_old,
                      "safeguard_would": would})


def rank_for_energy(trace, norm_a2, target, step=1, total=None):
    """Smallest prefix rank reaching energy >= target (§3.3 choosing mu per
    matrix), by the greedy prefix property: trace[j] is ||R||^2 after
    component j (step 1) or block j (step b).  0 for a zero matrix, -1 if no
    prefix reaches the target."""
    trace = np.asarray(trace, dtype=np.float64)
    if total is None:
        total = trace.size * step
    if norm_a2 == 0.0:
        return 0
    for j, t in enumerate(trace):
        if 1.0 - t / norm_a2 >= target:
            return min((j + 1) * step, total)
    return -1
