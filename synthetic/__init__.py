"""Seeded synthetic input matrices shaped like LLM weight matrices.

This module only draws inputs; it holds none of the decomposition's
arithmetic and is shared by the tests, the smoke check and the benchmark.
Every matrix is float32, generated on the host with numpy's PCG64 from a
fixed seed, so both the GPU path and the oracle receive the very same bytes.

Recipes (the pages measure on real checkpoints that are not available here;
these stand in for them with the same shapes):

* ``gaussian(m, n, seed, std)``: iid N(0, std^2).
* ``llm_like(m, n, seed)``: Student-t(5) entries scaled to std 0.02, rounded
  to bfloat16 (nearest-even), each row multiplied by exp(0.3 * N(0,1)), and
  16 distinct uniformly drawn columns multiplied by 10.
* ``low_rank_plus_noise(m, n, seed)``: U diag(s) V^T with U (m x 256) and
  V (n x 256) iid N(0,1), s_i = i^-0.8, plus iid N(0, 0.005^2).
* ``importance(n, seed, sigma)``: per-input-channel second moments standing
  in for an importance matrix (none is available): exp(sigma * N(0,1)),
  a skewed positive vector.
"""
import numpy as np

__all__ = ["gaussian", "llm_like", "low_rank_plus_noise", "importance", "round_bf16",
           "layer_shapes", "workload_matrix", "WORKLOADS"]


def round_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even), as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))
    out = ((bits + bias) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return out.view(np.float32)


def gaussian(m, n, seed, std=0.02):
    rng = np.random.Generator(np.random.PCG64(seed))
    return (std * rng.standard_normal((m, n))).astype(np.float32)


def llm_like(m, n, seed, std=0.02, row_sigma=0.3, n_outlier_cols=16, outlier_gain=10.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    nu = 5.0
    t = rng.standard_t(nu, size=(m, n))
    t *= std / np.sqrt(nu / (nu - 2.0))
    a = round_bf16(t.astype(np.float32)).astype(np.float64)
    rows = np.exp(row_sigma * rng.standard_normal(m))
    a *= rows[:, None]
    cols = rng.choice(n, size=min(n_outlier_cols, n), replace=False)
    a[:, cols] *= outlier_gain
    return a.astype(np.float32)


def low_rank_plus_noise(m, n, seed, rank=256, decay=0.8, noise=0.005):
    rng = np.random.Generator(np.random.PCG64(seed))
    r = min(rank, m, n)
    U = rng.standard_normal((m, r))
    V = rng.standard_normal((n, r))
    s = np.arange(1, r + 1, dtype=np.float64) ** (-decay)
    a = (U * s[None, :]) @ V.T + noise * rng.standard_normal((m, n))
    return a.astype(np.float32)


def importance(n, seed, sigma=1.5):
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.exp(sigma * rng.standard_normal(n)).astype(np.float32)


def layer_shapes():
    """The seven matrices of one 4B-class transformer layer (name, m, n)."""
    return [("q", 4096, 2560), ("k", 1024, 2560), ("v", 1024, 2560), ("o", 2560, 4096),
            ("gate", 9728, 2560), ("up", 9728, 2560), ("down", 2560, 9728)]


# The five workloads, by what they are: shapes, method knobs and the seed of
# each matrix.
#   gauss256     256 x 256 Gaussian, sequential
#   llm2560      2560 x 2560 LLM-shaped, sequential and block b = 64
#   mlp9728      9728 x 2560 LLM-shaped (an MLP matrix), block b = 128
#   layer        the seven matrices of one 4B-class transformer layer, b = 128
#   lowrank4096  4096 x 4096 low rank plus noise, mu and tau swept, b = 128
WORKLOADS = {
    "gauss256": dict(kind="gaussian", m=256, n=256, seed=0, mu=2.0, tau=0.7, iters=15, block=0),
    "llm2560": dict(kind="llm_like", m=2560, n=2560, seed=1, mu=2.0, tau=0.7, iters=15, block=64),
    "mlp9728": dict(kind="llm_like", m=9728, n=2560, seed=2, mu=3.0, tau=1.0, iters=15, block=128),
    "layer": dict(kind="layer", seed=3, mu=2.5, tau=0.7, iters=15, block=128),
    "lowrank4096": dict(kind="low_rank", m=4096, n=4096, seed=4, mus=(1.0, 2.0, 3.0, 3.5),
                        taus=(0.7, 1.0, 2.0), iters=15, block=128),
}


def workload_matrix(name, which=None):
    """Build the input matrix of workload `name` (for "layer", `which` names the layer matrix)."""
    c = WORKLOADS[name]
    if c["kind"] == "gaussian":
        return gaussian(c["m"], c["n"], c["seed"])
    if c["kind"] == "llm_like":
        return llm_like(c["m"], c["n"], c["seed"])
    if c["kind"] == "low_rank":
        return low_rank_plus_noise(c["m"], c["n"], c["seed"])
    if c["kind"] == "layer":
        names = [s[0] for s in layer_shapes()]
        j = names.index(which)
        _, m, n = layer_shapes()[j]
        return llm_like(m, n, 1000 * c["seed"] + j)
    raise ValueError(name)
