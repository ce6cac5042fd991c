"""Starting vector of each component (fp64 oracle side).

Test infrastructure: only tests, the smoke check and the benchmark's CPU
baseline may use this module.

The pages start the alternating fit from "u" without saying how u is chosen
(ExTernD, §2.3; the block variant in §2.4 likewise starts from some U).  The
reading used here: u0 is a dense +-1 (Rademacher) vector drawn from a
counter-based hash, keyed on the seed, the global component index i and the
row index r, so that sequential and block mode start component i from the same
vector and any component can be recomputed on its own.

Generator: SplitMix64's output function (Steele, Lea & Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), applied statelessly:
    mix(x) = finalise(x + 0x9E3779B97F4A7C15)   (mod 2**64)
    finalise(z): z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
                 z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31
    h(seed, i, r) = mix(mix(mix(seed) + i) + r)
    u0[r] = -1 if the top bit of h is set else +1
This module is written independently of the GPU path's copy of the same rule;
the two are cross-checked by the tests.
"""
import numpy as np

__all__ = ["splitmix64_mix", "init_hash", "init_signs", "init_block"]

_MASK = (1 << 64) - 1
_GOLDEN = 0x9E3779B97F4A7C15
_C1 = 0xBF58476D1CE4E5B9
_C2 = 0x94D049BB133111EB


def splitmix64_mix(x):
    """One SplitMix64 output for state x (Python int arithmetic mod 2**64)."""
    z = (int(x) + _GOLDEN) & _MASK
    z = ((z ^ (z >> 30)) * _C1) & _MASK
    z = ((z ^ (z >> 27)) * _C2) & _MASK
    return z ^ (z >> 31)


def init_hash(seed, i, r):
    """h(seed, i, r) as a Python int."""
    return splitmix64_mix((splitmix64_mix((splitmix64_mix(seed) + int(i)) & _MASK) + int(r)) & _MASK)


def _mix_array(x):
    """Vectorised SplitMix64 output over a uint64 numpy array (wrapping)."""
    z = (x + np.uint64(_GOLDEN)).astype(np.uint64)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(_C1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(_C2)
    return z ^ (z >> np.uint64(31))


def init_signs(seed, i, m):
    """u0 of component i: float64 vector of +-1 of length m."""
    base = splitmix64_mix((splitmix64_mix(seed) + int(i)) & _MASK)
    with np.errstate(over="ignore"):
        h = _mix_array(np.uint64(base) + np.arange(m, dtype=np.uint64))
    top = (h >> np.uint64(63)).astype(np.int64)
    return np.where(top == 1, -1.0, 1.0)


def init_block(seed, first, b, m):
    """U0 of a block whose first global component index is `first`: m x b."""
    return np.stack([init_signs(seed, first + j, m) for j in range(b)], axis=1)
