"""fp64 CPU oracle of ExTernD's greedy expanded-rank ternary decomposition.

TEST INFRASTRUCTURE ONLY.  Only code under tests/, the smoke check in
__graft_entry__.py and the CPU-baseline leg of bench.py may import or call
anything in this package.  The library in ternary_rank_weight_amd/ never
imports it and shares no code with it.

It is a plain, slow, step-by-step transcription of the method on the pages of
"ExTernD: Expanded-Rank Ternary Decomposition Ternary LLM PTQ with Accuracy
Approaching Any Quantization Level" (§2.1-§2.4, §2.6), in float64, with numpy
matrix products and Cholesky factorisations as the only library steps.

oracle/c/externd_oracle.c is a second, plain C transcription of T_tau, the
greedy sequential decomposition and the plain block ALS (loaded by
oracle/c_oracle.py, compiled by build() in __graft_entry__.py), pinned the
same way in tests/test_oracle_c.py.

Pins (tests/test_oracle_*.py) tie it to what the pages and mathematics fix:
hand-worked T_tau vectors, the Gaussian zero-fraction closed form, the
closed-form optimal projection against brute force, exact residual decrease,
brute-force rank-1 optima on tiny matrices, exact recovery of ternary rank-1
matrices, sign and power-of-two symmetries, the prefix property, block b=1 ==
sequential, and a known-answer value of the SplitMix64 generator.

Parity unpinned: the whole-trajectory energies on the synthetic workloads (the
pages print no worked example for them; the oracle's own result is the
reference) and the two free choices the pages leave open, the starting vector
rule and the ridge eps.
"""
from .ternarize import (mean_abs_threshold, ternarize, ternarize_columns, optimal_projection,
                        project_columns)
from .init_rule import splitmix64_mix, init_hash, init_signs, init_block
from .als import (rank_for, block_width, ridge, decompose_seq, decompose_block, rank1_fit,
                  rank_for_energy, importance_weights, weighted_norm2, block_u_target,
                  block_v_target, decorrelation_inverse, joint_scales, single_entry_bound)
from .factors import (reconstruct, apply_factors, energy_from_factors, pack2, unpack2,
                      zero_fraction, bpw_eff, bpw_packed2)

__all__ = [
    "mean_abs_threshold", "ternarize", "ternarize_columns", "optimal_projection", "project_columns",
    "splitmix64_mix", "init_hash", "init_signs", "init_block",
    "rank_for", "block_width", "ridge", "decompose_seq", "decompose_block", "rank1_fit",
    "rank_for_energy", "importance_weights", "weighted_norm2", "block_u_target",
    "block_v_target", "decorrelation_inverse", "joint_scales", "single_entry_bound",
    "reconstruct", "apply_factors", "energy_from_factors", "pack2", "unpack2", "zero_fraction",
    "bpw_eff", "bpw_packed2",
]
