"""CPU oracle of the POET layer (test infrastructure only; see poet_oracle)."""
from .poet_oracle import *  # noqa: F401,F403
from .poet_oracle import (MODE_BS, MODE_BSP, MODE_FS, SIDE_P, SIDE_R, Side, adamw_step, assemble, block_sizes,  # noqa
                          build_orthogonal, build_orthogonal_exact, hyperspherical_energy, hyperspherical_energy_rows,
                          optimizer_state_after_merge,
                          singular_value_entropy,
                          cayley_exact, cayley_neumann, factor, linear_bwd, linear_fwd, merge, neumann_adjoint,
                          pack_prims, prim_blocks, sample_indices, sample_permutation, skew_from_theta, skew_project, splitmix64,
                          theta_len)
