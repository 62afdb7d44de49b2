"""CPU oracle of the POET layer (test infrastructure only; see poet_oracle)."""
from .poet_oracle import *  # noqa: F401,F403
from .poet_oracle import (MODE_BS, MODE_FS, SIDE_P, SIDE_R, Side, assemble, block_sizes, build_orthogonal,  # noqa
                          cayley_exact, cayley_neumann, factor, linear_bwd, linear_fwd, merge, neumann_adjoint,
                          pack_prims, prim_blocks, sample_indices, skew_from_theta, skew_project, splitmix64,
                          theta_len)
