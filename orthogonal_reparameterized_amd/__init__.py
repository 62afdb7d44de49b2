"""POET reparameterized linear layer for MI355X (gfx950): HIP kernels behind a C ABI, with a thin Python binding.

Each weight is W = R W0 P with a fixed random W0 and orthogonal R, P built by the truncated Cayley-Neumann
series from skew-symmetric generators, as block-diagonal (POET-BS) or index-sampled (POET-FS) primitives. The
library provides the forward pass, the backward pass to the skew parameters and merge-then-reinitialize.
"""
from .binding import (POET_BF16, POET_BS, POET_F32, POET_FS, POET_OP_BUILD, POET_OP_BWD, POET_OP_FWD,  # noqa: F401
                      POET_OP_MERGE, POET_SIDE_P, POET_SIDE_R, PoetError, layer, lib, poet_build_orthogonal,
                      poet_build_workspace_bytes, poet_layer, poet_last_error, poet_linear_bwd, poet_linear_fwd,
                      poet_merge, poet_num_prims, poet_powers_len, poet_prim_len, poet_sample_indices,
                      poet_sample_workspace_bytes, poet_side, poet_status_string, poet_theta_len, poet_version,
                      poet_workspace_bytes, side, side_of)
from .layer import PoetLinear  # noqa: F401
