"""MoGA (Mixture-of-Groups Attention) forward hot path for AMD MI355X (gfx950).

The computation lives in libmoga.so (hand-written HIP kernels behind the C ABI
of include/moga.h); this package is its Python binding.  Importing it fails if
the library has not been built (`python sparse_attention_long_router_amd/build.py`).
"""

from ._lib import (MOGA_OP_BALANCE_STATS, MOGA_OP_GROUP_ATTENTION, MOGA_OP_PERMUTE,  # noqa: F401
                   MOGA_OP_ROUTE, MOGA_OP_STGA_ATTENTION, MOGA_OP_UNPERMUTE, LIB_PATH, MogaError, version)
from .binding import (MogaForward, MogaTraining, moga_balance_stats, moga_group_attention,  # noqa: F401
                      moga_attention_backward_staged, moga_attention_backward_staged_bytes,
                      moga_group_attention_backward, moga_group_attention_train, moga_route_backward,
                      moga_unpermute_backward,
                      moga_group_attention_fused, moga_group_attention_unpermute,
                      moga_group_attention_unpermute_vt, moga_group_attention_unpermute_vtq, moga_permute,
                      moga_permute_vt, moga_permute_vt_noalloc, moga_route,
                      moga_vt_row_length,
                      moga_stga_attention, moga_stga_shot_attention, moga_stga_shot_workspace_bytes, moga_unpermute,
                      moga_workspace_bytes)
