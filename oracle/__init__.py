"""CPU oracle for the MoGA forward hot path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call, link
or execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, helpers, tables or pre/post-processing)
and imports nothing from ``sparse_attention_long_router_amd``.

The method it follows is described on the page "MoGA: Mixture-of-Groups
Attention for End-to-End Long Video Generation" (architecture explainer of
arXiv 2510.18692); section names below refer to that page.
"""

from .moga_oracle import (  # noqa: F401
    router_logits,
    route,
    permute,
    gather_rows,
    group_attention,
    group_attention_rows,
    unpermute,
    stga_group_ids,
    stga_attention,
    stga_attention_rows,
    moga_forward,
    moga_output_rows,
    balance_stats,
    moga_backward,
    moga_backward_rows,
    shot_windows,
    stga_shot_attention,
    stga_shot_attention_rows,
    frame_attention,
    visual_block_forward,
)
