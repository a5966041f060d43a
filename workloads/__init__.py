"""Seeded synthetic workloads for the MoGA forward hot path.

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``: the only
module both the oracle side and the HIP side consume.  It draws inputs; it
computes none of the method (no routing decision, sort, attention or gate).
"""

from .configs import WORKLOADS, Workload, get_workload  # noqa: F401
from .gen import make_inputs, make_shots, top2_margin, sample_rows  # noqa: F401
