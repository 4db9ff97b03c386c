"""Seeded synthetic inputs for MoE token dispatch and combine.

This package only generates inputs: which experts each token picks, the router
weights, the token activations and the stand-in expert outputs.  It computes
none of the method's own results (no counts, offsets, permutations, row
gathers or weighted sums), so the CPU oracle and the HIP path can both be fed
from it without sharing any of the method's arithmetic.
"""

from .routing import (  # noqa: F401
    uniform_topk,
    k_hot_topk,
    zipf_topk,
    replica_topk,
    softmax_weights,
    normal_rows,
    fp8_blockscaled_rows,
)
from .configs import WORKLOADS, Workload, get_workload, build_inputs  # noqa: F401
