"""fp64 CPU oracle of the MiTA forward pass -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package; the HIP library never does.
"""
from .mita_oracle import (  # noqa: F401
    tau, pool_windows, landmark_queries, landmark_scores, expert_topk, softmax_rows,
    shared_values, route_queries, group_by_route, attend_head, mita_head, mita_forward,
    softmax_backward, mita_head_backward,
)
