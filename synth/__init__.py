"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the bench."""
from .workloads import (WORKLOADS, Workload, layer_temperatures, make_batch, make_context,
                        make_context_batch, make_head, make_use_batch, rope, tiny_workload,
                        uniform_budget, unrope)

__all__ = ["WORKLOADS", "Workload", "layer_temperatures", "make_batch", "make_context",
           "make_context_batch", "make_head", "make_use_batch", "rope", "tiny_workload",
           "uniform_budget", "unrope"]
