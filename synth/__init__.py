"""Seeded synthetic inputs for the Hybrid Block workloads.

This package only draws and lays out input tensors (queries, keys, values and
the planted retrieval structure). It holds none of the attention, scoring or
selection arithmetic; both the CPU oracle and the GPU library are fed from it.
"""
from .configs import CONFIGS, Workload, workload
from .inputs import (bridge_inputs, decode_step_inputs, grad_inputs, make_inputs,
                     random_index_rows, to_host)

__all__ = ["CONFIGS", "Workload", "workload", "make_inputs", "decode_step_inputs", "bridge_inputs",
           "grad_inputs", "random_index_rows", "to_host"]
