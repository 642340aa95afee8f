"""Seeded synthetic inputs for the MoE layer forward.

This package only draws random numbers and lays them out in the shapes of
the layer; it holds none of the layer's arithmetic (no router, no top-K, no
expert math).  Both the HIP path and the CPU oracle receive tensors made
here, so neither side can disagree with the other about its inputs.

Workloads follow the shapes of the Kimi K2 router card (OpenModelAtlas,
"Kimi K2 · Router": 7168-wide hidden state, 384 experts, top-8, x2.827) and
of the Kimi K3 table (lilting.ch essay on K3, table of K3 dimensions:
896 routed experts, top-16, 2 shared, latent 3584, intermediate 3072).
"""
from .workloads import WORKLOADS, Workload, get_workload
from .generate import (make_router_inputs, make_expert_weights,
                       make_layer_inputs, STREAM)

__all__ = ["WORKLOADS", "Workload", "get_workload", "make_router_inputs",
           "make_expert_weights", "make_layer_inputs", "STREAM"]
