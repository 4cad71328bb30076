"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

Holds none of the layer's arithmetic: only random draws and mask schedules.
"""
from .workloads import (WORKLOADS, SWEEP_FRACTIONS, SWEEP_R, Workload, workload, expert_weight, desc_fields,
                        shared_weight, router_weight, router_bias, layer_weights, decoded_masks,
                        force_masks, hidden_states, f32_to_bf16_bits, bf16_bits_to_f32, act_dtype,
                        decode_inputs)

__all__ = ["WORKLOADS", "SWEEP_FRACTIONS", "SWEEP_R", "Workload", "workload", "expert_weight", "desc_fields",
           "shared_weight", "router_weight", "router_bias", "layer_weights", "decoded_masks",
           "force_masks", "hidden_states", "f32_to_bf16_bits", "bf16_bits_to_f32", "act_dtype",
           "decode_inputs"]
