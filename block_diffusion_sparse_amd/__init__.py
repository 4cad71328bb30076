"""Liveness-sparse routed-expert MoE layer forward for MI355X (gfx950).

The compute path is libepoch.so (HIP kernels behind the C ABI in include/epoch.h);
`binding` marshals arguments to it and `plan.EpochPlan` owns the workspace.
"""
from . import binding  # noqa: F401

__all__ = ["binding"]
