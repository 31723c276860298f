"""FSDP data-parallel hot path on one MI355X (gfx950): a C-ABI HIP library
(libfsdp_mi355x.so, declared in include/fsdp_mi355x.h) and its ctypes binding.

The binding exposes the library's calls under the same names:
fsdp_plan_layout, fsdp_shard_pack, fsdp_gather_unflatten,
fsdp_reduce_scatter_avg, fsdp_adamw_shard_step (and fsdp_adamw_step_then_gather,
the step of one unit with the next unit's gather), and beyond the per-step path
fsdp_reshard_plan / fsdp_reshard / fsdp_reshard_batch (restore at another
world size), fsdp_grad_accumulate, fsdp_allreduce_avg (the DDP comparator)
and StepGraph (fsdp_step_graph_*: a unit loop replayed as one HIP graph).
rows and unit_buffers allocate device arrays placed so that the streams a
kernel touches at one offset do not share HBM channels.
"""
from .binding import (  # noqa: F401
    BF16, F32, FLAT, PER_PARAM, FsdpError, Plan, Resharder, StepGraph, bind_adamw_shard_step,
    bind_adamw_step_then_gather, bind_gather_unflatten, bind_reduce_scatter_avg, bind_shard_pack,
    fsdp_adamw_step_then_gather, bind_grad_accumulate, fsdp_adamw_shard_step,
    fsdp_adamw_shard_step_noalloc, fsdp_allreduce_avg,
    fsdp_gather_unflatten, fsdp_grad_accumulate, fsdp_plan_layout, fsdp_reduce_scatter_avg,
    fsdp_reshard, fsdp_reshard_batch, fsdp_reshard_plan, fsdp_shard_pack, lib,
)
from .buffers import rows, unit_buffers  # noqa: F401,E402
