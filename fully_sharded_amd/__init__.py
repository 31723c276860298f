"""FSDP data-parallel hot path on one MI355X (gfx950): a C-ABI HIP library
(libfsdp_hip.so, declared in include/fsdp_hip.h) and its ctypes binding.

The binding exposes the library's calls under the same names:
fsdp_plan_layout, fsdp_shard_pack, fsdp_gather_unflatten,
fsdp_reduce_scatter_avg, fsdp_adamw_shard_step.
"""
from .binding import (  # noqa: F401
    BF16, F32, FLAT, PER_PARAM, FsdpError, Plan, bind_adamw_shard_step, bind_gather_unflatten,
    fsdp_adamw_shard_step,
    fsdp_gather_unflatten, fsdp_plan_layout, fsdp_reduce_scatter_avg, fsdp_shard_pack, lib,
)
