"""Thin ctypes binding of libfsdp_mi355x.so, with the C ABI's names.

Only argument marshalling happens here: torch tensors become device
pointers and torch's current HIP stream becomes the stream argument.  Every
step of the path runs in the library's HIP kernels; if the library is missing
this module raises instead of computing anything itself.
"""

from __future__ import annotations

import ctypes
import os
import sys

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfsdp_mi355x.so")

PER_PARAM = 0
FLAT = 1
F32 = 0
BF16 = 1
MAX_RANKS = 64

_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "out of memory",
           -4: "HIP runtime error"}


class FsdpError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)} ({status})")
        self.status = status


class AdamWHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("numel_full", ctypes.c_int64), ("shard_numel", ctypes.c_int64),
                ("world", ctypes.c_int32), ("n_params", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("n_segments", ctypes.c_int32)]


_lib = None

# name -> (restype, argtypes); mirrors include/fsdp_mi355x.h
_SIGS = {
    "fsdp_plan_layout": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                        ctypes.POINTER(ctypes.c_int64), ctypes.c_int32,
                                        ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]),
    "fsdp_plan_destroy": (None, [ctypes.c_void_p]),
    "fsdp_plan_get_info": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(PlanInfo)]),
    "fsdp_plan_param": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.POINTER(ctypes.c_int64)]),
    "fsdp_plan_rank_valid": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_int64)]),
    "fsdp_plan_segments": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
                                          ctypes.c_int32]),
    "fsdp_plan_comm_ledger": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32,
                                             ctypes.POINTER(ctypes.c_int64)]),
    "fsdp_plan_state_bytes_per_rank": (ctypes.c_int64, [ctypes.c_void_p]),
    "fsdp_plan_prepare": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p]),
    "fsdp_shard_pack": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]),
    "fsdp_gather_unflatten": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                             ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p]),
    "fsdp_reduce_scatter_avg": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p),
                                               ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    "fsdp_adamw_shard_step": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(AdamWHParams),
                                             ctypes.c_int64, ctypes.POINTER(ctypes.c_void_p),
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_int32, ctypes.c_void_p]),
    "fsdp_adamw_shard_step_noalloc": (ctypes.c_int, [ctypes.c_void_p,
                                                     ctypes.POINTER(AdamWHParams), ctypes.c_int64,
                                                     ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.c_void_p, ctypes.c_void_p,
                                                     ctypes.c_void_p, ctypes.c_void_p,
                                                     ctypes.c_int32, ctypes.c_void_p]),
    "fsdp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fsdp_plan_work_items": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
                                            ctypes.POINTER(ctypes.c_int64)]),
    "fsdp_reshard_plan": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.POINTER(ctypes.c_void_p)]),
    "fsdp_reshard_destroy": (None, [ctypes.c_void_p]),
    "fsdp_reshard_items": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
                                          ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]),
    "fsdp_reshard": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int32, ctypes.c_void_p]),
    "fsdp_reshard_batch": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.POINTER(ctypes.c_void_p),
                                          ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32,
                                          ctypes.c_void_p]),
    "fsdp_adamw_step_then_gather": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(AdamWHParams),
                                                   ctypes.c_int64, ctypes.POINTER(ctypes.c_void_p),
                                                   ctypes.c_int32, ctypes.c_void_p,
                                                   ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.c_void_p, ctypes.c_int32,
                                                   ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.POINTER(ctypes.c_void_p),
                                                   ctypes.c_void_p]),
    "fsdp_step_graph_create": (ctypes.c_int, [ctypes.POINTER(AdamWHParams),
                                              ctypes.POINTER(ctypes.c_void_p)]),
    "fsdp_step_graph_destroy": (None, [ctypes.c_void_p]),
    "fsdp_step_graph_add_gather": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_int32,
                                                  ctypes.POINTER(ctypes.c_void_p)]),
    "fsdp_step_graph_add_adamw": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32,
                                                 ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_int32]),
    "fsdp_step_graph_add_adamw_gather": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p,
                                                        ctypes.POINTER(ctypes.c_void_p),
                                                        ctypes.c_int32, ctypes.c_void_p,
                                                        ctypes.c_void_p, ctypes.c_void_p,
                                                        ctypes.c_void_p, ctypes.c_int32,
                                                        ctypes.c_void_p, ctypes.c_void_p,
                                                        ctypes.POINTER(ctypes.c_void_p)]),
    "fsdp_step_graph_info": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
                                            ctypes.POINTER(ctypes.c_int64)]),
    "fsdp_step_graph_launch": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "fsdp_grad_accumulate": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p),
                                            ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p),
                                            ctypes.c_int32, ctypes.c_void_p]),
    "fsdp_allreduce_avg": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p),
                                          ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p),
                                          ctypes.c_int32, ctypes.c_void_p]),
}


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m fully_sharded_amd._build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise FsdpError(fn, status)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16 bits)")


def _dev(t: torch.Tensor, what: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    """hipStream_t argument: torch's current stream by default; a torch
    stream, or an already converted ctypes.c_void_p, otherwise."""
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, ctypes.c_void_p):
        return stream
    return ctypes.c_void_p(stream.cuda_stream)


class Plan:
    """A unit's sharding plan (host object owning the C plan)."""

    def __init__(self, shapes, R: int, layout):
        if isinstance(layout, str):
            layout = {"per_param": PER_PARAM, "flat": FLAT}[layout]
        shapes = [tuple(int(d) for d in s) for s in shapes]
        nd = (ctypes.c_int32 * len(shapes))(*[len(s) for s in shapes])
        flat = [d for s in shapes for d in s]
        dims = (ctypes.c_int64 * max(1, len(flat)))(*flat)
        h = ctypes.c_void_p()
        _check("fsdp_plan_layout",
               lib().fsdp_plan_layout(len(shapes), nd, dims, int(R), int(layout), ctypes.byref(h)))
        self._h = h
        info = PlanInfo()
        _check("fsdp_plan_get_info", lib().fsdp_plan_get_info(h, ctypes.byref(info)))
        self.shapes = shapes
        self.T = info.numel_full
        self.S = info.shard_numel
        self.R = info.world
        self.n_params = info.n_params
        self.layout = info.layout
        self.n_segments = info.n_segments

    @property
    def handle(self):
        return self._h

    def __del__(self):
        # at interpreter exit the HIP runtime may already be gone: leak then
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None and not sys.is_finalizing():
            _lib.fsdp_plan_destroy(h)
            self._h = None

    def param(self, p: int):
        out = (ctypes.c_int64 * 5)()
        _check("fsdp_plan_param", lib().fsdp_plan_param(self._h, p, out))
        return dict(flat_off=out[0], numel=out[1], shard_off=out[2], rows_per_shard=out[3],
                    row_numel=out[4])

    def rank_valid(self, r: int) -> int:
        v = ctypes.c_int64()
        _check("fsdp_plan_rank_valid", lib().fsdp_plan_rank_valid(self._h, r, ctypes.byref(v)))
        return v.value

    def segments(self):
        out = (ctypes.c_int64 * (4 * max(1, self.n_segments)))()
        _check("fsdp_plan_segments", lib().fsdp_plan_segments(self._h, out, self.n_segments))
        return [tuple(out[4 * i:4 * i + 4]) for i in range(self.n_segments)]

    def comm_ledger(self, reshard_after_forward: bool = True):
        out = (ctypes.c_int64 * 4)()
        _check("fsdp_plan_comm_ledger",
               lib().fsdp_plan_comm_ledger(self._h, int(bool(reshard_after_forward)), out))
        return dict(all_gather=out[0], reduce_scatter=out[1], optimizer=out[2], total=out[3])

    def state_bytes_per_rank(self) -> int:
        return lib().fsdp_plan_state_bytes_per_rank(self._h)

    def prepare(self, stream=None):
        _check("fsdp_plan_prepare", lib().fsdp_plan_prepare(self._h, _stream(stream)))

    def work_items(self, space: int):
        """Host copy of the per-workgroup work items: list of (dst, src, len);
        space 0 = shard space, 1 = flat space."""
        return _items(lambda out, cap, n: lib().fsdp_plan_work_items(self._h, space, out, cap, n),
                      "fsdp_plan_work_items")

    def unflatten(self, full: torch.Tensor):
        """Per-parameter views of a full-unit buffer [T] (no copy)."""
        views = []
        for p, shape in enumerate(self.shapes):
            q = self.param(p)
            views.append(full[q["flat_off"]:q["flat_off"] + q["numel"]].view(shape))
        return views


def _items(call, name):
    n = ctypes.c_int64()
    _check(name, call(None, 0, ctypes.byref(n)))
    out = (ctypes.c_int64 * (3 * max(1, n.value)))()
    _check(name, call(out, n.value, ctypes.byref(n)))
    return [tuple(out[3 * i:3 * i + 3]) for i in range(n.value)]


class Resharder:
    """Re-sharding of one unit from plan `src` to plan `dst` (other R and/or
    layout, same parameter shapes)."""

    def __init__(self, src: Plan, dst: Plan):
        h = ctypes.c_void_p()
        _check("fsdp_reshard_plan", lib().fsdp_reshard_plan(src.handle, dst.handle,
                                                            ctypes.byref(h)))
        self._h = h
        self.src_plan = src
        self.dst_plan = dst

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None and not sys.is_finalizing():
            _lib.fsdp_reshard_destroy(h)
            self._h = None

    def work_items(self):
        return _items(lambda out, cap, n: lib().fsdp_reshard_items(self._h, out, cap, n),
                      "fsdp_reshard_items")


def fsdp_reshard_plan(src: Plan, dst: Plan) -> Resharder:
    return Resharder(src, dst)


def fsdp_reshard(rs: Resharder, src: torch.Tensor, dst: torch.Tensor, stream=None):
    """src [R_from, S_from] -> dst [R_to, S_to], same dtype, bits copied."""
    if src.numel() != rs.src_plan.R * rs.src_plan.S or dst.numel() != rs.dst_plan.R * rs.dst_plan.S:
        raise ValueError("size mismatch with the plans")
    if _dtype_code(src) != _dtype_code(dst):
        raise ValueError("src and dst dtypes differ")
    _check("fsdp_reshard", lib().fsdp_reshard(rs.handle, _dev(src, "src"), _dev(dst, "dst"),
                                              _dtype_code(src), _stream(stream)))


def fsdp_reshard_batch(rs: Resharder, srcs, dsts, stream=None):
    """dsts[i] = reshard of srcs[i] for up to 64 same-dtype arrays, one launch."""
    if len(srcs) != len(dsts) or not srcs:
        raise ValueError("need as many destinations as sources")
    dt = _dtype_code(srcs[0])
    for a, b in zip(srcs, dsts):
        if a.numel() != rs.src_plan.R * rs.src_plan.S or b.numel() != rs.dst_plan.R * rs.dst_plan.S:
            raise ValueError("size mismatch with the plans")
        if _dtype_code(a) != dt or _dtype_code(b) != dt:
            raise ValueError("all arrays must have one dtype")
    _check("fsdp_reshard_batch",
           lib().fsdp_reshard_batch(rs.handle, len(srcs), _ptr_array(srcs, "srcs"),
                                    _ptr_array(dsts, "dsts"), dt, _stream(stream)))


def fsdp_grad_accumulate(plan: Plan, grads, acc, first: bool, stream=None):
    """acc[r] = grads[r] (first) or acc[r] + grads[r], fp32, over the unit."""
    if len(grads) != plan.R or len(acc) != plan.R:
        raise ValueError("need R gradients and R accumulators")
    dt = _dtype_code(grads[0])
    for g, a in zip(grads, acc):
        if g.numel() != plan.T or _dtype_code(g) != dt or a.numel() != plan.T \
                or a.dtype != torch.float32:
            raise ValueError("gradient or accumulator size/dtype mismatch")
    _check("fsdp_grad_accumulate",
           lib().fsdp_grad_accumulate(plan.handle, _ptr_array(grads, "grads"), dt,
                                      _ptr_array(acc, "acc"), int(bool(first)), _stream(stream)))


def fsdp_allreduce_avg(plan: Plan, grads, out, stream=None):
    """out[r] = rank-order mean of the R full-unit gradients, for every r."""
    if len(grads) != plan.R or len(out) != plan.R:
        raise ValueError("need R gradients and R outputs")
    dt = _dtype_code(grads[0])
    odt = _dtype_code(out[0])
    for g, o in zip(grads, out):
        if g.numel() != plan.T or _dtype_code(g) != dt or o.numel() != plan.T \
                or _dtype_code(o) != odt:
            raise ValueError("gradient or output size/dtype mismatch")
    _check("fsdp_allreduce_avg",
           lib().fsdp_allreduce_avg(plan.handle, _ptr_array(grads, "grads"), dt,
                                    _ptr_array(out, "out"), odt, _stream(stream)))


def fsdp_plan_layout(shapes, R: int, layout) -> Plan:
    return Plan(shapes, R, layout)


def _ptr_array(tensors, what):
    arr = (ctypes.c_void_p * len(tensors))()
    for i, t in enumerate(tensors):
        arr[i] = None if t is None else _dev(t, f"{what}[{i}]")
    return arr


def fsdp_shard_pack(plan: Plan, full: torch.Tensor, shards: torch.Tensor, stream=None):
    """full [T] -> shards [R, S] (same dtype: exact copy; f32 -> bf16: RNE)."""
    if full.numel() != plan.T or shards.numel() != plan.R * plan.S:
        raise ValueError("size mismatch with the plan")
    _check("fsdp_shard_pack",
           lib().fsdp_shard_pack(plan.handle, _dev(full, "full"), _dtype_code(full),
                                 _dev(shards, "shards"), _dtype_code(shards), _stream(stream)))


def fsdp_gather_unflatten(plan: Plan, shards: torch.Tensor, full_out, stream=None):
    """shards [R, S] -> R full-unit buffers (a list of R tensors of at least T
    elements, the first T written, or None to skip a receiver)."""
    _check_gather_args(plan, shards, full_out)
    arr = _ptr_array(full_out, "full_out")
    _check("fsdp_gather_unflatten",
           lib().fsdp_gather_unflatten(plan.handle, _dev(shards, "shards"), _dtype_code(shards),
                                       arr, _stream(stream)))


def fsdp_reduce_scatter_avg(plan: Plan, grads, out: torch.Tensor, stream=None):
    """R per-rank full-unit grads [T] -> averaged fp32 shards out [R, S]."""
    if len(grads) != plan.R or out.numel() != plan.R * plan.S or out.dtype != torch.float32:
        raise ValueError("size or dtype mismatch with the plan")
    dt = _dtype_code(grads[0])
    for g in grads:
        if g.numel() != plan.T or _dtype_code(g) != dt:
            raise ValueError("gradient size or dtype mismatch")
    arr = _ptr_array(grads, "grads")
    _check("fsdp_reduce_scatter_avg",
           lib().fsdp_reduce_scatter_avg(plan.handle, arr, dt, _dev(out, "out"), _stream(stream)))


def _adamw_args(plan: Plan, grads, master, m, v, param_out, grads_are_replicas):
    n = plan.R * plan.S
    for t, nm in ((master, "master"), (m, "m"), (v, "v")):
        if t.numel() != n or t.dtype != torch.float32:
            raise ValueError(f"{nm} must be fp32 with R*S elements")
    if param_out.numel() != n:
        raise ValueError("param_out must have R*S elements")
    if grads_are_replicas:
        if len(grads) != plan.R:
            raise ValueError("need R gradient replicas")
        dt = _dtype_code(grads[0])
        for g in grads:
            if g.numel() != plan.T or _dtype_code(g) != dt:
                raise ValueError("gradient size or dtype mismatch")
    else:
        if isinstance(grads, torch.Tensor):
            grads = [grads]
        if grads[0].numel() != n or grads[0].dtype != torch.float32:
            raise ValueError("reduced gradient must be fp32 [R, S]")
        dt = F32
    return _ptr_array(grads, "grads"), dt


def fsdp_adamw_shard_step(plan: Plan, hp: dict, step: int, grads, master, m, v, param_out,
                          grads_are_replicas: bool = True, stream=None):
    """AdamW on the [R, S] fp32 shards (in place) + recast into param_out.

    grads: list of R full-unit replicas [T] (fused reduce-scatter-average) or,
    with grads_are_replicas=False, one fp32 [R, S] tensor (or a 1-list)."""
    arr, dt = _adamw_args(plan, grads, master, m, v, param_out, grads_are_replicas)
    h = AdamWHParams(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"])
    _check("fsdp_adamw_shard_step",
           lib().fsdp_adamw_shard_step(plan.handle, ctypes.byref(h), int(step), arr, dt,
                                       int(bool(grads_are_replicas)), _dev(master, "master"),
                                       _dev(m, "m"), _dev(v, "v"), _dev(param_out, "param_out"),
                                       _dtype_code(param_out), _stream(stream)))


def fsdp_adamw_shard_step_noalloc(plan: Plan, hp: dict, step: int, grads, master, m, v,
                                  param_out, grads_are_replicas: bool = True, stream=None):
    """fsdp_adamw_shard_step through the entry point that allocates no device
    memory (the plan's work table goes to the library's static buffer)."""
    arr, dt = _adamw_args(plan, grads, master, m, v, param_out, grads_are_replicas)
    h = AdamWHParams(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"])
    _check("fsdp_adamw_shard_step_noalloc",
           lib().fsdp_adamw_shard_step_noalloc(plan.handle, ctypes.byref(h), int(step), arr, dt,
                                               int(bool(grads_are_replicas)),
                                               _dev(master, "master"), _dev(m, "m"),
                                               _dev(v, "v"), _dev(param_out, "param_out"),
                                               _dtype_code(param_out), _stream(stream)))


class BoundCall:
    """A library call with its pointer arguments marshalled once.

    For hot loops: the tensors are checked and their pointers cached at
    construction; calling the object only passes the cached arguments (plus
    the current stream and, for AdamW, the step) to the library."""

    def __init__(self, fn_name, args, keep):
        self._fn = getattr(lib(), fn_name)
        self._name = fn_name
        self._args = args
        self._keep = keep   # tensors whose memory the cached pointers refer to

    def _run(self, *args):
        _check(self._name, self._fn(*args))


def bind_gather_unflatten(plan: Plan, shards: torch.Tensor, full_out) -> "BoundCall":
    """fsdp_gather_unflatten with cached arguments; call as f(stream=None)."""
    _check_gather_args(plan, shards, full_out)
    arr = _ptr_array(full_out, "full_out")
    call = BoundCall("fsdp_gather_unflatten",
                     (plan.handle, ctypes.c_void_p(_dev(shards, "shards")),
                      _dtype_code(shards), arr), (plan, shards, list(full_out)))

    def run(stream=None):
        call._run(*call._args, _stream(stream))
    run.call = call
    return run


def bind_adamw_shard_step(plan: Plan, hp: dict, grads, master, m, v, param_out,
                          grads_are_replicas: bool = True):
    """fsdp_adamw_shard_step with cached arguments; call as
    f(step, stream=None).  grads: R gradient replicas (fused with the
    reduce-scatter), or with grads_are_replicas=False one fp32 [R*S] tensor
    (the reduce-scatter's output)."""
    n = plan.R * plan.S
    for t, nm in ((master, "master"), (m, "m"), (v, "v")):
        if t.numel() != n or t.dtype != torch.float32:
            raise ValueError(f"{nm} must be fp32 with R*S elements")
    if grads_are_replicas:
        if param_out.numel() != n or len(grads) != plan.R:
            raise ValueError("size mismatch with the plan")
        dt = _dtype_code(grads[0])
        for g in grads:
            if g.numel() != plan.T or _dtype_code(g) != dt:
                raise ValueError("gradient size or dtype mismatch")
        keep_g = list(grads)
    else:
        if param_out.numel() != n or grads.numel() != n or grads.dtype != torch.float32:
            raise ValueError("the reduced gradient must be fp32 with R*S elements")
        dt = F32
        keep_g = [grads]
    arr = _ptr_array(keep_g, "grads")
    h = AdamWHParams(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"])
    head = (plan.handle, ctypes.byref(h))
    tail = (arr, dt, int(bool(grads_are_replicas)), ctypes.c_void_p(_dev(master, "master")),
            ctypes.c_void_p(_dev(m, "m")), ctypes.c_void_p(_dev(v, "v")),
            ctypes.c_void_p(_dev(param_out, "param_out")), _dtype_code(param_out))
    call = BoundCall("fsdp_adamw_shard_step", None,
                     (plan, h, keep_g, master, m, v, param_out))

    def run(step, stream=None):
        call._run(*head, int(step), *tail, _stream(stream))
    run.call = call
    return run


def _check_step_args(plan: Plan, grads, master, m, v, param_out):
    n = plan.R * plan.S
    for t, nm in ((master, "master"), (m, "m"), (v, "v")):
        if t.numel() != n or t.dtype != torch.float32:
            raise ValueError(f"{nm} must be fp32 with R*S elements")
    if param_out.numel() != n or len(grads) != plan.R:
        raise ValueError("size mismatch with the plan")
    dt = _dtype_code(grads[0])
    for g in grads:
        if g.numel() != plan.T or _dtype_code(g) != dt:
            raise ValueError("gradient size or dtype mismatch")
    return dt


def _check_gather_args(plan: Plan, shards, full_out):
    if shards.numel() != plan.R * plan.S or len(full_out) != plan.R:
        raise ValueError("size mismatch with the plan")
    for t in full_out:
        if t is not None and (t.numel() < plan.T or t.dtype != shards.dtype):
            raise ValueError("receiver size or dtype mismatch")


def fsdp_adamw_step_then_gather(plan: Plan, hp: dict, step: int, grads, master, m, v, param_out,
                                next_plan: Plan, next_shards, full_out, stream=None):
    """The fused AdamW step of one unit, then the gather of the next unit's
    shards into full_out (one launch for short steps)."""
    bind_adamw_step_then_gather(plan, hp, grads, master, m, v, param_out, next_plan,
                                next_shards, full_out)(step, stream)


def bind_adamw_step_then_gather(plan: Plan, hp: dict, grads, master, m, v, param_out,
                                next_plan: Plan, next_shards, full_out):
    """fsdp_adamw_step_then_gather with cached arguments; call as
    f(step, stream=None)."""
    dt = _check_step_args(plan, grads, master, m, v, param_out)
    _check_gather_args(next_plan, next_shards, full_out)
    if next_shards.dtype != param_out.dtype:
        raise ValueError("the next unit's shards must have the parameter dtype")
    h = AdamWHParams(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"])
    head = (plan.handle, ctypes.byref(h))
    tail = (_ptr_array(grads, "grads"), dt, ctypes.c_void_p(_dev(master, "master")),
            ctypes.c_void_p(_dev(m, "m")), ctypes.c_void_p(_dev(v, "v")),
            ctypes.c_void_p(_dev(param_out, "param_out")), _dtype_code(param_out),
            next_plan.handle, ctypes.c_void_p(_dev(next_shards, "next_shards")),
            _ptr_array(full_out, "full_out"))
    call = BoundCall("fsdp_adamw_step_then_gather", None,
                     (plan, h, list(grads), master, m, v, param_out, next_plan, next_shards,
                      list(full_out)))

    def run(step, stream=None):
        call._run(*head, int(step), *tail, _stream(stream))
    run.call = call
    return run


def bind_reduce_scatter_avg(plan: Plan, grads, out: torch.Tensor):
    """fsdp_reduce_scatter_avg with cached arguments; call as f(stream=None)."""
    if len(grads) != plan.R or out.numel() != plan.R * plan.S or out.dtype != torch.float32:
        raise ValueError("need R gradients and an fp32 [R*S] output")
    dt = _dtype_code(grads[0])
    for g in grads:
        if g.numel() != plan.T or _dtype_code(g) != dt:
            raise ValueError("gradient size or dtype mismatch")
    arr = _ptr_array(grads, "grads")
    o = ctypes.c_void_p(_dev(out, "out"))
    call = BoundCall("fsdp_reduce_scatter_avg", None, (plan, list(grads), out))

    def run(stream=None):
        call._run(plan.handle, arr, dt, o, _stream(stream))
    run.call = call
    return run


def bind_shard_pack(plan: Plan, full: torch.Tensor, shards: torch.Tensor):
    """fsdp_shard_pack with cached arguments; call as f(stream=None)."""
    if full.numel() != plan.T or shards.numel() != plan.R * plan.S:
        raise ValueError("size mismatch with the plan")
    args = (plan.handle, ctypes.c_void_p(_dev(full, "full")), _dtype_code(full),
            ctypes.c_void_p(_dev(shards, "shards")), _dtype_code(shards))
    call = BoundCall("fsdp_shard_pack", None, (plan, full, shards))

    def run(stream=None):
        call._run(*args, _stream(stream))
    run.call = call
    return run


def bind_grad_accumulate(plan: Plan, grads, acc):
    """fsdp_grad_accumulate with cached arguments; call as f(first, stream=None)."""
    if len(grads) != plan.R or len(acc) != plan.R:
        raise ValueError("need R gradients and R accumulators")
    dt = _dtype_code(grads[0])
    for g, a in zip(grads, acc):
        if g.numel() != plan.T or _dtype_code(g) != dt or a.numel() != plan.T \
                or a.dtype != torch.float32:
            raise ValueError("gradient or accumulator size/dtype mismatch")
    ga = _ptr_array(grads, "grads")
    aa = _ptr_array(acc, "acc")
    call = BoundCall("fsdp_grad_accumulate", None, (plan, list(grads), list(acc)))

    def run(first, stream=None):
        call._run(plan.handle, ga, dt, aa, int(bool(first)), _stream(stream))
    run.call = call
    return run


class StepGraph:
    """fsdp_step_graph_*: a unit loop's gathers and AdamW steps recorded once
    and replayed per training step with one graph launch.

    The graph keeps the device pointers of every tensor added; this object
    holds references to them (and to the plans) so they stay alive."""

    def __init__(self, hp: dict):
        self._h = AdamWHParams(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                               hp["weight_decay"])
        h = ctypes.c_void_p()
        _check("fsdp_step_graph_create", lib().fsdp_step_graph_create(ctypes.byref(self._h),
                                                                       ctypes.byref(h)))
        self._handle = h
        self._keep = []

    @property
    def handle(self):
        return self._handle

    def __del__(self):
        h = getattr(self, "_handle", None)
        if h and h.value and _lib is not None and not sys.is_finalizing():
            _lib.fsdp_step_graph_destroy(h)
            self._handle = None

    def add_gather(self, plan: Plan, shards: torch.Tensor, full_out):
        """Record fsdp_gather_unflatten(plan, shards, full_out)."""
        _check_gather_args(plan, shards, full_out)
        _check("fsdp_step_graph_add_gather",
               lib().fsdp_step_graph_add_gather(self._handle, plan.handle,
                                                ctypes.c_void_p(_dev(shards, "shards")),
                                                _dtype_code(shards),
                                                _ptr_array(full_out, "full_out")))
        self._keep.append((plan, shards, list(full_out)))

    def add_adamw(self, plan: Plan, grads, master, m, v, param_out):
        """Record the fused fsdp_adamw_shard_step over R gradient replicas."""
        n = plan.R * plan.S
        for t, nm in ((master, "master"), (m, "m"), (v, "v")):
            if t.numel() != n or t.dtype != torch.float32:
                raise ValueError(f"{nm} must be fp32 with R*S elements")
        if param_out.numel() != n or len(grads) != plan.R:
            raise ValueError("size mismatch with the plan")
        dt = _dtype_code(grads[0])
        for g in grads:
            if g.numel() != plan.T or _dtype_code(g) != dt:
                raise ValueError("gradient size or dtype mismatch")
        _check("fsdp_step_graph_add_adamw",
               lib().fsdp_step_graph_add_adamw(
                   self._handle, plan.handle, _ptr_array(grads, "grads"), dt, 1,
                   ctypes.c_void_p(_dev(master, "master")), ctypes.c_void_p(_dev(m, "m")),
                   ctypes.c_void_p(_dev(v, "v")), ctypes.c_void_p(_dev(param_out, "param_out")),
                   _dtype_code(param_out)))
        self._keep.append((plan, list(grads), master, m, v, param_out))

    def add_adamw_gather(self, plan: Plan, grads, master, m, v, param_out, next_plan: Plan,
                         next_shards, full_out):
        """Record fsdp_adamw_step_then_gather: this unit's fused step with the
        next unit's gather."""
        dt = _check_step_args(plan, grads, master, m, v, param_out)
        _check_gather_args(next_plan, next_shards, full_out)
        if next_shards.dtype != param_out.dtype:
            raise ValueError("the next unit's shards must have the parameter dtype")
        _check("fsdp_step_graph_add_adamw_gather",
               lib().fsdp_step_graph_add_adamw_gather(
                   self._handle, plan.handle, _ptr_array(grads, "grads"), dt,
                   ctypes.c_void_p(_dev(master, "master")), ctypes.c_void_p(_dev(m, "m")),
                   ctypes.c_void_p(_dev(v, "v")), ctypes.c_void_p(_dev(param_out, "param_out")),
                   _dtype_code(param_out), next_plan.handle,
                   ctypes.c_void_p(_dev(next_shards, "next_shards")),
                   _ptr_array(full_out, "full_out")))
        self._keep.append((plan, list(grads), master, m, v, param_out, next_plan, next_shards,
                           list(full_out)))

    def info(self):
        """(kernel nodes, AdamW steps) recorded so far."""
        a, b = ctypes.c_int64(), ctypes.c_int64()
        _check("fsdp_step_graph_info",
               lib().fsdp_step_graph_info(self._handle, ctypes.byref(a), ctypes.byref(b)))
        return a.value, b.value

    def launch(self, step: int, stream=None):
        """Replay every recorded call with AdamW step counter `step`."""
        _check("fsdp_step_graph_launch",
               lib().fsdp_step_graph_launch(self._handle, int(step), _stream(stream)))
