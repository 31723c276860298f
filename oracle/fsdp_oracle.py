"""Plain CPU oracle for the FSDP data-parallel hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module.  It shares no
code with the HIP library and the library never calls it.

It computes, slowly and in the order the pages describe, what one FSDP unit
goes through in a training step with R ranks:

  plan_layout         which rank owns which elements (FSDP2 per-parameter
                      dim-0 split, or FSDP1 padded FlatParameter)
  shard_pack          full tensors -> per-rank shards
  gather_unflatten    per-rank shards -> full tensors (the all-gather)
  reduce_scatter_avg  R full per-rank gradients -> each rank's averaged slice
  adamw_step          AdamW on each rank's fp32 master / m / v shard
  bf16_rne            the bf16 recast of the updated master
  comm_ledger, ...    the per-rank communication and memory accounting
  reshard             shards under one plan -> shards under another world
                      size or layout (restoring at another world size)
  grad_accumulate     one rank's gradient summed over micro-batches
  allreduce_avg       DDP's averaged all-reduce (the comparator)

Sources (pages, by title and section):
  [WALK]  "FSDP Training Step Walkthrough" (astro-wiki): Setup, Initial state,
          Step 1.1 all-gather, Step 4.4 reduce-scatter, Step 6 optimizer
          update, and the one-step communication summary table.
  [FSDP2] "FSDP2 parameter all-gather, gradient reduce-scatter and memory peak"
          (zwjcode): sections 01 (memory formulas), 03 (two-rank, 8-element
          hand calculation), 04 (AdamW over the shards), 06 (reshard after
          forward), 08 (gradient accumulation), 09 (reduce-scatter = reduce
          then hand segment r to rank r; all-reduce for DDP), 10 (restore at
          another world size), 16 (exercises).
  [TINY]  "Understanding FSDP from source" (roger-lv, on Tiny-FSDP): 2.1
          intra-tensor dim-0 partition with a rounded-up shard size, 2.2
          gather (all-gather then concatenate non-empty shards along dim 0),
          2.3 reduce-scatter, 2.4 optimizer state shaped like the shard, 3.2
          the 16P/N memory account.
  [BLOCK] "FSDP Transformer Block Sharding Example" (astro-wiki): 4-GPU
          layout (FSDP2 per-parameter table, FSDP1 FlatParameter offsets),
          all-gather mechanics and per-GPU send volume, FSDP1 unflatten,
          backward reduce-scatter to averages, FSDP2 mixed-precision policy
          (bf16 params, fp32 reduction).

Readings taken where the pages are silent or disagree (each is repeated in
the design notes):
  * shards are zero-padded to one common length S per rank (FSDP1's even
    split; FSDP2 per-parameter pieces padded to ceil(d0/R) rows each);
  * a rank's shard buffer holds its per-parameter pieces in parameter order;
  * the reduce-scatter averages (the walkthroughs divide by the rank count;
    Tiny-FSDP's snippet sums), computed as an fp32 sum in rank order 0..R-1
    starting from rank 0's value, then one correctly rounded division by R;
  * AdamW is the textbook decoupled-weight-decay form with bias correction
    (the pages name torch.optim.AdamW but never print its update); evaluated
    here in float64 from the fp32 state, each result rounded once to fp32;
  * the bf16 recast rounds to nearest, ties to even; NaN stays NaN.

Floating point: the reduction is fp32 because the pages fix the reduction
dtype to float32 ([BLOCK], FSDP2 mixed-precision policy); AdamW is float64.
bf16 values are held as their uint16 bit patterns.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PER_PARAM = "per_param"
FLAT = "flat"


# --------------------------------------------------------------------- layout
@dataclass
class Plan:
    """Shapes-only sharding plan of one FSDP unit over R ranks."""
    shapes: list
    R: int
    layout: str
    numel: list = field(default_factory=list)      # per parameter
    d0: list = field(default_factory=list)         # rows (dim 0)
    row: list = field(default_factory=list)        # elements per row
    flat_off: list = field(default_factory=list)   # offset in the full-unit buffer
    k: list = field(default_factory=list)          # rows per shard (per-param layout)
    shard_off: list = field(default_factory=list)  # offset inside a rank's shard
    T: int = 0                                     # valid elements of the unit
    S: int = 0                                     # shard length incl. padding

    def pieces(self, r):
        """Rank r's pieces as (flat_start, shard_start, length) triples.

        Everything in [0, S) not covered by a piece is padding."""
        out = []
        if self.layout == PER_PARAM:
            for p in range(len(self.shapes)):
                lo = min(r * self.k[p], self.d0[p])
                hi = min(lo + self.k[p], self.d0[p])
                n = (hi - lo) * self.row[p]
                out.append((self.flat_off[p] + lo * self.row[p],
                            self.shard_off[p], n))
        else:
            lo = min(r * self.S, self.T)
            hi = min(lo + self.S, self.T)
            out.append((lo, 0, hi - lo))
        return out


def plan_layout(shapes, R: int, layout: str) -> Plan:
    """The shapes-only plan ([TINY] 2.1 and 4.1; [BLOCK] 4-GPU layout).

    FSDP2 per-parameter: every parameter is split along dim 0 into shards of
    ceil(d0 / R) rows; rank r owns rows [r*k, min(r*k + k, d0)), an empty
    range once r*k reaches d0 ([TINY] 2.1 partition).  Its piece of every
    parameter is stored, padded to k rows, one after the other in parameter
    order, so S = sum_p k_p * row_p.

    FSDP1 FlatParameter: the parameters are flattened and concatenated in
    order into one buffer of T elements, split evenly into R pieces of
    S = ceil(T / R); rank r owns [r*S, min((r+1)*S, T)) ([BLOCK] FSDP1).
    """
    if R < 1:
        raise ValueError("R must be >= 1")
    if layout not in (PER_PARAM, FLAT):
        raise ValueError(layout)
    pl = Plan(shapes=[tuple(int(d) for d in s) for s in shapes], R=R, layout=layout)
    off = 0
    soff = 0
    for shape in pl.shapes:
        if len(shape) < 1 or any(d <= 0 for d in shape):
            raise ValueError(f"bad shape {shape}")
        n = 1
        for d in shape:
            n *= d
        d0 = shape[0]
        row = n // d0
        k = (d0 + R - 1) // R          # shard size rounded up
        pl.numel.append(n)
        pl.d0.append(d0)
        pl.row.append(row)
        pl.flat_off.append(off)
        pl.k.append(k)
        pl.shard_off.append(soff)
        off += n
        soff += k * row
    pl.T = off
    pl.S = soff if layout == PER_PARAM else (off + R - 1) // R
    return pl


def rank_valid(pl: Plan, r: int) -> int:
    return sum(n for _, _, n in pl.pieces(r))


# ------------------------------------------------------------- pack / gather
def shard_pack(pl: Plan, full: np.ndarray) -> np.ndarray:
    """Full-unit buffer [T] -> shards [R, S], padding +0, dtype unchanged.

    Each rank slices its own rows out of the full tensor ([TINY] 2.1 and 4.2,
    slice own shard after the broadcast); FSDP1 slices the FlatParameter
    ([BLOCK] FSDP1)."""
    assert full.ndim == 1 and full.size == pl.T
    shards = np.zeros((pl.R, pl.S), dtype=full.dtype)
    if pl.layout == PER_PARAM:
        for p in range(len(pl.shapes)):
            W = full[pl.flat_off[p]:pl.flat_off[p] + pl.numel[p]].reshape(pl.d0[p], pl.row[p])
            for r in range(pl.R):
                lo = min(r * pl.k[p], pl.d0[p])
                hi = min(lo + pl.k[p], pl.d0[p])
                piece = W[lo:hi].reshape(-1)
                shards[r, pl.shard_off[p]:pl.shard_off[p] + piece.size] = piece
    else:
        for r in range(pl.R):
            lo = min(r * pl.S, pl.T)
            hi = min(lo + pl.S, pl.T)
            shards[r, :hi - lo] = full[lo:hi]
    return shards


def gather_unflatten(pl: Plan, shards: np.ndarray):
    """Shards [R, S] -> (full-unit buffer [T], list of per-parameter views).

    FSDP2: for every parameter, all ranks' row blocks are gathered and the
    non-empty ones concatenated along dim 0 in rank order ([TINY] 2.2
    gather).  FSDP1: the ranks' FlatParameter pieces are concatenated, then
    unflattened into views with the original shapes ([BLOCK] FSDP1
    all-gather).  Every rank receives this same full buffer."""
    assert shards.shape == (pl.R, pl.S)
    if pl.layout == PER_PARAM:
        parts = []
        for p in range(len(pl.shapes)):
            blocks = []
            for r in range(pl.R):
                lo = min(r * pl.k[p], pl.d0[p])
                hi = min(lo + pl.k[p], pl.d0[p])
                n = (hi - lo) * pl.row[p]
                blocks.append(shards[r, pl.shard_off[p]:pl.shard_off[p] + n]
                              .reshape(hi - lo, pl.row[p]))
            valid = [b for b in blocks if b.size > 0]
            parts.append(np.concatenate(valid, axis=0).reshape(-1))
        full = np.concatenate(parts) if parts else shards[:0, 0]
    else:
        full = np.concatenate([shards[r, :rank_valid(pl, r)] for r in range(pl.R)])
    views = [full[pl.flat_off[p]:pl.flat_off[p] + pl.numel[p]].reshape(pl.shapes[p])
             for p in range(len(pl.shapes))]
    return full, views


# -------------------------------------------------------------- precision
def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """bf16 bits -> fp32 (exact: the bf16 bits are the fp32 high half)."""
    return (u16.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest with ties to even.

    The low 16 bits are dropped; the result is rounded up when they exceed
    half of the last kept bit, or equal it and the kept part is odd.  Values
    past the largest bf16 round to infinity; NaN stays NaN (sign kept, quiet
    bit set)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    hi = u >> np.uint32(16)
    lo = u & np.uint32(0xFFFF)
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & np.uint32(1)) == 1))
    r = hi + up.astype(np.uint32)
    nan = np.isnan(x)
    r = np.where(nan, hi | np.uint32(0x0040), r)
    return r.astype(np.uint16)


def _as_f32(g: np.ndarray) -> np.ndarray:
    return bf16_to_f32(g) if g.dtype == np.uint16 else g.astype(np.float32, copy=False)


# ------------------------------------------------------------ reduce-scatter
def reduce_scatter_avg(pl: Plan, grads) -> np.ndarray:
    """R per-rank full-unit gradients [T] -> averaged shards [R, S] (fp32).

    Rank r keeps reduce(g_0[slice r], ..., g_{R-1}[slice r]) ([FSDP2] 03;
    [WALK] step 4.4 (g0 + g1) / 2; [BLOCK] backward: avg).  The reduction
    runs in fp32 ([BLOCK] mixed precision, reduce dtype float32): the sum is
    taken in rank order starting from rank 0's value, then divided by R.
    bf16 gradients (uint16 bits) are widened exactly.  Padding is +0."""
    assert len(grads) == pl.R
    out = np.zeros((pl.R, pl.S), np.float32)
    for r in range(pl.R):
        for f0, s0, n in pl.pieces(r):
            out[r, s0:s0 + n] = rank_order_mean([g[f0:f0 + n] for g in grads])
    return out


def rank_order_mean(values) -> np.ndarray:
    """Element-wise fp32 mean of R equally shaped arrays (fp32, or bf16 bits
    widened exactly): acc = v_0; acc = acc + v_q for q = 1..R-1; acc / R.
    The reduction every rank applies to its slice ([WALK] step 4.4)."""
    acc = _as_f32(values[0]).copy()
    for q in range(1, len(values)):
        acc = acc + _as_f32(values[q])
    return acc / np.float32(len(values))


def reduce_scatter_sum(pl: Plan, grads) -> np.ndarray:
    """The SUM variant of Tiny-FSDP's snippet ([TINY] 2.3, op=SUM), fp32,
    rank order; used only to pin the oracle against the SUM/AVG exercise."""
    g32 = [_as_f32(g) for g in grads]
    out = np.zeros((pl.R, pl.S), np.float32)
    for r in range(pl.R):
        for f0, s0, n in pl.pieces(r):
            acc = g32[0][f0:f0 + n].copy()
            for q in range(1, pl.R):
                acc = acc + g32[q][f0:f0 + n]
            out[r, s0:s0 + n] = acc
    return out


# ---------------------------------------------------------------------- AdamW
def adamw_step(master, m, v, g, t: int, lr, beta1, beta2, eps, weight_decay):
    """One AdamW step on fp32 shards, evaluated in float64.

    The pages run torch.optim.AdamW on the local shards, with state shaped
    like the shard and no communication ([FSDP2] 03-04; [TINY] 2.4; [WALK]
    step 6) but do not print the update.  Reading: decoupled weight decay,
    bias-corrected moments, eps added outside the square root:
        p1 = p * (1 - lr*wd)
        m' = b1*m + (1-b1)*g ;  v' = b2*v + (1-b2)*g^2
        p' = p1 - lr * (m'/(1-b1^t)) / (sqrt(v'/(1-b2^t)) + eps)
    Returns fp32 (p', m', v'), each rounded once from float64."""
    if t < 1:
        raise ValueError("step must be >= 1")
    p = np.asarray(master, np.float64)
    m = np.asarray(m, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    p1 = p * (1.0 - lr * weight_decay)
    m1 = beta1 * m + (1.0 - beta1) * g
    v1 = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m1 / (1.0 - beta1 ** t)
    v_hat = v1 / (1.0 - beta2 ** t)
    p2 = p1 - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p2.astype(np.float32), m1.astype(np.float32), v1.astype(np.float32)


def shard_step(pl: Plan, grads, master, m, v, t: int, hp: dict, param_dtype="bf16"):
    """One rank-local step for the whole unit: reduce-scatter-average the R
    per-rank gradients, AdamW on every rank's shard, recast the new master
    to the parameter dtype.  Returns (master', m', v', param')."""
    g = reduce_scatter_avg(pl, grads)
    p2, m2, v2 = adamw_step(master, m, v, g, t, hp["lr"], hp["beta1"], hp["beta2"],
                            hp["eps"], hp["weight_decay"])
    param = bf16_rne(p2) if param_dtype == "bf16" else p2.copy()
    return p2, m2, v2, param


# ------------------------------------------------------------------- ledgers
def comm_ledger(pl: Plan, reshard_after_forward: bool = True) -> dict:
    """Elements each rank sends for one unit in one step.

    All-gather: each rank's shard goes to the other R-1 ranks, (R-1)*S
    elements, once in forward and once more in backward when the full
    parameters were freed after forward ([WALK] summary table; [FSDP2] 06;
    [BLOCK] send volume (N-1)/N of the layer).  Reduce-scatter: (R-1)*S.
    The optimizer step sends nothing."""
    ag = (pl.R - 1) * pl.S
    n_ag = 2 if reshard_after_forward else 1
    return dict(all_gather=n_ag * ag, reduce_scatter=(pl.R - 1) * pl.S,
                optimizer=0, total=n_ag * ag + (pl.R - 1) * pl.S)


def ddp_allreduce_elems(P: int, R: int) -> float:
    """Elements a rank sends in a ring all-reduce of P gradients: 2(R-1)/R*P
    ([WALK] comparison with DDP)."""
    return 2.0 * (R - 1) / R * P


def state_bytes_per_rank(pl: Plan) -> int:
    """Resident bytes per rank for one unit: 16 per shard element (bf16
    param 2 + fp32 master 4 + fp32 m and v 8 + bf16 grad shard 2), the
    16P/N account of [TINY] 3.2 with padding included."""
    return 16 * pl.S


def peak_memory_lower_bound(state_total: float, R: int, largest_group: float,
                            prefetch: float) -> float:
    """M_peak >= M_state/R + largest unsharded group + prefetch buffer
    ([FSDP2] 01, activations and temporaries left out)."""
    return state_total / R + largest_group + prefetch


# ------------------------------------------------------ widening: next rows
def reshard(pl_from: Plan, pl_to: Plan, shards: np.ndarray) -> np.ndarray:
    """Shards of one unit under plan `pl_from` -> the same unit's shards under
    `pl_to` (another world size and/or layout), padding +0, bits unchanged.

    Restoring a checkpoint at a different world size ([FSDP2] 10) needs each
    new rank's shard of the same full tensors; by definition that is the
    all-gather under the old plan followed by the slicing under the new one
    ([TINY] 4.5 gathers full weights to save and re-shards to load)."""
    if pl_from.shapes != pl_to.shapes:
        raise ValueError("plans of different units")
    full, _ = gather_unflatten(pl_from, shards)
    return shard_pack(pl_to, full)


def grad_accumulate(micro_grads) -> np.ndarray:
    """One rank's full-unit gradient summed over K micro-batches in fp32, in
    micro-batch order starting from the first ([FSDP2] 08: every micro-batch
    runs forward and backward and the gradients add up before the update).
    bf16 inputs widen exactly."""
    acc = _as_f32(micro_grads[0]).copy()
    for g in micro_grads[1:]:
        acc = acc + _as_f32(g)
    return acc


def allreduce_avg(grads) -> list:
    """DDP's gradient all-reduce, averaged: every rank receives the rank-order
    fp32 mean of all ranks' full gradients ([WALK] comparison with DDP;
    [FSDP2] 09: the all-reduce gives every card the whole averaged gradient,
    of which the reduce-scatter keeps one slice per rank)."""
    mean = rank_order_mean(grads)
    return [mean.copy() for _ in grads]
