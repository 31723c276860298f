/*
 * fsdp_mi355x.h -- C ABI of the FSDP data-parallel hot path on one MI355X
 * (gfx950), with R virtual ranks held in one GPU's memory.
 *
 * A training step of fully sharded data parallelism, per FSDP unit, is:
 *   all-gather the rank shards into full parameters (forward, and again in
 *   backward), reduce-scatter the per-rank full gradients so that each rank
 *   keeps the average of its own slice, and run AdamW on each rank's shard
 *   with no communication, recasting the fp32 master to the bf16 parameter
 *   that the next all-gather sends.
 * Sources: "FSDP Training Step Walkthrough" (astro-wiki), steps 1-6;
 * "FSDP Transformer Block Sharding Example" (astro-wiki), 4-GPU shard layout,
 * all-gather mechanics, backward reduce-scatter; "Understanding FSDP from
 * source" (roger-lv, on Tiny-FSDP), 2.1-2.4; "FSDP2 parameter all-gather,
 * gradient reduce-scatter and memory peak" (zwjcode), sections 03, 04, 09.
 *
 * Conventions for every call below.
 *   Units and layouts.  A unit is an ordered list of parameters with shapes
 *   shape_p (ndim >= 1, every dim > 0).  Its full-unit buffer holds all
 *   parameters row-major, concatenated in order: T elements, parameter p at
 *   flat offset flat_off_p (the FSDP1 FlatParameter, unpadded).  "Unflatten"
 *   is a view of that buffer: parameter p is [flat_off_p, flat_off_p +
 *   numel_p) reshaped to shape_p.  Rank shards are one buffer [R][S], row r
 *   for rank r, S elements each including zero padding.
 *     FSDP_LAYOUT_PER_PARAM (FSDP2 per-parameter dim-0 sharding): with
 *       k_p = ceil(d0_p / R), rank r owns rows [min(r k_p, d0_p),
 *       min((r+1) k_p, d0_p)) of every parameter; its piece of parameter p
 *       sits at shard offset sum_{q<p} k_q row_q and is padded to k_p row_p
 *       elements, so S = sum_p k_p row_p.
 *     FSDP_LAYOUT_FLAT (FSDP1 FlatParameter): S = ceil(T / R); rank r owns
 *       [r S, min((r+1) S, T)) of the full-unit buffer; the tail is padded.
 *   Memory.  Every buffer argument is device memory owned by the caller,
 *   contiguous, on the current HIP device, aligned at least to its element
 *   size (16-byte alignment is the fast path).  Pointer arrays (grads,
 *   full_out) are host arrays of R device pointers.  The library never
 *   allocates in an operation, except that the first operation using a plan
 *   on a device uploads the plan's work tables there (hipMalloc, owned by
 *   the plan, freed by fsdp_plan_destroy); fsdp_plan_prepare does that
 *   upload ahead of time, e.g. before stream capture.
 *   Placement.  Any placement is correct.  For speed, do not give the
 *   arrays one kernel touches at the same element offset (the R gradient
 *   replicas, master, m, v, the parameter shards) base addresses that agree
 *   modulo a large power of two, as separate 2 MiB-aligned allocations do:
 *   those accesses then meet on the same HBM channels (on MI355X the fused
 *   step lost 3-6%).  Carving the replicas from one buffer, and master, m
 *   and v from another, with row strides that are not multiples of 4 KiB
 *   avoids it.
 *   Execution.  Operations are enqueued on `stream` (a hipStream_t; NULL is
 *   the null stream), asynchronous, in stream order, with no internal
 *   synchronisation.  Calls with the same plan may run concurrently on
 *   different streams.
 *   Errors.  Arguments are checked before anything is launched; on error
 *   nothing is enqueued and the status says why.  FSDP_ERR_HIP reports a
 *   failed launch or upload; faults inside a kernel surface at the caller's
 *   next synchronisation.  No C++ exception crosses this interface.
 *   Precision.  bf16 is stored as 16-bit patterns.  Reductions are fp32
 *   ("FSDP Transformer Block Sharding Example", FSDP2 mixed-precision
 *   policy: bf16 parameters, float32 reduction).  The bf16 recast rounds to
 *   nearest, ties to even.
 */
#ifndef FSDP_MI355X_H
#define FSDP_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fsdp_status {
  FSDP_OK = 0,
  FSDP_ERR_INVALID_ARG = -1,   /* bad pointer, size, dtype, overlap, hparam */
  FSDP_ERR_UNSUPPORTED = -2,   /* valid but not implemented (e.g. R > 64)  */
  FSDP_ERR_OUT_OF_MEMORY = -3, /* host or device table allocation failed   */
  FSDP_ERR_HIP = -4            /* a HIP runtime call or launch failed       */
} fsdp_status;

enum { FSDP_LAYOUT_PER_PARAM = 0, FSDP_LAYOUT_FLAT = 1 };
enum { FSDP_F32 = 0, FSDP_BF16 = 1 };
enum { FSDP_MAX_RANKS = 64 };

typedef struct fsdp_plan fsdp_plan; /* opaque; immutable once created */

typedef struct fsdp_adamw_hparams {
  double lr;            /* >= 0 */
  double beta1, beta2;  /* in [0, 1) */
  double eps;           /* > 0 */
  double weight_decay;  /* >= 0, decoupled: p <- p (1 - lr wd) */
} fsdp_adamw_hparams;

typedef struct fsdp_plan_info {
  int64_t numel_full;  /* T: valid elements of the unit */
  int64_t shard_numel; /* S: per-rank shard length incl. padding */
  int32_t world;       /* R */
  int32_t n_params;
  int32_t layout;      /* FSDP_LAYOUT_* */
  int32_t n_segments;  /* contiguous (rank, shard range, flat range) pieces */
} fsdp_plan_info;

/* Plan the layout of one unit (shapes only, host only, no device work).
 * Shard sizes round up: "Understanding FSDP from source" 2.1 (dim-0
 * partition with ceil shard size) and 4.1 (plan on shapes before
 * materialising); "FSDP Transformer Block Sharding Example", 4-GPU shard
 * layout (FSDP2 table, FSDP1 FlatParameter offsets).
 *   n_params >= 1 parameters; ndims[p] in [1, 8]; dims holds all shapes
 *   concatenated (sum of ndims entries, each > 0); 1 <= R <= 64; layout is
 *   FSDP_LAYOUT_*.  On success *out owns a new plan (free it with
 *   fsdp_plan_destroy); on error *out is set to NULL.  A unit whose work
 *   would not fit one launch's grid (16,777,215 workgroups of 1024
 *   elements: R*S above about 17.2G elements) returns
 *   FSDP_ERR_UNSUPPORTED. */
fsdp_status fsdp_plan_layout(int32_t n_params, const int32_t* ndims, const int64_t* dims,
                             int32_t R, int32_t layout, fsdp_plan** out);

/* Free a plan and its device tables.  No operation using it may still be in
 * flight.  NULL is ignored. */
void fsdp_plan_destroy(fsdp_plan* plan);

/* Plan queries (host only). */
fsdp_status fsdp_plan_get_info(const fsdp_plan* plan, fsdp_plan_info* out);
/* out[5] = {flat_off, numel, shard_off, rows_per_shard, row_numel} of
 * parameter p (rows_per_shard = ceil(d0/R); shard_off and rows_per_shard
 * describe the PER_PARAM layout and are reported for both layouts). */
fsdp_status fsdp_plan_param(const fsdp_plan* plan, int32_t p, int64_t* out);
/* Valid (non-padding) elements held by rank r. */
fsdp_status fsdp_plan_rank_valid(const fsdp_plan* plan, int32_t r, int64_t* valid);
/* The contiguous pieces, ordered by (rank, shard offset): out[4*i..4*i+3] =
 * {rank, shard_off, flat_off, len}.  capacity is the number of rows out can
 * hold and must be >= n_segments. */
fsdp_status fsdp_plan_segments(const fsdp_plan* plan, int64_t* out, int32_t capacity);
/* Elements one rank sends for this unit in one training step: out[4] =
 * {all_gather, reduce_scatter, optimizer (always 0), total}.  Each
 * all-gather sends the rank's shard to R-1 ranks, (R-1) S elements, twice
 * per step when reshard_after_forward != 0 (freed after forward, gathered
 * again in backward), once otherwise; the reduce-scatter sends (R-1) S.
 * "FSDP Training Step Walkthrough", one-step communication summary;
 * "FSDP Transformer Block Sharding Example", all-gather send volume;
 * zwjcode FSDP2 page, section 06. */
fsdp_status fsdp_plan_comm_ledger(const fsdp_plan* plan, int32_t reshard_after_forward,
                                  int64_t* out);
/* Resident bytes per rank for this unit: 16 S (bf16 param, fp32 master, m,
 * v, bf16 grad shard), the 16P/N account of "Understanding FSDP from
 * source" 3.2.  Returns -1 for a NULL plan. */
int64_t fsdp_plan_state_bytes_per_rank(const fsdp_plan* plan);
/* The plan's per-workgroup work items (host copy), for inspection and
 * host-side tests: space 0 = the shard space [0, R*S) used by pack,
 * reduce-scatter and the AdamW step (src = flat index, -1 for padding),
 * space 1 = the flat space [0, T) used by the gather (src = linear shard
 * index).  out[3*i..3*i+2] = {dst, src, len}; with out == NULL only *n is
 * set; otherwise capacity (rows) must be >= the item count. */
fsdp_status fsdp_plan_work_items(const fsdp_plan* plan, int32_t space, int64_t* out,
                                 int64_t capacity, int64_t* n);
/* Upload the plan's work tables to the current device now (synchronous).
 * Optional: operations do it on first use. */
fsdp_status fsdp_plan_prepare(const fsdp_plan* plan, void* stream);

/* Shard (pack): shards[r][j] = full[flat index of (r, j)], padding +0.
 * "Understanding FSDP from source" 4.2 (every rank slices its own shard
 * out of the full initial weight).
 *   full: [T] of full_dtype; shards: [R][S] of shard_dtype.  Same dtypes
 *   copy bits exactly; F32 -> BF16 rounds to nearest even; BF16 -> F32
 *   widens exactly.  full and shards must not overlap. */
fsdp_status fsdp_shard_pack(const fsdp_plan* plan, const void* full, int32_t full_dtype,
                            void* shards, int32_t shard_dtype, void* stream);

/* All-gather + unflatten: every receiver r' gets the whole unit,
 * full_out[r'][flat index of (r, j)] = shards[r][j] for every valid (r, j).
 * "Understanding FSDP from source" 2.2 (gather, concatenate the non-empty
 * shards along dim 0 in rank order); "FSDP Transformer Block Sharding
 * Example", all-gather mechanics and FSDP1 unflatten.
 *   shards: [R][S] of dtype; full_out: host array of R device pointers,
 *   each [T] of dtype, or NULL to skip that receiver.  Receivers must be
 *   distinct and must not overlap the shards or each other.  Bits are
 *   copied exactly. */
fsdp_status fsdp_gather_unflatten(const fsdp_plan* plan, const void* shards, int32_t dtype,
                                  void* const* full_out, void* stream);

/* Reduce-scatter-average: out[r][j] = (sum over q = 0..R-1 of
 * grads[q][flat index of (r, j)]) / R for valid (r, j), padding +0.  The
 * sum is fp32 in rank order starting from rank 0's value, then one
 * correctly rounded division by R; bf16 inputs widen exactly.
 * "FSDP Training Step Walkthrough", step 4.4; zwjcode FSDP2 page, sections
 * 03 and 09; "FSDP Transformer Block Sharding Example", backward
 * reduce-scatter.
 *   grads: host array of R device pointers, each a full-unit gradient [T]
 *   of grad_dtype (rank q's local gradient); out: [R][S] fp32, disjoint
 *   from every grads[q]. */
fsdp_status fsdp_reduce_scatter_avg(const fsdp_plan* plan, const void* const* grads,
                                    int32_t grad_dtype, float* out, void* stream);

/* AdamW on every rank's shard, then the parameter recast.  Per element,
 * with g the rank's averaged gradient and t = step:
 *   p1 = p (1 - lr wd); m' = b1 m + (1-b1) g; v' = b2 v + ((1-b2) g) g;
 *   p' = p1 - (lr (m'/(1-b1^t))) / (sqrt(v'/(1-b2^t)) + eps)
 * evaluated in IEEE double from the fp32 state and gradient, in that order
 * (products and sums left to right, 1-b1^t and 1-b2^t computed once),
 * each of p', m', v' rounded once to fp32; param_out = p' cast to
 * param_dtype.  The pages run
 * torch.optim.AdamW on the local shards with state shaped like the shard
 * and no communication ("FSDP Training Step Walkthrough", step 6; zwjcode
 * FSDP2 page, section 04; "Understanding FSDP from source" 2.4).
 *   grads_are_replicas = 1: grads is R device pointers, each rank's full-
 *     unit gradient [T] of grad_dtype; the reduce-scatter-average above is
 *     fused into the same pass (one read of every replica).
 *   grads_are_replicas = 0: grads[0] is the fp32 [R][S] output of
 *     fsdp_reduce_scatter_avg (grad_dtype must be FSDP_F32).
 *   master, m, v: [R][S] fp32, read and written in place; param_out: [R][S]
 *   of param_dtype.  master, m, v and param_out are pairwise disjoint and
 *   disjoint from the gradients.  step >= 1.  Padding stays +0 (with
 *   m = v = 0 there, eps > 0 keeps the update zero). */
fsdp_status fsdp_adamw_shard_step(const fsdp_plan* plan, const fsdp_adamw_hparams* hp,
                                  int64_t step, const void* const* grads, int32_t grad_dtype,
                                  int32_t grads_are_replicas, float* master, float* m, float* v,
                                  void* param_out, int32_t param_dtype, void* stream);

/* fsdp_adamw_shard_step for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, checks and results (bit for bit); the caller
 * still passes every input and output.  The call allocates nothing: the
 * plan's work table is copied (hipMemcpyAsync from the plan's host table,
 * on `stream`, before the step) into a static device buffer of the library
 * of 1 MiB, one per GPU, held until the process ends, instead of the
 * device copy the plan otherwise allocates on first use.
 *   Limit: with grads_are_replicas = 1 the plan's shard-space table must
 *   hold at most 43,690 work items (fsdp_plan_work_items, space 0: a shard
 *   space R*S of up to about 44.7M elements); larger plans give
 *   FSDP_ERR_UNSUPPORTED, checked before the other arguments.
 *   Every call on one GPU shares that GPU's buffer: calls enqueued on one
 *   stream are ordered, but calls that can overlap in time on one GPU (on
 *   different streams or from different threads) race on it.  Its
 *   contents are the last call's table; nothing in it needs clearing. */
fsdp_status fsdp_adamw_shard_step_noalloc(const fsdp_plan* plan, const fsdp_adamw_hparams* hp,
                                          int64_t step, const void* const* grads,
                                          int32_t grad_dtype, int32_t grads_are_replicas,
                                          float* master, float* m, float* v, void* param_out,
                                          int32_t param_dtype, void* stream);

/* ---- Beyond the per-step path: restore at another world size, gradient
 * accumulation, and the DDP all-reduce the pages compare FSDP with. ---- */

typedef struct fsdp_resharder fsdp_resharder; /* opaque; immutable once created */

/* Plan the re-sharding of one unit from plan `from` to plan `to`: another R
 * and/or the other layout, same parameter shapes (else
 * FSDP_ERR_INVALID_ARG).  Restoring a sharded checkpoint at a different
 * world size needs each new rank's shard of the same full tensors (zwjcode
 * FSDP2 page, section 10; "Understanding FSDP from source" 4.5 gathers the
 * full weights to save and re-shards them to load).  Host only; *out owns a
 * new object, freed by fsdp_reshard_destroy; the plans may be destroyed
 * afterwards.  FSDP_ERR_UNSUPPORTED when the copy would not fit one
 * launch's grid (16,777,215 workgroups of 2048 elements). */
fsdp_status fsdp_reshard_plan(const fsdp_plan* from, const fsdp_plan* to, fsdp_resharder** out);
void fsdp_reshard_destroy(fsdp_resharder* rs);
/* Its work items (host copy), as fsdp_plan_work_items: dst indexes `to`'s
 * [R_to][S_to], src `from`'s [R_from][S_from] (-1: padding). */
fsdp_status fsdp_reshard_items(const fsdp_resharder* rs, int64_t* out, int64_t capacity,
                               int64_t* n);

/* dst = the shards, under `to`, of the unit whose shards under `from` are
 * src: equal to gathering src with `from` and packing with `to`, without
 * materialising the full unit; padding +0, bits copied exactly.
 *   src: [R_from][S_from], dst: [R_to][S_to], both of dtype, disjoint.  Use
 *   it for the bf16 parameter and the fp32 master, m and v alike.  The
 *   first call on a device uploads the work table (as for a plan). */
fsdp_status fsdp_reshard(const fsdp_resharder* rs, const void* src, void* dst, int32_t dtype,
                         void* stream);

/* fsdp_reshard for n independent arrays of one dtype in one launch (e.g.
 * master, m and v of every unit sharing the plans): dst[i] = reshard of
 * src[i].  1 <= n <= 64 (larger n: FSDP_ERR_UNSUPPORTED); destinations
 * pairwise disjoint and disjoint from every source. */
fsdp_status fsdp_reshard_batch(const fsdp_resharder* rs, int32_t n, const void* const* srcs,
                               void* const* dsts, int32_t dtype, void* stream);

/* Gradient accumulation over micro-batches: acc[r][i] = g[r][i] when first
 * != 0, else acc[r][i] + g[r][i], in fp32, for every rank r < R and i < T
 * (zwjcode FSDP2 page, section 08: every micro-batch runs forward and
 * backward and the gradients add up before one update).  The accumulators
 * then feed fsdp_adamw_shard_step as FSDP_F32 replicas (or
 * fsdp_reduce_scatter_avg).
 *   grads: R device pointers, [T] each, of grad_dtype; acc: R device
 *   pointers, fp32 [T] each, pairwise disjoint and disjoint from the grads;
 *   first is 0 or 1 (first = 1 copies, so a -0 gradient stays -0). */
fsdp_status fsdp_grad_accumulate(const fsdp_plan* plan, const void* const* grads,
                                 int32_t grad_dtype, float* const* acc, int32_t first,
                                 void* stream);

/* DDP's averaged all-reduce: out[r][i] = (sum over q = 0..R-1 of
 * grads[q][i]) / R for every receiver r and i < T, with the same fp32
 * rank-order sum and division as fsdp_reduce_scatter_avg ("FSDP Training
 * Step Walkthrough", comparison with DDP; zwjcode FSDP2 page, section 09:
 * the all-reduce gives every card the whole averaged gradient).  out_dtype
 * FSDP_BF16 rounds the fp32 mean to nearest even.
 *   grads: R device pointers, [T] each; out: R device pointers, [T] each of
 *   out_dtype, pairwise disjoint and disjoint from the grads. */
fsdp_status fsdp_allreduce_avg(const fsdp_plan* plan, const void* const* grads,
                               int32_t grad_dtype, void* const* out, int32_t out_dtype,
                               void* stream);

/* The fused AdamW shard step of one unit (fsdp_adamw_shard_step with
 * grads_are_replicas = 1) and the all-gather + unflatten of the next unit's
 * parameter shards (fsdp_gather_unflatten of `next`, elements of
 * param_dtype), enqueued together: FSDP's prefetch, which all-gathers unit
 * k+1 while unit k's gradients are reduce-scattered and its shard updated
 * ("FSDP2 parameter all-gather, gradient reduce-scatter and memory peak",
 * section 07; "Understanding FSDP from source", section 5, overlap of
 * communication and computation).  The results
 * equal the two calls made one after the other.  When the step has at most
 * 65,536 work items (fsdp_plan_work_items, space 0) both run in one kernel
 * launch, the gather's workgroups after the step's, so the gather starts
 * while the step drains; longer steps take two launches.
 *   Arguments as in the two calls; in addition the two must not touch each
 *   other's outputs: full_out must be disjoint from the gradients, master,
 *   m, v and param_out, and param_out, master, m, v from next_shards (else
 *   FSDP_ERR_INVALID_ARG). */
fsdp_status fsdp_adamw_step_then_gather(const fsdp_plan* plan, const fsdp_adamw_hparams* hp,
                                        int64_t step, const void* const* grads,
                                        int32_t grad_dtype, float* master, float* m, float* v,
                                        void* param_out, int32_t param_dtype,
                                        const fsdp_plan* next, const void* next_shards,
                                        void* const* full_out, void* stream);

/* ---------------------------------------------------------------------
 * Step graph: a unit loop recorded once and replayed every step.
 *
 * The per-unit sequence of one training step ("FSDP Training Step
 * Walkthrough", steps 1-6: per unit, gather, then reduce-scatter and the
 * local AdamW step) is the same launches every step; only AdamW's step
 * counter changes.  A step graph records those launches once, as a HIP graph
 * of kernel nodes executed in the order they were added, and
 * fsdp_step_graph_launch replays it for step t with one graph launch.  Each
 * replay computes exactly what the stream calls compute, bit for bit.
 *
 * The graph owns a small device record of AdamW scalars (allocated by
 * fsdp_step_graph_create); every launch first writes step t's record with a
 * one-lane kernel on `stream`, then launches the graph on the same stream.
 * The graph keeps the device pointers it was given: the buffers and plans
 * must stay alive, at the same addresses, until it is destroyed.
 * Operations on one graph must not overlap: launches of one graph go to one
 * stream (or are ordered by the caller), and fsdp_step_graph_destroy
 * requires that no launch of it is still running.
 * --------------------------------------------------------------------- */
typedef struct fsdp_step_graph fsdp_step_graph; /* opaque */

/* An empty step graph on the current device whose AdamW nodes use hp
 * (checked as fsdp_adamw_shard_step checks it).  Allocates the scalar
 * record (FSDP_ERR_OUT_OF_MEMORY if that fails). */
fsdp_status fsdp_step_graph_create(const fsdp_adamw_hparams* hp, fsdp_step_graph** out);

/* Destroys the graph and frees its record.  NULL is ignored. */
void fsdp_step_graph_destroy(fsdp_step_graph* graph);

/* Appends the gather that fsdp_gather_unflatten would enqueue with these
 * arguments (same checks, same errors).  Uploads the plan's work tables
 * if needed.  After the graph's first launch, or on another device than
 * the graph's: FSDP_ERR_INVALID_ARG. */
fsdp_status fsdp_step_graph_add_gather(fsdp_step_graph* graph, const fsdp_plan* plan,
                                       const void* shards, int32_t dtype, void* const* full_out);

/* Appends the AdamW shard step that fsdp_adamw_shard_step would enqueue with
 * these arguments (same checks, same errors), taking its hyper-parameters
 * from the graph and its step counter from each launch. */
fsdp_status fsdp_step_graph_add_adamw(fsdp_step_graph* graph, const fsdp_plan* plan,
                                      const void* const* grads, int32_t grad_dtype,
                                      int32_t grads_are_replicas, float* master, float* m,
                                      float* v, void* param_out, int32_t param_dtype);

/* Appends what fsdp_adamw_step_then_gather would enqueue with these
 * arguments (same checks, same errors): one kernel node holding the step
 * and the next unit's gather, or two nodes for a long step. */
fsdp_status fsdp_step_graph_add_adamw_gather(fsdp_step_graph* graph, const fsdp_plan* plan,
                                             const void* const* grads, int32_t grad_dtype,
                                             float* master, float* m, float* v, void* param_out,
                                             int32_t param_dtype, const fsdp_plan* next,
                                             const void* next_shards, void* const* full_out);

/* Kernel nodes recorded so far, and how many AdamW steps they hold. */
fsdp_status fsdp_step_graph_info(const fsdp_step_graph* graph, int64_t* n_nodes,
                                 int64_t* n_adamw);

/* Runs every recorded operation, in order, with AdamW step counter `step`
 * (>= 1), on `stream`.  The first launch instantiates the graph and seals
 * it (no more nodes).  Must be called on the graph's device.  Consecutive
 * launches may use different streams: a launch on another stream than the
 * previous one first makes its stream wait (on the device, not the host)
 * for the work enqueued so far on the previous launch's stream, which must
 * therefore still exist; both replays use the graph's one record of AdamW
 * scalars.  Launches of one graph from several host threads at once are
 * not supported. */
fsdp_status fsdp_step_graph_launch(fsdp_step_graph* graph, int64_t step, void* stream);

/* Static, human-readable name of a status code (an fsdp_status value; any
 * other number gives "unknown status"). */
const char* fsdp_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* FSDP_MI355X_H */
