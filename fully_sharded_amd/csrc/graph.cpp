// The step graph: a unit loop's gathers and AdamW steps recorded once as a
// HIP graph (one kernel node per call, each depending on the one before) and
// replayed every training step with one hipGraphLaunch.
//
// A replay must run AdamW step t with t's bias corrections, but a graph's
// kernel arguments are fixed.  So the AdamW nodes read their float64
// scalars from a device record the graph owns, and every launch first
// enqueues, on the caller's stream, a one-lane kernel that writes step t's
// record (computed on the host exactly as the stream entry point computes
// it).  Stream order puts that write after the previous replay and before
// this one; a launch on another stream than the previous one first makes
// its stream wait for an event recorded, at that moment, on the previous
// launch's stream (so after that replay), and the write never races a
// replay still reading the record.  Launches on one stream record nothing:
// an event after every replay cost 4-5 us per step on the 12-layer model.
// No node's arguments change after instantiation.
#include <hip/hip_runtime.h>

#include <new>

#include "fsdp_mi355x.h"
#include "kernels.hpp"
#include "ops.hpp"
#include "plan.hpp"

struct fsdp_step_graph {
  int device = -1;
  fsdp_adamw_hparams hp{};
  fsdp::AdamScalars* scalars = nullptr;  // device record read by the AdamW nodes
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;  // instantiated at the first launch
  hipGraphNode_t last = nullptr;
  int64_t n_nodes = 0;
  int64_t n_adamw = 0;
  hipEvent_t replayed = nullptr;       // marks the previous launch's stream
  hipStream_t last_stream = nullptr;   // the stream of the previous launch
  bool launched = false;
};

namespace {

// Appends each launch as a kernel node after the graph's last node.
class GraphSink final : public fsdp::Sink {
 public:
  explicit GraphSink(fsdp_step_graph* g) : g_(g) {}
  hipError_t launch(const void* fn, dim3 grid, dim3 block, void** args,
                    unsigned lds) const override {
    hipKernelNodeParams p{};
    p.func = const_cast<void*>(fn);
    p.gridDim = grid;
    p.blockDim = block;
    p.sharedMemBytes = lds;
    p.kernelParams = args;
    p.extra = nullptr;
    hipGraphNode_t node = nullptr;
    const hipError_t e =
        hipGraphAddKernelNode(&node, g_->graph, g_->last ? &g_->last : nullptr,
                              g_->last ? 1 : 0, &p);
    if (e == hipSuccess) {
      g_->last = node;
      ++g_->n_nodes;
    }
    return e;
  }

 private:
  fsdp_step_graph* g_;
};

// The graph may still take nodes, on the device it was created on.
fsdp_status check_open(const fsdp_step_graph* g) {
  if (!g) return FSDP_ERR_INVALID_ARG;
  if (g->exec) return FSDP_ERR_INVALID_ARG;  // sealed by its first launch
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fsdp::status_of(hipErrorInvalidDevice);
  return dev == g->device ? FSDP_OK : FSDP_ERR_INVALID_ARG;
}

void destroy(fsdp_step_graph* g) {
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  if (g->replayed) (void)hipEventDestroy(g->replayed);
  if (g->scalars) (void)hipFree(g->scalars);
  delete g;
}

}  // namespace

extern "C" {

fsdp_status fsdp_step_graph_create(const fsdp_adamw_hparams* hp, fsdp_step_graph** out) {
  if (!out) return FSDP_ERR_INVALID_ARG;
  *out = nullptr;
  const fsdp_status st = fsdp::check_hparams(hp);
  if (st != FSDP_OK) return st;
  fsdp_step_graph* g = new (std::nothrow) fsdp_step_graph();
  if (!g) return FSDP_ERR_OUT_OF_MEMORY;
  g->hp = *hp;
  hipError_t e = hipGetDevice(&g->device);
  if (e == hipSuccess)
    e = hipMalloc(reinterpret_cast<void**>(&g->scalars), sizeof(fsdp::AdamScalars));
  if (e == hipSuccess) e = hipGraphCreate(&g->graph, 0);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&g->replayed, hipEventDisableTiming);
  if (e != hipSuccess) {
    destroy(g);
    return fsdp::status_of(e);
  }
  *out = g;
  return FSDP_OK;
}

void fsdp_step_graph_destroy(fsdp_step_graph* g) {
  if (g) destroy(g);
}

fsdp_status fsdp_step_graph_add_gather(fsdp_step_graph* g, const fsdp_plan* plan,
                                       const void* shards, int32_t dtype, void* const* full_out) {
  return fsdp::guarded([&]() -> fsdp_status {
    const fsdp_status st = check_open(g);
    if (st != FSDP_OK) return st;
    return fsdp::gather_impl(plan, shards, dtype, full_out, GraphSink(g));
  });
}

fsdp_status fsdp_step_graph_add_adamw(fsdp_step_graph* g, const fsdp_plan* plan,
                                      const void* const* grads, int32_t grad_dtype,
                                      int32_t grads_are_replicas, float* master, float* m,
                                      float* v, void* param_out, int32_t param_dtype) {
  return fsdp::guarded([&]() -> fsdp_status {
    const fsdp_status st = check_open(g);
    if (st != FSDP_OK) return st;
    const int64_t before = g->n_nodes;
    const fsdp::AdamScalars unused{};
    const fsdp_status r = fsdp::adamw_impl(plan, unused, g->scalars, grads, grad_dtype,
                                           grads_are_replicas, master, m, v, param_out, param_dtype,
                                           GraphSink(g));
    if (g->n_nodes > before) ++g->n_adamw;  // a node reads the record, even on a later error
    return r;
  });
}

fsdp_status fsdp_step_graph_add_adamw_gather(fsdp_step_graph* g, const fsdp_plan* plan,
                                             const void* const* grads, int32_t grad_dtype,
                                             float* master, float* m, float* v, void* param_out,
                                             int32_t param_dtype, const fsdp_plan* next,
                                             const void* next_shards, void* const* full_out) {
  return fsdp::guarded([&]() -> fsdp_status {
    const fsdp_status st = check_open(g);
    if (st != FSDP_OK) return st;
    const int64_t before = g->n_nodes;
    const fsdp::AdamScalars unused{};
    const fsdp_status r = fsdp::adamw_gather_impl(plan, unused, g->scalars, grads, grad_dtype,
                                                  master, m, v, param_out, param_dtype, next,
                                                  next_shards, full_out, GraphSink(g));
    if (g->n_nodes > before) ++g->n_adamw;  // a node reads the record, even on a later error
    return r;
  });
}

fsdp_status fsdp_step_graph_info(const fsdp_step_graph* g, int64_t* n_nodes, int64_t* n_adamw) {
  if (!g || !n_nodes || !n_adamw) return FSDP_ERR_INVALID_ARG;
  *n_nodes = g->n_nodes;
  *n_adamw = g->n_adamw;
  return FSDP_OK;
}

fsdp_status fsdp_step_graph_launch(fsdp_step_graph* g, int64_t step, void* stream) {
  if (!g) return FSDP_ERR_INVALID_ARG;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fsdp::status_of(hipErrorInvalidDevice);
  if (dev != g->device) return FSDP_ERR_INVALID_ARG;
  fsdp::AdamScalars sc;
  fsdp_status st = fsdp::adam_scalars(&g->hp, step, &sc);
  if (st != FSDP_OK) return st;
  if (g->n_nodes == 0) return FSDP_OK;
  if (!g->exec) {
    st = fsdp::status_of(hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0));
    if (st != FSDP_OK) {
      g->exec = nullptr;
      return st;
    }
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the previous replay, if it ran on another stream, ends before this
  // launch rewrites the scalar record
  if (g->launched && s != g->last_stream) {
    st = fsdp::status_of(hipEventRecord(g->replayed, g->last_stream));
    if (st == FSDP_OK) st = fsdp::status_of(hipStreamWaitEvent(s, g->replayed, 0));
    if (st != FSDP_OK) return st;
  }
  const fsdp::StreamSink sink(stream);
  if (g->n_adamw > 0) {
    st = fsdp::status_of(fsdp::launch_set_scalars(g->scalars, sc, sink));
    if (st != FSDP_OK) return st;
  }
  st = fsdp::status_of(hipGraphLaunch(g->exec, s));
  if (st != FSDP_OK) return st;
  g->launched = true;
  g->last_stream = s;
  return FSDP_OK;
}

}  // extern "C"
