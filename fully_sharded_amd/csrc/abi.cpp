// extern "C" boundary of the FSDP hot-path library: argument checks, then
// one kernel launch per call on the caller's stream.  Declarations and the
// contract of every entry point are in include/fsdp_mi355x.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <new>
#include <vector>

#include "fsdp_mi355x.h"
#include "kernels.hpp"
#include "ops.hpp"
#include "plan.hpp"

using fsdp::AdamScalars;
using fsdp::PtrArray;
using fsdp::Work;

namespace {

bool valid_dtype(int32_t dt) { return dt == FSDP_F32 || dt == FSDP_BF16; }
int64_t dtype_size(int32_t dt) { return dt == FSDP_F32 ? 4 : 2; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}
bool overlap(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}
// The address ranges one call reads or writes, kept inline: at most 64
// gradient replicas, receivers or arrays, plus the state arrays.  The
// argument checks allocate nothing.
struct Ranges {
  Range r[FSDP_MAX_RANKS + 8];
  int n = 0;
  void push_back(const Range& x) {
    if (n < FSDP_MAX_RANKS + 8) r[n++] = x;
  }
  const Range* begin() const { return r; }
  const Range* end() const { return r + n; }
  size_t size() const { return static_cast<size_t>(n); }
  const Range& operator[](size_t i) const { return r[i]; }
};

template <typename L>
bool any_overlap(const L& rs) {
  for (size_t i = 0; i < rs.size(); ++i)
    for (size_t j = i + 1; j < rs.size(); ++j)
      if (overlap(rs[i], rs[j])) return true;
  return false;
}

fsdp_status from_hip(hipError_t e) { return fsdp::status_of(e); }

}  // namespace

namespace fsdp {

fsdp_status status_of(hipError_t e) {
  if (e == hipSuccess) return FSDP_OK;
  (void)hipGetLastError();
  return e == hipErrorOutOfMemory ? FSDP_ERR_OUT_OF_MEMORY : FSDP_ERR_HIP;
}

fsdp_status check_hparams(const fsdp_adamw_hparams* hp) {
  if (!hp) return FSDP_ERR_INVALID_ARG;
  const double lr = hp->lr, b1 = hp->beta1, b2 = hp->beta2, eps = hp->eps,
               wd = hp->weight_decay;
  if (!std::isfinite(lr) || !std::isfinite(eps) || !std::isfinite(wd) || lr < 0 ||
      !(b1 >= 0 && b1 < 1) || !(b2 >= 0 && b2 < 1) || !(eps > 0) || wd < 0)
    return FSDP_ERR_INVALID_ARG;
  return FSDP_OK;
}

fsdp_status adam_scalars(const fsdp_adamw_hparams* hp, int64_t step, AdamScalars* sc) {
  const fsdp_status st = check_hparams(hp);
  if (st != FSDP_OK) return st;
  if (step < 1) return FSDP_ERR_INVALID_ARG;
  const double lr = hp->lr, b1 = hp->beta1, b2 = hp->beta2, eps = hp->eps,
               wd = hp->weight_decay;
  const double t = static_cast<double>(step);
  sc->decay = 1.0 - lr * wd;
  sc->beta1 = b1;
  sc->omb1 = 1.0 - b1;
  sc->beta2 = b2;
  sc->omb2 = 1.0 - b2;
  sc->bc1 = 1.0 - std::pow(b1, t);
  sc->bc2 = 1.0 - std::pow(b2, t);
  sc->lr = lr;
  sc->eps = eps;
  if (!(sc->bc1 > 0) || !(sc->bc2 > 0)) return FSDP_ERR_INVALID_ARG;
  // 1 / bc to about 2^-106: hi = RN(1 / bc); 1 - bc hi is exact in one
  // fused multiply-add (|1 - bc hi| <= 2^-53 and its bits fit 53), and
  // lo = RN((1 - bc hi) / bc).  The kernels divide by bc with these.
  sc->rbc1_hi = 1.0 / sc->bc1;
  sc->rbc1_lo = std::fma(-sc->bc1, sc->rbc1_hi, 1.0) / sc->bc1;
  sc->rbc2_hi = 1.0 / sc->bc2;
  sc->rbc2_lo = std::fma(-sc->bc2, sc->rbc2_hi, 1.0) / sc->bc2;
  return FSDP_OK;
}

namespace {

// A checked gather: its launch arguments and the memory it reads and writes.
struct GatherCall {
  const fsdp_plan* plan = nullptr;
  const Work* w = nullptr;
  int64_t n_work = 0;
  const void* src = nullptr;
  PtrArray dst{};
  int n_dst = 0;  // destinations given (NULL ones are skipped)
  int es = 0;
  int lane_bytes = 16;
  bool vec = false;
  Ranges reads, writes;
};

fsdp_status prep_gather(const fsdp_plan* plan, const void* shards, int32_t dtype,
                        void* const* full_out, GatherCall* c) {
  if (!plan || !shards || !full_out || !valid_dtype(dtype)) return FSDP_ERR_INVALID_ARG;
  const int64_t es = dtype_size(dtype);
  if (!aligned(shards, es)) return FSDP_ERR_INVALID_ARG;
  c->reads.push_back(range_of(shards, plan->R * plan->S * es));
  c->vec = aligned(shards, 16);
  for (int r = 0; r < plan->R; ++r) {
    void* d = full_out[r];
    c->dst.p[r] = d;
    if (!d) continue;
    if (!aligned(d, es)) return FSDP_ERR_INVALID_ARG;
    c->vec = c->vec && aligned(d, 16);
    c->writes.push_back(range_of(d, plan->T * es));
    ++c->n_dst;
  }
  Ranges all = c->writes;
  all.push_back(c->reads[0]);
  if (any_overlap(all)) return FSDP_ERR_INVALID_ARG;
  c->plan = plan;
  c->n_work = static_cast<int64_t>(plan->flat_work.host.size());
  c->src = shards;
  c->es = static_cast<int>(es);
  c->lane_bytes = plan->gather_lane_bytes;
  return FSDP_OK;
}

// The work table on the current device (uploaded on first use), once every
// check has passed.
fsdp_status attach(GatherCall* c) {
  return c->n_dst == 0 ? FSDP_OK : c->plan->flat_work.device(&c->w);
}

fsdp_status launch(const GatherCall& c, int R, const Sink& sink) {
  if (c.n_dst == 0) return FSDP_OK;
  return status_of(launch_copy(c.w, c.n_work, c.src, c.dst, R, c.es, c.lane_bytes, c.vec, sink));
}

// A checked AdamW shard step.
struct AdamCall {
  const fsdp_plan* plan = nullptr;
  bool replicas = true;
  PtrArray g{};
  int32_t grad_dt = 0, param_dt = 0;
  float *master = nullptr, *m = nullptr, *v = nullptr;
  void* param = nullptr;
  bool vec = false;
  const Work* w = nullptr;
  int64_t n_work = 0;
  Ranges reads, writes;
};

fsdp_status prep_adamw(const fsdp_plan* plan, const void* const* grads, int32_t grad_dtype,
                       int32_t grads_are_replicas, float* master, float* m, float* v,
                       void* param_out, int32_t param_dtype, AdamCall* c) {
  if (!plan || !grads || !master || !m || !v || !param_out) return FSDP_ERR_INVALID_ARG;
  if (!valid_dtype(grad_dtype) || !valid_dtype(param_dtype)) return FSDP_ERR_INVALID_ARG;
  if (grads_are_replicas != 0 && grads_are_replicas != 1) return FSDP_ERR_INVALID_ARG;
  const int64_t n = plan->R * plan->S;
  const int64_t pes = dtype_size(param_dtype);
  if (!aligned(master, 4) || !aligned(m, 4) || !aligned(v, 4) || !aligned(param_out, pes))
    return FSDP_ERR_INVALID_ARG;
  c->writes.push_back(range_of(master, n * 4));
  c->writes.push_back(range_of(m, n * 4));
  c->writes.push_back(range_of(v, n * 4));
  c->writes.push_back(range_of(param_out, n * pes));
  c->vec = aligned(master, 16) && aligned(m, 16) && aligned(v, 16) && aligned(param_out, 16);
  if (grads_are_replicas) {
    const int64_t ges = dtype_size(grad_dtype);
    for (int q = 0; q < plan->R; ++q) {
      if (!grads[q] || !aligned(grads[q], ges)) return FSDP_ERR_INVALID_ARG;
      c->reads.push_back(range_of(grads[q], plan->T * ges));
      c->vec = c->vec && aligned(grads[q], 16);
      c->g.p[q] = grads[q];
    }
  } else {
    if (grad_dtype != FSDP_F32 || !grads[0] || !aligned(grads[0], 4)) return FSDP_ERR_INVALID_ARG;
    c->reads.push_back(range_of(grads[0], n * 4));
    c->vec = c->vec && aligned(grads[0], 16);
    c->g.p[0] = grads[0];
  }
  for (const Range& o : c->writes)
    for (const Range& i : c->reads)
      if (overlap(o, i)) return FSDP_ERR_INVALID_ARG;
  if (any_overlap(c->writes)) return FSDP_ERR_INVALID_ARG;
  c->plan = plan;
  c->replicas = grads_are_replicas != 0;
  c->grad_dt = grad_dtype;
  c->param_dt = param_dtype;
  c->master = master;
  c->m = m;
  c->v = v;
  c->param = param_out;
  if (c->replicas) c->n_work = static_cast<int64_t>(plan->shard_work.host.size());
  return FSDP_OK;
}

fsdp_status attach(AdamCall* c) {
  return c->replicas ? c->plan->shard_work.device(&c->w) : FSDP_OK;
}

fsdp_status launch(const AdamCall& c, const AdamScalars& sc, const AdamScalars* scp,
                   const Sink& sink) {
  if (!c.replicas)
    return status_of(launch_adamw(c.plan->R * c.plan->S, static_cast<const float*>(c.g.p[0]),
                                  c.master, c.m, c.v, c.param, c.param_dt, sc, scp, c.vec, sink));
  return status_of(launch_fused(c.w, c.n_work, c.g, c.plan->R, c.grad_dt, c.master, c.m, c.v,
                                c.param, c.param_dt, sc, scp, c.vec, sink));
}

}  // namespace

fsdp_status gather_impl(const fsdp_plan* plan, const void* shards, int32_t dtype,
                        void* const* full_out, const Sink& sink) {
  GatherCall c;
  fsdp_status st = prep_gather(plan, shards, dtype, full_out, &c);
  if (st == FSDP_OK) st = attach(&c);
  return st != FSDP_OK ? st : launch(c, plan->R, sink);
}

fsdp_status adamw_impl(const fsdp_plan* plan, const AdamScalars& sc, const AdamScalars* scp,
                       const void* const* grads, int32_t grad_dtype, int32_t grads_are_replicas,
                       float* master, float* m, float* v, void* param_out, int32_t param_dtype,
                       const Sink& sink) {
  AdamCall c;
  fsdp_status st = prep_adamw(plan, grads, grad_dtype, grads_are_replicas, master, m, v,
                              param_out, param_dtype, &c);
  if (st == FSDP_OK) st = attach(&c);
  return st != FSDP_OK ? st : launch(c, sc, scp, sink);
}

fsdp_status adamw_gather_impl(const fsdp_plan* plan, const AdamScalars& sc,
                              const AdamScalars* scp, const void* const* grads,
                              int32_t grad_dtype, float* master, float* m, float* v,
                              void* param_out, int32_t param_dtype, const fsdp_plan* next,
                              const void* next_shards, void* const* full_out, const Sink& sink) {
  AdamCall a;
  fsdp_status st = prep_adamw(plan, grads, grad_dtype, 1, master, m, v, param_out, param_dtype, &a);
  if (st != FSDP_OK) return st;
  GatherCall g;
  st = prep_gather(next, next_shards, param_dtype, full_out, &g);
  if (st != FSDP_OK) return st;
  // the two run concurrently: neither may write what the other touches
  for (const Range& w : g.writes) {
    for (const Range& x : a.writes)
      if (overlap(w, x)) return FSDP_ERR_INVALID_ARG;
    for (const Range& x : a.reads)
      if (overlap(w, x)) return FSDP_ERR_INVALID_ARG;
  }
  for (const Range& w : a.writes)
    for (const Range& x : g.reads)
      if (overlap(w, x)) return FSDP_ERR_INVALID_ARG;
  if ((st = attach(&a)) != FSDP_OK || (st = attach(&g)) != FSDP_OK) return st;
  if (g.n_dst == 0) return launch(a, sc, scp, sink);
  // one launch when the step is short enough, the step's pointer slots also
  // hold the gather's receivers and the two fit in one grid
  const bool slots_fit = plan->R > kSmallPtrs || next->R <= kSmallPtrs;
  if (a.n_work > kPairMax || a.n_work == 0 || !slots_fit || a.n_work + g.n_work > kMaxItems) {
    // a long step: its own launch (with its occupancy cap), then the gather
    st = launch(a, sc, scp, sink);
    return st != FSDP_OK ? st : launch(g, next->R, sink);
  }
  return status_of(launch_fused_gather(a.w, a.n_work, a.g, plan->R, grad_dtype, master, m, v,
                                       param_out, param_dtype, sc, scp, a.vec, g.w, g.n_work,
                                       g.src, g.dst, next->R, g.lane_bytes, g.vec, sink));
}

}  // namespace fsdp

// ------------------------------------------ the entry point that allocates
// fsdp_adamw_shard_step_noalloc keeps the plan's work table in this static
// device array (one copy per GPU, held until the process ends) instead of
// device memory the plan allocates.  In host code `scratch` names a
// host-side stand-in, never the device array: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
namespace {
constexpr size_t kScratchBytes = size_t(1) << 20;
constexpr int64_t kScratchItems = static_cast<int64_t>(kScratchBytes / sizeof(Work));
constexpr int kScratchDevices = 64;
}  // namespace

static __device__ __align__(256) Work scratch[kScratchItems];

namespace {
std::mutex g_scratch_mu;
Work* g_scratch_ptr[kScratchDevices] = {};

// The device address of `scratch` on the current device, looked up on the
// first call there (with that device current) and kept.
fsdp_status scratch_on_current_device(Work** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fsdp::status_of(hipErrorInvalidDevice);
  if (dev < 0 || dev >= kScratchDevices) return FSDP_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return fsdp::status_of(e == hipSuccess ? hipErrorUnknown : e);
    g_scratch_ptr[dev] = static_cast<Work*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return FSDP_OK;
}
}  // namespace

extern "C" {

fsdp_status fsdp_plan_layout(int32_t n_params, const int32_t* ndims, const int64_t* dims,
                             int32_t R, int32_t layout, fsdp_plan** out) {
  if (!out) return FSDP_ERR_INVALID_ARG;
  *out = nullptr;
  if (n_params < 1 || !ndims || !dims) return FSDP_ERR_INVALID_ARG;
  if (R < 1) return FSDP_ERR_INVALID_ARG;
  if (R > FSDP_MAX_RANKS) return FSDP_ERR_UNSUPPORTED;
  if (layout != FSDP_LAYOUT_PER_PARAM && layout != FSDP_LAYOUT_FLAT) return FSDP_ERR_INVALID_ARG;
  fsdp_plan* pl = new (std::nothrow) fsdp_plan();
  if (!pl) return FSDP_ERR_OUT_OF_MEMORY;
  try {
    pl->R = R;
    pl->layout = layout;
    int64_t at = 0;
    for (int32_t p = 0; p < n_params; ++p) {
      if (ndims[p] < 1 || ndims[p] > 8) {
        delete pl;
        return FSDP_ERR_INVALID_ARG;
      }
      std::vector<int64_t> shape(dims + at, dims + at + ndims[p]);
      at += ndims[p];
      for (int64_t d : shape)
        if (d <= 0) {
          delete pl;
          return FSDP_ERR_INVALID_ARG;
        }
      pl->shapes.push_back(shape);
    }
    const fsdp_status st = fsdp::build_plan(pl);
    if (st != FSDP_OK) {
      delete pl;
      return st;
    }
  } catch (const std::bad_alloc&) {
    delete pl;
    return FSDP_ERR_OUT_OF_MEMORY;
  } catch (...) {
    delete pl;
    return FSDP_ERR_INVALID_ARG;
  }
  *out = pl;
  return FSDP_OK;
}

void fsdp_plan_destroy(fsdp_plan* plan) { delete plan; }

fsdp_status fsdp_plan_get_info(const fsdp_plan* plan, fsdp_plan_info* out) {
  if (!plan || !out) return FSDP_ERR_INVALID_ARG;
  out->numel_full = plan->T;
  out->shard_numel = plan->S;
  out->world = plan->R;
  out->n_params = static_cast<int32_t>(plan->params.size());
  out->layout = plan->layout;
  out->n_segments = static_cast<int32_t>(plan->segments.size());
  return FSDP_OK;
}

fsdp_status fsdp_plan_param(const fsdp_plan* plan, int32_t p, int64_t* out) {
  if (!plan || !out || p < 0 || p >= static_cast<int32_t>(plan->params.size()))
    return FSDP_ERR_INVALID_ARG;
  const fsdp::Param& q = plan->params[p];
  out[0] = q.flat_off;
  out[1] = q.numel;
  out[2] = q.shard_off;
  out[3] = q.k;
  out[4] = q.row;
  return FSDP_OK;
}

fsdp_status fsdp_plan_rank_valid(const fsdp_plan* plan, int32_t r, int64_t* valid) {
  if (!plan || !valid || r < 0 || r >= plan->R) return FSDP_ERR_INVALID_ARG;
  int64_t n = 0;
  for (const fsdp::Segment& s : plan->segments)
    if (s.rank == r) n += s.len;
  *valid = n;
  return FSDP_OK;
}

fsdp_status fsdp_plan_segments(const fsdp_plan* plan, int64_t* out, int32_t capacity) {
  if (!plan || !out || capacity < static_cast<int64_t>(plan->segments.size()))
    return FSDP_ERR_INVALID_ARG;
  for (size_t i = 0; i < plan->segments.size(); ++i) {
    const fsdp::Segment& s = plan->segments[i];
    out[4 * i + 0] = s.rank;
    out[4 * i + 1] = s.shard_off;
    out[4 * i + 2] = s.flat_off;
    out[4 * i + 3] = s.len;
  }
  return FSDP_OK;
}

fsdp_status fsdp_plan_comm_ledger(const fsdp_plan* plan, int32_t reshard_after_forward,
                                  int64_t* out) {
  if (!plan || !out) return FSDP_ERR_INVALID_ARG;
  const int64_t per_collective = (plan->R - 1) * plan->S;
  out[0] = (reshard_after_forward ? 2 : 1) * per_collective;
  out[1] = per_collective;
  out[2] = 0;
  out[3] = out[0] + out[1] + out[2];
  return FSDP_OK;
}

int64_t fsdp_plan_state_bytes_per_rank(const fsdp_plan* plan) {
  return plan ? 16 * plan->S : -1;
}

namespace {
fsdp_status copy_items(const std::vector<Work>& items, int64_t* out, int64_t capacity,
                       int64_t* n) {
  if (!n) return FSDP_ERR_INVALID_ARG;
  *n = static_cast<int64_t>(items.size());
  if (!out) return FSDP_OK;
  if (capacity < *n) return FSDP_ERR_INVALID_ARG;
  for (size_t i = 0; i < items.size(); ++i) {
    out[3 * i + 0] = items[i].dst;
    out[3 * i + 1] = items[i].src;
    out[3 * i + 2] = items[i].len;
  }
  return FSDP_OK;
}
}  // namespace

fsdp_status fsdp_plan_work_items(const fsdp_plan* plan, int32_t space, int64_t* out,
                                 int64_t capacity, int64_t* n) {
  if (!plan || (space != 0 && space != 1)) return FSDP_ERR_INVALID_ARG;
  return copy_items(space == 0 ? plan->shard_work.host : plan->flat_work.host, out, capacity, n);
}

fsdp_status fsdp_plan_prepare(const fsdp_plan* plan, void* stream) {
  return fsdp::guarded([&]() -> fsdp_status {
    (void)stream;
    if (!plan) return FSDP_ERR_INVALID_ARG;
    const Work* w = nullptr;
    const fsdp_status st = plan->shard_work.device(&w);
    return st != FSDP_OK ? st : plan->flat_work.device(&w);
  });
}

fsdp_status fsdp_shard_pack(const fsdp_plan* plan, const void* full, int32_t full_dtype,
                            void* shards, int32_t shard_dtype, void* stream) {
  return fsdp::guarded([&]() -> fsdp_status {
    if (!plan || !full || !shards) return FSDP_ERR_INVALID_ARG;
    if (!valid_dtype(full_dtype) || !valid_dtype(shard_dtype)) return FSDP_ERR_INVALID_ARG;
    if (!aligned(full, dtype_size(full_dtype)) || !aligned(shards, dtype_size(shard_dtype)))
      return FSDP_ERR_INVALID_ARG;
    if (overlap(range_of(full, plan->T * dtype_size(full_dtype)),
                range_of(shards, plan->R * plan->S * dtype_size(shard_dtype))))
      return FSDP_ERR_INVALID_ARG;
    const Work* w = nullptr;
    const fsdp_status st = plan->shard_work.device(&w);
    if (st != FSDP_OK) return st;
    const bool vec = aligned(full, 16) && aligned(shards, 16);
    const auto n_work = static_cast<int64_t>(plan->shard_work.host.size());
    const fsdp::StreamSink s(stream);
    if (full_dtype == shard_dtype) {
      PtrArray dst{};
      dst.p[0] = shards;
      return from_hip(fsdp::launch_copy(w, n_work, full, dst, 1,
                                        static_cast<int>(dtype_size(full_dtype)), 16, vec, s));
    }
    return from_hip(
        fsdp::launch_pack_cast(w, n_work, full, full_dtype, shards, shard_dtype, vec, s));
  });
}

fsdp_status fsdp_gather_unflatten(const fsdp_plan* plan, const void* shards, int32_t dtype,
                                  void* const* full_out, void* stream) {
  return fsdp::guarded([&]() -> fsdp_status {
    return fsdp::gather_impl(plan, shards, dtype, full_out, fsdp::StreamSink(stream));
  });
}

fsdp_status fsdp_reduce_scatter_avg(const fsdp_plan* plan, const void* const* grads,
                                    int32_t grad_dtype, float* out, void* stream) {
  return fsdp::guarded([&]() -> fsdp_status {
    if (!plan || !grads || !out || !valid_dtype(grad_dtype)) return FSDP_ERR_INVALID_ARG;
    const int64_t es = dtype_size(grad_dtype);
    if (!aligned(out, 4)) return FSDP_ERR_INVALID_ARG;
    const Range out_r = range_of(out, plan->R * plan->S * 4);
    PtrArray g{};
    bool vec = aligned(out, 16);
    for (int q = 0; q < plan->R; ++q) {
      if (!grads[q] || !aligned(grads[q], es)) return FSDP_ERR_INVALID_ARG;
      if (overlap(out_r, range_of(grads[q], plan->T * es))) return FSDP_ERR_INVALID_ARG;
      vec = vec && aligned(grads[q], 16);
      g.p[q] = grads[q];
    }
    const Work* w = nullptr;
    const fsdp_status st = plan->shard_work.device(&w);
    if (st != FSDP_OK) return st;
    return from_hip(fsdp::launch_rs_avg(w, static_cast<int64_t>(plan->shard_work.host.size()), g,
                                        plan->R, grad_dtype, out, vec,
                                        fsdp::StreamSink(stream)));
  });
}

fsdp_status fsdp_adamw_shard_step(const fsdp_plan* plan, const fsdp_adamw_hparams* hp,
                                  int64_t step, const void* const* grads, int32_t grad_dtype,
                                  int32_t grads_are_replicas, float* master, float* m, float* v,
                                  void* param_out, int32_t param_dtype, void* stream) {
  return fsdp::guarded([&]() -> fsdp_status {
    if (!plan || !hp) return FSDP_ERR_INVALID_ARG;
    AdamScalars sc;
    const fsdp_status st = fsdp::adam_scalars(hp, step, &sc);
    if (st != FSDP_OK) return st;
    return fsdp::adamw_impl(plan, sc, nullptr, grads, grad_dtype, grads_are_replicas, master, m, v,
                            param_out, param_dtype, fsdp::StreamSink(stream));
  });
}

fsdp_status fsdp_adamw_shard_step_noalloc(const fsdp_plan* plan, const fsdp_adamw_hparams* hp,
                                          int64_t step, const void* const* grads,
                                          int32_t grad_dtype, int32_t grads_are_replicas,
                                          float* master, float* m, float* v, void* param_out,
                                          int32_t param_dtype, void* stream) {
  return fsdp::guarded([&]() -> fsdp_status {
    if (!plan || !hp) return FSDP_ERR_INVALID_ARG;
    AdamScalars sc;
    fsdp_status st = fsdp::adam_scalars(hp, step, &sc);
    if (st != FSDP_OK) return st;
    const int64_t n_work = static_cast<int64_t>(plan->shard_work.host.size());
    if (grads_are_replicas == 1 && n_work > kScratchItems) return FSDP_ERR_UNSUPPORTED;
    fsdp::AdamCall c;
    st = fsdp::prep_adamw(plan, grads, grad_dtype, grads_are_replicas, master, m, v, param_out,
                          param_dtype, &c);
    if (st != FSDP_OK) return st;
    if (c.replicas && n_work > 0) {
      Work* table = nullptr;
      st = scratch_on_current_device(&table);
      if (st != FSDP_OK) return st;
      // the plan's table into the static array, in stream order before the step
      st = fsdp::status_of(hipMemcpyAsync(table, plan->shard_work.host.data(),
                                          static_cast<size_t>(n_work) * sizeof(Work),
                                          hipMemcpyHostToDevice,
                                          static_cast<hipStream_t>(stream)));
      if (st != FSDP_OK) return st;
      c.w = table;
    }
    return fsdp::launch(c, sc, nullptr, fsdp::StreamSink(stream));
  });
}

fsdp_status fsdp_adamw_step_then_gather(const fsdp_plan* plan, const fsdp_adamw_hparams* hp,
                                        int64_t step, const void* const* grads,
                                        int32_t grad_dtype, float* master, float* m, float* v,
                                        void* param_out, int32_t param_dtype,
                                        const fsdp_plan* next, const void* next_shards,
                                        void* const* full_out, void* stream) {
  return fsdp::guarded([&]() -> fsdp_status {
    if (!plan || !hp) return FSDP_ERR_INVALID_ARG;
    AdamScalars sc;
    const fsdp_status st = fsdp::adam_scalars(hp, step, &sc);
    if (st != FSDP_OK) return st;
    return fsdp::adamw_gather_impl(plan, sc, nullptr, grads, grad_dtype, master, m, v, param_out,
                                   param_dtype, next, next_shards, full_out,
                                   fsdp::StreamSink(stream));
  });
}

fsdp_status fsdp_reshard_plan(const fsdp_plan* from, const fsdp_plan* to, fsdp_resharder** out) {
  if (!out) return FSDP_ERR_INVALID_ARG;
  *out = nullptr;
  if (!from || !to) return FSDP_ERR_INVALID_ARG;
  fsdp_resharder* rs = new (std::nothrow) fsdp_resharder();
  if (!rs) return FSDP_ERR_OUT_OF_MEMORY;
  fsdp_status st;
  try {
    st = fsdp::build_reshard(from, to, rs);
  } catch (const std::bad_alloc&) {
    st = FSDP_ERR_OUT_OF_MEMORY;
  }
  if (st != FSDP_OK) {
    delete rs;
    return st;
  }
  *out = rs;
  return FSDP_OK;
}

void fsdp_reshard_destroy(fsdp_resharder* rs) { delete rs; }

fsdp_status fsdp_reshard_items(const fsdp_resharder* rs, int64_t* out, int64_t capacity,
                               int64_t* n) {
  if (!rs) return FSDP_ERR_INVALID_ARG;
  return copy_items(rs->work.host, out, capacity, n);
}

fsdp_status fsdp_reshard(const fsdp_resharder* rs, const void* src, void* dst, int32_t dtype,
                         void* stream) {
  return fsdp::guarded([&]() -> fsdp_status {
    if (!rs || !src || !dst || !valid_dtype(dtype)) return FSDP_ERR_INVALID_ARG;
    const int64_t es = dtype_size(dtype);
    if (!aligned(src, es) || !aligned(dst, es)) return FSDP_ERR_INVALID_ARG;
    if (overlap(range_of(src, rs->R_from * rs->S_from * es),
                range_of(dst, rs->R_to * rs->S_to * es)))
      return FSDP_ERR_INVALID_ARG;
    const Work* w = nullptr;
    const fsdp_status st = rs->work.device(&w);
    if (st != FSDP_OK) return st;
    PtrArray d{};
    d.p[0] = dst;
    const bool vec = aligned(src, 16) && aligned(dst, 16);
    return from_hip(fsdp::launch_copy(w, static_cast<int64_t>(rs->work.host.size()), src, d, 1,
                                      static_cast<int>(es), 16, vec, fsdp::StreamSink(stream)));
  });
}

fsdp_status fsdp_reshard_batch(const fsdp_resharder* rs, int32_t n, const void* const* srcs,
                               void* const* dsts, int32_t dtype, void* stream) {
  return fsdp::guarded([&]() -> fsdp_status {
    if (!rs || !srcs || !dsts || !valid_dtype(dtype)) return FSDP_ERR_INVALID_ARG;
    if (n < 1 || n > FSDP_MAX_RANKS) return n < 1 ? FSDP_ERR_INVALID_ARG : FSDP_ERR_UNSUPPORTED;
    const int64_t es = dtype_size(dtype);
    std::vector<Range> ins, outs;
    PtrArray s{}, d{};
    bool vec = true;
    for (int i = 0; i < n; ++i) {
      if (!srcs[i] || !dsts[i] || !aligned(srcs[i], es) || !aligned(dsts[i], es))
        return FSDP_ERR_INVALID_ARG;
      vec = vec && aligned(srcs[i], 16) && aligned(dsts[i], 16);
      ins.push_back(range_of(srcs[i], rs->R_from * rs->S_from * es));
      outs.push_back(range_of(dsts[i], rs->R_to * rs->S_to * es));
      s.p[i] = srcs[i];
      d.p[i] = dsts[i];
    }
    if (any_overlap(outs)) return FSDP_ERR_INVALID_ARG;
    for (const Range& o : outs)
      for (const Range& x : ins)
        if (overlap(o, x)) return FSDP_ERR_INVALID_ARG;
    const Work* w = nullptr;
    const fsdp_status st = rs->work.device(&w);
    if (st != FSDP_OK) return st;
    return from_hip(fsdp::launch_copy_pairs(w, static_cast<int64_t>(rs->work.host.size()), s, d, n,
                                            static_cast<int>(es), vec,
                                            fsdp::StreamSink(stream)));
  });
}

fsdp_status fsdp_grad_accumulate(const fsdp_plan* plan, const void* const* grads,
                                 int32_t grad_dtype, float* const* acc, int32_t first,
                                 void* stream) {
  return fsdp::guarded([&]() -> fsdp_status {
    if (!plan || !grads || !acc || !valid_dtype(grad_dtype)) return FSDP_ERR_INVALID_ARG;
    if (first != 0 && first != 1) return FSDP_ERR_INVALID_ARG;
    const int64_t ges = dtype_size(grad_dtype);
    std::vector<Range> outs;
    std::vector<Range> ins;
    PtrArray g{}, a{};
    bool vec = true;
    for (int r = 0; r < plan->R; ++r) {
      if (!grads[r] || !acc[r] || !aligned(grads[r], ges) || !aligned(acc[r], 4))
        return FSDP_ERR_INVALID_ARG;
      vec = vec && aligned(grads[r], 16) && aligned(acc[r], 16);
      ins.push_back(range_of(grads[r], plan->T * ges));
      outs.push_back(range_of(acc[r], plan->T * 4));
      g.p[r] = grads[r];
      a.p[r] = acc[r];
    }
    if (any_overlap(outs)) return FSDP_ERR_INVALID_ARG;
    for (const Range& o : outs)
      for (const Range& i : ins)
        if (overlap(o, i)) return FSDP_ERR_INVALID_ARG;
    return from_hip(fsdp::launch_accumulate(plan->T, plan->R, g, grad_dtype, a, first != 0, vec,
                                            fsdp::StreamSink(stream)));
  });
}

fsdp_status fsdp_allreduce_avg(const fsdp_plan* plan, const void* const* grads,
                               int32_t grad_dtype, void* const* out, int32_t out_dtype,
                               void* stream) {
  return fsdp::guarded([&]() -> fsdp_status {
    if (!plan || !grads || !out || !valid_dtype(grad_dtype) || !valid_dtype(out_dtype))
      return FSDP_ERR_INVALID_ARG;
    const int64_t ges = dtype_size(grad_dtype), oes = dtype_size(out_dtype);
    std::vector<Range> outs;
    std::vector<Range> ins;
    PtrArray g{}, o{};
    bool vec = true;
    for (int r = 0; r < plan->R; ++r) {
      if (!grads[r] || !out[r] || !aligned(grads[r], ges) || !aligned(out[r], oes))
        return FSDP_ERR_INVALID_ARG;
      vec = vec && aligned(grads[r], 16) && aligned(out[r], 16);
      ins.push_back(range_of(grads[r], plan->T * ges));
      outs.push_back(range_of(out[r], plan->T * oes));
      g.p[r] = grads[r];
      o.p[r] = out[r];
    }
    if (any_overlap(outs)) return FSDP_ERR_INVALID_ARG;
    for (const Range& x : outs)
      for (const Range& i : ins)
        if (overlap(x, i)) return FSDP_ERR_INVALID_ARG;
    return from_hip(fsdp::launch_allreduce(plan->T, plan->R, g, grad_dtype, o, out_dtype, vec,
                                           fsdp::StreamSink(stream)));
  });
}

const char* fsdp_status_string(int32_t status) {
  switch (status) {
    case FSDP_OK: return "ok";
    case FSDP_ERR_INVALID_ARG: return "invalid argument";
    case FSDP_ERR_UNSUPPORTED: return "unsupported";
    case FSDP_ERR_OUT_OF_MEMORY: return "out of memory";
    case FSDP_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

}  // extern "C"
