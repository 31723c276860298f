// Launchers of the gfx950 kernels (internal; the C ABI validates first).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fsdp_mi355x.h"
#include "plan.hpp"

namespace fsdp {

struct PtrArray {
  const void* p[FSDP_MAX_RANKS];
};

// Scalars of one AdamW step, in float64, each computed on the host with the
// same expression the definition uses (1 - lr*wd, 1 - b1, 1 - b1^t, ...).
struct AdamScalars {
  double decay;  // 1 - lr * wd
  double beta1, omb1;  // b1, 1 - b1
  double beta2, omb2;  // b2, 1 - b2
  double bc1, bc2;     // 1 - b1^t, 1 - b2^t
  double lr, eps;
  // 1 / bc1 and 1 / bc2 as unevaluated sums hi + lo: hi the correctly
  // rounded reciprocal, lo the correctly rounded (1 - bc hi) / bc
  double rbc1_hi, rbc1_lo, rbc2_hi, rbc2_lo;
};
static_assert(sizeof(AdamScalars) == 13 * sizeof(double), "AdamScalars: 13 doubles, no padding");

// Where a launcher sends its kernel: enqueued on a stream, or appended to a
// graph under construction.  args follows hipLaunchKernel: one pointer per
// kernel argument, read before launch() returns; lds is the dynamic LDS
// (shared memory) bytes per workgroup.
class Sink {
 public:
  virtual ~Sink() = default;
  virtual hipError_t launch(const void* fn, dim3 grid, dim3 block, void** args,
                            unsigned lds) const = 0;
};

class StreamSink final : public Sink {
 public:
  explicit StreamSink(hipStream_t s) : stream_(s) {}
  explicit StreamSink(void* s) : stream_(static_cast<hipStream_t>(s)) {}
  hipError_t launch(const void* fn, dim3 grid, dim3 block, void** args,
                    unsigned lds) const override;

 private:
  hipStream_t stream_;
};

// Copy along work items; es = element size in bytes (2 or 4), lane_bytes
// = 8 or 16 bytes per lane.  dst holds n_dst pointers (NULL entries are
// skipped); padding items write zeros.
hipError_t launch_copy(const Work* work, int64_t n_work, const void* src, const PtrArray& dst,
                       int n_dst, int es, int lane_bytes, bool vec, const Sink& stream);

// Pack with a dtype change (F32 -> BF16 round to nearest even, BF16 -> F32).
hipError_t launch_pack_cast(const Work* work, int64_t n_work, const void* src, int src_dt,
                            void* dst, int dst_dt, bool vec, const Sink& stream);

// Reduce-scatter-average over shard-space work items.
hipError_t launch_rs_avg(const Work* work, int64_t n_work, const PtrArray& grads, int R,
                         int grad_dt, float* out, bool vec, const Sink& stream);

// The AdamW launchers take the step's scalars by value (sc), or, when scp is
// non-null, read them from that device record when they run.

// AdamW on n contiguous elements with an fp32 gradient of the same indexing.
hipError_t launch_adamw(int64_t n, const float* g, float* master, float* m, float* v,
                        void* param, int param_dt, const AdamScalars& sc,
                        const AdamScalars* scp, bool vec, const Sink& stream);

// Fused reduce-scatter-average + AdamW + recast over shard-space work items.
hipError_t launch_fused(const Work* work, int64_t n_work, const PtrArray& grads, int R,
                        int grad_dt, float* master, float* m, float* v, void* param,
                        int param_dt, const AdamScalars& sc, const AdamScalars* scp,
                        bool vec, const Sink& stream);

// acc[r] = g[r] (first) or acc[r] + g[r], fp32, for r < R over [0, T).
hipError_t launch_accumulate(int64_t T, int R, const PtrArray& grads, int grad_dt,
                             const PtrArray& acc, bool first, bool vec, const Sink& stream);

// out[r] = rank-order mean of the R gradients, for every receiver r, over
// [0, T).
hipError_t launch_allreduce(int64_t T, int R, const PtrArray& grads, int grad_dt,
                            const PtrArray& out, int out_dt, bool vec, const Sink& stream);

// The copy for n_pairs (source, destination) pairs sharing one work table
// (one destination each), 16 bytes per lane.
hipError_t launch_copy_pairs(const Work* work, int64_t n_work, const PtrArray& src,
                             const PtrArray& dst, int n_pairs, int es, bool vec,
                             const Sink& stream);

// Write sc to the device record dst (one single-lane kernel).
hipError_t launch_set_scalars(AdamScalars* dst, const AdamScalars& sc, const Sink& stream);

// launch_fused's step of one unit (n_fused work items), then in the same
// launch launch_copy's gather of another (n_gather items, n_dst
// destinations, elements of the parameter dtype).  Both counts > 0.
hipError_t launch_fused_gather(const Work* fwork, int64_t n_fused, const PtrArray& grads, int R,
                               int grad_dt, float* master, float* m, float* v, void* param,
                               int param_dt, const AdamScalars& sc, const AdamScalars* scp,
                               bool vec_f, const Work* gwork, int64_t n_gather,
                               const void* shards, const PtrArray& dst, int n_dst,
                               int lane_bytes, bool vec_g, const Sink& stream);

// Pointer-array slots of the kernels specialised for R <= 8 (a paired launch
// with such a step carries the gather's receivers in the same 8 slots).
constexpr int kSmallPtrs = 8;

// Fused-step work items at or below which a launch keeps full occupancy
// (no workgroup cap).
constexpr int64_t kSmallFusedLaunch = 4096;

// Fused-step work items up to which a step shares its launch with the next
// unit's gather (with the step's own workgroup cap).  Longer steps take the
// tighter cap of 3 per CU, which the gather does not want, and are long
// enough that one more launch boundary costs little.  Measured on MI355X,
// the 12-layer model at R = 8 as 6 units of 2 blocks (6,146 items): 398.8
// µs per step with two launches per unit, 390.0 µs paired.
constexpr int64_t kPairMax = 65536;

}  // namespace fsdp
