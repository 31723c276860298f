// Internal plan structures: the shard layout of one FSDP unit, its
// contiguous (rank, shard range, flat range) segments, and the
// per-workgroup work tables the kernels consume (host copies, and device
// copies uploaded lazily per device).
#pragma once

#include <cstdint>
#include <map>
#include <mutex>
#include <vector>

#include "fsdp_mi355x.h"

namespace fsdp {

// One workgroup's contiguous range.  dst indexes the destination index space
// of the operation (the [R][S] shard buffer linearly, or the full-unit
// buffer), src the source space.  src < 0 marks padding (no source: the
// destination gets +0).
struct Work {
  int64_t dst;
  int64_t src;
  int64_t len;
};

struct Segment {
  int64_t rank;
  int64_t shard_off;  // inside the rank's shard
  int64_t flat_off;   // in the full-unit buffer
  int64_t len;
};

struct Param {
  int64_t numel, d0, row, flat_off, k, shard_off;
};

// A work table: host copy plus one device copy per HIP device.
class WorkTable {
 public:
  std::vector<Work> host;
  // Device copy for the current device, uploaded on first use (hipMalloc +
  // hipMemcpy, synchronous).  Returns FSDP_OK and sets *out, or an error.
  fsdp_status device(const Work** out) const;
  void release();  // free every device copy
  ~WorkTable() { release(); }

 private:
  mutable std::mutex mu_;
  mutable std::map<int, Work*> dev_;
};

// Append [dst, dst+len) <- [src, src+len) to a list of runs, merging it with
// the previous run when both are contiguous in the destination and (both
// padding or) contiguous in the source.
void push_run(std::vector<Work>& runs, int64_t dst, int64_t src, int64_t len);

// Cut runs into work items of at most `chunk` elements, at multiples of
// chunk in the destination space.
void emit_items(const std::vector<Work>& runs, int64_t chunk, std::vector<Work>& out);

}  // namespace fsdp

struct fsdp_plan {
  int32_t R = 0;
  int32_t layout = 0;
  int64_t T = 0;
  int64_t S = 0;
  std::vector<std::vector<int64_t>> shapes;
  std::vector<fsdp::Param> params;
  std::vector<fsdp::Segment> segments;  // ordered by (rank, shard_off)
  std::vector<fsdp::Work> shard_runs;   // shard space [0, R*S): pieces and padding
  std::vector<fsdp::Work> flat_runs;    // flat space [0, T) -> shard space
  fsdp::WorkTable shard_work;           // shard_runs cut into work items
  fsdp::WorkTable flat_work;            // flat_runs cut into work items
  int32_t gather_lane_bytes = 16;       // bytes per lane of the gather copy
};

struct fsdp_resharder {
  int32_t R_from = 0, R_to = 0;
  int64_t T = 0, S_from = 0, S_to = 0;
  fsdp::WorkTable work;  // destination shard space [0, R_to*S_to) <- source shard space
};

namespace fsdp {

// Elements per work item (one workgroup): exactly one pass of its 256
// lanes, at every size -- 1024 for the 4-element lanes of the arithmetic
// kernels (shard space), 2048 for the 16-byte lanes of the bf16 copy.
// Workgroups are dispatched in order, so the ones in flight then cover one
// compact window of every stream; giving each workgroup 16 consecutive
// passes spread the in-flight window over ~60 MB per stream and cost 8% on
// an 872M-element unit (5.27 vs 5.68 TB/s), and even 2 passes cost 7% on a
// 3M-element one.
constexpr int64_t kShardChunk = 1024;
constexpr int64_t kFlatChunk = 2048;

// The gather copies 16 bytes per lane up to this many elements per unit and
// 8 bytes per lane (1024-element work items) above it.  Measured on MI355X
// (bf16, 8 receivers): 16-byte lanes lead at 3M and 6M elements (5.40 vs
// 5.15, 5.60 vs 5.05 TB/s), tie at 12.6M, and trail from 25M on (4.67 vs
// 5.26 TB/s at 25M, 4.96 vs 5.68 at 100M).
constexpr int64_t kWideGatherMax = 12582912;

// At R = 8 the 16-byte gather stores its 8 receivers from an unrolled
// sequence, which keeps 16-byte lanes ahead further: up to this many
// elements per unit.  Measured against 8-byte lanes (alternating runs on
// one machine): the 12-layer model as 4-block units (12.6M elements)
// gather 42.3 -> 40.1 us and step 393.6 -> 386.3 us (serial), 403.8 ->
// 385.2 us (overlap, which then pairs each step with the next gather); as
// one unit (37.8M) gather 129.3 -> 126.2 us.  Larger units keep 8-byte
// lanes (untested with the unrolled stores).
constexpr int64_t kWideGatherMaxR8 = 41943040;

// A launch covers at most 2^32 - 1 lanes along x: 16,777,215 workgroups of
// 256 lanes.  A plan (or re-shard) whose work table would need more items
// than that is refused with FSDP_ERR_UNSUPPORTED.  The shard space holds at
// least ceil(T / 1024) items, so the same bound covers the kernels that
// cut the full unit into 1024-element blocks (accumulate, all-reduce).
constexpr int64_t kMaxItems = 0xFFFFFFFFLL / 256;

// Number of work items emit_items would cut `runs` into.
int64_t count_items(const std::vector<Work>& runs, int64_t chunk);

// Build every host-side table of a plan; returns FSDP_OK or an error.
fsdp_status build_plan(fsdp_plan* pl);

// Build the work table that re-shards `from`'s layout into `to`'s.
fsdp_status build_reshard(const fsdp_plan* from, const fsdp_plan* to, fsdp_resharder* rs);

}  // namespace fsdp
