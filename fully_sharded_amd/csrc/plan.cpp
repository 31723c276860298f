// Host-side planning of one FSDP unit: the shard layout, its contiguous
// segments and the per-workgroup work tables.
//
// Layout rules ("Understanding FSDP from source" 2.1; "FSDP Transformer
// Block Sharding Example", 4-GPU shard layout):
//   per-parameter (FSDP2): k_p = ceil(d0_p / R) rows per shard, rank r owns
//     rows [min(r k_p, d0_p), min((r+1) k_p, d0_p)); its pieces sit one after
//     the other in parameter order, each padded to k_p * row_p elements.
//   flat (FSDP1): S = ceil(T / R), rank r owns [r S, min((r+1) S, T)).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>

#include "plan.hpp"

namespace fsdp {
namespace {

// Elements per work item (one workgroup): exactly one pass of its 256
// lanes, at every size -- 1024 for the 4-element lanes of the arithmetic
// kernels (shard space), 2048 for the 16-byte lanes of the bf16 copy (flat
// space).  Workgroups are dispatched in order, so the ones in flight then
// cover one compact window of every stream; giving each workgroup 16
// consecutive passes spread the in-flight window over ~60 MB per stream and
// cost 8% on an 872M-element unit (5.27 vs 5.68 TB/s), and even 2 passes
// cost 7% on a 3M-element one.
constexpr int64_t kShardChunk = 1024;
constexpr int64_t kFlatChunk = 2048;

// Append [dst, dst+len) <- [src, src+len) as work items cut at multiples of
// chunk in the destination index space.
void emit(std::vector<Work>& out, int64_t dst, int64_t src, int64_t len, int64_t chunk) {
  while (len > 0) {
    const int64_t next = (dst / chunk + 1) * chunk;
    const int64_t n = std::min(len, next - dst);
    out.push_back(Work{dst, src < 0 ? -1 : src, n});
    dst += n;
    if (src >= 0) src += n;
    len -= n;
  }
}

// Append a run to a list of runs, merging it with the previous one when both
// are contiguous in the destination and (both padding or) contiguous in the
// source.
void push_run(std::vector<Work>& runs, int64_t dst, int64_t src, int64_t len) {
  if (len <= 0) return;
  if (!runs.empty()) {
    Work& b = runs.back();
    const bool dst_next = b.dst + b.len == dst;
    const bool both_pad = b.src < 0 && src < 0;
    const bool src_next = b.src >= 0 && src >= 0 && b.src + b.len == src;
    if (dst_next && (both_pad || src_next)) {
      b.len += len;
      return;
    }
  }
  runs.push_back(Work{dst, src < 0 ? -1 : src, len});
}

}  // namespace

fsdp_status build_plan(fsdp_plan* pl) {
  const int64_t R = pl->R;
  // parameters
  int64_t off = 0, soff = 0;
  for (const auto& shape : pl->shapes) {
    Param p{};
    p.numel = 1;
    for (int64_t d : shape) {
      if (p.numel > (int64_t(1) << 62) / d) return FSDP_ERR_INVALID_ARG;
      p.numel *= d;
    }
    p.d0 = shape[0];
    p.row = p.numel / p.d0;
    p.k = (p.d0 + R - 1) / R;
    p.flat_off = off;
    p.shard_off = soff;
    off += p.numel;
    soff += p.k * p.row;
    if (off > (int64_t(1) << 62) || soff > (int64_t(1) << 62)) return FSDP_ERR_INVALID_ARG;
    pl->params.push_back(p);
  }
  pl->T = off;
  pl->S = pl->layout == FSDP_LAYOUT_PER_PARAM ? soff : (off + R - 1) / R;
  if (pl->S > (int64_t(1) << 62) / R) return FSDP_ERR_INVALID_ARG;

  // segments, ordered by (rank, shard offset), merged inside a rank
  for (int64_t r = 0; r < R; ++r) {
    auto add = [&](int64_t shard_off, int64_t flat_off, int64_t len) {
      if (len <= 0) return;
      if (!pl->segments.empty()) {
        Segment& b = pl->segments.back();
        if (b.rank == r && b.shard_off + b.len == shard_off && b.flat_off + b.len == flat_off) {
          b.len += len;
          return;
        }
      }
      pl->segments.push_back(Segment{r, shard_off, flat_off, len});
    };
    if (pl->layout == FSDP_LAYOUT_PER_PARAM) {
      for (const Param& p : pl->params) {
        const int64_t lo = std::min(r * p.k, p.d0);
        const int64_t hi = std::min(lo + p.k, p.d0);
        add(p.shard_off, p.flat_off + lo * p.row, (hi - lo) * p.row);
      }
    } else {
      const int64_t lo = std::min(r * pl->S, pl->T);
      const int64_t hi = std::min(lo + pl->S, pl->T);
      add(0, lo, hi - lo);
    }
  }

  // shard-space runs: every position of [0, R*S), pieces and padding
  std::vector<Work> runs;
  {
    size_t i = 0;
    for (int64_t r = 0; r < R; ++r) {
      int64_t pos = 0;
      for (; i < pl->segments.size() && pl->segments[i].rank == r; ++i) {
        const Segment& s = pl->segments[i];
        push_run(runs, r * pl->S + pos, -1, s.shard_off - pos);
        push_run(runs, r * pl->S + s.shard_off, s.flat_off, s.len);
        pos = s.shard_off + s.len;
      }
      push_run(runs, r * pl->S + pos, -1, pl->S - pos);
    }
  }
  pl->shard_chunk = kShardChunk;
  for (const Work& w : runs) emit(pl->shard_work, w.dst, w.src, w.len, pl->shard_chunk);

  // flat-space runs: the same segments ordered by flat offset; they tile
  // [0, T) exactly
  std::vector<Segment> by_flat = pl->segments;
  std::sort(by_flat.begin(), by_flat.end(),
            [](const Segment& a, const Segment& b) { return a.flat_off < b.flat_off; });
  runs.clear();
  int64_t expect = 0;
  for (const Segment& s : by_flat) {
    if (s.flat_off != expect) return FSDP_ERR_INVALID_ARG;  // cannot happen
    push_run(runs, s.flat_off, s.rank * pl->S + s.shard_off, s.len);
    expect += s.len;
  }
  if (expect != pl->T) return FSDP_ERR_INVALID_ARG;
  pl->flat_chunk = kFlatChunk;
  for (const Work& w : runs) emit(pl->flat_work, w.dst, w.src, w.len, pl->flat_chunk);
  return FSDP_OK;
}

fsdp_status device_tables(const fsdp_plan* pl, const DeviceTables** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FSDP_ERR_HIP;
  std::lock_guard<std::mutex> lock(pl->mu);
  auto it = pl->device.find(dev);
  if (it != pl->device.end()) {
    *out = &it->second;
    return FSDP_OK;
  }
  const size_t n_shard = pl->shard_work.size();
  const size_t n_flat = pl->flat_work.size();
  void* mem = nullptr;
  if (hipMalloc(&mem, (n_shard + n_flat) * sizeof(Work)) != hipSuccess) {
    (void)hipGetLastError();
    return FSDP_ERR_OUT_OF_MEMORY;
  }
  Work* w = static_cast<Work*>(mem);
  if (hipMemcpy(w, pl->shard_work.data(), n_shard * sizeof(Work), hipMemcpyHostToDevice) !=
          hipSuccess ||
      hipMemcpy(w + n_shard, pl->flat_work.data(), n_flat * sizeof(Work),
                hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(mem);
    return FSDP_ERR_HIP;
  }
  DeviceTables t;
  t.shard_work = w;
  t.flat_work = w + n_shard;
  auto res = pl->device.emplace(dev, t);
  *out = &res.first->second;
  return FSDP_OK;
}

}  // namespace fsdp
