// Host-side planning of one FSDP unit: the shard layout, its contiguous
// segments and the per-workgroup work tables; and the table that re-shards
// one plan's layout into another's.
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

void emit_items(const std::vector<Work>& runs, int64_t chunk, std::vector<Work>& out) {
  for (const Work& w : runs) {
    int64_t dst = w.dst, src = w.src, len = w.len;
    while (len > 0) {
      const int64_t next = (dst / chunk + 1) * chunk;
      const int64_t n = std::min(len, next - dst);
      out.push_back(Work{dst, src < 0 ? -1 : src, n});
      dst += n;
      if (src >= 0) src += n;
      len -= n;
    }
  }
}

int64_t count_items(const std::vector<Work>& runs, int64_t chunk) {
  int64_t n = 0;
  for (const Work& w : runs)
    if (w.len > 0) n += (w.dst + w.len - 1) / chunk - w.dst / chunk + 1;
  return n;
}

fsdp_status WorkTable::device(const Work** out) const {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return FSDP_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(mu_);
  auto it = dev_.find(dev);
  if (it != dev_.end()) {
    *out = it->second;
    return FSDP_OK;
  }
  const size_t bytes = std::max<size_t>(1, host.size()) * sizeof(Work);
  void* mem = nullptr;
  if (hipMalloc(&mem, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return FSDP_ERR_OUT_OF_MEMORY;
  }
  if (!host.empty() &&
      hipMemcpy(mem, host.data(), host.size() * sizeof(Work), hipMemcpyHostToDevice) !=
          hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(mem);
    return FSDP_ERR_HIP;
  }
  dev_.emplace(dev, static_cast<Work*>(mem));
  *out = static_cast<Work*>(mem);
  return FSDP_OK;
}

void WorkTable::release() {
  std::lock_guard<std::mutex> lock(mu_);
  for (auto& kv : dev_) (void)hipFree(kv.second);
  dev_.clear();
}

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
  {
    size_t i = 0;
    for (int64_t r = 0; r < R; ++r) {
      int64_t pos = 0;
      for (; i < pl->segments.size() && pl->segments[i].rank == r; ++i) {
        const Segment& s = pl->segments[i];
        push_run(pl->shard_runs, r * pl->S + pos, -1, s.shard_off - pos);
        push_run(pl->shard_runs, r * pl->S + s.shard_off, s.flat_off, s.len);
        pos = s.shard_off + s.len;
      }
      push_run(pl->shard_runs, r * pl->S + pos, -1, pl->S - pos);
    }
  }
  if (count_items(pl->shard_runs, kShardChunk) > kMaxItems) return FSDP_ERR_UNSUPPORTED;
  emit_items(pl->shard_runs, kShardChunk, pl->shard_work.host);

  // flat-space runs: the same segments ordered by flat offset; they tile
  // [0, T) exactly
  std::vector<Segment> by_flat = pl->segments;
  std::sort(by_flat.begin(), by_flat.end(),
            [](const Segment& a, const Segment& b) { return a.flat_off < b.flat_off; });
  int64_t expect = 0;
  for (const Segment& s : by_flat) {
    if (s.flat_off != expect) return FSDP_ERR_INVALID_ARG;  // cannot happen
    push_run(pl->flat_runs, s.flat_off, s.rank * pl->S + s.shard_off, s.len);
    expect += s.len;
  }
  if (expect != pl->T) return FSDP_ERR_INVALID_ARG;
  pl->gather_lane_bytes =
      pl->T <= kWideGatherMax || (R == 8 && pl->T <= kWideGatherMaxR8) ? 16 : 8;
  const int64_t flat_chunk = pl->gather_lane_bytes == 16 ? kFlatChunk : kFlatChunk / 2;
  if (count_items(pl->flat_runs, flat_chunk) > kMaxItems) return FSDP_ERR_UNSUPPORTED;
  emit_items(pl->flat_runs, flat_chunk, pl->flat_work.host);
  return FSDP_OK;
}

fsdp_status build_reshard(const fsdp_plan* from, const fsdp_plan* to, fsdp_resharder* rs) {
  if (from->shapes != to->shapes) return FSDP_ERR_INVALID_ARG;
  rs->R_from = from->R;
  rs->R_to = to->R;
  rs->T = from->T;
  rs->S_from = from->S;
  rs->S_to = to->S;
  // Destination: `to`'s shard space, runs in order (pieces map to flat
  // offsets, padding has none).  Each piece's flat range is looked up in
  // `from`'s flat runs (which tile [0, T) in order), split where those runs
  // end.
  const std::vector<Work>& fr = from->flat_runs;
  std::vector<Work> runs;
  for (const Work& d : to->shard_runs) {
    if (d.src < 0) {
      push_run(runs, d.dst, -1, d.len);
      continue;
    }
    int64_t f = d.src, dst = d.dst, left = d.len;
    // first run of `from` whose flat range ends after f
    size_t k = static_cast<size_t>(
        std::upper_bound(fr.begin(), fr.end(), f,
                         [](int64_t x, const Work& w) { return x < w.dst + w.len; }) -
        fr.begin());
    while (left > 0) {
      if (k >= fr.size()) return FSDP_ERR_INVALID_ARG;  // cannot happen
      const Work& s = fr[k];
      const int64_t take = std::min(left, s.dst + s.len - f);
      push_run(runs, dst, s.src + (f - s.dst), take);
      dst += take;
      f += take;
      left -= take;
      ++k;
    }
  }
  if (count_items(runs, kFlatChunk) > kMaxItems) return FSDP_ERR_UNSUPPORTED;
  emit_items(runs, kFlatChunk, rs->work.host);
  return FSDP_OK;
}

}  // namespace fsdp
