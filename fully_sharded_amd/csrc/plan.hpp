// Internal plan structure of one FSDP unit: shapes, the shard layout, the
// contiguous (rank, shard range, flat range) segments, and the per-workgroup
// work tables the kernels consume.  Host-side; the device copies of the work
// tables are uploaded lazily per device.
#pragma once

#include <cstdint>
#include <map>
#include <mutex>
#include <vector>

#include "fsdp_hip.h"

namespace fsdp {

// One workgroup's contiguous range.  In the shard space (pack,
// reduce-scatter, AdamW) dst indexes the [R][S] shard buffer linearly and
// src the full-unit buffer; in the flat space (gather) dst indexes the
// full-unit buffer and src the shard buffer.  src < 0 marks padding (no
// source: the destination gets +0 / is left as padding).
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

struct DeviceTables {
  Work* shard_work = nullptr;  // device copy of shard_work
  Work* flat_work = nullptr;   // device copy of flat_work
};

}  // namespace fsdp

struct fsdp_plan {
  int32_t R = 0;
  int32_t layout = 0;
  int64_t T = 0;
  int64_t S = 0;
  std::vector<std::vector<int64_t>> shapes;
  std::vector<fsdp::Param> params;
  std::vector<fsdp::Segment> segments;      // ordered by (rank, shard_off)
  std::vector<fsdp::Work> shard_work;       // covers [0, R*S) in order
  std::vector<fsdp::Work> flat_work;        // covers [0, T) in order
  int64_t shard_chunk = 0;                  // max elements per work item
  int64_t flat_chunk = 0;

  mutable std::mutex mu;
  mutable std::map<int, fsdp::DeviceTables> device;  // by HIP device id
};

namespace fsdp {

// Build every host-side table of a plan; returns FSDP_OK or an error.
fsdp_status build_plan(fsdp_plan* pl);

// Device tables for the current device (uploaded on first use).
fsdp_status device_tables(const fsdp_plan* pl, const DeviceTables** out);

}  // namespace fsdp
