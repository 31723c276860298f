// The plan, re-shard and argument-check code of the library, exercised on
// the host under AddressSanitizer and UndefinedBehaviorSanitizer (built by
// tests/test_sanitize_host.py with the kernel launchers stubbed out, see
// launch_stub.cpp).  Through the C ABI only:
//   random N  -- N seeded random units (1-5 parameters of 1-4 dimensions,
//                R in 1..64, both layouts): every plan query, with its
//                invariants (items and segments tile their spaces, the
//                item sources agree with the segments, the ledgers'
//                closed forms), capacity errors, and the re-shard table to
//                another R and layout (every destination element's source
//                holds the same flat element); then every entry point's
//                argument checks, and valid calls that stop at the first
//                device call (there is none).
//   dump R layout n nd_0..nd_{n-1} dims...  -- prints T, S and the segments
//                of one plan, for comparison with the oracle.
// Exit status 0 when every check holds.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string_view>
#include <vector>

#include "fsdp_mi355x.h"

static int g_failures = 0;
#define EXPECT(c)                                                             \
  do {                                                                        \
    if (!(c)) {                                                               \
      std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);       \
      ++g_failures;                                                           \
    }                                                                         \
  } while (0)

struct Unit {
  std::vector<int32_t> nd;
  std::vector<int64_t> dims;
};

static fsdp_plan* make_plan(const Unit& u, int R, int layout) {
  fsdp_plan* p = nullptr;
  const fsdp_status st = fsdp_plan_layout(static_cast<int32_t>(u.nd.size()), u.nd.data(),
                                          u.dims.data(), R, layout, &p);
  EXPECT(st == FSDP_OK);
  return st == FSDP_OK ? p : nullptr;
}

struct Seg {
  int64_t rank, shard_off, flat_off, len;
};

static std::vector<Seg> segments_of(const fsdp_plan* p) {
  fsdp_plan_info info;
  EXPECT(fsdp_plan_get_info(p, &info) == FSDP_OK);
  std::vector<int64_t> raw(4 * static_cast<size_t>(info.n_segments) + 4);
  EXPECT(fsdp_plan_segments(p, raw.data(), info.n_segments) == FSDP_OK);
  if (info.n_segments > 0) EXPECT(fsdp_plan_segments(p, raw.data(), info.n_segments - 1) != FSDP_OK);
  std::vector<Seg> s;
  for (int i = 0; i < info.n_segments; ++i)
    s.push_back({raw[4 * i], raw[4 * i + 1], raw[4 * i + 2], raw[4 * i + 3]});
  return s;
}

static std::vector<int64_t> items_of(const fsdp_plan* p, int space) {
  int64_t n = -1;
  EXPECT(fsdp_plan_work_items(p, space, nullptr, 0, &n) == FSDP_OK);
  std::vector<int64_t> it(3 * static_cast<size_t>(std::max<int64_t>(n, 0)) + 3);
  int64_t m = -1;
  EXPECT(fsdp_plan_work_items(p, space, it.data(), n, &m) == FSDP_OK && m == n);
  if (n > 0) EXPECT(fsdp_plan_work_items(p, space, it.data(), n - 1, &m) != FSDP_OK);
  it.resize(3 * static_cast<size_t>(std::max<int64_t>(n, 0)));
  return it;
}

// Flat index of shard-space position x (-1: padding), from the segments.
static int64_t flat_of(const std::vector<Seg>& seg, int64_t S, int64_t x) {
  const int64_t r = x / S, j = x % S;
  for (const Seg& s : seg)
    if (s.rank == r && j >= s.shard_off && j < s.shard_off + s.len) return s.flat_off + (j - s.shard_off);
  return -1;
}

static void check_plan(const fsdp_plan* p, const Unit& u, int R, int layout) {
  fsdp_plan_info info;
  EXPECT(fsdp_plan_get_info(p, &info) == FSDP_OK);
  const int64_t T = info.numel_full, S = info.shard_numel;
  EXPECT(info.world == R && info.layout == layout);
  EXPECT(info.n_params == static_cast<int32_t>(u.nd.size()));
  // parameters: offsets, rows per shard, the per-parameter shard size
  int64_t off = 0, soff = 0;
  size_t at = 0;
  for (int32_t q = 0; q < info.n_params; ++q) {
    int64_t o[5];
    EXPECT(fsdp_plan_param(p, q, o) == FSDP_OK);
    int64_t numel = 1;
    for (int d = 0; d < u.nd[q]; ++d) numel *= u.dims[at + d];
    const int64_t d0 = u.dims[at];
    at += u.nd[q];
    EXPECT(o[0] == off && o[1] == numel && o[2] == soff);
    EXPECT(o[3] == (d0 + R - 1) / R && o[4] == numel / d0);
    off += numel;
    soff += o[3] * o[4];
  }
  int64_t bad[5];
  EXPECT(fsdp_plan_param(p, info.n_params, bad) != FSDP_OK);
  EXPECT(fsdp_plan_param(p, -1, bad) != FSDP_OK);
  EXPECT(T == off);
  EXPECT(S == (layout == FSDP_LAYOUT_PER_PARAM ? soff : (T + R - 1) / R));
  // valid elements per rank
  int64_t sum = 0, v = 0;
  for (int r = 0; r < R; ++r) {
    EXPECT(fsdp_plan_rank_valid(p, r, &v) == FSDP_OK && v >= 0 && v <= S);
    sum += v;
  }
  EXPECT(sum == T);
  EXPECT(fsdp_plan_rank_valid(p, R, &v) != FSDP_OK);
  // segments tile the flat space once, each inside its rank's shard
  std::vector<Seg> seg = segments_of(p);
  std::vector<Seg> by_flat = seg;
  std::sort(by_flat.begin(), by_flat.end(),
            [](const Seg& a, const Seg& b) { return a.flat_off < b.flat_off; });
  int64_t expect = 0;
  for (const Seg& s : by_flat) {
    EXPECT(s.flat_off == expect && s.len > 0);
    EXPECT(s.rank >= 0 && s.rank < R && s.shard_off >= 0 && s.shard_off + s.len <= S);
    expect += s.len;
  }
  EXPECT(expect == T);
  // shard-space items tile [0, R*S) in order, within 1024-element chunks,
  // and their sources agree with the segments at both ends
  std::vector<int64_t> it = items_of(p, 0);
  int64_t pos = 0;
  for (size_t i = 0; i + 2 < it.size(); i += 3) {
    const int64_t d = it[i], s = it[i + 1], n = it[i + 2];
    EXPECT(d == pos && n > 0 && n <= 1024 && d / 1024 == (d + n - 1) / 1024);
    EXPECT(s == flat_of(seg, S, d));
    EXPECT((s < 0) == (flat_of(seg, S, d + n - 1) < 0));
    if (s >= 0) EXPECT(flat_of(seg, S, d + n - 1) == s + n - 1);
    pos += n;
  }
  EXPECT(pos == R * S);
  // flat-space items tile [0, T); their sources are the same elements
  it = items_of(p, 1);
  pos = 0;
  for (size_t i = 0; i + 2 < it.size(); i += 3) {
    const int64_t d = it[i], s = it[i + 1], n = it[i + 2];
    EXPECT(d == pos && n > 0 && s >= 0 && s + n <= R * S);
    EXPECT(flat_of(seg, S, s) == d && flat_of(seg, S, s + n - 1) == d + n - 1);
    pos += n;
  }
  EXPECT(pos == T);
  int64_t dummy = 0;
  EXPECT(fsdp_plan_work_items(p, 2, nullptr, 0, &dummy) != FSDP_OK);
  // ledgers
  int64_t led[4];
  for (int raf = 0; raf < 2; ++raf) {
    EXPECT(fsdp_plan_comm_ledger(p, raf, led) == FSDP_OK);
    EXPECT(led[0] == (raf ? 2 : 1) * (R - 1) * S && led[1] == (R - 1) * S && led[2] == 0);
    EXPECT(led[3] == led[0] + led[1]);
  }
  EXPECT(fsdp_plan_state_bytes_per_rank(p) == 16 * S);
}

static void check_reshard(const fsdp_plan* a, const fsdp_plan* b) {
  fsdp_resharder* rs = nullptr;
  EXPECT(fsdp_reshard_plan(a, b, &rs) == FSDP_OK);
  if (!rs) return;
  fsdp_plan_info ia, ib;
  fsdp_plan_get_info(a, &ia);
  fsdp_plan_get_info(b, &ib);
  const std::vector<Seg> sa = segments_of(a), sb = segments_of(b);
  int64_t n = -1;
  EXPECT(fsdp_reshard_items(rs, nullptr, 0, &n) == FSDP_OK);
  std::vector<int64_t> it(3 * static_cast<size_t>(std::max<int64_t>(n, 0)) + 3);
  int64_t m = -1;
  EXPECT(fsdp_reshard_items(rs, it.data(), n, &m) == FSDP_OK && m == n);
  if (n > 0) EXPECT(fsdp_reshard_items(rs, it.data(), n - 1, &m) != FSDP_OK);
  int64_t pos = 0;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t d = it[3 * i], s = it[3 * i + 1], len = it[3 * i + 2];
    EXPECT(d == pos && len > 0);
    for (int64_t e : {d, d + len - 1}) {
      const int64_t f = flat_of(sb, ib.shard_numel, e);
      if (s < 0)
        EXPECT(f < 0);
      else
        EXPECT(f >= 0 && flat_of(sa, ia.shard_numel, s + (e - d)) == f);
    }
    pos += len;
  }
  EXPECT(pos == static_cast<int64_t>(ib.world) * ib.shard_numel);
  fsdp_reshard_destroy(rs);
}

static Unit random_unit(std::mt19937_64& rng, int R) {
  Unit u;
  const int np = 1 + static_cast<int>(rng() % 5);
  for (int q = 0; q < np; ++q) {
    const int nd = 1 + static_cast<int>(rng() % 4);
    u.nd.push_back(nd);
    u.dims.push_back(1 + static_cast<int64_t>(rng() % (3 * R + 3)));
    for (int d = 1; d < nd; ++d) u.dims.push_back(1 + static_cast<int64_t>(rng() % 40));
  }
  return u;
}

// Fake device addresses: never dereferenced on the host, 4 GiB apart.
static void* fake(int i, int64_t off = 0) {
  return reinterpret_cast<void*>((uintptr_t{1} << 40) + (uintptr_t(i) << 32) + uintptr_t(off));
}

static void check_entry_points() {
  const Unit u{{2, 1}, {64, 8, 8}};
  fsdp_plan* p = make_plan(u, 4, FSDP_LAYOUT_PER_PARAM);
  fsdp_plan* q = make_plan(u, 2, FSDP_LAYOUT_FLAT);
  if (!p || !q) return;
  const fsdp_adamw_hparams hp{1e-3, 0.9, 0.999, 1e-8, 0.01};
  const fsdp_adamw_hparams bad_b1{1e-3, 1.0, 0.999, 1e-8, 0.01};
  const fsdp_adamw_hparams bad_eps{1e-3, 0.9, 0.999, 0.0, 0.01};
  void* g[4] = {fake(1), fake(2), fake(3), fake(4)};
  void* recv[4] = {fake(10), fake(11), fake(12), fake(13)};
  float* master = static_cast<float*>(fake(20));
  float* m = static_cast<float*>(fake(21));
  float* v = static_cast<float*>(fake(22));
  void* param = fake(23);
  const int E = FSDP_ERR_INVALID_ARG, H = FSDP_ERR_HIP;
  // plan creation
  fsdp_plan* x = reinterpret_cast<fsdp_plan*>(1);
  int32_t nd0[1] = {0}, nd9[1] = {9}, nd1[1] = {1};
  int64_t d0[1] = {0}, d5[1] = {5}, huge[2] = {int64_t(1) << 40, int64_t(1) << 40};
  int32_t nd2[1] = {2};
  EXPECT(fsdp_plan_layout(1, nd0, d5, 2, 0, &x) == E && x == nullptr);
  EXPECT(fsdp_plan_layout(1, nd9, d5, 2, 0, &x) == E);
  EXPECT(fsdp_plan_layout(1, nd1, d0, 2, 0, &x) == E);
  EXPECT(fsdp_plan_layout(1, nd1, d5, 0, 0, &x) == E);
  EXPECT(fsdp_plan_layout(1, nd1, d5, 65, 0, &x) == FSDP_ERR_UNSUPPORTED);
  EXPECT(fsdp_plan_layout(1, nd1, d5, 2, 7, &x) == E);
  EXPECT(fsdp_plan_layout(0, nd1, d5, 2, 0, &x) == E);
  EXPECT(fsdp_plan_layout(1, nd2, huge, 2, 0, &x) != FSDP_OK);
  EXPECT(fsdp_plan_layout(1, nullptr, d5, 2, 0, &x) == E);
  EXPECT(fsdp_plan_layout(1, nd1, d5, 2, 0, nullptr) == E);
  EXPECT(fsdp_plan_get_info(nullptr, nullptr) == E);
  EXPECT(fsdp_plan_state_bytes_per_rank(nullptr) == -1);
  fsdp_plan_destroy(nullptr);
  // pack / gather / reduce-scatter
  EXPECT(fsdp_shard_pack(nullptr, fake(30), FSDP_F32, master, FSDP_F32, nullptr) == E);
  EXPECT(fsdp_shard_pack(p, fake(30), 5, master, FSDP_F32, nullptr) == E);
  EXPECT(fsdp_shard_pack(p, fake(30, 1), FSDP_F32, master, FSDP_F32, nullptr) == E);
  EXPECT(fsdp_shard_pack(p, master, FSDP_F32, fake(20, 4), FSDP_F32, nullptr) == E);
  EXPECT(fsdp_shard_pack(p, fake(30), FSDP_F32, master, FSDP_F32, nullptr) == H);
  EXPECT(fsdp_gather_unflatten(p, param, FSDP_BF16, nullptr, nullptr) == E);
  void* dup[4] = {recv[0], recv[0], recv[2], recv[3]};
  EXPECT(fsdp_gather_unflatten(p, param, FSDP_BF16, dup, nullptr) == E);
  void* into[4] = {param, recv[1], recv[2], recv[3]};
  EXPECT(fsdp_gather_unflatten(p, param, FSDP_BF16, into, nullptr) == E);
  EXPECT(fsdp_gather_unflatten(p, param, FSDP_BF16, recv, nullptr) == H);
  EXPECT(fsdp_reduce_scatter_avg(p, g, FSDP_BF16, nullptr, nullptr) == E);
  EXPECT(fsdp_reduce_scatter_avg(p, g, FSDP_BF16, static_cast<float*>(g[1]), nullptr) == E);
  EXPECT(fsdp_reduce_scatter_avg(p, g, FSDP_BF16, master, nullptr) == H);
  // AdamW, both entry points
  for (int na = 0; na < 2; ++na) {
    auto step = [&](const fsdp_adamw_hparams* h, int64_t t, void* const* gg, int32_t gdt,
                    int32_t rep, float* mm, void* pp) {
      return na ? fsdp_adamw_shard_step_noalloc(p, h, t, gg, gdt, rep, master, mm, v, pp,
                                                FSDP_BF16, nullptr)
                : fsdp_adamw_shard_step(p, h, t, gg, gdt, rep, master, mm, v, pp, FSDP_BF16,
                                        nullptr);
    };
    EXPECT(step(&hp, 0, g, FSDP_BF16, 1, m, param) == E);
    EXPECT(step(&bad_b1, 1, g, FSDP_BF16, 1, m, param) == E);
    EXPECT(step(&bad_eps, 1, g, FSDP_BF16, 1, m, param) == E);
    EXPECT(step(nullptr, 1, g, FSDP_BF16, 1, m, param) == E);
    EXPECT(step(&hp, 1, g, FSDP_BF16, 2, m, param) == E);
    EXPECT(step(&hp, 1, g, FSDP_BF16, 1, master, param) == E);
    EXPECT(step(&hp, 1, g, FSDP_BF16, 1, m, g[0]) == E);
    EXPECT(step(&hp, 1, g, FSDP_BF16, 1, m, fake(23, 1)) == E);
    EXPECT(step(&hp, 1, g, FSDP_BF16, 0, m, param) == E);     // reduced grads must be fp32
    EXPECT(step(&hp, 1, g, FSDP_BF16, 1, m, param) == H);
    EXPECT(step(&hp, 1, g, FSDP_F32, 0, m, param) == H);
  }
  // the paired call
  EXPECT(fsdp_adamw_step_then_gather(p, &hp, 1, g, FSDP_BF16, master, m, v, param, FSDP_BF16,
                                     nullptr, param, recv, nullptr) == E);
  EXPECT(fsdp_adamw_step_then_gather(p, &hp, 1, g, FSDP_BF16, master, m, v, param, FSDP_BF16, p,
                                     param, recv, nullptr) == E);   // reads what it writes
  EXPECT(fsdp_adamw_step_then_gather(p, &hp, 1, g, FSDP_BF16, master, m, v, param, FSDP_BF16, p,
                                     fake(31), recv, nullptr) == H);
  // re-shard, accumulation, all-reduce
  fsdp_resharder* rs = nullptr;
  EXPECT(fsdp_reshard_plan(p, nullptr, &rs) == E && rs == nullptr);
  const Unit other{{1}, {64}};
  fsdp_plan* o = make_plan(other, 2, FSDP_LAYOUT_FLAT);
  EXPECT(fsdp_reshard_plan(p, o, &rs) == E);
  fsdp_plan_destroy(o);
  EXPECT(fsdp_reshard_plan(p, q, &rs) == FSDP_OK);
  EXPECT(fsdp_reshard(rs, fake(40), fake(40, 8), FSDP_F32, nullptr) == E);   // overlap
  EXPECT(fsdp_reshard(rs, fake(40), fake(41), 9, nullptr) == E);
  EXPECT(fsdp_reshard(rs, fake(40), fake(41), FSDP_F32, nullptr) == H);
  void* srcs[2] = {fake(42), fake(43)};
  void* dsts[2] = {fake(44), fake(44)};
  EXPECT(fsdp_reshard_batch(rs, 2, srcs, dsts, FSDP_F32, nullptr) == E);
  EXPECT(fsdp_reshard_batch(rs, 65, srcs, dsts, FSDP_F32, nullptr) != FSDP_OK);
  void* dsts2[2] = {fake(44), fake(45)};
  EXPECT(fsdp_reshard_batch(rs, 2, srcs, dsts2, FSDP_F32, nullptr) == H);
  fsdp_reshard_destroy(rs);
  float* acc[4] = {static_cast<float*>(fake(50)), static_cast<float*>(fake(51)),
                   static_cast<float*>(fake(52)), static_cast<float*>(fake(53))};
  EXPECT(fsdp_grad_accumulate(p, g, FSDP_BF16, acc, 2, nullptr) == E);
  float* acc_dup[4] = {acc[0], acc[0], acc[2], acc[3]};
  EXPECT(fsdp_grad_accumulate(p, g, FSDP_BF16, acc_dup, 1, nullptr) == E);
  EXPECT(fsdp_grad_accumulate(p, g, FSDP_BF16, acc, 1, nullptr) == H);
  void* out[4] = {fake(60), fake(61), fake(62), g[0]};
  EXPECT(fsdp_allreduce_avg(p, g, FSDP_BF16, out, FSDP_F32, nullptr) == E);
  out[3] = fake(63);
  EXPECT(fsdp_allreduce_avg(p, g, FSDP_BF16, out, FSDP_F32, nullptr) == H);
  // the step graph's checks (creation needs a device)
  fsdp_step_graph* sg = reinterpret_cast<fsdp_step_graph*>(1);
  EXPECT(fsdp_step_graph_create(&bad_eps, &sg) == E && sg == nullptr);
  EXPECT(fsdp_step_graph_create(&hp, &sg) != FSDP_OK);
  EXPECT(fsdp_step_graph_add_gather(nullptr, p, param, FSDP_BF16, recv) == E);
  EXPECT(fsdp_step_graph_launch(nullptr, 1, nullptr) == E);
  fsdp_step_graph_destroy(nullptr);
  // status strings
  for (int32_t s = -5; s <= 1; ++s) EXPECT(fsdp_status_string(s) != nullptr);
  fsdp_plan_destroy(p);
  fsdp_plan_destroy(q);
}

int main(int argc, char** argv) {
  if (argc >= 3 && std::string_view(argv[1]) == "random") {
    const int n = std::atoi(argv[2]);
    std::mt19937_64 rng(20261203);
    const int Rs[] = {1, 2, 3, 4, 5, 7, 8, 13, 16, 64};
    for (int i = 0; i < n; ++i) {
      const int R = Rs[i % 10];
      const int layout = (i / 10) % 2;
      const Unit u = random_unit(rng, R);
      fsdp_plan* p = make_plan(u, R, layout);
      if (!p) continue;
      check_plan(p, u, R, layout);
      const int R2 = Rs[(i * 7 + 3) % 10];
      fsdp_plan* p2 = make_plan(u, R2, 1 - layout);
      if (p2) {
        check_plan(p2, u, R2, 1 - layout);
        check_reshard(p, p2);
        check_reshard(p2, p);
        fsdp_plan_destroy(p2);
      }
      fsdp_plan_destroy(p);
    }
    check_entry_points();
    std::printf("checked %d random units, failures %d\n", n, g_failures);
    return g_failures == 0 ? 0 : 1;
  }
  if (argc >= 4 && std::string_view(argv[1]) == "dump") {
    const int R = std::atoi(argv[2]), layout = std::atoi(argv[3]);
    const int np = std::atoi(argv[4]);
    Unit u;
    int a = 5;
    for (int q = 0; q < np; ++q) u.nd.push_back(std::atoi(argv[a++]));
    while (a < argc) u.dims.push_back(std::atoll(argv[a++]));
    fsdp_plan* p = make_plan(u, R, layout);
    if (!p) return 1;
    check_plan(p, u, R, layout);
    fsdp_plan_info info;
    fsdp_plan_get_info(p, &info);
    std::printf("%lld %lld\n", static_cast<long long>(info.numel_full),
                static_cast<long long>(info.shard_numel));
    for (const Seg& s : segments_of(p))
      std::printf("%lld %lld %lld %lld\n", static_cast<long long>(s.rank),
                  static_cast<long long>(s.shard_off), static_cast<long long>(s.flat_off),
                  static_cast<long long>(s.len));
    fsdp_plan_destroy(p);
    return g_failures == 0 ? 0 : 1;
  }
  std::fprintf(stderr, "usage: %s random N | dump R layout n nd... dims...\n", argv[0]);
  return 2;
}
