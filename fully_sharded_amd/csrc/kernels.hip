// gfx950 kernels of the FSDP data-parallel hot path.
//
// All of them stream through HBM with no data reuse, so each is bound by
// HBM bandwidth, not by arithmetic.  Design, as measured on MI355X:
//   * one workgroup (256 lanes) owns one work item: a contiguous range that
//     never crosses a shard/parameter boundary, so the source offset is one
//     constant per workgroup;
//   * the arithmetic kernels move 4 consecutive elements per lane per pass
//     (8-byte bf16 and 16-byte fp32 accesses), the copy kernels 16 bytes per
//     lane; 4 elements per lane beat 8 because twice as many waves keep
//     requests in flight for the same registers.  At R >= 8 the fused step
//     takes one element per lane in short launches of its own
//     (k_fused_one) and two adjacent ones in longer launches and in the
//     launch it shares with a gather (k_fused_pair, k_fused_two_gather);
//     so do short launches at R = 3 and 4, and the short reduce-scatter
//     (R >= 8) and AdamW launches: where those measured faster;
//   * every streaming access is nontemporal: the data is touched once, and
//     keeping it out of the caches raised the fused kernel from 4.8 to
//     5.6 TB/s in isolation (the overlapping word pairs of misaligned
//     windows below are the exception);
//   * work items whose source is misaligned relative to the destination
//     funnel each lane's window out of two aligned vector loads; lanes
//     whose chunk is cut by the ends of the range take an element-by-element
//     path with the same arithmetic;
//   * long fused, unfused AdamW and all-reduce launches cap their resident
//     workgroups per CU (fused_lds, adamw_lds, allreduce_lds), and a fused
//     step of up to 65,536 work items can share its launch with the next
//     unit's gather (k_fused_two_gather at R >= 8, else k_fused_gather),
//     which then starts while the step drains.
//
// Reductions are fp32, in rank order 0..R-1 starting from rank 0's value,
// then one correctly rounded division by R: one lane owns an element and
// nothing is reassociated, so results are deterministic and independent of
// the launch shape.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace fsdp {
namespace {

constexpr int kThreads = 256;
constexpr int kEPL = 4;  // elements per lane per pass, arithmetic kernels
// A grid dimension holds at most 2^32 - 1 lanes.
constexpr int64_t kMaxBlocks = 0xFFFFFFFFLL / kThreads;

// Pointer arrays passed by value in the kernel arguments.  Kernels
// specialised for R <= 8 carry 8 slots, the others FSDP_MAX_RANKS: the
// argument block is copied at every launch, and the smaller one took ~1% off
// the 12-layer step (403.2 vs 407.0 us) and the fused kernel (24.40 vs 24.67
// us).
template <int N>
struct Ptrs {
  const void* p[N];
};
constexpr int ptr_cap(int rt) { return rt > 0 && rt <= kSmallPtrs ? kSmallPtrs : FSDP_MAX_RANKS; }

template <int N>
Ptrs<N> narrow(const PtrArray& a) {
  Ptrs<N> r{};
  for (int i = 0; i < N; ++i) r.p[i] = a.p[i];
  return r;
}

using u16 = uint16_t;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------ nontemporal access
__device__ __forceinline__ u32x2 ld_nt8(const void* p) {
  return __builtin_nontemporal_load(static_cast<const u32x2*>(p));
}
__device__ __forceinline__ u32x4 ld_nt16(const void* p) {
  return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st_nt8(void* p, u32x2 x) {
  __builtin_nontemporal_store(x, static_cast<u32x2*>(p));
}
__device__ __forceinline__ void st_nt16(void* p, u32x4 x) {
  __builtin_nontemporal_store(x, static_cast<u32x4*>(p));
}

// Misaligned source windows.  A work item whose source offset is not a
// multiple of the lane's element count relative to its destination still
// takes vector loads: the W bytes a lane needs start k elements past an
// aligned W-byte word, so it loads that word and the next one and funnels
// the wanted bytes out of the pair (v_alignbit).  Both words hold at least
// one element the lane needs, so nothing outside them is read and no extra
// page is touched.  A lane's second word is its neighbour's first, so these
// two loads are ordinary cached loads, not nontemporal ones: on the R = 3
// hidden-512 block (every rank but 0 misaligned) the step took 28.7-29.1
// instead of 29.6-29.8 us, the fused kernel 21.0-21.3 instead of 21.5-21.7
// (the standalone reduce-scatter 8.8 instead of 8.6), alternating A/B runs.
template <int NW, int Q>
__device__ __forceinline__ void funnel_words(const uint32_t (&w)[2 * NW], uint32_t shift,
                                             uint32_t (&r)[NW]) {
#pragma unroll
  for (int j = 0; j < NW; ++j) r[j] = __builtin_amdgcn_alignbit(w[j + Q + 1], w[j + Q], shift);
}

// Words [byte, byte + 4*NW) of the 2*NW-word window w (byte uniform).
template <int NW>
__device__ __forceinline__ void funnel(const uint32_t (&w)[2 * NW], int byte, uint32_t (&r)[NW]) {
  const uint32_t shift = static_cast<uint32_t>(byte & 3) * 8u;
  switch (byte >> 2) {
    case 0: funnel_words<NW, 0>(w, shift, r); break;
    case 1: funnel_words<NW, 1>(w, shift, r); break;
    default:
      if constexpr (NW == 4) {
        if ((byte >> 2) == 2)
          funnel_words<NW, 2>(w, shift, r);
        else
          funnel_words<NW, 3>(w, shift, r);
      }
      break;
  }
}

// 8 or 16 bytes starting `byte` bytes (0 < byte < W, element-aligned) past
// the W-aligned address p.
__device__ __forceinline__ u32x2 ld8_shifted(const char* p, int byte) {
  const u32x2 a = *reinterpret_cast<const u32x2*>(p);
  const u32x2 b = *reinterpret_cast<const u32x2*>(p + 8);
  const uint32_t w[4] = {a.x, a.y, b.x, b.y};
  uint32_t r[2];
  funnel<2>(w, byte, r);
  return u32x2{r[0], r[1]};
}
__device__ __forceinline__ u32x4 ld16_shifted(const char* p, int byte) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(p);
  const u32x4 b = *reinterpret_cast<const u32x4*>(p + 16);
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t r[4];
  funnel<4>(w, byte, r);
  return u32x4{r[0], r[1], r[2], r[3]};
}

// ------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round to nearest, ties to even; NaN stays NaN (quiet bit set, sign kept);
// values beyond the largest bf16 become infinity.
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// 4 elements of T <-> 4 floats.  vec: one aligned nontemporal access;
// otherwise element by element.
template <typename T>
struct Io;

template <>
struct Io<float> {
  __device__ __forceinline__ static void load4(const float* p, bool vec, float (&x)[4]) {
    if (vec) {
      const u32x4 u = ld_nt16(p);
      x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
      x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) x[k] = p[k];
    }
  }
  __device__ __forceinline__ static void store4(float* p, bool vec, const float (&x)[4]) {
    if (vec) {
      u32x4 u;
      u.x = __float_as_uint(x[0]); u.y = __float_as_uint(x[1]);
      u.z = __float_as_uint(x[2]); u.w = __float_as_uint(x[3]);
      st_nt16(p, u);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) p[k] = x[k];
    }
  }
  // elements [s, s+4) with s % 4 == k != 0
  __device__ __forceinline__ static void load4s(const float* p, int64_t s, int k, float (&x)[4]) {
    const u32x4 u = ld16_shifted(reinterpret_cast<const char*>(p + (s - k)), 4 * k);
    x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
  }
  __device__ __forceinline__ static float load1(const float* p) { return *p; }
  __device__ __forceinline__ static void store1(float* p, float x) { *p = x; }
};

template <>
struct Io<u16> {
  __device__ __forceinline__ static void load4(const u16* p, bool vec, float (&x)[4]) {
    if (vec) {
      const u32x2 u = ld_nt8(p);
      x[0] = __uint_as_float(u.x << 16); x[1] = __uint_as_float(u.x & 0xffff0000u);
      x[2] = __uint_as_float(u.y << 16); x[3] = __uint_as_float(u.y & 0xffff0000u);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) x[k] = bf16_to_f32(p[k]);
    }
  }
  __device__ __forceinline__ static void store4(u16* p, bool vec, const float (&x)[4]) {
    if (vec) {
      u32x2 u;
      u.x = f32_to_bf16(x[0]) | (f32_to_bf16(x[1]) << 16);
      u.y = f32_to_bf16(x[2]) | (f32_to_bf16(x[3]) << 16);
      st_nt8(p, u);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) p[k] = static_cast<u16>(f32_to_bf16(x[k]));
    }
  }
  // elements [s, s+4) with s % 4 == k != 0
  __device__ __forceinline__ static void load4s(const u16* p, int64_t s, int k, float (&x)[4]) {
    const u32x2 u = ld8_shifted(reinterpret_cast<const char*>(p + (s - k)), 2 * k);
    x[0] = __uint_as_float(u.x << 16); x[1] = __uint_as_float(u.x & 0xffff0000u);
    x[2] = __uint_as_float(u.y << 16); x[3] = __uint_as_float(u.y & 0xffff0000u);
  }
  __device__ __forceinline__ static float load1(const u16* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store1(u16* p, float x) {
    *p = static_cast<u16>(f32_to_bf16(x));
  }
};

// ------------------------------------------------- one element per lane
// A second form of the fused step for short launches at R >= 8
// (fused_one_lane) gives each lane one element (every access one naturally
// aligned 2- or 4-byte element, so no alignment case exists) and each
// 1024-element work item four workgroups.  A wave's float64 arithmetic
// after its loads return is then a quarter of what it is with four elements
// per lane, and that arithmetic of the last workgroups is what a short
// launch waits for at its end.  Measured on MI355X, back-to-back launches
// on the 12-layer model's 3.1M-element units (R = 8, bf16 gradients): 23.15
// against 24.05 us.  In the reduce-scatter and AdamW kernels alone, in the
// launch shared with a gather, in long capped launches at R >= 8 and in
// short ones at R = 3 and 4, two adjacent elements per lane measured
// faster (paired: 31.2 us, against 31.8 with one or four).
template <typename T>
struct One;
template <>
struct One<float> {
  __device__ __forceinline__ static float load(const float* p) {
    return __builtin_nontemporal_load(p);
  }
  __device__ __forceinline__ static void store(float* p, float x) {
    __builtin_nontemporal_store(x, p);
  }
};
template <>
struct One<u16> {
  __device__ __forceinline__ static float load(const u16* p) {
    return bf16_to_f32(__builtin_nontemporal_load(p));
  }
  __device__ __forceinline__ static void store(u16* p, float x) {
    __builtin_nontemporal_store(static_cast<u16>(f32_to_bf16(x)), p);
  }
};

// Two adjacent elements [e, e + 2) of T <-> 2 floats, e even: one naturally
// aligned nontemporal access of 4 (bf16) or 8 (fp32) bytes.
template <typename T>
struct Two;
template <>
struct Two<float> {
  __device__ __forceinline__ static void load(const float* p, float (&x)[2]) {
    const u32x2 u = ld_nt8(p);
    x[0] = __uint_as_float(u.x);
    x[1] = __uint_as_float(u.y);
  }
  __device__ __forceinline__ static void store(float* p, const float (&x)[2]) {
    st_nt8(p, u32x2{__float_as_uint(x[0]), __float_as_uint(x[1])});
  }
};
template <>
struct Two<u16> {
  __device__ __forceinline__ static void load(const u16* p, float (&x)[2]) {
    const uint32_t u = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    x[0] = __uint_as_float(u << 16);
    x[1] = __uint_as_float(u & 0xffff0000u);
  }
  __device__ __forceinline__ static void store(u16* p, const float (&x)[2]) {
    __builtin_nontemporal_store(f32_to_bf16(x[0]) | (f32_to_bf16(x[1]) << 16),
                                reinterpret_cast<uint32_t*>(p));
  }
};

// Workgroups per shard-space work item in the one-element form: item
// b / kSplit, its elements [(b % kSplit) * 256, + 256).
constexpr int kSplit = 1024 / kThreads;

// Ask for the work descriptor and the data pointers in scalar registers at
// the top of a kernel, in one asm statement: the compiler then issues all
// of their scalar loads in one round after the kernel arguments', where it
// otherwise loads the descriptor's length, tests it, and only then loads
// its offsets and the pointers -- one more memory round trip before the
// first data load of every workgroup.  One statement, because each
// volatile asm is a scheduling barrier: with one per value the loads for
// the later ones were issued a round after the descriptor's.  An empty asm
// statement: no instruction is emitted.
template <int RT, bool REC, typename A>
__device__ __forceinline__ void args_in_sgprs(const Work& w, const A& a) {
  // REC: the address of the scalar record too (the record itself is only
  // needed for the arithmetic, so its load is not waited for here)
  const void* rec = REC ? static_cast<const void*>(a.scp) : static_cast<const void*>(a.param);
  if constexpr (RT == 8) {
    asm volatile("" ::"s"(w.dst), "s"(w.src), "s"(w.len), "s"(a.g.p[0]), "s"(a.g.p[1]),
                 "s"(a.g.p[2]), "s"(a.g.p[3]), "s"(a.g.p[4]), "s"(a.g.p[5]), "s"(a.g.p[6]),
                 "s"(a.g.p[7]), "s"(a.master), "s"(a.m), "s"(a.v), "s"(a.param), "s"(rec));
  } else if constexpr (RT == 3) {
    asm volatile("" ::"s"(w.dst), "s"(w.src), "s"(w.len), "s"(a.g.p[0]), "s"(a.g.p[1]),
                 "s"(a.g.p[2]), "s"(a.master), "s"(a.m), "s"(a.v), "s"(a.param), "s"(rec));
  } else if constexpr (RT == 4) {
    asm volatile("" ::"s"(w.dst), "s"(w.src), "s"(w.len), "s"(a.g.p[0]), "s"(a.g.p[1]),
                 "s"(a.g.p[2]), "s"(a.g.p[3]), "s"(a.master), "s"(a.m), "s"(a.v), "s"(a.param),
                 "s"(rec));
  } else {
    asm volatile("" ::"s"(w.dst), "s"(w.src), "s"(w.len), "s"(a.master), "s"(a.m), "s"(a.v),
                 "s"(a.param), "s"(rec));
  }
}

// (g_0[s] + g_1[s] + ... + g_{R-1}[s]) / R, fp32, left to right, every
// load issued before the first add.
template <typename G, int RT, typename PA>
__device__ __forceinline__ float grad_avg_one(const PA& g, int R, int64_t s) {
  if constexpr (RT > 0) {
    float x[RT];
#pragma unroll
    for (int q = 0; q < RT; ++q) x[q] = One<G>::load(static_cast<const G*>(g.p[q]) + s);
    float acc = x[0];
#pragma unroll
    for (int q = 1; q < RT; ++q) acc = acc + x[q];
    return acc / static_cast<float>(RT);
  } else {
    float acc = One<G>::load(static_cast<const G*>(g.p[0]) + s);
#pragma unroll 8
    for (int q = 1; q < R; ++q) acc = acc + One<G>::load(static_cast<const G*>(g.p[q]) + s);
    return acc / static_cast<float>(R);
  }
}

// The same for the two adjacent elements s, s + 1 (s even), each replica's
// pair in one access.
template <typename G, int RT, typename PA>
__device__ __forceinline__ void grad_avg_two(const PA& g, int R, int64_t s, float (&avg)[2]) {
  if constexpr (RT > 0) {
    float x[RT][2];
#pragma unroll
    for (int q = 0; q < RT; ++q) Two<G>::load(static_cast<const G*>(g.p[q]) + s, x[q]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float acc = x[0][j];
#pragma unroll
      for (int q = 1; q < RT; ++q) acc = acc + x[q][j];
      avg[j] = acc / static_cast<float>(RT);
    }
  } else {
    float acc[2];
    Two<G>::load(static_cast<const G*>(g.p[0]) + s, acc);
#pragma unroll 8
    for (int q = 1; q < R; ++q) {
      float x[2];
      Two<G>::load(static_cast<const G*>(g.p[q]) + s, x);
      acc[0] = acc[0] + x[0];
      acc[1] = acc[1] + x[1];
    }
    avg[0] = acc[0] / static_cast<float>(R);
    avg[1] = acc[1] / static_cast<float>(R);
  }
}

// ------------------------------------------------------ rank-order average
// avg[k] = (g_0[s+k] + g_1[s+k] + ... + g_{R-1}[s+k]) / R, fp32, left to
// right.  RT > 0: R known at compile time (all R loads issued before the
// adds); RT == 0: any R.
template <typename G, int RT, bool SHIFT = false, typename PA>
__device__ __forceinline__ void grad_load4(const PA& g, int q, int64_t s, int k, float (&x)[4]) {
  const G* p = static_cast<const G*>(g.p[q]);
  if constexpr (SHIFT)
    Io<G>::load4s(p, s, k, x);
  else
    Io<G>::load4(p + s, true, x);
}

// SHIFT: s % 4 == k != 0 (misaligned source, funnelled vector loads).
template <typename G, int RT, bool SHIFT = false, typename PA>
__device__ __forceinline__ void grad_avg4(const PA& g, int R, int64_t s, int k, float (&avg)[4]) {
  if constexpr (RT > 0) {
    float x[RT][4];
#pragma unroll
    for (int q = 0; q < RT; ++q) grad_load4<G, RT, SHIFT>(g, q, s, k, x[q]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float acc = x[0][j];
#pragma unroll
      for (int q = 1; q < RT; ++q) acc = acc + x[q][j];
      avg[j] = acc / static_cast<float>(RT);
    }
  } else {
    grad_load4<G, RT, SHIFT>(g, 0, s, k, avg);
    for (int q = 1; q < R; ++q) {
      float x[4];
      grad_load4<G, RT, SHIFT>(g, q, s, k, x);
#pragma unroll
      for (int j = 0; j < 4; ++j) avg[j] = avg[j] + x[j];
    }
    const float fr = static_cast<float>(R);
#pragma unroll
    for (int j = 0; j < 4; ++j) avg[j] = avg[j] / fr;
  }
}

template <typename G, int RT, typename PA>
__device__ __forceinline__ float grad_avg1(const PA& g, int R, int64_t s) {
  const int n = RT > 0 ? RT : R;
  float acc = Io<G>::load1(static_cast<const G*>(g.p[0]) + s);
  for (int q = 1; q < n; ++q) acc = acc + Io<G>::load1(static_cast<const G*>(g.p[q]) + s);
  return acc / static_cast<float>(n);
}

// ------------------------------------------------------------------ AdamW
// a / b, correctly rounded, for b one of the step's bias corrections
// (2^-53 <= b <= 1) and 1 / b = hi + lo to about 2^-106 (hi = RN(1 / b)):
//   q0 = RN(a hi + RN(a lo))  is within 1/2 ulp + 2^-104 |a/b| of a / b, so
//                             it is one of the two doubles around a / b;
//   r  = RN(a - b q0)         is then exact (the remainder of a faithful
//                             quotient fits a double);
//   q  = RN(q0 + r hi)        is RN(a / b) by Markstein's theorem (hi within
//                             1/2 ulp of 1 / b, q0 within 1 ulp of a / b).
// A multiply and three fused multiply-adds, where an IEEE division is a
// reciprocal estimate, two scaling steps, five multiply-adds and a fix-up.
// The steps need a lo and r in the normal range.  Here a is m' or v', made
// from fp32 values and betas in [0, 1): a nonzero a is at least 2^-404 in
// magnitude (at most 2^257) unless the gradient is zero and a beta is below
// 2^-651, and then b = 1 - beta^t rounds to 1, hi = 1, lo = 0 and q = a
// exactly.  Zero, infinity and NaN, for which a / b is a itself, take a.
constexpr int kZeroInfNan = 0x267;  // v_cmp_class: +-0, +-inf, quiet and signalling NaN

__device__ __forceinline__ double div_bias(double a, double b, double hi, double lo) {
  const double q0 = fma(a, hi, a * lo);
  const double r = fma(-b, q0, a);
  const double q = fma(r, hi, q0);
  return __builtin_amdgcn_class(a, kZeroInfNan) ? a : q;
}

// One element, in float64 from the fp32 state, in the order the update is
// defined:
//   p1 = p (1 - lr wd);  m' = b1 m + (1-b1) g;  v' = b2 v + ((1-b2) g) g;
//   m^ = m' / (1 - b1^t);  v^ = v' / (1 - b2^t);
//   p' = p1 - (lr m^) / (sqrt(v^) + eps)
// with correctly rounded double operations (no contraction), then each
// result rounded once to fp32, which makes the result the definition's
// exactly.  The two divisions by the bias corrections are IEEE divisions
// (FASTDIV false) or div_bias (true): the same bits, 55 instead of 65
// double operations per element.  Which one a kernel takes was measured on
// MI355X in alternating runs of both: div_bias made the one-element fused
// step 1%, the short unfused AdamW 2-4% and the two-element step-and-gather
// launch 0.6% faster; in the four-element fused forms it gained nothing on
// the 872M-parameter group (within 0.5%) and made their step-and-gather
// launch slower (31.9-32.2 against 31.7-32.0 us), so those and the long
// AdamW launches keep IEEE division.
template <bool FASTDIV>
__device__ __forceinline__ void adamw1(float gf, float& pf, float& mf, float& vf,
                                       const AdamScalars& c) {
  const double g = gf;
  const double p1 = static_cast<double>(pf) * c.decay;
  const double m1 = c.beta1 * static_cast<double>(mf) + c.omb1 * g;
  const double v1 = c.beta2 * static_cast<double>(vf) + (c.omb2 * g) * g;
  const double mh = FASTDIV ? div_bias(m1, c.bc1, c.rbc1_hi, c.rbc1_lo) : m1 / c.bc1;
  const double vh = FASTDIV ? div_bias(v1, c.bc2, c.rbc2_hi, c.rbc2_lo) : v1 / c.bc2;
  const double p2 = p1 - (c.lr * mh) / (sqrt(vh) + c.eps);
  pf = static_cast<float>(p2);
  mf = static_cast<float>(m1);
  vf = static_cast<float>(v1);
}

// The step's scalars.  Stream launches carry them in the kernel arguments;
// graph nodes (REC) read the device record written before each replay, in
// scalar loads issued beside the work descriptor's.  A single kernel
// choosing between the two at run time compiled to nine dependent 8-byte
// loads before the descriptor's, which slowed every graph node's
// workgroups; the choice is therefore made at compile time.
template <bool REC>
__device__ __forceinline__ AdamScalars scalars_of(const AdamScalars& own,
                                                  const AdamScalars* __restrict__ rec) {
  if constexpr (REC) {
    // Only a separate launch writes the record, so it is constant for the
    // whole kernel: read through the constant address space, whose uniform
    // loads the compiler always issues as scalar loads (through a global
    // pointer it proves that only where no store can precede the load).
    using ConstScalars = const __attribute__((address_space(4))) AdamScalars;
    const ConstScalars* c = reinterpret_cast<const ConstScalars*>(reinterpret_cast<uintptr_t>(rec));
    AdamScalars r;
    r.decay = c->decay;
    r.beta1 = c->beta1;
    r.omb1 = c->omb1;
    r.beta2 = c->beta2;
    r.omb2 = c->omb2;
    r.bc1 = c->bc1;
    r.bc2 = c->bc2;
    r.lr = c->lr;
    r.eps = c->eps;
    r.rbc1_hi = c->rbc1_hi;
    r.rbc1_lo = c->rbc1_lo;
    r.rbc2_hi = c->rbc2_hi;
    r.rbc2_lo = c->rbc2_lo;
    return r;
  } else {
    return own;
  }
}

// ------------------------------------------------------------------ copy
// Bit copy, W bytes per lane (W/ES elements), from one source to up to R
// destinations.  Each workgroup starts its round of stores at a different
// destination (rotation by workgroup), which spreads the concurrent stores
// over the destinations: +10% for 8-byte lanes on a 100M-element gather.
// The loop waits for each destination's pointer, and then for the previous
// store, before the next store: a wave keeps one store in flight, which on
// large gathers is faster than issuing all stores back to back.  With
// exactly 4 or 8 destinations (a gather at R = 4 or 8; in the
// step-and-gather launch at R = 8) separate instances unroll the stores in
// destination order, still one in flight per wave: on the 12-layer model's 3.1M-element units
// (16-byte lanes) the gather took 9.63 instead of 10.45 us, the
// step-and-gather launch 31.9 instead of 33.1 us and the whole step 385.2
// instead of 398.6 us; on the 872M-element group (8-byte lanes) the gather
// took 2.38-2.61 instead of 2.61-2.74 ms; on the hidden-512 block at R = 4
// the gather took 6.5-7.0 instead of 7.1-8.1 us (alternating runs on one
// machine).  Unrolling for any count from 2 to 8 behind a switch
// (gather 11.3 us), or with the stores back to back after one explicit wait
// (11.9 us), was slower; so was the unrolled code in the same instance as
// the single-destination copy, whose scalar registers it raised from 45 to
// 78 (fp32 pack 3% slower).
template <int ES>
struct Raw;
template <>
struct Raw<2> {
  using E = u16;
};
template <>
struct Raw<4> {
  using E = uint32_t;
};

template <int W>
struct Lane;
template <>
struct Lane<8> {
  using V = u32x2;
  __device__ __forceinline__ static V load(const void* p) { return ld_nt8(p); }
  __device__ __forceinline__ static void store(void* p, V x) { st_nt8(p, x); }
};
template <>
struct Lane<16> {
  using V = u32x4;
  __device__ __forceinline__ static V load(const void* p) { return ld_nt16(p); }
  __device__ __forceinline__ static void store(void* p, V x) { st_nt16(p, x); }
};

template <int N>
struct CopyArgs {
  const void* src;
  Ptrs<N> dst;
  int n_dst;
  int vec;
};

// s_waitcnt operand: vector memory counter 0, the export and LGKM counters
// not waited for (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8).
constexpr int kWaitVmcnt0 = (0x7 << 4) | (0xF << 8);

// v to element e0 of destinations 0..ND-1 (NULL ones skipped), unrolled.
template <int ND, int ES, int W, typename V, int N_>
__device__ __forceinline__ void store_each(const CopyArgs<N_>& a, int64_t e0, const V& v) {
  using E = typename Raw<ES>::E;
#pragma unroll
  for (int r = 0; r < ND; ++r) {
    E* d = static_cast<E*>(const_cast<void*>(a.dst.p[r]));
    if (d) Lane<W>::store(d + e0, v);
  }
}

// One work item of the copy; wg numbers the item (it picks the first
// destination of the rotation).  UNROLL > 0: the unrolled stores for
// exactly that many destinations (8 pointer slots); 0: the loop.
template <int ES, int W, int N_, int UNROLL = 0>
__device__ __forceinline__ void copy_item(const Work& w, const CopyArgs<N_>& a, unsigned wg) {
  using E = typename Raw<ES>::E;
  using V = typename Lane<W>::V;
  constexpr int N = W / ES;  // elements per lane
  const E* __restrict__ src = static_cast<const E*>(a.src);
  const bool pad = w.src < 0;
  const int64_t delta = w.src - w.dst;
  const int k = static_cast<int>(((delta % N) + N) % N);  // source misalignment
  const bool vec = a.vec != 0;
  const int64_t end = w.dst + w.len;
  const int first = static_cast<int>(wg % static_cast<unsigned>(a.n_dst));
  for (int64_t c = w.dst / N + threadIdx.x; c * N < end; c += kThreads) {
    const int64_t e0 = c * N;
    if (vec && e0 >= w.dst && e0 + N <= end) {
      V v = {};
      if (!pad) {
        const E* sp = src + e0 + delta;
        if (k == 0) {
          v = Lane<W>::load(sp);
        } else {
          const char* al = reinterpret_cast<const char*>(sp - k);
          if constexpr (W == 8)
            v = ld8_shifted(al, k * ES);
          else
            v = ld16_shifted(al, k * ES);
        }
      }
      bool stored = false;
      if constexpr (UNROLL > 0 && N_ == kSmallPtrs) {
        if (a.n_dst == UNROLL) {  // UNROLL receivers: unrolled, in receiver order
          store_each<UNROLL, ES, W>(a, e0, v);
          stored = true;
        }
      }
      if (!stored)
        for (int i = 0, r = first; i < a.n_dst; ++i, r = r + 1 == a.n_dst ? 0 : r + 1) {
          E* d = static_cast<E*>(const_cast<void*>(a.dst.p[r]));
          if (d) Lane<W>::store(d + e0, v);
        }
    } else {
      const int64_t lo = e0 > w.dst ? e0 : w.dst;
      const int64_t hi = e0 + N < end ? e0 + N : end;
      for (int64_t e = lo; e < hi; ++e) {
        const E x = pad ? E(0) : src[e + delta];
        for (int i = 0; i < a.n_dst; ++i) {
          E* d = static_cast<E*>(const_cast<void*>(a.dst.p[i]));
          if (d) d[e] = x;
        }
      }
    }
  }
}

template <int ES, int W, int N, int UNROLL = 0>
__global__ __launch_bounds__(kThreads) void k_copy(const Work* __restrict__ work,
                                                   CopyArgs<N> a) {
  copy_item<ES, W, N, UNROLL>(work[blockIdx.x], a, blockIdx.x);
}

// The same copy for up to 64 independent (source, destination) pairs that
// share one work table: blockIdx.y picks the pair.
struct PairArgs {
  Ptrs<FSDP_MAX_RANKS> src;
  Ptrs<FSDP_MAX_RANKS> dst;
  int vec;
};

template <int ES>
__global__ __launch_bounds__(kThreads) void k_copy_pairs(const Work* __restrict__ work,
                                                         PairArgs a) {
  using E = typename Raw<ES>::E;
  constexpr int N = 16 / ES;
  const Work w = work[blockIdx.x];
  const E* __restrict__ src = static_cast<const E*>(a.src.p[blockIdx.y]);
  E* __restrict__ dst = static_cast<E*>(const_cast<void*>(a.dst.p[blockIdx.y]));
  const bool pad = w.src < 0;
  const int64_t delta = w.src - w.dst;
  const int k = static_cast<int>(((delta % N) + N) % N);
  const int64_t end = w.dst + w.len;
  for (int64_t c = w.dst / N + threadIdx.x; c * N < end; c += kThreads) {
    const int64_t e0 = c * N;
    if (a.vec && e0 >= w.dst && e0 + N <= end) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (!pad) {
        const E* sp = src + e0 + delta;
        v = k == 0 ? ld_nt16(sp) : ld16_shifted(reinterpret_cast<const char*>(sp - k), k * ES);
      }
      st_nt16(dst + e0, v);
    } else {
      const int64_t lo = e0 > w.dst ? e0 : w.dst;
      const int64_t hi = e0 + N < end ? e0 + N : end;
      for (int64_t e = lo; e < hi; ++e) dst[e] = pad ? E(0) : src[e + delta];
    }
  }
}

// Loop of the arithmetic kernels over one work item: lane chunks of kEPL
// elements aligned in the destination index space.  body4(e0) handles a
// whole aligned chunk, body1(e) one element.
template <typename Body4, typename Body1>
__device__ __forceinline__ void for_chunks(const Work& w, bool vec, Body4 body4, Body1 body1) {
  const int64_t end = w.dst + w.len;
  for (int64_t c = w.dst / kEPL + threadIdx.x; c * kEPL < end; c += kThreads) {
    const int64_t e0 = c * kEPL;
    if (vec && e0 >= w.dst && e0 + kEPL <= end) {
      body4(e0);
    } else {
      const int64_t lo = e0 > w.dst ? e0 : w.dst;
      const int64_t hi = e0 + kEPL < end ? e0 + kEPL : end;
      for (int64_t e = lo; e < hi; ++e) body1(e);
    }
  }
}

// --------------------------------------------------------------- pack+cast
struct CastArgs {
  const void* src;
  void* dst;
  int vec;
};

template <typename S, typename D>
__global__ __launch_bounds__(kThreads) void k_pack_cast(const Work* __restrict__ work,
                                                        CastArgs a) {
  const Work w = work[blockIdx.x];
  const S* __restrict__ src = static_cast<const S*>(a.src);
  D* __restrict__ dst = static_cast<D*>(a.dst);
  const bool pad = w.src < 0;
  const int64_t delta = w.src - w.dst;
  const int k = static_cast<int>(((delta % kEPL) + kEPL) % kEPL);  // source misalignment
  for_chunks(
      w, a.vec != 0,
      [&](int64_t e0) {
        float x[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (!pad) {
          if (k == 0)
            Io<S>::load4(src + e0 + delta, true, x);
          else
            Io<S>::load4s(src, e0 + delta, k, x);
        }
        Io<D>::store4(dst + e0, true, x);
      },
      [&](int64_t e) { Io<D>::store1(dst + e, pad ? 0.0f : Io<S>::load1(src + e + delta)); });
}

// ------------------------------------------------------ reduce-scatter-avg
template <int N>
struct RsArgs {
  Ptrs<N> g;
  float* out;
  int R;
  int vec;
};

template <typename G, int RT, bool PAD, bool SHIFT>
__device__ __forceinline__ void rs_item(const Work& w, const RsArgs<ptr_cap(RT)>& a, int k) {
  const int64_t delta = w.src - w.dst;
  for_chunks(
      w, a.vec != 0,
      [&](int64_t e0) {
        float avg[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (!PAD) grad_avg4<G, RT, SHIFT>(a.g, a.R, e0 + delta, k, avg);
        Io<float>::store4(a.out + e0, true, avg);
      },
      [&](int64_t e) { a.out[e] = PAD ? 0.0f : grad_avg1<G, RT>(a.g, a.R, e + delta); });
}

template <typename G, int RT>
__global__ __launch_bounds__(kThreads) void k_rs_avg(const Work* __restrict__ work,
                                                     RsArgs<ptr_cap(RT)> a) {
  const Work w = work[blockIdx.x];
  const int k = static_cast<int>((((w.src - w.dst) % kEPL) + kEPL) % kEPL);
  if (w.src < 0)
    rs_item<G, RT, true, false>(w, a, 0);
  else if (k == 0)
    rs_item<G, RT, false, false>(w, a, 0);
  else
    rs_item<G, RT, false, true>(w, a, k);
}

// The reduce-scatter alone in short launches at R >= 8: two adjacent
// elements per lane and two workgroups per item, on fused_pair_wg's layout
// (two strided elements where an item's offsets, length or the bases do
// not allow the pair), the descriptor and pointers in one round of scalar
// loads.  The 12-layer model's units: 11.6-11.8 us against 12.1 us with
// four elements per lane (alternating runs on one machine); on the
// 872M-parameter group the two forms measured level, so long launches keep
// four.
template <typename G, int RT>
__global__ __launch_bounds__(kThreads) void k_rs_two(const Work* __restrict__ work,
                                                     RsArgs<ptr_cap(RT)> a) {
  const int b = static_cast<int>(blockIdx.x);
  const Work w = work[b / 2];
  if constexpr (RT == 8) {
    asm volatile("" ::"s"(w.dst), "s"(w.src), "s"(w.len), "s"(a.g.p[0]), "s"(a.g.p[1]),
                 "s"(a.g.p[2]), "s"(a.g.p[3]), "s"(a.g.p[4]), "s"(a.g.p[5]), "s"(a.g.p[6]),
                 "s"(a.g.p[7]), "s"(a.out));
  } else {
    asm volatile("" ::"s"(w.dst), "s"(w.src), "s"(w.len), "s"(a.out));
  }
  const int64_t half = static_cast<int64_t>(b % 2) * (2 * kThreads);
  const bool even =
      a.vec != 0 && ((w.dst | w.len) & 1) == 0 && (w.src < 0 || (w.src & 1) == 0);
  if (even) {
    const int64_t off = half + 2 * threadIdx.x;
    if (off >= w.len) return;
    float avg[2] = {0.0f, 0.0f};
    if (w.src >= 0) grad_avg_two<G, RT>(a.g, a.R, w.src + off, avg);
    Two<float>::store(a.out + w.dst + off, avg);
    return;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t off = half + j * kThreads + threadIdx.x;
    if (off >= w.len) return;
    const float x = w.src < 0 ? 0.0f : grad_avg_one<G, RT>(a.g, a.R, w.src + off);
    One<float>::store(a.out + w.dst + off, x);
  }
}

// ------------------------------------------------------------------ AdamW
struct AdamArgs {
  const float* g;
  float* master;
  float* m;
  float* v;
  void* param;
  AdamScalars sc;
  const AdamScalars* scp;  // non-null: take the scalars from device memory
  int64_t n;
  int vec;
};

// One pass per workgroup: lane c of the grid owns elements [4c, 4c + 4)
// (long launches; IEEE division).
template <typename P, bool REC>
__global__ __launch_bounds__(kThreads) void k_adamw(AdamArgs a) {
  P* __restrict__ param = static_cast<P*>(a.param);
  const AdamScalars sc = scalars_of<REC>(a.sc, a.scp);
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t e0 = c * kEPL;
  if (e0 >= a.n) return;
  if (a.vec && e0 + kEPL <= a.n) {
    float g[4], p[4], m[4], v[4];
    Io<float>::load4(a.g + e0, true, g);
    Io<float>::load4(a.master + e0, true, p);
    Io<float>::load4(a.m + e0, true, m);
    Io<float>::load4(a.v + e0, true, v);
#pragma unroll
    for (int k = 0; k < 4; ++k) adamw1<false>(g[k], p[k], m[k], v[k], sc);
    Io<float>::store4(a.master + e0, true, p);
    Io<float>::store4(a.m + e0, true, m);
    Io<float>::store4(a.v + e0, true, v);
    Io<P>::store4(param + e0, true, p);
  } else {
    const int64_t hi = e0 + kEPL < a.n ? e0 + kEPL : a.n;
    for (int64_t e = e0; e < hi; ++e) {
      float p = a.master[e], m = a.m[e], v = a.v[e];
      adamw1<false>(a.g[e], p, m, v, sc);
      a.master[e] = p;
      a.m[e] = m;
      a.v[e] = v;
      Io<P>::store1(param + e, p);
    }
  }
}

// AdamW alone in short launches (up to 4,096 four-element workgroups): two
// adjacent elements per lane (8-byte state and gradient accesses when the
// bases are 16-byte aligned), the division of div_bias.  The 12-layer
// model's units: 17.9-18.0 us against 18.5-18.6 us with four elements per
// lane (alternating runs on one machine); on the 872M-parameter group four
// elements at 4 per CU stayed faster (4.25 against 4.29-4.33 ms).
template <typename P, bool REC>
__global__ __launch_bounds__(kThreads) void k_adamw_two(AdamArgs a) {
  const AdamScalars sc = scalars_of<REC>(a.sc, a.scp);
  const int64_t e = 2 * (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x);
  if (e >= a.n) return;
  if (a.vec && e + 1 < a.n) {
    float g[2], p[2], m[2], v[2];
    Two<float>::load(a.g + e, g);
    Two<float>::load(a.master + e, p);
    Two<float>::load(a.m + e, m);
    Two<float>::load(a.v + e, v);
    adamw1<true>(g[0], p[0], m[0], v[0], sc);
    adamw1<true>(g[1], p[1], m[1], v[1], sc);
    Two<float>::store(a.master + e, p);
    Two<float>::store(a.m + e, m);
    Two<float>::store(a.v + e, v);
    Two<P>::store(static_cast<P*>(a.param) + e, p);
    return;
  }
  const int64_t hi = e + 2 < a.n ? e + 2 : a.n;
  for (int64_t i = e; i < hi; ++i) {
    float p = a.master[i], m = a.m[i], v = a.v[i];
    adamw1<true>(a.g[i], p, m, v, sc);
    a.master[i] = p;
    a.m[i] = m;
    a.v[i] = v;
    Io<P>::store1(static_cast<P*>(a.param) + i, p);
  }
}

// -------------------------------------- fused reduce-scatter + AdamW + cast
template <int N>
struct FusedArgs {
  Ptrs<N> g;
  float* master;
  float* m;
  float* v;
  void* param;
  AdamScalars sc;
  const AdamScalars* scp;  // non-null: take the scalars from device memory
  int R;
  int vec;
};

// One work item of the fused step.  In a whole chunk every load (master, m,
// v, then the R gradient replicas) is issued before any of them is used, so
// a wave waits for memory once per chunk.  PAD: padding, no gradient (g = 0).
template <typename G, typename P, int RT, bool PAD, bool SHIFT>
__device__ __forceinline__ void fused_item(const Work& w, const FusedArgs<ptr_cap(RT)>& a,
                                           const AdamScalars& sc, int k) {
  P* __restrict__ param = static_cast<P*>(a.param);
  const int64_t delta = w.src - w.dst;
  for_chunks(
      w, a.vec != 0,
      [&](int64_t e0) {
        float p[4], m[4], v[4];
        Io<float>::load4(a.master + e0, true, p);
        Io<float>::load4(a.m + e0, true, m);
        Io<float>::load4(a.v + e0, true, v);
        float g[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (!PAD) grad_avg4<G, RT, SHIFT>(a.g, a.R, e0 + delta, k, g);
#pragma unroll
        for (int j = 0; j < 4; ++j) adamw1<false>(g[j], p[j], m[j], v[j], sc);
        Io<float>::store4(a.master + e0, true, p);
        Io<float>::store4(a.m + e0, true, m);
        Io<float>::store4(a.v + e0, true, v);
        Io<P>::store4(param + e0, true, p);
      },
      [&](int64_t e) {
        const float g = PAD ? 0.0f : grad_avg1<G, RT>(a.g, a.R, e + delta);
        float p = a.master[e], m = a.m[e], v = a.v[e];
        adamw1<false>(g, p, m, v, sc);
        a.master[e] = p;
        a.m[e] = m;
        a.v[e] = v;
        Io<P>::store1(param + e, p);
      });
}

template <typename G, typename P, int RT>
__device__ __forceinline__ void fused_wg(const Work& w, const FusedArgs<ptr_cap(RT)>& a,
                                         const AdamScalars& sc) {
  const int k = static_cast<int>((((w.src - w.dst) % kEPL) + kEPL) % kEPL);
  if (w.src < 0)
    fused_item<G, P, RT, true, false>(w, a, sc, 0);
  else if (k == 0)
    fused_item<G, P, RT, false, false>(w, a, sc, 0);
  else
    fused_item<G, P, RT, false, true>(w, a, sc, k);
}

template <typename G, typename P, int RT, bool REC>
__global__ __launch_bounds__(kThreads) void k_fused(const Work* __restrict__ work,
                                                    FusedArgs<ptr_cap(RT)> a) {
  const AdamScalars sc = scalars_of<REC>(a.sc, a.scp);
  fused_wg<G, P, RT>(work[blockIdx.x], a, sc);
}

// The one-element form: part b % kSplit of work item b / kSplit.  master,
// m and v are loaded, then the R gradient replicas (none for padding, whose
// gradient is 0), all before the first use.
template <typename G, typename P, int RT, bool REC>
__global__ __launch_bounds__(kThreads) void k_fused_one(const Work* __restrict__ work,
                                                        FusedArgs<ptr_cap(RT)> a) {
  const Work w = work[blockIdx.x / kSplit];
  // the step's scalars (REC: the record's scalar loads, which the compiler
  // issues after the data loads, while they are in flight)
  const AdamScalars sc = scalars_of<REC>(a.sc, a.scp);
  args_in_sgprs<RT, REC>(w, a);
  const int64_t off = static_cast<int64_t>(blockIdx.x % kSplit) * kThreads + threadIdx.x;
  if (off >= w.len) return;
  const int64_t e = w.dst + off;
  float p = One<float>::load(a.master + e), m = One<float>::load(a.m + e),
        v = One<float>::load(a.v + e);
  const float g = w.src < 0 ? 0.0f : grad_avg_one<G, RT>(a.g, a.R, w.src + off);
  adamw1<true>(g, p, m, v, sc);
  One<float>::store(a.master + e, p);
  One<float>::store(a.m + e, m);
  One<float>::store(a.v + e, v);
  One<P>::store(static_cast<P*>(a.param) + e, p);
}

// The fused step with NE elements per lane at off, off + 256, ...: each
// 1024-element work item takes 1024 / (256 NE) workgroups; every access is
// one naturally aligned element.  A lane past the end of its item reloads
// its first element (in range) and skips the stores.  FD: the division of
// div_bias (else IEEE division).
template <typename G, typename P, int RT, bool REC, int NE, bool FD>
__device__ __forceinline__ void fused_ne_wg(const Work* __restrict__ work,
                                            const FusedArgs<ptr_cap(RT)>& a, int b) {
  constexpr int kS = 1024 / (kThreads * NE);
  const Work w = work[b / kS];
  const AdamScalars sc = scalars_of<REC>(a.sc, a.scp);
  args_in_sgprs<RT, REC>(w, a);
  const int64_t base = static_cast<int64_t>(b % kS) * kThreads * NE + threadIdx.x;
  if (base >= w.len) return;
  float p[NE], m[NE], v[NE], g[NE];
  int64_t off[NE];
  bool ok[NE];
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    const int64_t o = base + j * kThreads;
    ok[j] = o < w.len;
    off[j] = ok[j] ? o : base;
    const int64_t e = w.dst + off[j];
    p[j] = One<float>::load(a.master + e);
    m[j] = One<float>::load(a.m + e);
    v[j] = One<float>::load(a.v + e);
  }
#pragma unroll
  for (int j = 0; j < NE; ++j)
    g[j] = w.src < 0 ? 0.0f : grad_avg_one<G, RT>(a.g, a.R, w.src + off[j]);
#pragma unroll
  for (int j = 0; j < NE; ++j) adamw1<FD>(g[j], p[j], m[j], v[j], sc);
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    if (!ok[j]) continue;
    const int64_t e = w.dst + off[j];
    One<float>::store(a.master + e, p[j]);
    One<float>::store(a.m + e, m[j]);
    One<float>::store(a.v + e, v[j]);
    One<P>::store(static_cast<P*>(a.param) + e, p[j]);
  }
}

// The fused step with two adjacent elements per lane: workgroup b takes
// elements [512 (b % 2), + 512) of work item b / 2, lane t the pair at
// 2t, so every state, gradient and parameter access moves a lane's two
// elements at once (8 or 4 bytes, naturally aligned).  That needs 16-byte
// aligned bases (a.vec) and an even destination offset, length and source
// offset; otherwise (an odd-sized piece of a parameter, a base aligned to
// its element only) the item takes fused_ne_wg's two strided elements, on
// the same workgroup-to-item mapping.  div_bias divides.
template <typename G, typename P, int RT, bool REC>
__device__ __forceinline__ void fused_pair_wg(const Work* __restrict__ work,
                                              const FusedArgs<ptr_cap(RT)>& a, int b) {
  const Work w = work[b / 2];
  const AdamScalars sc = scalars_of<REC>(a.sc, a.scp);
  args_in_sgprs<RT, REC>(w, a);
  const bool even =
      a.vec != 0 && ((w.dst | w.len) & 1) == 0 && (w.src < 0 || (w.src & 1) == 0);
  if (!even) {
    fused_ne_wg<G, P, RT, REC, 2, true>(work, a, b);
    return;
  }
  const int64_t off = static_cast<int64_t>(b % 2) * (2 * kThreads) + 2 * threadIdx.x;
  if (off >= w.len) return;
  const int64_t e = w.dst + off;
  float p[2], m[2], v[2], g[2] = {0.0f, 0.0f};
  Two<float>::load(a.master + e, p);
  Two<float>::load(a.m + e, m);
  Two<float>::load(a.v + e, v);
  if (w.src >= 0) grad_avg_two<G, RT>(a.g, a.R, w.src + off, g);
  adamw1<true>(g[0], p[0], m[0], v[0], sc);
  adamw1<true>(g[1], p[1], m[1], v[1], sc);
  Two<float>::store(a.master + e, p);
  Two<float>::store(a.m + e, m);
  Two<float>::store(a.v + e, v);
  Two<P>::store(static_cast<P*>(a.param) + e, p);
}

// The fused step alone in the two-element form (fused_pair_lane): launches
// of more than 4,096 work items at R >= 8, two workgroups per item, 4 per
// CU (fused_pair_lds); short launches at R = 3 and 4, uncapped.  On the
// 872M-parameter group (852k items, alternating
// runs on one machine): 5.66-5.72 ms against 5.93-5.96 ms with four
// elements per lane at 3 per CU, 6.40-6.48 TB/s; the cap at 3, 5-6 or 8
// per CU: 6.12, 5.77-5.79 and 6.14 ms.  The 12-layer model in 2-block
// units (6,260 items): 43.5-43.6 against 44.3-44.7 us; in 4-block units
// (12,520): 87.7-88.7 against 88.9-90.0 us.
template <typename G, typename P, int RT, bool REC>
__global__ __launch_bounds__(kThreads) void k_fused_pair(const Work* __restrict__ work,
                                                         FusedArgs<ptr_cap(RT)> a) {
  fused_pair_wg<G, P, RT, REC>(work, a, static_cast<int>(blockIdx.x));
}

// The fused step of one unit and the gather of another in one launch:
// workgroups [0, n_fused) take the step's work items, the rest the
// gather's, in that order.  Dispatch follows the workgroup order, so the
// gather starts while the step's last workgroups drain instead of after
// them.  wide: 16-byte gather lanes (else 8).  The gather copies the
// parameter dtype P.
// The pairing with the fused step in the two-element form (fused_pair_wg,
// adjacent pairs, div_bias): workgroups [0, n_fused) are two per work item
// of the step.  On the 12-layer model's per-parameter units at R = 8,
// alternating runs on one machine: 31.2 us against 31.35 with two elements
// strided by 256 (fused_ne_wg) and 31.7-31.8 with four per lane, the step
// 375.5-375.6 against 377.5-377.8 us (two strided) and 381.3-381.9 (four).
// Two strided elements had lost to four on FSDP1 units and on longer steps;
// adjacent pairs gain there too: the FSDP1 12-layer step 374.3-374.4
// against 374.8-375.5 us, the model in 4-block units (12,520 items, capped
// at 4 per CU) 381.3-381.6 against 382.9-383.6 us; in 2-block units (6,260
// items) 376.3-376.8 against 375.9-376.4 us.
template <typename G, typename P, int RT, bool REC>
__global__ __launch_bounds__(kThreads) void k_fused_two_gather(
    const Work* __restrict__ fwork, FusedArgs<ptr_cap(RT)> fa, int n_fused,
    const Work* __restrict__ gwork, CopyArgs<ptr_cap(RT)> ca, int wide) {
  const int b = static_cast<int>(blockIdx.x);
  if (b < n_fused) {
    fused_pair_wg<G, P, RT, REC>(fwork, fa, b);
    return;
  }
  const int i = b - n_fused;
  if (wide)
    copy_item<sizeof(P), 16, ptr_cap(RT), kSmallPtrs>(gwork[i], ca, static_cast<unsigned>(i));
  else
    copy_item<sizeof(P), 8>(gwork[i], ca, static_cast<unsigned>(i));
}

template <typename G, typename P, int RT, bool REC>
__global__ __launch_bounds__(kThreads) void k_fused_gather(const Work* __restrict__ fwork,
                                                           FusedArgs<ptr_cap(RT)> fa,
                                                           int n_fused,
                                                           const Work* __restrict__ gwork,
                                                           CopyArgs<ptr_cap(RT)> ca, int wide) {
  const int b = static_cast<int>(blockIdx.x);
  if (b < n_fused) {
    fused_wg<G, P, RT>(fwork[b], fa, scalars_of<REC>(fa.sc, fa.scp));
    return;
  }
  const int i = b - n_fused;
  if (wide)
    copy_item<sizeof(P), 16, ptr_cap(RT), kSmallPtrs>(gwork[i], ca, static_cast<unsigned>(i));
  else
    copy_item<sizeof(P), 8>(gwork[i], ca, static_cast<unsigned>(i));
}

// ------------------------------------------------- gradient accumulation
// acc[r][i] = g[r][i] (first micro-batch) or acc[r][i] + g[r][i], fp32, for
// every rank r (blockIdx.y) and i < T.  Elementwise: no layout involved.
template <int N>
struct AccArgs {
  Ptrs<N> g;
  Ptrs<N> acc;
  int64_t T;
  int first;
  int vec;
};

template <typename G, int N>
__global__ __launch_bounds__(kThreads) void k_accumulate(AccArgs<N> a) {
  const G* __restrict__ g = static_cast<const G*>(a.g.p[blockIdx.y]);
  float* __restrict__ acc = static_cast<float*>(const_cast<void*>(a.acc.p[blockIdx.y]));
  const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * kEPL;
  if (e0 >= a.T) return;
  if (a.vec && e0 + kEPL <= a.T) {
    float x[4];
    Io<G>::load4(g + e0, true, x);
    if (!a.first) {
      float y[4];
      Io<float>::load4(acc + e0, true, y);
#pragma unroll
      for (int k = 0; k < 4; ++k) x[k] = y[k] + x[k];
    }
    Io<float>::store4(acc + e0, true, x);
  } else {
    const int64_t hi = e0 + kEPL < a.T ? e0 + kEPL : a.T;
    for (int64_t e = e0; e < hi; ++e) {
      const float x = Io<G>::load1(g + e);
      acc[e] = a.first ? x : acc[e] + x;
    }
  }
}

// ------------------------------------------------------ all-reduce-average
// out[r][i] = (g_0[i] + ... + g_{R-1}[i]) / R for every receiver r and
// i < T: DDP's averaged all-reduce, the rank-order mean of the
// reduce-scatter over the whole unit.
template <int N>
struct ArArgs {
  Ptrs<N> g;
  Ptrs<N> out;
  int64_t T;
  int R;
  int vec;
};

template <typename G, typename O, int RT>
__global__ __launch_bounds__(kThreads) void k_allreduce(ArArgs<ptr_cap(RT)> a) {
  const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * kEPL;
  if (e0 >= a.T) return;
  const int R = RT > 0 ? RT : a.R;
  if (a.vec && e0 + kEPL <= a.T) {
    float avg[4];
    grad_avg4<G, RT>(a.g, a.R, e0, 0, avg);
    // one store in flight per wave: each waits for the one before (the
    // loaded gradients are consumed by then, so only stores are counted)
    for (int r = 0; r < R; ++r) {
      Io<O>::store4(static_cast<O*>(const_cast<void*>(a.out.p[r])) + e0, true, avg);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
  } else {
    const int64_t hi = e0 + kEPL < a.T ? e0 + kEPL : a.T;
    for (int64_t e = e0; e < hi; ++e) {
      const float avg = grad_avg1<G, RT>(a.g, a.R, e);
      for (int r = 0; r < R; ++r)
        Io<O>::store1(static_cast<O*>(const_cast<void*>(a.out.p[r])) + e, avg);
    }
  }
}

// -------------------------------------------- AdamW scalars into memory
// One lane writes the step's scalar record, for kernels that read it from
// device memory (a step graph replays the same kernel arguments every step).
__global__ __launch_bounds__(64) void k_set_scalars(AdamScalars* __restrict__ dst,
                                                    AdamScalars sc) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *dst = sc;
}

// ----------------------------------------------------------------- launch
template <typename Args>
hipError_t launch_work(const void* fn, const Work* work, int64_t n_work, Args& a, const Sink& sink,
                       unsigned lds = 0) {
  if (n_work <= 0) return hipSuccess;
  if (n_work > kMaxBlocks) return hipErrorInvalidValue;
  void* args[] = {const_cast<Work**>(&work), &a};
  return sink.launch(fn, dim3(static_cast<unsigned>(n_work)), dim3(kThreads), args, lds);
}

// Workgroups of the fused step resident per CU, set through LDS: the kernel
// uses none, so asking for L bytes per workgroup lets at most
// floor(LDS per CU / L) of them share a CU.  Measured on MI355X with
// per-workgroup timestamps: without LDS the kernel's own resources allow 5
// per CU (1,280 resident); 32 KB gives 4, 48 KB 3, 64 KB 2.  GB/s at 5 / 4
// / 3 per CU (R = 8, hidden-512 blocks, bf16 gradients, 4+ GB of buffers
// cycled so the last-level cache serves nothing): 1 block (3,073 items)
// 5353 / 5300 / 5219; 4 blocks 5767 / 5836 / 5763; 16 blocks (49k items)
// 5920 / 6136 / 6031; 32 blocks 5704 / 5885 / 6086; 128 blocks (394k items)
// 5404 / 5641 / 5824; the 872M-parameter group (852k items)
// 5674 / 5931 / 6205.  Fifteen streams per workgroup (8 gradients, 3 states
// read; 4 arrays written) are far more than the DRAM pages one channel
// keeps open; fewer workgroups in flight keep fewer pages busy while still
// covering the latency, once the launch is long enough that its ramp does
// not dominate.
unsigned fused_lds(int64_t n_work) {
  if (n_work <= kSmallFusedLaunch) return 0;  // short: the kernel's own 5 per CU
  if (n_work <= 65536) return 32 * 1024;        // 4 per CU
  return 48 * 1024;                             // 3 per CU
}

// The cap of the two-element form (fused_pair_wg: alone or paired with a
// gather), whose own resources allow 8 per CU: none up to 4,096 items, 4
// per CU above at every length.
unsigned fused_pair_lds(int64_t n_work) { return n_work <= kSmallFusedLaunch ? 0 : 32 * 1024; }

// The same cap for the unfused AdamW step (8 streams per workgroup: the
// reduced gradient, master, m and v read; master, m, v and the parameter
// written), whose best is 4 per CU.  One pass per workgroup, on the
// 872M-parameter group (852k workgroups): GB/s uncapped 5,652-5,764; 4 per
// CU 5,997; 3 per CU 5,754-5,765; 2 per CU 5,055 -- and 5,119 for the
// earlier grid-stride loop over 65,536 workgroups.  Short launches take no
// cap, as for the fused step.
unsigned adamw_lds(int64_t blocks) { return blocks <= kSmallFusedLaunch ? 0 : 32 * 1024; }

// DDP's all-reduce (R gradient replicas read, R averaged copies written per
// element) keeps one of its R stores in flight per wave and, above 4,096
// workgroups, 3 workgroups per CU.  Alternating A/B runs on MI355X, R = 8,
// bf16 gradients, fp32 outputs: with stores back to back, capping took
// 3.1M elements (3,073 workgroups) 28.66 -> 27.90 us, 12.6M 121.0 ->
// 116.2 us, 37.8M 358-366 -> 348-349 us; pacing the stores then took them
// (capped) to 27.65, 113.3 and 335.3 us, and uncapped to 27.10, 112.5 and
// 345.5 us.
unsigned allreduce_lds(int64_t blocks) { return blocks <= kSmallFusedLaunch ? 0 : 48 * 1024; }

// The AdamW kernel for the parameter dtype and the scalars' source: the
// two-element form (TWO) or the four-element one.
template <bool TWO>
const void* adamw_fn(int param_dt, bool rec) {
  if constexpr (TWO) {
    if (rec)
      return param_dt == FSDP_BF16 ? reinterpret_cast<const void*>(&k_adamw_two<u16, true>)
                                   : reinterpret_cast<const void*>(&k_adamw_two<float, true>);
    return param_dt == FSDP_BF16 ? reinterpret_cast<const void*>(&k_adamw_two<u16, false>)
                                 : reinterpret_cast<const void*>(&k_adamw_two<float, false>);
  } else {
    if (rec)
      return param_dt == FSDP_BF16 ? reinterpret_cast<const void*>(&k_adamw<u16, true>)
                                   : reinterpret_cast<const void*>(&k_adamw<float, true>);
    return param_dt == FSDP_BF16 ? reinterpret_cast<const void*>(&k_adamw<u16, false>)
                                 : reinterpret_cast<const void*>(&k_adamw<float, false>);
  }
}

template <typename G>
const void* pick_rs(int R) {
  switch (R) {
    case 1: return reinterpret_cast<const void*>(&k_rs_avg<G, 1>);
    case 2: return reinterpret_cast<const void*>(&k_rs_avg<G, 2>);
    case 3: return reinterpret_cast<const void*>(&k_rs_avg<G, 3>);
    case 4: return reinterpret_cast<const void*>(&k_rs_avg<G, 4>);
    case 5: return reinterpret_cast<const void*>(&k_rs_avg<G, 5>);
    case 6: return reinterpret_cast<const void*>(&k_rs_avg<G, 6>);
    case 7: return reinterpret_cast<const void*>(&k_rs_avg<G, 7>);
    case 8: return reinterpret_cast<const void*>(&k_rs_avg<G, 8>);
    default: return reinterpret_cast<const void*>(&k_rs_avg<G, 0>);
  }
}

template <typename G>
const void* pick_rs_two(int R) {
  return R == 8 ? reinterpret_cast<const void*>(&k_rs_two<G, 8>)
                : reinterpret_cast<const void*>(&k_rs_two<G, 0>);
}

template <typename G, typename O>
const void* pick_allreduce(int R) {
  switch (R) {
    case 1: return reinterpret_cast<const void*>(&k_allreduce<G, O, 1>);
    case 2: return reinterpret_cast<const void*>(&k_allreduce<G, O, 2>);
    case 4: return reinterpret_cast<const void*>(&k_allreduce<G, O, 4>);
    case 8: return reinterpret_cast<const void*>(&k_allreduce<G, O, 8>);
    default: return reinterpret_cast<const void*>(&k_allreduce<G, O, 0>);
  }
}

template <typename G, typename P, bool REC>
const void* pick_fused(int R) {
  switch (R) {
    case 1: return reinterpret_cast<const void*>(&k_fused<G, P, 1, REC>);
    case 2: return reinterpret_cast<const void*>(&k_fused<G, P, 2, REC>);
    case 3: return reinterpret_cast<const void*>(&k_fused<G, P, 3, REC>);
    case 4: return reinterpret_cast<const void*>(&k_fused<G, P, 4, REC>);
    case 5: return reinterpret_cast<const void*>(&k_fused<G, P, 5, REC>);
    case 6: return reinterpret_cast<const void*>(&k_fused<G, P, 6, REC>);
    case 7: return reinterpret_cast<const void*>(&k_fused<G, P, 7, REC>);
    default: return nullptr;  // R >= 8 takes the one- or two-element forms
  }
}

template <typename G, typename P, bool REC>
const void* pick_fused_one(int R) {
  return R == 8 ? reinterpret_cast<const void*>(&k_fused_one<G, P, 8, REC>)
                : reinterpret_cast<const void*>(&k_fused_one<G, P, 0, REC>);
}

template <typename G, typename P, bool REC>
const void* pick_fused_pair(int R) {
  return R == 8 ? reinterpret_cast<const void*>(&k_fused_pair<G, P, 8, REC>)
       : R == 4 ? reinterpret_cast<const void*>(&k_fused_pair<G, P, 4, REC>)
       : R == 3 ? reinterpret_cast<const void*>(&k_fused_pair<G, P, 3, REC>)
                : reinterpret_cast<const void*>(&k_fused_pair<G, P, 0, REC>);
}

template <bool REC>
const void* fused_pair_fn(int grad_dt, int param_dt, int R) {
  if (grad_dt == FSDP_BF16)
    return param_dt == FSDP_BF16 ? pick_fused_pair<u16, u16, REC>(R)
                                 : pick_fused_pair<u16, float, REC>(R);
  return param_dt == FSDP_BF16 ? pick_fused_pair<float, u16, REC>(R)
                               : pick_fused_pair<float, float, REC>(R);
}

template <bool REC>
const void* fused_one_fn(int grad_dt, int param_dt, int R) {
  if (grad_dt == FSDP_BF16)
    return param_dt == FSDP_BF16 ? pick_fused_one<u16, u16, REC>(R)
                                 : pick_fused_one<u16, float, REC>(R);
  return param_dt == FSDP_BF16 ? pick_fused_one<float, u16, REC>(R)
                               : pick_fused_one<float, float, REC>(R);
}

// Which form runs a standalone fused step.  One element per lane: short
// launches at R >= 8.  Two adjacent elements (k_fused_pair): longer ones at
// R >= 8 (4 per CU), and short ones at R = 3 and 4.  Four: everything else
// (R = 5..7, unmeasured in the other forms, and long launches below R = 8).
// On the hidden-512 block (3.1M parameters, short launches), alternating
// runs on one machine: at R = 4 four elements 20.7-21.5 us, one 19.9-20.1,
// two 19.8-20.1 (the step 27.3-27.9 -> 26.6-26.9 us); at R = 3 four
// 20.4-20.5, one 19.6-20.0, two 19.1-19.6 us; in the FSDP1 layout at R = 4
// one 20.8-21.0, two 21.0-21.3 us (the step level at 27.8-28.3 us), at R = 3
// one 19.4-20.2, two 19.0-19.2 us (the step 25.7-26.5 -> 24.9-25.1 us).
bool fused_one_lane(int64_t n_work, int R) { return R >= 8 && n_work <= kSmallFusedLaunch; }
bool fused_pair_lane(int64_t n_work, int R) {
  return R >= 8 ? n_work > kSmallFusedLaunch
                : (R == 3 || R == 4) && n_work <= kSmallFusedLaunch;
}

template <typename G, typename P, bool REC>
const void* pick_fused_gather(int R) {
  switch (R) {
    case 1: return reinterpret_cast<const void*>(&k_fused_gather<G, P, 1, REC>);
    case 2: return reinterpret_cast<const void*>(&k_fused_gather<G, P, 2, REC>);
    case 3: return reinterpret_cast<const void*>(&k_fused_gather<G, P, 3, REC>);
    case 4: return reinterpret_cast<const void*>(&k_fused_gather<G, P, 4, REC>);
    case 5: return reinterpret_cast<const void*>(&k_fused_gather<G, P, 5, REC>);
    case 6: return reinterpret_cast<const void*>(&k_fused_gather<G, P, 6, REC>);
    case 7: return reinterpret_cast<const void*>(&k_fused_gather<G, P, 7, REC>);
    default: return nullptr;  // R >= 8 takes k_fused_two_gather
  }
}

// The fused kernel (or the fused step + gather kernel) for the dtypes, R
// and the scalars' source.
template <bool REC>
const void* fused_fn(int grad_dt, int param_dt, int R) {
  if (grad_dt == FSDP_BF16)
    return param_dt == FSDP_BF16 ? pick_fused<u16, u16, REC>(R) : pick_fused<u16, float, REC>(R);
  return param_dt == FSDP_BF16 ? pick_fused<float, u16, REC>(R) : pick_fused<float, float, REC>(R);
}

template <typename G, typename P, bool REC>
const void* pick_fused_two_gather(int R) {
  return R == 8 ? reinterpret_cast<const void*>(&k_fused_two_gather<G, P, 8, REC>)
                : reinterpret_cast<const void*>(&k_fused_two_gather<G, P, 0, REC>);
}

template <bool REC>
const void* fused_two_gather_fn(int grad_dt, int param_dt, int R) {
  if (grad_dt == FSDP_BF16)
    return param_dt == FSDP_BF16 ? pick_fused_two_gather<u16, u16, REC>(R)
                                 : pick_fused_two_gather<u16, float, REC>(R);
  return param_dt == FSDP_BF16 ? pick_fused_two_gather<float, u16, REC>(R)
                               : pick_fused_two_gather<float, float, REC>(R);
}

template <bool REC>
const void* fused_gather_fn(int grad_dt, int param_dt, int R) {
  if (grad_dt == FSDP_BF16)
    return param_dt == FSDP_BF16 ? pick_fused_gather<u16, u16, REC>(R)
                                 : pick_fused_gather<u16, float, REC>(R);
  return param_dt == FSDP_BF16 ? pick_fused_gather<float, u16, REC>(R)
                               : pick_fused_gather<float, float, REC>(R);
}

// The copy kernel for up to 8 destinations: the unrolled instance for 4 or
// 8 of them, the loop otherwise.
template <int ES, int W>
const void* copy_fn(int n_dst) {
  switch (n_dst) {
    case 4: return reinterpret_cast<const void*>(&k_copy<ES, W, kSmallPtrs, 4>);
    case 8: return reinterpret_cast<const void*>(&k_copy<ES, W, kSmallPtrs, 8>);
    default: return reinterpret_cast<const void*>(&k_copy<ES, W, kSmallPtrs, 0>);
  }
}

}  // namespace

hipError_t launch_copy(const Work* work, int64_t n_work, const void* src, const PtrArray& dst,
                       int n_dst, int es, int lane_bytes, bool vec, const Sink& stream) {
  if (n_dst < 1 || n_dst > FSDP_MAX_RANKS) return hipErrorInvalidValue;
  const bool wide = lane_bytes != 8;
  if (n_dst <= kSmallPtrs) {
    CopyArgs<kSmallPtrs> a{src, narrow<kSmallPtrs>(dst), n_dst, vec ? 1 : 0};
    const void* fn = es == 2 ? (wide ? copy_fn<2, 16>(n_dst) : copy_fn<2, 8>(n_dst))
                             : (wide ? copy_fn<4, 16>(n_dst) : copy_fn<4, 8>(n_dst));
    return launch_work(fn, work, n_work, a, stream);
  }
  CopyArgs<FSDP_MAX_RANKS> a{src, narrow<FSDP_MAX_RANKS>(dst), n_dst, vec ? 1 : 0};
  const void* fn =
      es == 2 ? (wide ? reinterpret_cast<const void*>(&k_copy<2, 16, FSDP_MAX_RANKS>)
                      : reinterpret_cast<const void*>(&k_copy<2, 8, FSDP_MAX_RANKS>))
              : (wide ? reinterpret_cast<const void*>(&k_copy<4, 16, FSDP_MAX_RANKS>)
                      : reinterpret_cast<const void*>(&k_copy<4, 8, FSDP_MAX_RANKS>));
  return launch_work(fn, work, n_work, a, stream);
}

hipError_t launch_pack_cast(const Work* work, int64_t n_work, const void* src, int src_dt,
                            void* dst, int dst_dt, bool vec, const Sink& stream) {
  CastArgs a{src, dst, vec ? 1 : 0};
  const void* fn = nullptr;
  if (src_dt == FSDP_F32 && dst_dt == FSDP_BF16)
    fn = reinterpret_cast<const void*>(&k_pack_cast<float, u16>);
  else if (src_dt == FSDP_BF16 && dst_dt == FSDP_F32)
    fn = reinterpret_cast<const void*>(&k_pack_cast<u16, float>);
  else
    return hipErrorInvalidValue;
  return launch_work(fn, work, n_work, a, stream);
}

hipError_t launch_rs_avg(const Work* work, int64_t n_work, const PtrArray& grads, int R,
                         int grad_dt, float* out, bool vec, const Sink& stream) {
  if (R >= 8 && n_work > 0 && n_work <= kSmallFusedLaunch) {  // short: two per lane
    const void* fn = grad_dt == FSDP_BF16 ? pick_rs_two<u16>(R) : pick_rs_two<float>(R);
    const dim3 grid(static_cast<unsigned>(2 * n_work));
    if (R <= kSmallPtrs) {
      RsArgs<kSmallPtrs> a{narrow<kSmallPtrs>(grads), out, R, vec ? 1 : 0};
      void* args[] = {const_cast<Work**>(&work), &a};
      return stream.launch(fn, grid, dim3(kThreads), args, 0);
    }
    RsArgs<FSDP_MAX_RANKS> a{narrow<FSDP_MAX_RANKS>(grads), out, R, vec ? 1 : 0};
    void* args[] = {const_cast<Work**>(&work), &a};
    return stream.launch(fn, grid, dim3(kThreads), args, 0);
  }
  const void* fn = grad_dt == FSDP_BF16 ? pick_rs<u16>(R) : pick_rs<float>(R);
  if (R <= kSmallPtrs) {
    RsArgs<kSmallPtrs> a{narrow<kSmallPtrs>(grads), out, R, vec ? 1 : 0};
    return launch_work(fn, work, n_work, a, stream);
  }
  RsArgs<FSDP_MAX_RANKS> a{narrow<FSDP_MAX_RANKS>(grads), out, R, vec ? 1 : 0};
  return launch_work(fn, work, n_work, a, stream);
}

hipError_t launch_adamw(int64_t n, const float* g, float* master, float* m, float* v,
                        void* param, int param_dt, const AdamScalars& sc,
                        const AdamScalars* scp, bool vec, const Sink& stream) {
  if (n <= 0) return hipSuccess;
  AdamArgs a{g, master, m, v, param, sc, scp, n, vec ? 1 : 0};
  const int64_t chunks = (n + kEPL - 1) / kEPL;
  const int64_t blocks = (chunks + kThreads - 1) / kThreads;
  if (blocks > kMaxBlocks) return hipErrorInvalidValue;
  void* args[] = {&a};
  if (blocks <= kSmallFusedLaunch) {  // short: two elements per lane
    const int64_t blocks2 = (n + 2 * kThreads - 1) / (2 * kThreads);
    return stream.launch(adamw_fn<true>(param_dt, scp != nullptr),
                         dim3(static_cast<unsigned>(blocks2)), dim3(kThreads), args, 0);
  }
  return stream.launch(adamw_fn<false>(param_dt, scp != nullptr),
                       dim3(static_cast<unsigned>(blocks)), dim3(kThreads), args,
                       adamw_lds(blocks));
}

hipError_t launch_fused(const Work* work, int64_t n_work, const PtrArray& grads, int R,
                        int grad_dt, float* master, float* m, float* v, void* param,
                        int param_dt, const AdamScalars& sc, const AdamScalars* scp,
                        bool vec, const Sink& stream) {
  // one element per lane, kSplit workgroups per item, or two, two per item
  const bool one = fused_one_lane(n_work, R);
  if (one || fused_pair_lane(n_work, R)) {
    if (n_work <= 0) return hipSuccess;
    const int64_t split = one ? kSplit : 2;
    if (n_work > kMaxBlocks / split) return hipErrorInvalidValue;
    const void* fn = one ? (scp ? fused_one_fn<true>(grad_dt, param_dt, R)
                                : fused_one_fn<false>(grad_dt, param_dt, R))
                         : (scp ? fused_pair_fn<true>(grad_dt, param_dt, R)
                                : fused_pair_fn<false>(grad_dt, param_dt, R));
    const unsigned lds = one ? 0 : fused_pair_lds(n_work);
    const dim3 grid(static_cast<unsigned>(n_work * split));
    if (R <= kSmallPtrs) {
      FusedArgs<kSmallPtrs> a{narrow<kSmallPtrs>(grads), master, m, v, param, sc, scp, R,
                              vec ? 1 : 0};
      void* args[] = {const_cast<Work**>(&work), &a};
      return stream.launch(fn, grid, dim3(kThreads), args, lds);
    }
    FusedArgs<FSDP_MAX_RANKS> a{narrow<FSDP_MAX_RANKS>(grads), master, m, v, param, sc, scp, R,
                                vec ? 1 : 0};
    void* args[] = {const_cast<Work**>(&work), &a};
    return stream.launch(fn, grid, dim3(kThreads), args, lds);
  }
  const void* fn = scp ? fused_fn<true>(grad_dt, param_dt, R)
                       : fused_fn<false>(grad_dt, param_dt, R);
  if (fn == nullptr) return hipErrorInvalidValue;
  if (R <= kSmallPtrs) {
    FusedArgs<kSmallPtrs> a{narrow<kSmallPtrs>(grads), master, m, v, param, sc, scp, R,
                            vec ? 1 : 0};
    return launch_work(fn, work, n_work, a, stream, fused_lds(n_work));
  }
  FusedArgs<FSDP_MAX_RANKS> a{narrow<FSDP_MAX_RANKS>(grads), master, m, v, param, sc, scp, R,
                              vec ? 1 : 0};
  return launch_work(fn, work, n_work, a, stream, fused_lds(n_work));
}

hipError_t launch_accumulate(int64_t T, int R, const PtrArray& grads, int grad_dt,
                             const PtrArray& acc, bool first, bool vec, const Sink& stream) {
  if (T <= 0) return hipSuccess;
  const int64_t blocks = (T + kThreads * kEPL - 1) / (kThreads * kEPL);
  if (blocks > kMaxBlocks || R < 1 || R > FSDP_MAX_RANKS) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(R));
  if (R <= kSmallPtrs) {
    AccArgs<kSmallPtrs> a{narrow<kSmallPtrs>(grads), narrow<kSmallPtrs>(acc), T, first ? 1 : 0,
                          vec ? 1 : 0};
    const void* fn =
        grad_dt == FSDP_BF16 ? reinterpret_cast<const void*>(&k_accumulate<u16, kSmallPtrs>)
                             : reinterpret_cast<const void*>(&k_accumulate<float, kSmallPtrs>);
    void* args[] = {&a};
    return stream.launch(fn, grid, dim3(kThreads), args, 0);
  }
  AccArgs<FSDP_MAX_RANKS> a{narrow<FSDP_MAX_RANKS>(grads), narrow<FSDP_MAX_RANKS>(acc), T,
                            first ? 1 : 0, vec ? 1 : 0};
  const void* fn =
      grad_dt == FSDP_BF16 ? reinterpret_cast<const void*>(&k_accumulate<u16, FSDP_MAX_RANKS>)
                           : reinterpret_cast<const void*>(&k_accumulate<float, FSDP_MAX_RANKS>);
  void* args[] = {&a};
  return stream.launch(fn, grid, dim3(kThreads), args, 0);
}

hipError_t launch_allreduce(int64_t T, int R, const PtrArray& grads, int grad_dt,
                            const PtrArray& out, int out_dt, bool vec, const Sink& stream) {
  if (T <= 0) return hipSuccess;
  const int64_t blocks = (T + kThreads * kEPL - 1) / (kThreads * kEPL);
  if (blocks > kMaxBlocks) return hipErrorInvalidValue;
  const void* fn;
  if (grad_dt == FSDP_BF16)
    fn = out_dt == FSDP_BF16 ? pick_allreduce<u16, u16>(R) : pick_allreduce<u16, float>(R);
  else
    fn = out_dt == FSDP_BF16 ? pick_allreduce<float, u16>(R) : pick_allreduce<float, float>(R);
  // the specialised kernels (R = 1, 2, 4, 8) carry 8 slots, the generic one 64
  if (R == 1 || R == 2 || R == 4 || R == 8) {
    ArArgs<kSmallPtrs> a{narrow<kSmallPtrs>(grads), narrow<kSmallPtrs>(out), T, R, vec ? 1 : 0};
    void* args[] = {&a};
    return stream.launch(fn, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), args,
                         allreduce_lds(blocks));
  }
  ArArgs<FSDP_MAX_RANKS> a{narrow<FSDP_MAX_RANKS>(grads), narrow<FSDP_MAX_RANKS>(out), T, R,
                           vec ? 1 : 0};
  void* args[] = {&a};
  return stream.launch(fn, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), args,
                       allreduce_lds(blocks));
}

hipError_t launch_copy_pairs(const Work* work, int64_t n_work, const PtrArray& src,
                             const PtrArray& dst, int n_pairs, int es, bool vec,
                             const Sink& stream) {
  if (n_work <= 0 || n_pairs <= 0) return hipSuccess;
  if (n_work > kMaxBlocks || n_pairs > FSDP_MAX_RANKS) return hipErrorInvalidValue;
  PairArgs a{narrow<FSDP_MAX_RANKS>(src), narrow<FSDP_MAX_RANKS>(dst), vec ? 1 : 0};
  const void* fn = es == 2 ? reinterpret_cast<const void*>(&k_copy_pairs<2>)
                           : reinterpret_cast<const void*>(&k_copy_pairs<4>);
  void* args[] = {const_cast<Work**>(&work), &a};
  return stream.launch(fn, dim3(static_cast<unsigned>(n_work), static_cast<unsigned>(n_pairs)),
                       dim3(kThreads), args, 0);
}

hipError_t launch_set_scalars(AdamScalars* dst, const AdamScalars& sc, const Sink& stream) {
  AdamScalars v = sc;
  void* args[] = {&dst, &v};
  return stream.launch(reinterpret_cast<const void*>(&k_set_scalars), dim3(1), dim3(64), args, 0);
}

hipError_t StreamSink::launch(const void* fn, dim3 grid, dim3 block, void** args,
                              unsigned lds) const {
  return hipLaunchKernel(fn, grid, block, args, lds, stream_);
}

hipError_t launch_fused_gather(const Work* fwork, int64_t n_fused, const PtrArray& grads, int R,
                               int grad_dt, float* master, float* m, float* v, void* param,
                               int param_dt, const AdamScalars& sc, const AdamScalars* scp,
                               bool vec_f, const Work* gwork, int64_t n_gather,
                               const void* shards, const PtrArray& dst, int n_dst,
                               int lane_bytes, bool vec_g, const Sink& stream) {
  if (n_fused <= 0 || n_gather <= 0 || n_dst < 1) return hipErrorInvalidValue;
  // R >= 8: the two-element form of the step, two workgroups per item
  const bool two = R >= 8;
  const int64_t fused_blocks = two ? n_fused * 2 : n_fused;
  if (fused_blocks + n_gather > kMaxBlocks) return hipErrorInvalidValue;
  int nf = static_cast<int>(fused_blocks);
  int wide = lane_bytes == 16 ? 1 : 0;
  const void* fn = two ? (scp ? fused_two_gather_fn<true>(grad_dt, param_dt, R)
                              : fused_two_gather_fn<false>(grad_dt, param_dt, R))
                       : (scp ? fused_gather_fn<true>(grad_dt, param_dt, R)
                              : fused_gather_fn<false>(grad_dt, param_dt, R));
  if (fn == nullptr) return hipErrorInvalidValue;
  const unsigned lds = two ? fused_pair_lds(n_fused) : fused_lds(n_fused);
  const dim3 grid(static_cast<unsigned>(fused_blocks + n_gather));
  if (R <= kSmallPtrs) {   // the specialised kernel: 8 slots for both arrays
    if (n_dst > kSmallPtrs) return hipErrorInvalidValue;
    FusedArgs<kSmallPtrs> fa{narrow<kSmallPtrs>(grads), master, m, v, param, sc, scp, R,
                             vec_f ? 1 : 0};
    CopyArgs<kSmallPtrs> ca{shards, narrow<kSmallPtrs>(dst), n_dst, vec_g ? 1 : 0};
    void* args[] = {const_cast<Work**>(&fwork), &fa, &nf, const_cast<Work**>(&gwork), &ca,
                    &wide};
    return stream.launch(fn, grid, dim3(kThreads), args, lds);
  }
  FusedArgs<FSDP_MAX_RANKS> fa{narrow<FSDP_MAX_RANKS>(grads), master, m, v, param, sc, scp, R,
                               vec_f ? 1 : 0};
  CopyArgs<FSDP_MAX_RANKS> ca{shards, narrow<FSDP_MAX_RANKS>(dst), n_dst, vec_g ? 1 : 0};
  void* args[] = {const_cast<Work**>(&fwork), &fa, &nf, const_cast<Work**>(&gwork), &ca, &wide};
  return stream.launch(fn, grid, dim3(kThreads), args, lds);
}

}  // namespace fsdp
