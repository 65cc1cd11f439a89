// fingerprint_device.h -- device code of the fingerprint scan shared by the
// list scan and the single-tensor scan: per-lane accumulation of (S, W, X,
// NF) over 16-byte vectors, the item body loop, head/tail elements, wave and
// workgroup reductions, the wave-item scan and the merge of partial rows.
#pragma once

#include "scan_device.h"

namespace sdc {
namespace {

// acc + lo(d)*lo(w) + hi(d)*hi(w): 16x16 -> 32-bit products (v_dot2_u32_u16 /
// v_dot2_i32_i16, the latter with sign-extended halves), no clamping.
__device__ __forceinline__ uint32_t udot2(uint32_t d, uint32_t w, uint32_t acc) {
  return __builtin_amdgcn_udot2(as_us2(d), as_us2(w), acc, false);
}
__device__ __forceinline__ int32_t sdot2(uint32_t d, uint32_t w, int32_t acc) {
  return __builtin_amdgcn_sdot2(as_s2(d), as_s2(w), acc, false);
}
// acc + sum over the 4 bytes of d*w (v_dot4_u32_u8).
__device__ __forceinline__ uint32_t udot4(uint32_t d, uint32_t w, uint32_t acc) {
  return __builtin_amdgcn_udot4(d, w, acc, false);
}

// ---- per-lane accumulation ------------------------------------------------------
// Per-lane partial state of one item.
struct Lane {
  uint64_t s = 0;   // sum of widened x over the lane's elements
  uint64_t w = 0;   // sum of (j+1) x over the lane's elements (j: index in the item)
  uint64_t x = 0;   // xor of the raw words / elements (folded to the width later)
  uint64_t nf = 0;  // exact non-finite count
};

// Per vector of E = 16/ES elements: a = sum x, c = sum k x (k = slot in the
// vector), q = running sum of a after each vector, x = xor of raw words.
// 32-bit a and c cannot overflow within an item (<= 1024 vectors per lane).
template <uint32_t ES, bool SIGNED, int CHK>
struct Acc;

template <bool SIGNED, int CHK>
struct Acc<1, SIGNED, CHK> {  // 16 bytes per vector; 1-byte elements are never sign-extended
  uint32_t a = 0, c = 0, x = 0;
  uint64_t q = 0;
  Chk<CHK> chk;
  __device__ __forceinline__ explicit Acc(const NfRule& r) : chk(r) {}
  __device__ __forceinline__ void add(u32x4 v) {
    a = udot4(v.x, 0x01010101u, a);
    a = udot4(v.y, 0x01010101u, a);
    a = udot4(v.z, 0x01010101u, a);
    a = udot4(v.w, 0x01010101u, a);
    c = udot4(v.x, 0x03020100u, c);
    c = udot4(v.y, 0x07060504u, c);
    c = udot4(v.z, 0x0B0A0908u, c);
    c = udot4(v.w, 0x0F0E0D0Cu, c);
    q += a;
    x ^= v.x ^ v.y ^ v.z ^ v.w;
    chk.add(v);
  }
  __device__ __forceinline__ uint64_t sum() const { return a; }
  __device__ __forceinline__ uint64_t csum() const { return c; }
};

template <int CHK>
struct Acc<2, false, CHK> {
  uint32_t a = 0, c = 0, x = 0;
  uint64_t q = 0;
  Chk<CHK> chk;
  __device__ __forceinline__ explicit Acc(const NfRule& r) : chk(r) {}
  __device__ __forceinline__ void add(u32x4 v) {
    a = udot2(v.x, 0x00010001u, a);
    a = udot2(v.y, 0x00010001u, a);
    a = udot2(v.z, 0x00010001u, a);
    a = udot2(v.w, 0x00010001u, a);
    c = udot2(v.x, 0x00010000u, c);
    c = udot2(v.y, 0x00030002u, c);
    c = udot2(v.z, 0x00050004u, c);
    c = udot2(v.w, 0x00070006u, c);
    q += a;
    x ^= v.x ^ v.y ^ v.z ^ v.w;
    chk.add(v);
  }
  __device__ __forceinline__ uint64_t sum() const { return a; }
  __device__ __forceinline__ uint64_t csum() const { return c; }
};

template <int CHK>
struct Acc<2, true, CHK> {  // halves read as int16 (sign-extended products)
  int32_t a = 0, c = 0;
  uint32_t x = 0;
  uint64_t q = 0;
  Chk<CHK> chk;
  __device__ __forceinline__ explicit Acc(const NfRule& r) : chk(r) {}
  __device__ __forceinline__ void add(u32x4 v) {
    a = sdot2(v.x, 0x00010001u, a);
    a = sdot2(v.y, 0x00010001u, a);
    a = sdot2(v.z, 0x00010001u, a);
    a = sdot2(v.w, 0x00010001u, a);
    c = sdot2(v.x, 0x00010000u, c);
    c = sdot2(v.y, 0x00030002u, c);
    c = sdot2(v.z, 0x00050004u, c);
    c = sdot2(v.w, 0x00070006u, c);
    q += (uint64_t)(int64_t)a;
    x ^= v.x ^ v.y ^ v.z ^ v.w;
    chk.add(v);
  }
  __device__ __forceinline__ uint64_t sum() const { return (uint64_t)(int64_t)a; }
  __device__ __forceinline__ uint64_t csum() const { return (uint64_t)(int64_t)c; }
};

template <bool SIGNED, int CHK>
struct Acc<4, SIGNED, CHK> {
  uint64_t a = 0, c = 0, q = 0;
  uint32_t x = 0;
  Chk<CHK> chk;
  __device__ __forceinline__ explicit Acc(const NfRule& r) : chk(r) {}
  __device__ __forceinline__ static uint64_t wid(uint32_t v) {
    if constexpr (SIGNED) return (uint64_t)(int64_t)(int32_t)v;
    return (uint64_t)v;
  }
  __device__ __forceinline__ void add(u32x4 v) {
    a += wid(v.x) + wid(v.y) + wid(v.z) + wid(v.w);
    c += wid(v.y) + 2ull * wid(v.z) + 3ull * wid(v.w);
    q += a;
    x ^= v.x ^ v.y ^ v.z ^ v.w;
    chk.add(v);
  }
  __device__ __forceinline__ uint64_t sum() const { return a; }
  __device__ __forceinline__ uint64_t csum() const { return c; }
};

template <bool SIGNED, int CHK>
struct Acc<8, SIGNED, CHK> {  // 2 elements per vector, full 64-bit patterns
  uint64_t a = 0, c = 0, q = 0, x = 0;
  Chk<CHK> chk;
  __device__ __forceinline__ explicit Acc(const NfRule& r) : chk(r) {}
  __device__ __forceinline__ void add(u32x4 v) {
    const uint64_t x0 = lohi(v.x, v.y), x1 = lohi(v.z, v.w);
    a += x0 + x1;
    c += x1;
    q += a;
    x ^= x0 ^ x1;
    chk.add(v);
  }
  __device__ __forceinline__ uint64_t sum() const { return a; }
  __device__ __forceinline__ uint64_t csum() const { return c; }
};

// Shape of the body loop: U vector loads per lane per round; with PIPE the
// loads of round r+1 are issued before round r is consumed, so a wave keeps
// loads in flight while it computes.
template <int U_, bool PIPE_>
struct BodyCfg {
  static constexpr int U = U_;
  static constexpr bool PIPE = PIPE_;
};
typedef BodyCfg<4, true> DefaultBody;  // ~104 VGPRs: 4 workgroups per CU
typedef BodyCfg<8, true> DeepBody;     // ~188 VGPRs: deeper pipeline, 2 workgroups per CU
typedef BodyCfg<kWideU, false> WideBody;  // the wide shape: one workgroup per CU
// Plans whose items average at least this many bytes use DeepBody (measured:
// better for items of ~170 KiB and more, worse for lists of small tensors).
constexpr uint64_t kDeepItemBytes = 96ull << 10;
// NaN/Inf exact counts: bodies of at least this many vectors per lane per
// round count a flagged round from its registers; shorter rounds (where a
// check per round measurably slows lists of small tensors) keep one flag per
// item and, when it is set, re-read the lane's vectors in a second pass.
constexpr int kRoundCheckMinU = 8;
// Body of one item: nvec aligned vectors at `body`.  Lane t handles vectors
// 256*it + t, it = 0 .. T-1 with T = rounds*U (uniform over the workgroup);
// vectors past the end are not loaded and count as zero vectors, which leave
// every partial sum unchanged (and keep T*A - Q exact).
template <class Ty, class Cfg>
__device__ __forceinline__ void scan_body(const unsigned char* body, uint32_t nvec, uint32_t h,
                                          const NfRule& rule, Lane& ln) {
  typedef Acc<Ty::ES, Ty::SIGNED, Ty::CHK> A_t;
  constexpr int U = Cfg::U;
  constexpr uint32_t E = kVecBytes / Ty::ES;    // elements per vector
  const uint32_t t = threadIdx.x;
  A_t acc(rule);
  uint32_t nf = 0;
  uint32_t rounds;
  if constexpr (U >= kRoundCheckMinU) {
    rounds = stream_body<U, Cfg::PIPE>(
        body, nvec, [&](u32x4 v) { acc.add(v); },
        [&](const u32x4 (&v)[U]) { count_flagged_round(acc.chk, v, nf); });
  } else {
    rounds = stream_body<U, Cfg::PIPE>(body, nvec, [&](u32x4 v) { acc.add(v); });
    if (acc.chk.flagged())  // rare: a second, pipelined pass over this lane's vectors
      stream_body<U, Cfg::PIPE>(body, nvec, [&](u32x4 v) { nf += acc.chk.exact(v); });
  }
  const uint64_t T = (uint64_t)rounds * U;
  const uint64_t A = acc.sum();
  ln.s += A;
  ln.w += (uint64_t)(h + 1u + E * t) * A + (uint64_t)(kBlock * E) * (T * A - acc.q) + acc.csum();
  ln.x ^= acc.x;
  ln.nf += nf;
}

template <uint32_t ES, bool SIGNED>
__device__ __forceinline__ uint64_t widen(uint64_t raw) {
  if constexpr (SIGNED && ES == 2) return (uint64_t)(int64_t)(int16_t)(uint16_t)raw;
  if constexpr (SIGNED && ES == 4) return (uint64_t)(int64_t)(int32_t)(uint32_t)raw;
  return raw;
}

// Head/tail element j (index within the item) with raw pattern `raw`.  A zero
// pattern adds nothing to any column (zero is never NaN/Inf).
template <class Ty>
__device__ __forceinline__ void add_scalar(uint64_t raw, uint32_t j, const NfRule& rule, Lane& ln) {
  const uint64_t v = widen<Ty::ES, Ty::SIGNED>(raw);
  ln.s += v;
  ln.w += (uint64_t)(j + 1u) * v;
  ln.x ^= raw;
  if constexpr (Ty::CHK != kChkNone) ln.nf += nf_exact(raw, rule);
}

// xor of raw words -> xor of the elements' widened patterns.
template <class Ty>
__device__ __forceinline__ uint64_t finish_xor(uint64_t x) {
  if constexpr (Ty::ES == 1) {
    x ^= x >> 16;
    x = (x ^ (x >> 8)) & 0xFFu;
  } else if constexpr (Ty::ES == 2) {
    x = (x & 0xFFFFu) ^ (x >> 16);
  }
  return widen<Ty::ES, Ty::SIGNED>(x);
}

__device__ __forceinline__ void wave_reduce(Lane& ln) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    ln.s += __shfl_xor(ln.s, off);
    ln.w += __shfl_xor(ln.w, off);
    ln.x ^= __shfl_xor(ln.x, off);
    ln.nf += __shfl_xor(ln.nf, off);
  }
}

__device__ __forceinline__ void block_reduce(Lane& ln) {
  wave_reduce(ln);
  __shared__ uint64_t ls[kWaves], lw[kWaves], lx[kWaves], ln_[kWaves];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    ls[wave] = ln.s;
    lw[wave] = ln.w;
    lx[wave] = ln.x;
    ln_[wave] = ln.nf;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 1; i < kWaves; ++i) {
      ln.s += ls[i];
      ln.w += lw[i];
      ln.x ^= lx[i];
      ln.nf += ln_[i];
    }
  }
}

// Scan of one item by a workgroup; lane 0 ends with the item's
// (S, sum (j+1) x_j with j local to the item, X, NF).
template <class Ty, class Cfg>
__device__ __forceinline__ void scan_item(const PlanItem& it, Lane& ln) {
  constexpr uint32_t es = Ty::ES;
  const Span sp = span_of<es>(it);
  const NfRule rule = nf_rule(it.dtype_flags & kItemDtypeMask);
  const uint32_t t = threadIdx.x;
  const ItemEnds<es> ends(sp, t);
  if (sp.nvec) scan_body<Ty, Cfg>(sp.base + (uint64_t)sp.h * es, sp.nvec, sp.h, rule, ln);
  add_scalar<Ty>(ends.head, t, rule, ln);
  add_scalar<Ty>(ends.tail, ends.tail_index(sp, t), rule, ln);
  block_reduce(ln);
  ln.x = finish_xor<Ty>(ln.x);
}

// ---- wave items: small tensors, one group of lanes each ---------------------------
// The aligned body has at most LANES x kWaveVecs vectors; lane l loads vectors
// LANES*u + l for u = 0 .. kWaveVecs-1 all at once (T = kWaveVecs, missing
// vectors count as zero), then W_lane = (h+1+E*l)*A + LANES*E*(T*A - Q) + C.
// Loads go through per-lane addresses: the groups of a wave (up to 8) read
// different tensors.
template <uint32_t LANES>
__device__ __forceinline__ void part_reduce(Lane& ln) {
#pragma unroll
  for (uint32_t off = LANES / 2; off > 0; off >>= 1) {  // stays within the LANES lanes
    ln.s += __shfl_xor(ln.s, off);
    ln.w += __shfl_xor(ln.w, off);
    ln.x ^= __shfl_xor(ln.x, off);
    ln.nf += __shfl_xor(ln.nf, off);
  }
}

template <class Ty, uint32_t LANES>
__device__ __forceinline__ void scan_small(const PlanItem& it, uint32_t l, Lane& ln) {
  typedef Acc<Ty::ES, Ty::SIGNED, Ty::CHK> A_t;
  constexpr uint32_t es = Ty::ES;
  constexpr uint32_t E = kVecBytes / es;
  const Span sp = span_of<es>(it);
  const NfRule rule = nf_rule(it.dtype_flags & kItemDtypeMask);
  const WaveItemLoads<es, LANES> ld(sp, l);
#pragma unroll
  for (uint32_t k = 0; k < ld.kHT; ++k) {
    const uint32_t j = k * LANES + l;
    add_scalar<Ty>(ld.head[k], j, rule, ln);
    add_scalar<Ty>(ld.tail[k], sp.tail0 + j, rule, ln);
  }
  // No branch on the body's size (the compiler would sink the loads into
  // it): zero vectors add nothing.
  A_t acc(rule);
#pragma unroll
  for (uint32_t u = 0; u < kWaveVecs; ++u) acc.add(ld.v[u]);
  const uint64_t T = kWaveVecs;
  const uint64_t A = acc.sum();
  ln.s += A;
  ln.w += (uint64_t)(sp.h + 1u + E * l) * A + (uint64_t)(LANES * E) * (T * A - acc.q) + acc.csum();
  ln.x ^= acc.x;
  if (acc.chk.flagged()) {  // rare: count this lane's vectors exactly (zero vectors count none)
    uint32_t c = 0;
#pragma unroll
    for (uint32_t u = 0; u < kWaveVecs; ++u) c += acc.chk.exact(ld.v[u]);
    ln.nf += c;
  }
  part_reduce<LANES>(ln);
  ln.x = finish_xor<Ty>(ln.x);
}

// kLanes lanes combine `count` partial rows at p (+, +, ^, +), lane l taking
// rows l, l + kLanes, ...; kMergeUnroll independent row loads per lane are in
// flight, so a tensor split into thousands of items is merged in a few
// memory latencies.  The lanes' results still have to be reduced.
template <uint32_t kLanes = 64>
__device__ __forceinline__ Lane merge_slots(const sdc_row* __restrict__ rows, uint32_t count,
                                            uint32_t l) {
  Lane ln;
  const ulonglong2* p = reinterpret_cast<const ulonglong2*>(rows);
  for (uint32_t i0 = 0; i0 < count; i0 += kLanes * kMergeUnroll) {
    ulonglong2 a[kMergeUnroll], b[kMergeUnroll];
#pragma unroll
    for (uint32_t u = 0; u < kMergeUnroll; ++u) {
      const uint32_t i = i0 + u * kLanes + l;
      a[u] = (i < count) ? p[2 * i] : ulonglong2{0, 0};
      b[u] = (i < count) ? p[2 * i + 1] : ulonglong2{0, 0};
    }
#pragma unroll
    for (uint32_t u = 0; u < kMergeUnroll; ++u) {
      ln.s += a[u].x;
      ln.w += a[u].y;
      ln.x ^= b[u].x;
      ln.nf += b[u].y;
    }
  }
  return ln;
}

}  // namespace
}  // namespace sdc
