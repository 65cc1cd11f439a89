// scan.hip -- the fused multi-tensor integrity scan for gfx950.
//
// Computes, for every tensor of a list, the row (S, W, X, NF) defined in
// include/sdc.h: the plain and position-weighted 64-bit sums of the raw bit
// patterns (AWS Machine Learning Blog, "Detecting and recovering from silent
// data corruption on Amazon SageMaker HyperPod", section "Compare by
// fingerprint"), the xorsum (AEGIS review page, section "core method" item 4)
// and the NaN/Inf count (same blog, section "Check 1").
//
// Structure (HBM-bound streaming reduction, no matrix cores):
//   * The host packs the list into self-contained work items (<= 4 MiB of one
//     tensor each); one 256-lane workgroup scans one item.  Item boundaries
//     inside a tensor are 16-byte aligned, so only an item that starts a
//     tensor can have a misaligned head and only the last one a tail.
//   * The aligned body is read with coalesced 16-byte non-temporal buffer
//     loads (lane t of the workgroup takes vector 256*it + t of the body),
//     U per lane in flight.
//   * Per lane the 16-bit path keeps 32-bit partial sums built with
//     v_dot2_u32_u16 (two elements per instruction): A = sum x,
//     C = sum (k x) with k the element's slot in its 8-element vector, and a
//     running sum Q of A after each vector, from which sum_it it*s_it =
//     T*A - Q.  The lane's weighted sum is then
//       W_lane = (h + 1 + E*t) * A + 256*E*(T*A - Q) + C   (mod 2^64),
//     so the only 64-bit multiplies happen once per lane per item.
//   * NaN/Inf: a sticky fma(x, 0, acc) stays +0 unless an element is NaN or
//     Inf (the packed fp16 form flags every bf16/fp16 NaN/Inf, and possibly a
//     few huge finite bf16 values); a lane whose flag is set rescans its own
//     vectors with the exact exponent test.  So the count is exact.
//   * Lane results are combined with wave shuffles, then across the 4 waves
//     through LDS.  The item's row is W_item = start*S_item + sum_j (j+1) x_j
//     (the concatenation identity W(A||B) = W(A) + W(B) + |A| S(B) in additive
//     form); a tensor scanned by one item stores its row, each item of a
//     split tensor stores a partial row in its own slot, and one wave per
//     split tensor combines its slots (+, +, ^, +: order independent, so the
//     result is bit-exact, and no atomics share an address).
#include <algorithm>
#include <cstring>
#include <vector>

#include "sdc_internal.h"

namespace sdc {
namespace {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef short s2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// By-value reinterpretations.  (Bit-casting a vector component in place is
// avoided on purpose: clang lowers __builtin_bit_cast(T, v.y) as a read of
// the vector's first component.)
__device__ __forceinline__ us2 as_us2(uint32_t w) { return __builtin_bit_cast(us2, w); }
__device__ __forceinline__ s2 as_s2(uint32_t w) { return __builtin_bit_cast(s2, w); }
__device__ __forceinline__ h2 as_h2(uint32_t w) { return __builtin_bit_cast(h2, w); }
__device__ __forceinline__ uint32_t h2_bits(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ uint64_t lohi(uint32_t lo, uint32_t hi) {
  return (uint64_t)lo | ((uint64_t)hi << 32);
}

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

// Raw buffer over [base, base + bytes): loads beyond `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Cache policy of the streaming loads: the non-temporal bit (CPol NT on
// gfx94x/gfx950).  Every byte is read exactly once, and with this hint the
// chip's streaming-read rate rises from about 6.3 to about 7.1 TB/s.
constexpr int kLoadPolicy = 2;

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, kLoadPolicy));
}

// ---- NaN/Inf ------------------------------------------------------------------
// Exact rule: an element is NaN/Inf when (x & mask) == val; mask 0: never.
struct NfRule {
  uint64_t mask, val;
};

__device__ __forceinline__ NfRule nf_rule(uint32_t dtype) {
  switch (dtype) {
    case SDC_F32: return NfRule{0x7F800000ull, 0x7F800000ull};
    case SDC_BF16: return NfRule{0x7F80ull, 0x7F80ull};
    case SDC_F16: return NfRule{0x7C00ull, 0x7C00ull};
    case SDC_F64: return NfRule{0x7FF0000000000000ull, 0x7FF0000000000000ull};
    case SDC_FP8_E4M3: return NfRule{0x7Full, 0x7Full};  // no Inf; NaN is S.1111.111
    case SDC_FP8_E5M2: return NfRule{0x7Cull, 0x7Cull};
    case SDC_FP8_E4M3FNUZ: case SDC_FP8_E5M2FNUZ: return NfRule{0xFFull, 0x80ull};  // the one NaN
    default: return NfRule{0ull, 1ull};  // raw integers
  }
}

__device__ __forceinline__ uint32_t nf_exact(uint64_t x, const NfRule& r) {
  return (x & r.mask) == r.val;
}

// Exact count over one 16-byte vector of ES-byte elements.
template <uint32_t ES>
__device__ __forceinline__ uint32_t nf_vec(u32x4 v, const NfRule& r) {
  uint32_t c = 0;
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
  if constexpr (ES == 8) {
    c = nf_exact(lohi(d[0], d[1]), r) + nf_exact(lohi(d[2], d[3]), r);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (uint32_t b = 0; b < 32; b += 8 * ES) c += nf_exact((d[i] >> b) & ((1ull << (8 * ES)) - 1), r);
    }
  }
  return c;
}

// Fast "may contain NaN/Inf" flag, per element-type family.  Every NaN/Inf
// sets it; a set flag triggers the exact recount, so false alarms only cost
// time.
enum : int { kChkNone = 0, kChkHalf = 1, kChkF32 = 2, kChkF64 = 3, kChkFp8Top = 4, kChkFp8Eq = 5 };

template <int CHK>
struct Chk;

template <>
struct Chk<kChkNone> {  // raw integers: never NaN/Inf
  __device__ __forceinline__ explicit Chk(const NfRule&) {}
  __device__ __forceinline__ void add(u32x4) {}
  __device__ __forceinline__ bool flagged() const { return false; }
};

// bf16 / fp16: fma(x, 0, acc) on the dword read as two fp16 halves stays +0
// unless a half is fp16 NaN/Inf (exponent bits 14..10 all ones) -- which every
// fp16 and bf16 NaN/Inf is (for bf16 also finite values >= 2^121).
template <>
struct Chk<kChkHalf> {
  h2 nf = {0, 0};
  __device__ __forceinline__ explicit Chk(const NfRule&) {}
  __device__ __forceinline__ void add(u32x4 v) {
    const h2 z = {0, 0};
    nf = __builtin_elementwise_fma(as_h2(v.x), z, nf);
    nf = __builtin_elementwise_fma(as_h2(v.y), z, nf);
    nf = __builtin_elementwise_fma(as_h2(v.z), z, nf);
    nf = __builtin_elementwise_fma(as_h2(v.w), z, nf);
  }
  __device__ __forceinline__ bool flagged() const { return h2_bits(nf) != 0; }
};

template <>
struct Chk<kChkF32> {  // exact: fma(x, 0, acc) is NaN iff x is NaN/Inf
  float nf = 0.0f;
  __device__ __forceinline__ explicit Chk(const NfRule&) {}
  __device__ __forceinline__ void add(u32x4 v) {
    nf = __builtin_fmaf(__uint_as_float(v.x), 0.0f, nf);
    nf = __builtin_fmaf(__uint_as_float(v.y), 0.0f, nf);
    nf = __builtin_fmaf(__uint_as_float(v.z), 0.0f, nf);
    nf = __builtin_fmaf(__uint_as_float(v.w), 0.0f, nf);
  }
  __device__ __forceinline__ bool flagged() const { return __float_as_uint(nf) != 0u; }
};

template <>
struct Chk<kChkF64> {  // exact, as for fp32
  double nf = 0.0;
  __device__ __forceinline__ explicit Chk(const NfRule&) {}
  __device__ __forceinline__ void add(u32x4 v) {
    nf = __builtin_fma(__longlong_as_double((long long)lohi(v.x, v.y)), 0.0, nf);
    nf = __builtin_fma(__longlong_as_double((long long)lohi(v.z, v.w)), 0.0, nf);
  }
  __device__ __forceinline__ bool flagged() const { return __double_as_longlong(nf) != 0; }
};

// fp8 whose NaN/Inf are "all ones under a mask m < 0x80" (E4M3: m = 0x7F,
// E5M2: m = 0x7C): per byte, (b & m) + (0x80 - m) reaches 0x80 exactly when
// (b & m) == m, without carrying into the next byte.  Exact.
template <>
struct Chk<kChkFp8Top> {
  uint32_t flag = 0, m4, k4;
  __device__ __forceinline__ explicit Chk(const NfRule& r)
      : m4((uint32_t)r.mask * 0x01010101u), k4((0x80u - (uint32_t)r.mask) * 0x01010101u) {}
  __device__ __forceinline__ void add(u32x4 v) {
    flag |= ((v.x & m4) + k4) & 0x80808080u;
    flag |= ((v.y & m4) + k4) & 0x80808080u;
    flag |= ((v.z & m4) + k4) & 0x80808080u;
    flag |= ((v.w & m4) + k4) & 0x80808080u;
  }
  __device__ __forceinline__ bool flagged() const { return flag != 0; }
};

// fp8 "fnuz": the single NaN 0x80; a byte of d ^ 0x80808080 is zero.  Exact.
template <>
struct Chk<kChkFp8Eq> {
  uint32_t flag = 0, v4;
  __device__ __forceinline__ explicit Chk(const NfRule& r) : v4((uint32_t)r.val * 0x01010101u) {}
  __device__ __forceinline__ void one(uint32_t d) {
    const uint32_t t = d ^ v4;
    flag |= (t - 0x01010101u) & ~t & 0x80808080u;
  }
  __device__ __forceinline__ void add(u32x4 v) {
    one(v.x);
    one(v.y);
    one(v.z);
    one(v.w);
  }
  __device__ __forceinline__ bool flagged() const { return flag != 0; }
};

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

// Element type of an item, resolved once per workgroup (or wave) into the
// compile-time width / signedness / NaN-check family.
template <uint32_t ES_, bool SIGNED_, int CHK_>
struct TypeTag {
  static constexpr uint32_t ES = ES_;
  static constexpr bool SIGNED = SIGNED_;
  static constexpr int CHK = CHK_;
};

template <class F>
__device__ __forceinline__ void dispatch_type(uint32_t df, F&& f) {
  const bool sg = (df & kItemSigned) != 0;
  switch (df & kItemDtypeMask) {
    case SDC_F32:
      if (sg) f(TypeTag<4, true, kChkF32>()); else f(TypeTag<4, false, kChkF32>());
      break;
    case SDC_U32:
      if (sg) f(TypeTag<4, true, kChkNone>()); else f(TypeTag<4, false, kChkNone>());
      break;
    case SDC_BF16: case SDC_F16:
      if (sg) f(TypeTag<2, true, kChkHalf>()); else f(TypeTag<2, false, kChkHalf>());
      break;
    case SDC_U16:
      if (sg) f(TypeTag<2, true, kChkNone>()); else f(TypeTag<2, false, kChkNone>());
      break;
    case SDC_F64: f(TypeTag<8, false, kChkF64>()); break;
    case SDC_U64: f(TypeTag<8, false, kChkNone>()); break;
    case SDC_FP8_E4M3: case SDC_FP8_E5M2: f(TypeTag<1, false, kChkFp8Top>()); break;
    case SDC_FP8_E4M3FNUZ: case SDC_FP8_E5M2FNUZ: f(TypeTag<1, false, kChkFp8Eq>()); break;
    default: f(TypeTag<1, false, kChkNone>()); break;  // SDC_U8
  }
}

// Shape of the body loop: U vector loads per lane per round; with PIPE the
// loads of round r+1 are issued before round r is consumed, so a wave keeps
// loads in flight while it computes.
template <int U_, bool PIPE_>
struct BodyCfg {
  static constexpr int U = U_;
  static constexpr bool PIPE = PIPE_;
};
typedef BodyCfg<4, true> DefaultBody;  // ~106 VGPRs: 4 workgroups per CU
typedef BodyCfg<8, true> DeepBody;     // ~188 VGPRs: deeper pipeline, 2 workgroups per CU
// Plans whose items average at least this many bytes use DeepBody (measured:
// better for items of ~170 KiB and more, worse for lists of small tensors).
constexpr uint64_t kDeepItemBytes = 96ull << 10;
// Vectors of the nonfinite-only loop per lane per round.
constexpr int kUnroll = 4;

// Loads round r (vectors r*256*U .. of the body) into v.  Rounds below
// `full` are complete; the last, partial round masks lanes past the end,
// whose vectors then read as zero.
template <int U>
__device__ __forceinline__ void load_round(const unsigned char* body, uint32_t nvec, uint32_t full,
                                           uint32_t r, u32x4 (&v)[U]) {
  constexpr uint32_t kRound = kBlock * U;
  const uint32_t t = threadIdx.x;
  const uint32_t v0 = r * kRound;
  if (r < full) {
    __amdgpu_buffer_rsrc_t rs = make_rsrc(body + (uint64_t)v0 * kVecBytes, kRound * kVecBytes);
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load16(rs, (u * kBlock + t) * kVecBytes);
  } else {
    const uint32_t left = nvec - v0;
    __amdgpu_buffer_rsrc_t rs = make_rsrc(body + (uint64_t)v0 * kVecBytes, left * kVecBytes);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t vi = u * kBlock + t;
      v[u] = (vi < left) ? load16(rs, vi * kVecBytes) : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

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
  constexpr uint32_t kRound = kBlock * U;      // vectors per round
  const uint32_t t = threadIdx.x;
  A_t acc(rule);
  const uint32_t full = nvec / kRound;
  const uint32_t rounds = full + ((nvec % kRound) ? 1u : 0u);
  if constexpr (!Cfg::PIPE) {
    for (uint32_t r = 0; r < rounds; ++r) {
      u32x4 v[U];
      load_round<U>(body, nvec, full, r, v);
#pragma unroll
      for (int u = 0; u < U; ++u) acc.add(v[u]);
    }
  } else {
    // Two register sets, alternating, so no copies are needed.
    u32x4 va[U], vb[U];
    load_round<U>(body, nvec, full, 0, va);
    uint32_t r = 0;
    for (;;) {
      if (r + 1 < rounds) load_round<U>(body, nvec, full, r + 1, vb);
#pragma unroll
      for (int u = 0; u < U; ++u) acc.add(va[u]);
      if (++r == rounds) break;
      if (r + 1 < rounds) load_round<U>(body, nvec, full, r + 1, va);
#pragma unroll
      for (int u = 0; u < U; ++u) acc.add(vb[u]);
      if (++r == rounds) break;
    }
  }
  const uint64_t T = (uint64_t)rounds * U;
  const uint64_t A = acc.sum();
  ln.s += A;
  ln.w += (uint64_t)(h + 1u + E * t) * A + (uint64_t)(kBlock * E) * (T * A - acc.q) + acc.csum();
  ln.x ^= acc.x;
  if (acc.chk.flagged()) {
    // Rare: some element may be NaN/Inf.  Recount this lane's vectors exactly.
    uint32_t c = 0;
    for (uint32_t vi = t; vi < nvec; vi += kBlock) {
      __amdgpu_buffer_rsrc_t rs = make_rsrc(body + (uint64_t)vi * kVecBytes, kVecBytes);
      c += nf_vec<Ty::ES>(load16(rs, 0), rule);
    }
    ln.nf += c;
  }
}

// Raw pattern of the ES-byte element at p.
template <uint32_t ES>
__device__ __forceinline__ uint64_t load_elem(const unsigned char* p) {
  if constexpr (ES == 1) return *p;
  if constexpr (ES == 2) return *reinterpret_cast<const unsigned short*>(p);
  if constexpr (ES == 4) return *reinterpret_cast<const uint32_t*>(p);
  return *reinterpret_cast<const uint64_t*>(p);
}

template <uint32_t ES, bool SIGNED>
__device__ __forceinline__ uint64_t widen(uint64_t raw) {
  if constexpr (SIGNED && ES == 2) return (uint64_t)(int64_t)(int16_t)(uint16_t)raw;
  if constexpr (SIGNED && ES == 4) return (uint64_t)(int64_t)(int32_t)(uint32_t)raw;
  return raw;
}

// Head/tail element j (index within the item) at p.
template <class Ty>
__device__ __forceinline__ void scan_scalar(const unsigned char* p, uint32_t j, const NfRule& rule,
                                            Lane& ln) {
  const uint64_t raw = load_elem<Ty::ES>(p);
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

// Index of the calling wave over the grid (4*block + wave), wave-uniform.
__device__ __forceinline__ uint32_t wave_item_index() {
  return __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6));
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

// Head, aligned body and tail of an item of ES-byte elements.
struct Span {
  const unsigned char* base;
  uint32_t h, nvec, tail0, ntail;
};

template <uint32_t ES>
__device__ __forceinline__ Span span_of(const PlanItem& it) {
  Span sp;
  sp.base = reinterpret_cast<const unsigned char*>(it.addr);
  const uint32_t len = it.len;
  const uint32_t mis = (uint32_t)(it.addr & 15u);
  sp.h = mis ? min(len, (16u - mis) / ES) : 0u;
  sp.nvec = (uint32_t)(((uint64_t)(len - sp.h) * ES) / kVecBytes);
  sp.tail0 = sp.h + sp.nvec * (kVecBytes / ES);
  sp.ntail = len - sp.tail0;
  return sp;
}

// Scan of one item by a workgroup; lane 0 ends with the item's
// (S, sum (j+1) x_j with j local to the item, X, NF).
template <class Ty, class Cfg>
__device__ __forceinline__ void scan_item(const PlanItem& it, Lane& ln) {
  constexpr uint32_t es = Ty::ES;
  const Span sp = span_of<es>(it);
  const NfRule rule = nf_rule(it.dtype_flags & kItemDtypeMask);
  const uint32_t t = threadIdx.x;
  if (t < sp.h) scan_scalar<Ty>(sp.base + (uint64_t)t * es, t, rule, ln);
  if (t >= 128u && t - 128u < sp.ntail) {
    const uint32_t j = sp.tail0 + (t - 128u);
    scan_scalar<Ty>(sp.base + (uint64_t)j * es, j, rule, ln);
  }
  if (sp.nvec) scan_body<Ty, Cfg>(sp.base + (uint64_t)sp.h * es, sp.nvec, sp.h, rule, ln);
  block_reduce(ln);
  ln.x = finish_xor<Ty>(ln.x);
}

template <class Cfg>
__global__ void __launch_bounds__(kBlock) fingerprint_kernel(const PlanItem* __restrict__ items,
                                                             sdc_row* __restrict__ partials,
                                                             sdc_row* __restrict__ out) {
  const PlanItem it = items[blockIdx.x];
  Lane ln;
  dispatch_type(it.dtype_flags, [&](auto ty) { scan_item<decltype(ty), Cfg>(it, ln); });
  if (threadIdx.x != 0) return;
  const uint64_t S = ln.s;
  const uint64_t W = ln.w + it.start * S;
  // A whole tensor stores its row; an item of a split tensor stores its
  // partial row in its own slot (plain stores: no two workgroups ever write
  // the same address, so there is no contention and no clearing).
  sdc_row* dst = (it.dtype_flags & kItemWhole) ? out + it.row : partials + it.slot;
  ulonglong2* d = reinterpret_cast<ulonglong2*>(dst);
  d[0] = ulonglong2{S, W};
  d[1] = ulonglong2{ln.x, ln.nf};
}

// ---- wave items: small tensors, one wave each ---------------------------------
// The aligned body has at most 64 x kWaveVecs vectors; lane l loads vectors
// 64*u + l for u = 0 .. kWaveVecs-1 all at once (T = kWaveVecs, missing
// vectors count as zero), then W_lane = (h+1+E*l)*A + 64*E*(T*A - Q) + C.
template <class Ty>
__device__ __forceinline__ void scan_small(const PlanItem& it, uint32_t l, Lane& ln) {
  typedef Acc<Ty::ES, Ty::SIGNED, Ty::CHK> A_t;
  constexpr uint32_t es = Ty::ES;
  constexpr uint32_t E = kVecBytes / es;
  const Span sp = span_of<es>(it);
  const NfRule rule = nf_rule(it.dtype_flags & kItemDtypeMask);
  if (l < sp.h) scan_scalar<Ty>(sp.base + (uint64_t)l * es, l, rule, ln);
  if (l >= 32u && l - 32u < sp.ntail) {
    const uint32_t j = sp.tail0 + (l - 32u);
    scan_scalar<Ty>(sp.base + (uint64_t)j * es, j, rule, ln);
  }
  if (sp.nvec) {
    const unsigned char* body = sp.base + (uint64_t)sp.h * es;
    __amdgpu_buffer_rsrc_t rs = make_rsrc(body, sp.nvec * kVecBytes);
    u32x4 v[kWaveVecs];
#pragma unroll
    for (uint32_t u = 0; u < kWaveVecs; ++u) {
      const uint32_t vi = u * 64u + l;
      v[u] = (vi < sp.nvec) ? load16(rs, vi * kVecBytes) : u32x4{0u, 0u, 0u, 0u};
    }
    A_t acc(rule);
#pragma unroll
    for (uint32_t u = 0; u < kWaveVecs; ++u) acc.add(v[u]);
    const uint64_t T = kWaveVecs;
    const uint64_t A = acc.sum();
    ln.s += A;
    ln.w += (uint64_t)(sp.h + 1u + E * l) * A + (uint64_t)(64u * E) * (T * A - acc.q) + acc.csum();
    ln.x ^= acc.x;
    if (acc.chk.flagged()) {  // rare: reload this lane's vectors and count exactly
      uint32_t c = 0;
      for (uint32_t vi = l; vi < sp.nvec; vi += 64u) c += nf_vec<es>(load16(rs, vi * kVecBytes), rule);
      ln.nf += c;
    }
  }
  wave_reduce(ln);
  ln.x = finish_xor<Ty>(ln.x);
}

__global__ void __launch_bounds__(kBlock) fingerprint_small_kernel(const PlanItem* __restrict__ items,
                                                                   uint32_t n,
                                                                   sdc_row* __restrict__ out) {
  const uint32_t i = wave_item_index();
  if (i >= n) return;  // the whole wave leaves; no workgroup barrier in this kernel
  const PlanItem it = items[i];
  const uint32_t l = threadIdx.x & 63u;
  Lane ln;
  dispatch_type(it.dtype_flags, [&](auto ty) { scan_small<decltype(ty)>(it, l, ln); });
  if (l != 0) return;
  ulonglong2* d = reinterpret_cast<ulonglong2*>(out + it.row);
  d[0] = ulonglong2{ln.s, ln.w};
  d[1] = ulonglong2{ln.x, ln.nf};
}

// Row of each split tensor from its items' partial rows: sums of S and of the
// already position-offset W (the concatenation identity in additive form),
// xor of X, sum of NF.  A tensor with no items gets the zero row.  One wave
// per split tensor (entry 4*block + wave).
__global__ void __launch_bounds__(kBlock) merge_rows_kernel(const PlanSplit* __restrict__ split,
                                                            uint32_t n_split,
                                                            const sdc_row* __restrict__ partials,
                                                            sdc_row* __restrict__ out) {
  const uint32_t e = wave_item_index();
  if (e >= n_split) return;
  const PlanSplit sp = split[e];
  const uint32_t l = threadIdx.x & 63u;
  Lane ln;
  for (uint32_t i = l; i < sp.count; i += 64u) {
    const ulonglong2* p = reinterpret_cast<const ulonglong2*>(partials + sp.first + i);
    const ulonglong2 a = p[0], b = p[1];
    ln.s += a.x;
    ln.w += a.y;
    ln.x ^= b.x;
    ln.nf += b.y;
  }
  wave_reduce(ln);
  if (l != 0) return;
  ulonglong2* d = reinterpret_cast<ulonglong2*>(out + sp.row);
  d[0] = ulonglong2{ln.s, ln.w};
  d[1] = ulonglong2{ln.x, ln.nf};
}

// ---- NaN/Inf count only ----------------------------------------------------------
template <class Ty>
__device__ __forceinline__ uint32_t nonfinite_item(const PlanItem& it) {
  constexpr uint32_t es = Ty::ES;
  constexpr uint32_t kRound = kBlock * kUnroll;
  const uint32_t t = threadIdx.x;
  uint32_t c = 0;
  if constexpr (Ty::CHK != kChkNone) {  // raw integers are never NaN/Inf: nothing to read
    const Span sp = span_of<es>(it);
    const NfRule rule = nf_rule(it.dtype_flags & kItemDtypeMask);
    if (t < sp.h) c += nf_exact(load_elem<es>(sp.base + (uint64_t)t * es), rule);
    if (t >= 128u && t - 128u < sp.ntail)
      c += nf_exact(load_elem<es>(sp.base + (uint64_t)(sp.tail0 + t - 128u) * es), rule);
    if (sp.nvec) {
      const unsigned char* body = sp.base + (uint64_t)sp.h * es;
      Chk<Ty::CHK> chk(rule);
      for (uint32_t v0 = 0; v0 < sp.nvec; v0 += kRound) {
        const uint32_t left = min(sp.nvec - v0, kRound);
        __amdgpu_buffer_rsrc_t rs = make_rsrc(body + (uint64_t)v0 * kVecBytes, left * kVecBytes);
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const uint32_t vi = u * kBlock + t;
          v[u] = (vi < left) ? load16(rs, vi * kVecBytes) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) chk.add(v[u]);
      }
      if (chk.flagged()) {
        for (uint32_t vi = t; vi < sp.nvec; vi += kBlock) {
          __amdgpu_buffer_rsrc_t rs = make_rsrc(body + (uint64_t)vi * kVecBytes, kVecBytes);
          c += nf_vec<es>(load16(rs, 0), rule);
        }
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  __shared__ uint32_t lc[kWaves];
  if ((t & 63) == 0) lc[t >> 6] = c;
  __syncthreads();
  if (t == 0) {
    for (int i = 1; i < kWaves; ++i) c += lc[i];
  }
  return c;
}

// Signedness does not change the NaN/Inf count; it is dropped here.
template <class Ty>
struct Unsigned {
  typedef TypeTag<Ty::ES, false, Ty::CHK> type;
};

__global__ void __launch_bounds__(kBlock) nonfinite_kernel(const PlanItem* __restrict__ items,
                                                           sdc_row* __restrict__ partials,
                                                           uint64_t* __restrict__ counts,
                                                           uint64_t* __restrict__ total) {
  const PlanItem it = items[blockIdx.x];
  uint32_t c = 0;
  dispatch_type(it.dtype_flags & ~kItemSigned,
                [&](auto ty) { c = nonfinite_item<typename Unsigned<decltype(ty)>::type>(it); });
  if (threadIdx.x != 0) return;
  if (counts) {
    if (it.dtype_flags & kItemWhole) counts[it.row] = c;
    else partials[it.slot].nonfinite = c;
  }
  // NaN/Inf are rare, so the total's atomics are too.
  if (c) atomicAdd(reinterpret_cast<unsigned long long*>(total), (unsigned long long)c);
}

template <class Ty>
__device__ __forceinline__ uint32_t nonfinite_small(const PlanItem& it, uint32_t l) {
  constexpr uint32_t es = Ty::ES;
  uint32_t c = 0;
  if constexpr (Ty::CHK != kChkNone) {
    const Span sp = span_of<es>(it);
    const NfRule rule = nf_rule(it.dtype_flags & kItemDtypeMask);
    if (l < sp.h) c += nf_exact(load_elem<es>(sp.base + (uint64_t)l * es), rule);
    if (l >= 32u && l - 32u < sp.ntail)
      c += nf_exact(load_elem<es>(sp.base + (uint64_t)(sp.tail0 + l - 32u) * es), rule);
    if (sp.nvec) {
      __amdgpu_buffer_rsrc_t rs = make_rsrc(sp.base + (uint64_t)sp.h * es, sp.nvec * kVecBytes);
#pragma unroll
      for (uint32_t u = 0; u < kWaveVecs; ++u) {
        const uint32_t vi = u * 64u + l;
        if (vi < sp.nvec) c += nf_vec<es>(load16(rs, vi * kVecBytes), rule);
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  return c;
}

__global__ void __launch_bounds__(kBlock) nonfinite_small_kernel(const PlanItem* __restrict__ items,
                                                                 uint32_t n,
                                                                 uint64_t* __restrict__ counts,
                                                                 uint64_t* __restrict__ total) {
  const uint32_t i = wave_item_index();
  if (i >= n) return;
  const PlanItem it = items[i];
  const uint32_t l = threadIdx.x & 63u;
  uint32_t c = 0;
  dispatch_type(it.dtype_flags & ~kItemSigned,
                [&](auto ty) { c = nonfinite_small<typename Unsigned<decltype(ty)>::type>(it, l); });
  if (l != 0) return;
  if (counts) counts[it.row] = c;
  if (c) atomicAdd(reinterpret_cast<unsigned long long*>(total), (unsigned long long)c);
}

__global__ void __launch_bounds__(kBlock) merge_counts_kernel(const PlanSplit* __restrict__ split,
                                                              uint32_t n_split,
                                                              const sdc_row* __restrict__ partials,
                                                              uint64_t* __restrict__ counts) {
  const uint32_t e = wave_item_index();
  if (e >= n_split) return;
  const PlanSplit sp = split[e];
  const uint32_t l = threadIdx.x & 63u;
  uint64_t c = 0;
  for (uint32_t i = l; i < sp.count; i += 64u) c += partials[sp.first + i].nonfinite;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  if (l == 0) counts[sp.row] = c;
}

__global__ void clear_total_kernel(uint64_t* total) { *total = 0; }

// ---- squared norm (the norm-based check) --------------------------------------------
// Element values decoded exactly (every format here converts to double without
// rounding), squared and summed in double in a fixed order: per lane in index
// order, then fixed shuffle / LDS trees, partial slots in slot order, and one
// workgroup for the total -- so a plan gives the same bits on every run.
template <uint32_t DT>
struct DtTag {
  static constexpr uint32_t DTYPE = DT;
};

template <class F>
__device__ __forceinline__ void dispatch_dtype(uint32_t df, F&& f) {
  switch (df & kItemDtypeMask) {
    case SDC_F32: f(DtTag<SDC_F32>()); break;
    case SDC_BF16: f(DtTag<SDC_BF16>()); break;
    case SDC_F16: f(DtTag<SDC_F16>()); break;
    case SDC_F64: f(DtTag<SDC_F64>()); break;
    case SDC_FP8_E4M3: f(DtTag<SDC_FP8_E4M3>()); break;
    case SDC_FP8_E5M2: f(DtTag<SDC_FP8_E5M2>()); break;
    case SDC_FP8_E4M3FNUZ: f(DtTag<SDC_FP8_E4M3FNUZ>()); break;
    case SDC_FP8_E5M2FNUZ: f(DtTag<SDC_FP8_E5M2FNUZ>()); break;
    default: break;  // raw integers carry no floating-point value: contribute 0
  }
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
}

// fp8 with a 4-bit exponent (bias B, 3 mantissa bits): normal numbers map to
// fp32 bits directly, subnormals are m * 2^(-(B+2)).
template <int B>
__device__ __forceinline__ float e4m3_to_float(uint32_t x) {
  const uint32_t e = (x >> 3) & 15u, m = x & 7u;
  const float mag = e ? __uint_as_float(((e + 127u - B) << 23) | (m << 20)) : (float)m * __uint_as_float((uint32_t)(127 - B - 2) << 23);
  return (x & 0x80u) ? -mag : mag;
}

template <uint32_t DT>
__device__ __forceinline__ double value_of(uint64_t x) {
  if constexpr (DT == SDC_F32) return (double)__uint_as_float((uint32_t)x);
  if constexpr (DT == SDC_BF16) return (double)__uint_as_float((uint32_t)x << 16);
  if constexpr (DT == SDC_F16) return (double)half_bits_to_float((uint32_t)x);
  if constexpr (DT == SDC_F64) return __longlong_as_double((long long)x);
  if constexpr (DT == SDC_FP8_E5M2) return (double)half_bits_to_float((uint32_t)x << 8);
  if constexpr (DT == SDC_FP8_E4M3) {
    if ((x & 0x7Fu) == 0x7Fu) return __longlong_as_double(0x7FF8000000000000ll);
    return (double)e4m3_to_float<7>((uint32_t)x);
  }
  if constexpr (DT == SDC_FP8_E4M3FNUZ) {
    if (x == 0x80u) return __longlong_as_double(0x7FF8000000000000ll);
    return (double)e4m3_to_float<8>((uint32_t)x);
  }
  if constexpr (DT == SDC_FP8_E5M2FNUZ) {
    if (x == 0x80u) return __longlong_as_double(0x7FF8000000000000ll);
    const uint32_t e = (x >> 2) & 31u, m = x & 3u;
    const float mag = e ? __uint_as_float(((e + 111u) << 23) | (m << 21)) : (float)m * 0x1p-17f;
    return (double)((x & 0x80u) ? -mag : mag);
  }
  return 0.0;
}

template <uint32_t DT>
constexpr uint32_t dt_size() {
  return DT == SDC_F32 ? 4u : (DT == SDC_BF16 || DT == SDC_F16) ? 2u : DT == SDC_F64 ? 8u : 1u;
}

// acc += value^2 over the elements of one vector, in index order.
template <uint32_t DT>
__device__ __forceinline__ double sq_vec(u32x4 v, double acc) {
  constexpr uint32_t es = dt_size<DT>();
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
  if constexpr (es == 8) {
    const double a = value_of<DT>(lohi(d[0], d[1])), b = value_of<DT>(lohi(d[2], d[3]));
    acc = __builtin_fma(a, a, acc);
    acc = __builtin_fma(b, b, acc);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (uint32_t sh = 0; sh < 32; sh += 8 * es) {
        const double y = value_of<DT>((d[i] >> sh) & ((1ull << (8 * es)) - 1));
        acc = __builtin_fma(y, y, acc);
      }
    }
  }
  return acc;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ double block_sum_d(double v) {
  v = wave_sum_d(v);
  __shared__ double lw[kWaves];
  if ((threadIdx.x & 63) == 0) lw[threadIdx.x >> 6] = v;
  __syncthreads();
  double all = lw[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) all += lw[i];
  return all;
}

template <class Dt>
__device__ __forceinline__ double sq_item(const PlanItem& it) {
  constexpr uint32_t DT = Dt::DTYPE, es = dt_size<DT>();
  constexpr uint32_t kRound = kBlock * kUnroll;
  const Span sp = span_of<es>(it);
  const uint32_t t = threadIdx.x;
  double acc = 0.0;
  if (t < sp.h) {
    const double y = value_of<DT>(load_elem<es>(sp.base + (uint64_t)t * es));
    acc = y * y;
  }
  if (t >= 128u && t - 128u < sp.ntail) {
    const double y = value_of<DT>(load_elem<es>(sp.base + (uint64_t)(sp.tail0 + t - 128u) * es));
    acc = __builtin_fma(y, y, acc);
  }
  const unsigned char* body = sp.base + (uint64_t)sp.h * es;
  for (uint32_t v0 = 0; v0 < sp.nvec; v0 += kRound) {
    const uint32_t left = min(sp.nvec - v0, kRound);
    __amdgpu_buffer_rsrc_t rs = make_rsrc(body + (uint64_t)v0 * kVecBytes, left * kVecBytes);
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t vi = u * kBlock + t;
      v[u] = (vi < left) ? load16(rs, vi * kVecBytes) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc = sq_vec<DT>(v[u], acc);
  }
  return acc;
}

__global__ void __launch_bounds__(kBlock) sqnorm_kernel(const PlanItem* __restrict__ items,
                                                        sdc_row* __restrict__ partials,
                                                        double* __restrict__ sq) {
  const PlanItem it = items[blockIdx.x];
  double acc = 0.0;
  dispatch_dtype(it.dtype_flags, [&](auto dt) { acc = sq_item<decltype(dt)>(it); });
  acc = block_sum_d(acc);
  if (threadIdx.x != 0) return;
  if (it.dtype_flags & kItemWhole) sq[it.row] = acc;
  else partials[it.slot].sum = (uint64_t)__double_as_longlong(acc);
}

template <class Dt>
__device__ __forceinline__ double sq_small(const PlanItem& it, uint32_t l) {
  constexpr uint32_t DT = Dt::DTYPE, es = dt_size<DT>();
  const Span sp = span_of<es>(it);
  double acc = 0.0;
  if (l < sp.h) {
    const double y = value_of<DT>(load_elem<es>(sp.base + (uint64_t)l * es));
    acc = y * y;
  }
  if (l >= 32u && l - 32u < sp.ntail) {
    const double y = value_of<DT>(load_elem<es>(sp.base + (uint64_t)(sp.tail0 + l - 32u) * es));
    acc = __builtin_fma(y, y, acc);
  }
  if (sp.nvec) {
    __amdgpu_buffer_rsrc_t rs = make_rsrc(sp.base + (uint64_t)sp.h * es, sp.nvec * kVecBytes);
#pragma unroll
    for (uint32_t u = 0; u < kWaveVecs; ++u) {
      const uint32_t vi = u * 64u + l;
      if (vi < sp.nvec) acc = sq_vec<DT>(load16(rs, vi * kVecBytes), acc);
    }
  }
  return acc;
}

__global__ void __launch_bounds__(kBlock) sqnorm_small_kernel(const PlanItem* __restrict__ items,
                                                              uint32_t n, double* __restrict__ sq) {
  const uint32_t i = wave_item_index();
  if (i >= n) return;
  const PlanItem it = items[i];
  const uint32_t l = threadIdx.x & 63u;
  double acc = 0.0;
  dispatch_dtype(it.dtype_flags, [&](auto dt) { acc = sq_small<decltype(dt)>(it, l); });
  acc = wave_sum_d(acc);
  if (l == 0) sq[it.row] = acc;
}

__global__ void __launch_bounds__(kBlock) merge_sq_kernel(const PlanSplit* __restrict__ split,
                                                          uint32_t n_split,
                                                          const sdc_row* __restrict__ partials,
                                                          double* __restrict__ sq) {
  const uint32_t e = wave_item_index();
  if (e >= n_split) return;
  const PlanSplit sp = split[e];
  const uint32_t l = threadIdx.x & 63u;
  double acc = 0.0;
  for (uint32_t i = l; i < sp.count; i += 64u)
    acc += __longlong_as_double((long long)partials[sp.first + i].sum);
  acc = wave_sum_d(acc);
  if (l == 0) sq[sp.row] = acc;
}

// Total over all tensors in a fixed order, and the decision: the squared sum
// rounded to fp32 is not finite.
__global__ void __launch_bounds__(kBlock) sq_total_kernel(const double* __restrict__ sq, uint64_t n,
                                                          double* __restrict__ total,
                                                          uint32_t* __restrict__ flag) {
  double acc = 0.0;
  for (uint64_t k = threadIdx.x; k < n; k += kBlock) acc += sq[k];
  acc = block_sum_d(acc);
  if (threadIdx.x == 0) {
    *total = acc;
    if (flag) *flag = !__builtin_isfinite((float)acc);
  }
}

// ---- host side: plan layout --------------------------------------------------
struct Layout {
  uint64_t n_items = 0, n_small = 0, n_split = 0, n_slots = 0, total_elems = 0, total_bytes = 0;
  uint64_t item_bytes = 0;
  PlanOffsets off{};
};

uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// Items of one tensor: [0, min(n, h + IE)), then IE elements at a time, where
// h is the misaligned head and IE = item_bytes / es.  Calls f(start, len).
template <typename F>
void split_tensor(uint64_t ptr, uint64_t numel, uint32_t es, uint64_t item_bytes, F&& f) {
  const uint64_t mis = ptr & 15u;
  const uint64_t h = mis ? std::min<uint64_t>(numel, (16u - mis) / es) : 0u;
  const uint64_t ie = item_bytes / es;
  uint64_t end = std::min<uint64_t>(numel, h + ie);
  f(0, end);
  for (uint64_t s = end; s < numel; s += ie) f(s, std::min<uint64_t>(numel - s, ie));
}

uint64_t items_of(uint64_t ptr, uint64_t numel, uint32_t es, uint64_t item_bytes) {
  const uint64_t mis = ptr & 15u;
  const uint64_t h = mis ? std::min<uint64_t>(numel, (16u - mis) / es) : 0u;
  const uint64_t ie = item_bytes / es;
  const uint64_t first = std::min<uint64_t>(numel, h + ie);
  return 1 + (numel - first + ie - 1) / ie;
}

bool has_data(const sdc_tensor& t) { return t.ptr != nullptr && t.numel != 0; }

// A tensor scanned whole by one wave: it is a single item anyway and its
// aligned body has at most 64 x kWaveVecs vectors.
bool is_wave_item(uint64_t ptr, uint64_t numel, uint32_t es, uint64_t item_bytes) {
  if (items_of(ptr, numel, es, item_bytes) != 1) return false;
  const uint64_t mis = ptr & 15u;
  const uint64_t h = mis ? std::min<uint64_t>(numel, (16u - mis) / es) : 0u;
  return (numel - h) * es / kVecBytes <= kWaveBodyVecs;
}

int32_t layout_plan(const sdc_tensor* t, uint64_t n, uint64_t item_bytes, Layout* L) {
  if (n > 0 && t == nullptr) return SDC_ERR_INVALID;
  if (n >= (1ull << 31)) return SDC_ERR_RANGE;
  if (item_bytes % kVecBytes != 0 || item_bytes > kItemBytesMax) return SDC_ERR_INVALID;
  uint64_t elems = 0, bytes = 0;
  for (uint64_t k = 0; k < n; ++k) {
    if ((t[k].flags & ~(uint32_t)SDC_FLAG_SIGNED) != 0) return SDC_ERR_INVALID;
    const uint32_t es = element_size(t[k].dtype);
    if (es == 0) return SDC_ERR_DTYPE;
    if (!has_data(t[k])) continue;
    if (t[k].numel >= (1ull << 62)) return SDC_ERR_RANGE;
    if (reinterpret_cast<uintptr_t>(t[k].ptr) % es != 0) return SDC_ERR_ALIGN;
    elems += t[k].numel;
    bytes += t[k].numel * es;
  }
  if (item_bytes == 0) {
    uint64_t ib = align_up(std::max<uint64_t>(bytes / kAutoTargetItems, 1), 4096);
    item_bytes = std::min(kAutoMax, std::max(kAutoMin, ib));
  }
  uint64_t items = 0, small = 0, split = 0, slots = 0;
  for (uint64_t k = 0; k < n; ++k) {
    if (!has_data(t[k])) {
      split++;
      continue;
    }
    const uint64_t ptr = reinterpret_cast<uintptr_t>(t[k].ptr);
    const uint32_t es = element_size(t[k].dtype);
    const uint64_t c = items_of(ptr, t[k].numel, es, item_bytes);
    items += c;
    if (is_wave_item(ptr, t[k].numel, es, item_bytes)) small++;
    if (c > 1) {
      split++;
      slots += c;
    }
  }
  if (items > kMaxGrid || slots >= (1ull << 32)) return SDC_ERR_RANGE;
  L->n_items = items;
  L->n_small = small;
  L->n_split = split;
  L->n_slots = slots;
  L->total_elems = elems;
  L->total_bytes = bytes;
  L->item_bytes = item_bytes;
  L->off = plan_offsets(items, split, slots);
  return SDC_OK;
}

// Host image of the plan (the partial-row slots are left uninitialised).
// Workgroup items come first, then wave items; each group is in list order
// and in address order within a tensor.
void pack_plan(const sdc_tensor* t, uint64_t n, const Layout& L, std::vector<unsigned char>& img) {
  img.assign(L.off.partials, 0);
  PlanHeader* hd = reinterpret_cast<PlanHeader*>(img.data());
  hd->magic = kPlanMagic;
  hd->n_tensors = n;
  hd->n_items = L.n_items;
  hd->n_split = L.n_split;
  hd->n_slots = L.n_slots;
  hd->total_bytes = L.total_bytes;
  hd->item_bytes = L.item_bytes;
  hd->n_small = L.n_small;
  PlanItem* items = reinterpret_cast<PlanItem*>(img.data() + L.off.items);
  PlanSplit* split = reinterpret_cast<PlanSplit*>(img.data() + L.off.split);
  uint64_t ni = 0, nw = L.n_items - L.n_small, ns = 0, slot = 0;
  for (uint64_t k = 0; k < n; ++k) {
    if (!has_data(t[k])) {
      split[ns++] = PlanSplit{(uint32_t)k, 0u, 0u, 0u};
      continue;
    }
    const uint32_t es = element_size(t[k].dtype);
    const uint64_t ptr = reinterpret_cast<uintptr_t>(t[k].ptr);
    const uint64_t c = items_of(ptr, t[k].numel, es, L.item_bytes);
    const uint32_t whole = (c == 1) ? kItemWhole : 0u;
    const bool wave = is_wave_item(ptr, t[k].numel, es, L.item_bytes);
    if (c > 1) split[ns++] = PlanSplit{(uint32_t)k, (uint32_t)slot, (uint32_t)c, 0u};
    split_tensor(ptr, t[k].numel, es, L.item_bytes, [&](uint64_t s, uint64_t len) {
      PlanItem& it = items[wave ? nw++ : ni++];
      it.addr = ptr + s * es;
      it.start = s;
      it.len = (uint32_t)len;
      it.row = (uint32_t)k;
      it.slot = whole ? 0u : (uint32_t)slot++;
      it.dtype_flags = t[k].dtype | whole | ((t[k].flags & SDC_FLAG_SIGNED) ? kItemSigned : 0u);
    });
  }
}

bool info_ok(const sdc_plan_info* h) {
  if (h == nullptr || h->magic != kPlanMagic || h->n_items > kMaxGrid ||
      h->n_split > h->n_tensors || h->n_small > h->n_items)
    return false;
  return h->plan_bytes >= plan_offsets(h->n_items, h->n_split, h->n_slots).end;
}

struct PlanView {
  const PlanItem* items;
  const PlanSplit* split;
  sdc_row* partials;
};

PlanView view_of(const void* d_plan, const sdc_plan_info* h) {
  unsigned char* base = reinterpret_cast<unsigned char*>(const_cast<void*>(d_plan));
  const PlanOffsets o = plan_offsets(h->n_items, h->n_split, h->n_slots);
  return PlanView{reinterpret_cast<const PlanItem*>(base + o.items),
                  reinterpret_cast<const PlanSplit*>(base + o.split),
                  reinterpret_cast<sdc_row*>(base + o.partials)};
}

int32_t launch_scan(const void* d_plan, const sdc_plan_info* h, sdc_row* out, hipStream_t s) {
  const PlanView v = view_of(d_plan, h);
  const uint64_t n_block = h->n_items - h->n_small;
  int32_t st;
  if (h->n_small) {
    hipLaunchKernelGGL(fingerprint_small_kernel, dim3((uint32_t)((h->n_small + kWaves - 1) / kWaves)),
                       dim3(kBlock), 0, s, v.items + n_block, (uint32_t)h->n_small, out);
    if ((st = launch_status())) return st;
  }
  if (n_block) {
    if (h->total_bytes / h->n_items >= kDeepItemBytes)
      hipLaunchKernelGGL(fingerprint_kernel<DeepBody>, dim3((uint32_t)n_block), dim3(kBlock), 0, s,
                         v.items, v.partials, out);
    else
      hipLaunchKernelGGL(fingerprint_kernel<DefaultBody>, dim3((uint32_t)n_block), dim3(kBlock), 0,
                         s, v.items, v.partials, out);
    if ((st = launch_status())) return st;
  }
  if (h->n_split) {
    hipLaunchKernelGGL(merge_rows_kernel, dim3((uint32_t)((h->n_split + kWaves - 1) / kWaves)),
                       dim3(kBlock), 0, s, v.split, (uint32_t)h->n_split, v.partials, out);
    return launch_status();
  }
  return SDC_OK;
}

}  // namespace
}  // namespace sdc

using namespace sdc;

extern "C" int32_t sdc_plan_bytes(const sdc_tensor* h_tensors, uint64_t n, uint64_t item_bytes,
                                  uint64_t* h_bytes) {
  if (h_bytes == nullptr) return SDC_ERR_INVALID;
  Layout L;
  int32_t st = layout_plan(h_tensors, n, item_bytes, &L);
  if (st) return st;
  *h_bytes = L.off.end;
  return SDC_OK;
}

extern "C" int32_t sdc_plan_build(const sdc_tensor* h_tensors, uint64_t n, uint64_t item_bytes,
                                  void* d_plan, uint64_t plan_bytes, sdc_plan_info* h_info,
                                  sdc_stream_t stream) {
  if (d_plan == nullptr || h_info == nullptr) return SDC_ERR_INVALID;
  Layout L;
  int32_t st = layout_plan(h_tensors, n, item_bytes, &L);
  if (st) return st;
  if (plan_bytes < L.off.end) return SDC_ERR_WORKSPACE;
  std::vector<unsigned char> img;
  try {
    pack_plan(h_tensors, n, L, img);
  } catch (...) {
    return SDC_ERR_RANGE;  // host allocation failed
  }
  hipStream_t s = as_stream(stream);
  st = hip_status(hipMemcpyAsync(d_plan, img.data(), img.size(), hipMemcpyHostToDevice, s));
  if (st) return st;
  st = hip_status(hipStreamSynchronize(s));
  if (st) return st;
  h_info->magic = kPlanMagic;
  h_info->n_tensors = n;
  h_info->n_items = L.n_items;
  h_info->n_small = L.n_small;
  h_info->n_split = L.n_split;
  h_info->n_slots = L.n_slots;
  h_info->total_elems = L.total_elems;
  h_info->total_bytes = L.total_bytes;
  h_info->plan_bytes = L.off.end;
  h_info->item_bytes = L.item_bytes;
  return SDC_OK;
}

extern "C" int32_t sdc_plan_pack_host(const sdc_tensor* h_tensors, uint64_t n, uint64_t item_bytes,
                                      void* h_plan, uint64_t plan_bytes, sdc_plan_info* h_info) {
  if (h_plan == nullptr || h_info == nullptr) return SDC_ERR_INVALID;
  Layout L;
  int32_t st = layout_plan(h_tensors, n, item_bytes, &L);
  if (st) return st;
  if (plan_bytes < L.off.partials) return SDC_ERR_WORKSPACE;
  std::vector<unsigned char> img;
  try {
    pack_plan(h_tensors, n, L, img);
  } catch (...) {
    return SDC_ERR_RANGE;
  }
  std::memcpy(h_plan, img.data(), img.size());
  h_info->magic = kPlanMagic;
  h_info->n_tensors = n;
  h_info->n_items = L.n_items;
  h_info->n_small = L.n_small;
  h_info->n_split = L.n_split;
  h_info->n_slots = L.n_slots;
  h_info->total_elems = L.total_elems;
  h_info->total_bytes = L.total_bytes;
  h_info->plan_bytes = L.off.end;
  h_info->item_bytes = L.item_bytes;
  return SDC_OK;
}

extern "C" int32_t sdc_fingerprint_plan(const void* d_plan, const sdc_plan_info* h_info,
                                        sdc_row* d_out, sdc_stream_t stream) {
  if (d_plan == nullptr || h_info == nullptr) return SDC_ERR_INVALID;
  if (!info_ok(h_info)) return SDC_ERR_PLAN;
  if (h_info->n_tensors > 0 && d_out == nullptr) return SDC_ERR_INVALID;
  return launch_scan(d_plan, h_info, d_out, as_stream(stream));
}

extern "C" int32_t sdc_nonfinite(const void* d_plan, const sdc_plan_info* h_info,
                                 uint64_t* d_counts, uint64_t* d_total, sdc_stream_t stream) {
  if (d_plan == nullptr || h_info == nullptr || d_total == nullptr) return SDC_ERR_INVALID;
  if (!info_ok(h_info)) return SDC_ERR_PLAN;
  hipStream_t s = as_stream(stream);
  const PlanView v = view_of(d_plan, h_info);
  hipLaunchKernelGGL(clear_total_kernel, dim3(1), dim3(1), 0, s, d_total);
  int32_t st = launch_status();
  if (st) return st;
  const uint64_t n_block = h_info->n_items - h_info->n_small;
  if (h_info->n_small) {
    hipLaunchKernelGGL(nonfinite_small_kernel,
                       dim3((uint32_t)((h_info->n_small + kWaves - 1) / kWaves)), dim3(kBlock), 0, s,
                       v.items + n_block, (uint32_t)h_info->n_small, d_counts, d_total);
    if ((st = launch_status())) return st;
  }
  if (n_block) {
    hipLaunchKernelGGL(nonfinite_kernel, dim3((uint32_t)n_block), dim3(kBlock), 0, s, v.items,
                       v.partials, d_counts, d_total);
    if ((st = launch_status())) return st;
  }
  if (d_counts && h_info->n_split) {
    hipLaunchKernelGGL(merge_counts_kernel,
                       dim3((uint32_t)((h_info->n_split + kWaves - 1) / kWaves)), dim3(kBlock), 0, s,
                       v.split, (uint32_t)h_info->n_split, v.partials, d_counts);
    return launch_status();
  }
  return SDC_OK;
}

extern "C" int32_t sdc_fingerprint(const sdc_tensor* h_tensors, uint64_t n, void* d_ws,
                                   uint64_t ws_bytes, sdc_row* d_out, sdc_stream_t stream) {
  sdc_plan_info info;
  int32_t st = sdc_plan_build(h_tensors, n, 0, d_ws, ws_bytes, &info, stream);
  if (st) return st;
  return sdc_fingerprint_plan(d_ws, &info, d_out, stream);
}

extern "C" int32_t sdc_sqnorm(const void* d_plan, const sdc_plan_info* h_info, double* d_sq,
                              double* d_total, uint32_t* d_flag, sdc_stream_t stream) {
  if (d_plan == nullptr || h_info == nullptr || d_total == nullptr) return SDC_ERR_INVALID;
  if (!info_ok(h_info)) return SDC_ERR_PLAN;
  if (h_info->n_tensors > 0 && d_sq == nullptr) return SDC_ERR_INVALID;
  hipStream_t s = as_stream(stream);
  const PlanView v = view_of(d_plan, h_info);
  const uint64_t n_block = h_info->n_items - h_info->n_small;
  int32_t st;
  if (h_info->n_small) {
    hipLaunchKernelGGL(sqnorm_small_kernel,
                       dim3((uint32_t)((h_info->n_small + kWaves - 1) / kWaves)), dim3(kBlock), 0, s,
                       v.items + n_block, (uint32_t)h_info->n_small, d_sq);
    if ((st = launch_status())) return st;
  }
  if (n_block) {
    hipLaunchKernelGGL(sqnorm_kernel, dim3((uint32_t)n_block), dim3(kBlock), 0, s, v.items,
                       v.partials, d_sq);
    if ((st = launch_status())) return st;
  }
  if (h_info->n_split) {
    hipLaunchKernelGGL(merge_sq_kernel, dim3((uint32_t)((h_info->n_split + kWaves - 1) / kWaves)),
                       dim3(kBlock), 0, s, v.split, (uint32_t)h_info->n_split, v.partials, d_sq);
    if ((st = launch_status())) return st;
  }
  hipLaunchKernelGGL(sq_total_kernel, dim3(1), dim3(kBlock), 0, s, d_sq, h_info->n_tensors, d_total,
                     d_flag);
  return launch_status();
}
