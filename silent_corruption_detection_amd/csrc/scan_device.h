// scan_device.h -- device building blocks shared by the scan-family kernels
// (fingerprint, NaN/Inf count, squared norm): raw non-temporal buffer loads,
// the exact per-type NaN/Inf rules and their fast pre-checks, element-type
// dispatch, the pipelined body stream of workgroup items, the head / aligned
// body / tail split of a work item, and the lane groups of wave items.
#pragma once

#include <type_traits>

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
// sets it; a set flag triggers an exact count of the vectors it covers (then
// reset()), so false alarms only cost time.
enum : int { kChkNone = 0, kChkHalf = 1, kChkF32 = 2, kChkF64 = 3, kChkFp8Top = 4, kChkFp8Eq = 5 };

template <int CHK>
struct Chk;

template <>
struct Chk<kChkNone> {  // raw integers: never NaN/Inf
  __device__ __forceinline__ explicit Chk(const NfRule&) {}
  __device__ __forceinline__ void add(u32x4) {}
  __device__ __forceinline__ bool flagged() const { return false; }
  __device__ __forceinline__ void reset() {}
  __device__ __forceinline__ uint32_t exact(u32x4) const { return 0u; }
};

// bf16 / fp16: fma(x, 0, acc) on the dword read as two fp16 halves stays +0
// unless a half is fp16 NaN/Inf (exponent bits 14..10 all ones) -- which every
// fp16 and bf16 NaN/Inf is (for bf16 also finite values >= 2^121).
template <>
struct Chk<kChkHalf> {
  h2 nf = {0, 0};
  uint32_t m2, k2;  // the exponent mask in both halves; 0x8000 - mask in both halves
  __device__ __forceinline__ explicit Chk(const NfRule& r)
      : m2((uint32_t)r.mask * 0x10001u), k2((0x8000u - (uint32_t)r.mask) * 0x10001u) {}
  __device__ __forceinline__ void add(u32x4 v) {
    const h2 z = {0, 0};
    nf = __builtin_elementwise_fma(as_h2(v.x), z, nf);
    nf = __builtin_elementwise_fma(as_h2(v.y), z, nf);
    nf = __builtin_elementwise_fma(as_h2(v.z), z, nf);
    nf = __builtin_elementwise_fma(as_h2(v.w), z, nf);
  }
  __device__ __forceinline__ bool flagged() const { return h2_bits(nf) != 0; }
  __device__ __forceinline__ void reset() { nf = h2{0, 0}; }
  // Exact count: per half, (x & m) + (0x8000 - m) reaches bit 15 exactly when
  // every exponent bit is set, and never carries into the other half.
  __device__ __forceinline__ uint32_t one(uint32_t d) const {
    return (uint32_t)__builtin_popcount(((d & m2) + k2) & 0x80008000u);
  }
  __device__ __forceinline__ uint32_t exact(u32x4 v) const {
    return one(v.x) + one(v.y) + one(v.z) + one(v.w);
  }
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
  __device__ __forceinline__ void reset() { nf = 0.0f; }
  // exponent bits 30..23 all ones: adding 1 at bit 23 carries into bit 31
  __device__ __forceinline__ static uint32_t one(uint32_t d) {
    return ((d & 0x7F800000u) + 0x00800000u) >> 31;
  }
  __device__ __forceinline__ uint32_t exact(u32x4 v) const {
    return one(v.x) + one(v.y) + one(v.z) + one(v.w);
  }
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
  __device__ __forceinline__ void reset() { nf = 0.0; }
  // exponent bits 62..52 = bits 30..20 of the high word
  __device__ __forceinline__ static uint32_t one(uint32_t hi) {
    return ((hi & 0x7FF00000u) + 0x00100000u) >> 31;
  }
  __device__ __forceinline__ uint32_t exact(u32x4 v) const { return one(v.y) + one(v.w); }
};

// fp8 whose NaN/Inf are "all ones under a mask m < 0x80" (E4M3: m = 0x7F,
// E5M2: m = 0x7C): per byte, (b & m) + (0x80 - m) reaches 0x80 exactly when
// (b & m) == m, without carrying into the next byte.  Exact.
template <>
struct Chk<kChkFp8Top> {
  uint32_t flag = 0, m4, k4;
  __device__ __forceinline__ explicit Chk(const NfRule& r)
      : m4((uint32_t)r.mask * 0x01010101u), k4((0x80u - (uint32_t)r.mask) * 0x01010101u) {}
  __device__ __forceinline__ uint32_t bits(uint32_t d) const { return ((d & m4) + k4) & 0x80808080u; }
  __device__ __forceinline__ void add(u32x4 v) {
    flag |= bits(v.x);
    flag |= bits(v.y);
    flag |= bits(v.z);
    flag |= bits(v.w);
  }
  __device__ __forceinline__ bool flagged() const { return flag != 0; }
  __device__ __forceinline__ void reset() { flag = 0; }
  __device__ __forceinline__ uint32_t exact(u32x4 v) const {
    return (uint32_t)(__builtin_popcount(bits(v.x)) + __builtin_popcount(bits(v.y)) +
                      __builtin_popcount(bits(v.z)) + __builtin_popcount(bits(v.w)));
  }
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
  __device__ __forceinline__ void reset() { flag = 0; }
  // Exact count: 0x80 in every byte of d ^ v4 that is zero (no borrow between
  // bytes, unlike the any-zero test above).
  __device__ __forceinline__ uint32_t zeros(uint32_t d) const {
    const uint32_t t = d ^ v4;
    return (uint32_t)__builtin_popcount(~(((t & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | t | 0x7F7F7F7Fu));
  }
  __device__ __forceinline__ uint32_t exact(u32x4 v) const {
    return zeros(v.x) + zeros(v.y) + zeros(v.z) + zeros(v.w);
  }
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

// Slot loads per lane in flight in the merge of a split tensor's partial rows.
constexpr uint32_t kMergeUnroll = 8;

// Vectors per lane per round of the pipelined NaN/Inf-count and squared-norm
// loops: kCheckU in general, kCheckDeepU for plans whose items average at
// least kCheckDeepItemBytes (measured: 16 is 2 % faster on lists of large
// tensors and 11 % slower on lists of small ones).
constexpr int kCheckU = 8;
constexpr int kCheckDeepU = 16;
constexpr uint64_t kCheckDeepItemBytes = 96ull << 10;

// "Wide" launch shape of every scan-family kernel for plans whose items
// average at least kWideItemBytes: kWideU vectors per lane per round, not
// pipelined (a wave issues a round's loads, waits for them and consumes
// them), and one workgroup per CU.  The launch reserves kWideLdsBytes of
// dynamic LDS that no kernel touches: a CU has 160 KiB, so a second
// workgroup never fits.  HBM streams best with about 8-12 MiB of reads in
// flight over the chip, issued by as few concurrent workgroups as can keep
// that many in flight (each reads its own region): the default shapes (2-4
// workgroups per CU, pipelined rounds) lose 4-5 % to it, and so do 2-4
// workgroups per CU with the same reads in flight in shallower rounds.
// Measured on the 141 GB Llama-70B bf16 list (1 MiB items, median of 10
// scans, one box): this shape 7.46 TB/s, two workgroups per CU with pipelined
// 8-vector rounds (the shape used below the threshold) 7.13; 10 / 14 / 16
// vectors per round 7.40 / 7.39 / 7.41; pipelined rounds at one workgroup per
// CU 7.29; 6 vectors at two workgroups per CU 7.12.  With 128 KiB items one
// workgroup per CU loses 25 % (each item's start-up latency is then
// exposed), hence the threshold.
constexpr int kWideU = 12;
constexpr uint64_t kWideItemBytes = 512ull << 10;
constexpr uint32_t kWideLdsBytes = 96u << 10;

// Launch shape of a plan's workgroup items from their average size.
enum ItemShape : int { kShapeShort = 0, kShapeDeep = 1, kShapeWide = 2 };
inline int item_shape(uint64_t total_bytes, uint64_t n_items, uint64_t deep_bytes) {
  const uint64_t avg = n_items ? total_bytes / n_items : 0;
  return avg >= kWideItemBytes ? kShapeWide : (avg >= deep_bytes ? kShapeDeep : kShapeShort);
}

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

struct NoRoundHook {
  template <int U>
  __device__ __forceinline__ void operator()(const u32x4 (&)[U]) const {}
};

// Streams the nvec aligned 16-byte vectors at `body` through consume(v):
// round r holds vectors r*256*U .. r*256*U + 256*U - 1, lane t taking
// vectors u*256 + t of each round.  Lanes past the end consume zero vectors.
// After a round is consumed, done(v) sees the lane's U vectors of that round
// while they are still in registers.  With PIPE the loads of round r+1 are
// issued before round r is consumed (two register sets, alternating), so a
// wave keeps loads in flight while it computes.  Requires nvec > 0.  Returns
// the number of rounds (uniform over the workgroup).
template <int U, bool PIPE, class F, class G = NoRoundHook>
__device__ __forceinline__ uint32_t stream_body(const unsigned char* body, uint32_t nvec, F&& consume,
                                                G&& done = G()) {
  constexpr uint32_t kRound = kBlock * U;
  const uint32_t full = nvec / kRound;
  const uint32_t rounds = full + ((nvec % kRound) ? 1u : 0u);
  if constexpr (!PIPE) {
    for (uint32_t r = 0; r < rounds; ++r) {
      u32x4 v[U];
      load_round<U>(body, nvec, full, r, v);
#pragma unroll
      for (int u = 0; u < U; ++u) consume(v[u]);
      done(v);
    }
  } else {
    u32x4 va[U], vb[U];
    load_round<U>(body, nvec, full, 0, va);
    uint32_t r = 0;
    for (;;) {
      if (r + 1 < rounds) load_round<U>(body, nvec, full, r + 1, vb);
#pragma unroll
      for (int u = 0; u < U; ++u) consume(va[u]);
      done(va);
      if (++r == rounds) break;
      if (r + 1 < rounds) load_round<U>(body, nvec, full, r + 1, va);
#pragma unroll
      for (int u = 0; u < U; ++u) consume(vb[u]);
      done(vb);
      if (++r == rounds) break;
    }
  }
  return rounds;
}

// Exact NaN/Inf count (chk.exact) of a round's vectors when the lane's fast flag is set
// (rare), then the flag is cleared for the next round.  The vectors are the
// ones just loaded, so nothing is read again.
template <int U, class C>
__device__ __forceinline__ void count_flagged_round(C& chk, const u32x4 (&v)[U], uint32_t& count) {
  if (chk.flagged()) {
#pragma unroll
    for (int u = 0; u < U; ++u) count += chk.exact(v[u]);
    chk.reset();
  }
}

// Per-lane loads go through global-address-space pointers (every pointer
// here is device memory): global loads wait on the vector-memory counter
// alone, where flat loads of a generic pointer also hold the scalar one.
#define SDC_GLOBAL __attribute__((address_space(1)))

// Raw pattern of the ES-byte element at p.
template <uint32_t ES>
__device__ __forceinline__ uint64_t load_elem(const unsigned char* p) {
  if constexpr (ES == 1) return *(const SDC_GLOBAL unsigned char*)p;
  if constexpr (ES == 2) return *(const SDC_GLOBAL unsigned short*)p;
  if constexpr (ES == 4) return *(const SDC_GLOBAL uint32_t*)p;
  return *(const SDC_GLOBAL uint64_t*)p;
}

// Item of workgroup b among the n workgroup items of a launch on a device
// with `xcds` XCDs.  Workgroups go to the XCDs round-robin (b to XCD
// b % xcds); within each window of xcds * kXcdRun items, XCD k takes the
// kXcdRun adjacent items k*kXcdRun .. (k+1)*kXcdRun - 1, so each XCD reads
// runs of neighbouring items while all XCDs advance through the list
// together.  Items past the last whole window keep their order, and with one
// XCD the map is the identity.  A bijection on [0, n).  Measured on the full
// MI355X (8 XCDs) against items in workgroup order on plan scans: lists of
// 128 KiB items 1.1-1.9 % faster, lists of small tensors 1 %, 1 MiB items
// unchanged; giving each XCD one contiguous eighth of the list instead is
// 2-3 % faster on the first and 5-7 % slower on a 141 GB list of 1 MiB
// items.  (The single-tensor scan keeps workgroup order: its 512 KiB items
// measured 5 % slower with this mapping.)
constexpr uint32_t kXcdRun = 16;

__device__ __forceinline__ uint32_t xcd_item(uint32_t b, uint32_t n, uint32_t xcds) {
  const uint32_t win = xcds * kXcdRun;
  if (xcds <= 1u || b >= n / win * win) return b;
  const uint32_t o = b % win;
  return (b - o) + (o % xcds) * kXcdRun + o / xcds;
}

// Index of the calling wave over the grid (4*block + wave), wave-uniform.
__device__ __forceinline__ uint32_t wave_item_index() {
  return __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6));
}

// The launch of a plan's wave items.  Class c's items (1 << c per wave,
// 4 << c per workgroup) take workgroups [group[c], group[c+1]); their indices
// among the wave items start at first[c].
struct WaveLaunch {
  uint32_t first[kWaveClasses], count[kWaveClasses], group[kWaveClasses + 1];
};

inline WaveLaunch wave_launch(const uint64_t* n_wave) {
  WaveLaunch w;
  uint64_t first = 0, group = 0;
  for (uint32_t c = 0; c < kWaveClasses; ++c) {
    w.first[c] = (uint32_t)first;
    w.count[c] = (uint32_t)n_wave[c];
    w.group[c] = (uint32_t)group;
    first += n_wave[c];
    group += (n_wave[c] + (kWaves << c) - 1) / (kWaves << c);
  }
  w.group[kWaveClasses] = (uint32_t)group;
  return w;
}

template <uint32_t C, class F>
__device__ __forceinline__ void run_wave_class(const WaveLaunch& w, F& f) {
  constexpr uint32_t kLanes = class_lanes(C);
  uint32_t j = ((blockIdx.x - w.group[C]) * kWaves + (threadIdx.x >> 6)) * (1u << C) +
               ((threadIdx.x & 63u) / kLanes);
  // one item per wave: the index is wave-uniform, so its descriptor can come
  // through scalar loads and the item's base address through scalar registers
  if constexpr (kLanes == 64) j = __builtin_amdgcn_readfirstlane(j);
  if (j < w.count[C])
    f(w.first[C] + j, threadIdx.x & (kLanes - 1u), std::integral_constant<uint32_t, kLanes>());
}

// Calls f(item, lane, lanes) for the calling lane's wave item, lanes (the
// group width) as a compile-time constant; lanes without an item do nothing.
// The class is uniform over a workgroup.  No workgroup barrier may follow.
template <class F>
__device__ __forceinline__ void for_wave_item(const WaveLaunch& w, F&& f) {
  if (blockIdx.x < w.group[1]) run_wave_class<0>(w, f);
  else if (blockIdx.x < w.group[2]) run_wave_class<1>(w, f);
  else if (blockIdx.x < w.group[3]) run_wave_class<2>(w, f);
  else run_wave_class<3>(w, f);
}

// Non-temporal 16-byte load through a per-lane address (the two halves of a
// wave read different tensors, so their base addresses are not uniform).
__device__ __forceinline__ u32x4 load16_nt(const unsigned char* p) {
  return __builtin_nontemporal_load((const SDC_GLOBAL u32x4*)p);
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

// Sixteen zero bytes in device memory, read by wave-item lanes that have
// nothing of their item to load at a place.
static __device__ __align__(16) u32x4 g_zero16;

// Every load of a wave-item lane, issued before any value is used and with
// no branch, so an item costs one memory latency after its descriptor: the
// lane's elements of the head and of the tail (each has fewer than E = 16/ES
// elements: element k*LANES + l of each, for k < kHT) and its kWaveVecs body
// vectors (vector LANES*u + l).  Where the lane has nothing to read it loads
// the zero vector instead, which adds nothing to a fingerprint, a NaN/Inf
// count or a squared norm.  Patterns of up to 4 bytes stay 32-bit: a
// widening right after a load would make the wave wait for it there.
template <uint32_t ES, uint32_t LANES>
struct WaveItemLoads {
  static constexpr uint32_t kHT = (kVecBytes / ES - 1u + LANES - 1u) / LANES;
  typedef std::conditional_t<(ES == 8), uint64_t, uint32_t> raw_t;
  raw_t head[kHT], tail[kHT];
  u32x4 v[kWaveVecs];
  __device__ __forceinline__ WaveItemLoads(const Span& sp, uint32_t l) {
    const unsigned char* zero = reinterpret_cast<const unsigned char*>(&g_zero16);
#pragma unroll
    for (uint32_t k = 0; k < kHT; ++k) {
      const uint32_t j = k * LANES + l;
      head[k] = (raw_t)load_elem<ES>(j < sp.h ? sp.base + (uint64_t)j * ES : zero);
      tail[k] = (raw_t)load_elem<ES>(j < sp.ntail ? sp.base + (uint64_t)(sp.tail0 + j) * ES : zero);
    }
    const unsigned char* body = sp.base + (uint64_t)sp.h * ES;
#pragma unroll
    for (uint32_t u = 0; u < kWaveVecs; ++u) {
      const uint32_t vi = u * LANES + l;
      v[u] = load16_nt(vi < sp.nvec ? body + (uint64_t)vi * kVecBytes : zero);
    }
  }
};

// The head element t and the tail element t - 128 of a workgroup item's
// thread t (heads and tails have fewer than 16 elements), loaded with no
// branch before the item's body loads are issued and used after them, so an
// item's start costs one memory latency instead of three: a thread with no
// such element loads the zero vector, which adds nothing.
template <uint32_t ES>
struct ItemEnds {
  typedef std::conditional_t<(ES == 8), uint64_t, uint32_t> raw_t;
  raw_t head, tail;
  __device__ __forceinline__ ItemEnds(const Span& sp, uint32_t t) {
    const unsigned char* zero = reinterpret_cast<const unsigned char*>(&g_zero16);
    const uint32_t k = t - 128u;  // wraps for t < 128: no tail element there
    head = (raw_t)load_elem<ES>(t < sp.h ? sp.base + (uint64_t)t * ES : zero);
    tail = (raw_t)load_elem<ES>(k < sp.ntail ? sp.base + (uint64_t)(sp.tail0 + k) * ES : zero);
  }
  // index in the item of the tail element (any value where tail is zero)
  __device__ __forceinline__ static uint32_t tail_index(const Span& sp, uint32_t t) {
    return sp.tail0 + (t - 128u);
  }
};

}  // namespace
}  // namespace sdc
