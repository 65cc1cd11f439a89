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
typedef BodyCfg<4, true> DefaultBody;  // ~106 VGPRs: 4 workgroups per CU
typedef BodyCfg<8, true> DeepBody;     // ~188 VGPRs: deeper pipeline, 2 workgroups per CU
// Plans whose items average at least this many bytes use DeepBody (measured:
// better for items of ~170 KiB and more, worse for lists of small tensors).
constexpr uint64_t kDeepItemBytes = 96ull << 10;
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
  const uint32_t rounds = stream_body<U, Cfg::PIPE>(body, nvec, [&](u32x4 v) { acc.add(v); });
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

// One wave combines `count` partial rows at p (+, +, ^, +), lane l taking
// rows l, l + 64, ...; kMergeUnroll independent row loads per lane are in
// flight, so a tensor split into thousands of items is merged in a few
// memory latencies.  The wave's lanes still have to be reduced.
__device__ __forceinline__ Lane merge_slots(const sdc_row* __restrict__ rows, uint32_t count,
                                            uint32_t l) {
  Lane ln;
  const ulonglong2* p = reinterpret_cast<const ulonglong2*>(rows);
  for (uint32_t i0 = 0; i0 < count; i0 += 64u * kMergeUnroll) {
    ulonglong2 a[kMergeUnroll], b[kMergeUnroll];
#pragma unroll
    for (uint32_t u = 0; u < kMergeUnroll; ++u) {
      const uint32_t i = i0 + u * 64u + l;
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
  Lane ln = merge_slots(partials + sp.first, sp.count, l);
  wave_reduce(ln);
  if (l != 0) return;
  ulonglong2* d = reinterpret_cast<ulonglong2*>(out + sp.row);
  d[0] = ulonglong2{ln.s, ln.w};
  d[1] = ulonglong2{ln.x, ln.nf};
}

// ---- one tensor, no plan ---------------------------------------------------------
// The items of a single tensor follow from the workgroup index alone (the same
// split a plan makes): item 0 covers the misaligned head and the next ie
// elements, item i >= 1 the elements [h + i*ie, h + (i+1)*ie).  So the scan
// needs no plan upload and no host synchronisation.  Every item stores its
// partial row in slot i of the caller's workspace; one wave merges them.
struct TensorJob {
  uint64_t addr, numel, ie;  // base address, elements, elements per item
  uint32_t h, df;            // misaligned head elements; dtype | kItemSigned
  uint32_t es, pad;
};

__device__ __forceinline__ PlanItem job_item(const TensorJob& j, uint32_t i) {
  const uint64_t start = i ? j.h + (uint64_t)i * j.ie : 0u;
  const uint64_t end = min(j.numel, (uint64_t)j.h + (uint64_t)(i + 1) * j.ie);
  PlanItem it;
  it.addr = j.addr + start * j.es;
  it.start = start;
  it.len = (uint32_t)(end - start);
  it.row = 0;
  it.slot = i;
  it.dtype_flags = j.df;
  return it;
}

template <class Cfg>
__global__ void __launch_bounds__(kBlock) fingerprint_tensor_kernel(TensorJob j,
                                                                    sdc_row* __restrict__ partials) {
  const PlanItem it = job_item(j, blockIdx.x);
  Lane ln;
  dispatch_type(it.dtype_flags, [&](auto ty) { scan_item<decltype(ty), Cfg>(it, ln); });
  if (threadIdx.x != 0) return;
  ulonglong2* d = reinterpret_cast<ulonglong2*>(partials + blockIdx.x);
  d[0] = ulonglong2{ln.s, ln.w + it.start * ln.s};
  d[1] = ulonglong2{ln.x, ln.nf};
}

__device__ __forceinline__ bool rows_differ(const sdc_row& a, const sdc_row& b, uint32_t mask) {
  return ((mask & SDC_COL_SUM) && a.sum != b.sum) || ((mask & SDC_COL_WSUM) && a.wsum != b.wsum) ||
         ((mask & SDC_COL_XOR) && a.xorsum != b.xorsum) ||
         ((mask & SDC_COL_NONFINITE) && a.nonfinite != b.nonfinite);
}

// One wave: the tensor's row from its n partial rows; with a reference row,
// a difference under the mask adds 1 to *mismatch.
__global__ void __launch_bounds__(64) merge_check_kernel(const sdc_row* __restrict__ partials,
                                                         uint32_t n, sdc_row* __restrict__ out,
                                                         const sdc_row* __restrict__ ref,
                                                         uint32_t mask, uint32_t* __restrict__ mismatch) {
  const uint32_t l = threadIdx.x;
  Lane ln = merge_slots(partials, n, l);
  wave_reduce(ln);
  if (l != 0) return;
  const sdc_row r{ln.s, ln.w, ln.x, ln.nf};
  ulonglong2* d = reinterpret_cast<ulonglong2*>(out);
  d[0] = ulonglong2{r.sum, r.wsum};
  d[1] = ulonglong2{r.xorsum, r.nonfinite};
  if (ref && rows_differ(r, *ref, mask)) atomicAdd(mismatch, 1u);
}

// Launch shape of the single-tensor scan: items and the split of item 0.
struct TensorShape {
  uint64_t n_items, ie;
  uint32_t h, es;
};

int32_t tensor_shape(const sdc_tensor* t, uint64_t item_bytes, TensorShape* sh) {
  if (t == nullptr) return SDC_ERR_INVALID;
  if (item_bytes % kVecBytes != 0 || item_bytes > kItemBytesMax) return SDC_ERR_INVALID;
  if ((t->flags & ~(uint32_t)SDC_FLAG_SIGNED) != 0) return SDC_ERR_INVALID;
  const uint32_t es = element_size(t->dtype);
  if (es == 0) return SDC_ERR_DTYPE;
  if (t->numel >= (1ull << 62)) return SDC_ERR_RANGE;
  const uint64_t numel = t->ptr ? t->numel : 0u;
  const uint64_t ptr = reinterpret_cast<uintptr_t>(t->ptr);
  if (ptr % es != 0) return SDC_ERR_ALIGN;
  const uint64_t ie = (item_bytes ? item_bytes : tensor_item_bytes(numel * es)) / es;
  const uint64_t mis = ptr & 15u;
  const uint64_t h = mis ? std::min<uint64_t>(numel, (16u - mis) / es) : 0u;
  const uint64_t first = std::min<uint64_t>(numel, h + ie);
  sh->n_items = numel ? 1 + (numel - first + ie - 1) / ie : 0;
  if (sh->n_items > kMaxGrid) return SDC_ERR_RANGE;
  sh->ie = ie;
  sh->h = (uint32_t)h;
  sh->es = es;
  return SDC_OK;
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

extern "C" int32_t sdc_fingerprint_plan(const void* d_plan, const sdc_plan_info* h_info,
                                        sdc_row* d_out, sdc_stream_t stream) {
  if (d_plan == nullptr || h_info == nullptr) return SDC_ERR_INVALID;
  if (!info_ok(h_info)) return SDC_ERR_PLAN;
  if (h_info->n_tensors > 0 && d_out == nullptr) return SDC_ERR_INVALID;
  return launch_scan(d_plan, h_info, d_out, as_stream(stream));
}

extern "C" int32_t sdc_fingerprint(const sdc_tensor* h_tensors, uint64_t n, void* d_ws,
                                   uint64_t ws_bytes, sdc_row* d_out, sdc_stream_t stream) {
  sdc_plan_info info;
  int32_t st = sdc_plan_build(h_tensors, n, 0, d_ws, ws_bytes, &info, stream);
  if (st) return st;
  return sdc_fingerprint_plan(d_ws, &info, d_out, stream);
}

extern "C" int32_t sdc_tensor_ws_bytes(const sdc_tensor* h_tensor, uint64_t item_bytes,
                                       uint64_t* h_bytes) {
  if (h_bytes == nullptr) return SDC_ERR_INVALID;
  TensorShape sh;
  const int32_t st = tensor_shape(h_tensor, item_bytes, &sh);
  if (st) return st;
  *h_bytes = std::max<uint64_t>(sh.n_items, 1) * sizeof(sdc_row);
  return SDC_OK;
}

extern "C" int32_t sdc_fingerprint_tensor(const sdc_tensor* h_tensor, uint64_t item_bytes, void* d_ws,
                                          uint64_t ws_bytes, const sdc_row* d_ref, uint32_t col_mask,
                                          sdc_row* d_out, uint32_t* d_mismatch, sdc_stream_t stream) {
  TensorShape sh;
  int32_t st = tensor_shape(h_tensor, item_bytes, &sh);
  if (st) return st;
  if (d_out == nullptr || d_ws == nullptr) return SDC_ERR_INVALID;
  if (d_ref && (d_mismatch == nullptr || (col_mask & SDC_COL_ALL) == 0 ||
                (col_mask & ~(uint32_t)SDC_COL_ALL) != 0))
    return SDC_ERR_INVALID;
  if (ws_bytes < std::max<uint64_t>(sh.n_items, 1) * sizeof(sdc_row)) return SDC_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  sdc_row* partials = reinterpret_cast<sdc_row*>(d_ws);
  if (sh.n_items) {
    TensorJob j;
    j.addr = reinterpret_cast<uintptr_t>(h_tensor->ptr);
    j.numel = h_tensor->numel;
    j.ie = sh.ie;
    j.h = sh.h;
    j.df = h_tensor->dtype | ((h_tensor->flags & SDC_FLAG_SIGNED) ? kItemSigned : 0u);
    j.es = sh.es;
    j.pad = 0;
    if (sh.ie * sh.es >= kDeepItemBytes)
      hipLaunchKernelGGL(fingerprint_tensor_kernel<DeepBody>, dim3((uint32_t)sh.n_items), dim3(kBlock),
                         0, s, j, partials);
    else
      hipLaunchKernelGGL(fingerprint_tensor_kernel<DefaultBody>, dim3((uint32_t)sh.n_items),
                         dim3(kBlock), 0, s, j, partials);
    if ((st = launch_status())) return st;
  }
  hipLaunchKernelGGL(merge_check_kernel, dim3(1), dim3(64), 0, s, partials, (uint32_t)sh.n_items,
                     d_out, d_ref, col_mask, d_mismatch);
  return launch_status();
}
