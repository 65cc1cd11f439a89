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
//   * The aligned body is read with coalesced 16-byte buffer loads (lane t of
//     the workgroup takes vector 256*it + t of the body), U per lane in flight.
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
//     form); a tensor scanned by one item stores its row, a split tensor adds
//     into a row cleared beforehand with 64-bit atomics (+, +, ^, +), which
//     are order independent, so the result is bit-exact.
#include <algorithm>
#include <cstring>
#include <vector>

#include "sdc_internal.h"

namespace sdc {
namespace {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// By-value reinterpretations.  (Bit-casting a vector component in place is
// avoided on purpose: clang lowers __builtin_bit_cast(T, v.y) as a read of
// the vector's first component.)
__device__ __forceinline__ us2 as_us2(uint32_t w) { return __builtin_bit_cast(us2, w); }
__device__ __forceinline__ h2 as_h2(uint32_t w) { return __builtin_bit_cast(h2, w); }
__device__ __forceinline__ uint32_t h2_bits(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// acc + lo(d)*lo(w) + hi(d)*hi(w), 16x16 -> 32-bit products, no clamping.
__device__ __forceinline__ uint32_t dot2(uint32_t d, uint32_t w, uint32_t acc) {
  return __builtin_amdgcn_udot2(as_us2(d), as_us2(w), acc, false);
}

// Raw buffer over [base, base + bytes): loads beyond `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

// Exact NaN/Inf tests on raw patterns (exponent field all ones).
template <uint32_t DT>
__device__ __forceinline__ uint32_t nonfinite_bits(uint32_t x) {
  if constexpr (DT == SDC_F32) return (x & 0x7F800000u) == 0x7F800000u;
  if constexpr (DT == SDC_BF16) return (x & 0x7F80u) == 0x7F80u;
  return (x & 0x7C00u) == 0x7C00u;  // SDC_F16
}

// Exact count of non-finite elements in one 16-byte vector.
template <uint32_t DT>
__device__ __forceinline__ uint32_t nonfinite_vec(u32x4 v) {
  uint32_t c = 0;
  uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (DT == SDC_F32) {
      c += nonfinite_bits<DT>(d[i]);
    } else {
      c += nonfinite_bits<DT>(d[i] & 0xFFFFu) + nonfinite_bits<DT>(d[i] >> 16);
    }
  }
  return c;
}

// Per-lane partial state of one item.
struct Lane {
  uint64_t s = 0;   // sum of x over the lane's elements
  uint64_t w = 0;   // sum of (j+1) x over the lane's elements (j: index in the item)
  uint32_t x = 0;   // xor of the lane's 32-bit words and scalar elements
  uint32_t nf = 0;  // exact non-finite count
};

// ---- 16-bit elements (bf16, fp16): 8 per vector ---------------------------
struct Acc16 {
  uint32_t a = 0;  // sum x
  uint32_t c = 0;  // sum k x, k = slot 0..7 in the vector
  uint64_t q = 0;  // running sum of a after each vector
  uint32_t x = 0;  // xor of dwords
  h2 nf = {0, 0};  // sticky NaN flag (+0 until a NaN/Inf is seen)

  __device__ __forceinline__ void add(u32x4 v) {
    a = dot2(v.x, 0x00010001u, a);
    a = dot2(v.y, 0x00010001u, a);
    a = dot2(v.z, 0x00010001u, a);
    a = dot2(v.w, 0x00010001u, a);
    c = dot2(v.x, 0x00010000u, c);
    c = dot2(v.y, 0x00030002u, c);
    c = dot2(v.z, 0x00050004u, c);
    c = dot2(v.w, 0x00070006u, c);
    q += a;
    x ^= v.x ^ v.y ^ v.z ^ v.w;
    const h2 z = {0, 0};
    nf = __builtin_elementwise_fma(as_h2(v.x), z, nf);
    nf = __builtin_elementwise_fma(as_h2(v.y), z, nf);
    nf = __builtin_elementwise_fma(as_h2(v.z), z, nf);
    nf = __builtin_elementwise_fma(as_h2(v.w), z, nf);
  }
  __device__ __forceinline__ bool flagged() const { return h2_bits(nf) != 0; }
  __device__ __forceinline__ uint64_t sum() const { return a; }
  __device__ __forceinline__ uint64_t csum() const { return c; }
};

// ---- 32-bit elements (fp32): 4 per vector ---------------------------------
struct Acc32 {
  uint64_t a = 0;  // sum x
  uint64_t c = 0;  // sum k x, k = slot 0..3
  uint64_t q = 0;  // running sum of a after each vector
  uint32_t x = 0;
  float nf = 0.0f;

  __device__ __forceinline__ void add(u32x4 v) {
    a += (uint64_t)v.x + (uint64_t)v.y + (uint64_t)v.z + (uint64_t)v.w;
    c += (uint64_t)v.y + 2ull * v.z + 3ull * v.w;
    q += a;
    x ^= v.x ^ v.y ^ v.z ^ v.w;
    nf = __builtin_fmaf(__uint_as_float(v.x), 0.0f, nf);
    nf = __builtin_fmaf(__uint_as_float(v.y), 0.0f, nf);
    nf = __builtin_fmaf(__uint_as_float(v.z), 0.0f, nf);
    nf = __builtin_fmaf(__uint_as_float(v.w), 0.0f, nf);
  }
  __device__ __forceinline__ bool flagged() const { return __float_as_uint(nf) != 0u; }
  __device__ __forceinline__ uint64_t sum() const { return a; }
  __device__ __forceinline__ uint64_t csum() const { return c; }
};

template <uint32_t DT>
struct AccOf { typedef Acc16 type; };
template <>
struct AccOf<SDC_F32> { typedef Acc32 type; };

constexpr int kUnroll = 4;

// Body of one item: nvec aligned vectors at `body`.  Lane t handles vectors
// 256*it + t, it = 0 .. T-1 with T = rounds*U (uniform over the workgroup);
// vectors past the end are not loaded and count as zero vectors, which leave
// every partial sum unchanged (and keep T*A - Q exact).
template <uint32_t DT>
__device__ __forceinline__ void scan_body(const unsigned char* body, uint32_t nvec, uint32_t h,
                                          Lane& ln) {
  typedef typename AccOf<DT>::type Acc;
  constexpr uint32_t E = (DT == SDC_F32) ? 4u : 8u;  // elements per vector
  constexpr uint32_t kRound = kBlock * kUnroll;      // vectors per round
  const uint32_t t = threadIdx.x;
  Acc acc;
  const uint32_t full = nvec / kRound;
  const uint32_t rounds = full + ((nvec % kRound) ? 1u : 0u);
  for (uint32_t r = 0; r < full; ++r) {
    const uint32_t v0 = r * kRound;
    __amdgpu_buffer_rsrc_t rs = make_rsrc(body + (uint64_t)v0 * kVecBytes, kRound * kVecBytes);
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load16(rs, (u * kBlock + t) * kVecBytes);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc.add(v[u]);
  }
  if (full < rounds) {
    const uint32_t v0 = full * kRound;
    const uint32_t left = nvec - v0;
    __amdgpu_buffer_rsrc_t rs = make_rsrc(body + (uint64_t)v0 * kVecBytes, left * kVecBytes);
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t vi = u * kBlock + t;
      v[u] = (vi < left) ? load16(rs, vi * kVecBytes) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc.add(v[u]);
  }
  const uint64_t T = (uint64_t)rounds * kUnroll;
  const uint64_t A = acc.sum();
  ln.s += A;
  ln.w += (uint64_t)(h + 1u + E * t) * A + (uint64_t)(kBlock * E) * (T * A - acc.q) + acc.csum();
  ln.x ^= acc.x;
  if (acc.flagged()) {
    // Rare: some element may be NaN/Inf.  Recount this lane's vectors exactly.
    uint32_t c = 0;
    for (uint32_t vi = t; vi < nvec; vi += kBlock) {
      __amdgpu_buffer_rsrc_t rs = make_rsrc(body + (uint64_t)vi * kVecBytes, kVecBytes);
      c += nonfinite_vec<DT>(load16(rs, 0));
    }
    ln.nf += c;
  }
}

// Head/tail element j (index within the item) at p.
template <uint32_t DT>
__device__ __forceinline__ void scan_scalar(const unsigned char* p, uint32_t j, Lane& ln) {
  uint32_t x;
  if constexpr (DT == SDC_F32) x = *reinterpret_cast<const uint32_t*>(p);
  else x = *reinterpret_cast<const unsigned short*>(p);
  ln.s += x;
  ln.w += (uint64_t)(j + 1u) * x;
  ln.x ^= x;
  ln.nf += nonfinite_bits<DT>(x);
}

__device__ __forceinline__ void block_reduce(Lane& ln) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    ln.s += __shfl_xor(ln.s, off);
    ln.w += __shfl_xor(ln.w, off);
    ln.x ^= __shfl_xor(ln.x, off);
    ln.nf += __shfl_xor(ln.nf, off);
  }
  __shared__ uint64_t ls[kWaves], lw[kWaves];
  __shared__ uint32_t lx[kWaves], ln_[kWaves];
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

// Scan of one item into a lane-partial; returns in lane 0 the item's
// (S, sum (j+1) x_j with j local to the item, X folded to element width, NF).
template <uint32_t DT>
__device__ __forceinline__ void scan_item(const PlanItem& it, Lane& ln) {
  constexpr uint32_t es = (DT == SDC_F32) ? 4u : 2u;
  const unsigned char* base = reinterpret_cast<const unsigned char*>(it.addr);
  const uint32_t len = it.len;
  const uint32_t mis = (uint32_t)(it.addr & 15u);
  const uint32_t h = mis ? min(len, (16u - mis) / es) : 0u;
  const uint32_t nvec = (uint32_t)(((uint64_t)(len - h) * es) / kVecBytes);
  const uint32_t tail0 = h + nvec * (kVecBytes / es);
  const uint32_t ntail = len - tail0;
  const uint32_t t = threadIdx.x;
  if (t < h) scan_scalar<DT>(base + (uint64_t)t * es, t, ln);
  if (t >= 128u && t - 128u < ntail) {
    const uint32_t j = tail0 + (t - 128u);
    scan_scalar<DT>(base + (uint64_t)j * es, j, ln);
  }
  if (nvec) scan_body<DT>(base + (uint64_t)h * es, nvec, h, ln);
  block_reduce(ln);
  if constexpr (es == 2) ln.x = (ln.x & 0xFFFFu) ^ (ln.x >> 16);
}

__global__ void __launch_bounds__(kBlock) fingerprint_kernel(const PlanItem* __restrict__ items,
                                                             sdc_row* __restrict__ out) {
  const PlanItem it = items[blockIdx.x];
  Lane ln;
  switch (it.dtype) {
    case SDC_F32: scan_item<SDC_F32>(it, ln); break;
    case SDC_BF16: scan_item<SDC_BF16>(it, ln); break;
    default: scan_item<SDC_F16>(it, ln); break;
  }
  if (threadIdx.x != 0) return;
  const uint64_t S = ln.s;
  const uint64_t W = ln.w + it.start * S;
  sdc_row* row = out + it.row;
  if (it.flags & kItemWhole) {
    row->sum = S;
    row->wsum = W;
    row->xorsum = ln.x;
    row->nonfinite = ln.nf;
  } else {
    atomicAdd(reinterpret_cast<unsigned long long*>(&row->sum), (unsigned long long)S);
    atomicAdd(reinterpret_cast<unsigned long long*>(&row->wsum), (unsigned long long)W);
    if (ln.x) atomicXor(reinterpret_cast<unsigned long long*>(&row->xorsum), (unsigned long long)ln.x);
    if (ln.nf) atomicAdd(reinterpret_cast<unsigned long long*>(&row->nonfinite), (unsigned long long)ln.nf);
  }
}

// ---- NaN/Inf count only ----------------------------------------------------
template <uint32_t DT>
__device__ __forceinline__ uint32_t nonfinite_item(const PlanItem& it) {
  constexpr uint32_t es = (DT == SDC_F32) ? 4u : 2u;
  constexpr uint32_t kRound = kBlock * kUnroll;
  const unsigned char* base = reinterpret_cast<const unsigned char*>(it.addr);
  const uint32_t len = it.len;
  const uint32_t mis = (uint32_t)(it.addr & 15u);
  const uint32_t h = mis ? min(len, (16u - mis) / es) : 0u;
  const uint32_t nvec = (uint32_t)(((uint64_t)(len - h) * es) / kVecBytes);
  const uint32_t tail0 = h + nvec * (kVecBytes / es);
  const uint32_t ntail = len - tail0;
  const uint32_t t = threadIdx.x;
  uint32_t c = 0;
  if (t < h) {
    const unsigned char* p = base + (uint64_t)t * es;
    c += nonfinite_bits<DT>(es == 4 ? *reinterpret_cast<const uint32_t*>(p)
                                    : *reinterpret_cast<const unsigned short*>(p));
  }
  if (t >= 128u && t - 128u < ntail) {
    const unsigned char* p = base + (uint64_t)(tail0 + t - 128u) * es;
    c += nonfinite_bits<DT>(es == 4 ? *reinterpret_cast<const uint32_t*>(p)
                                    : *reinterpret_cast<const unsigned short*>(p));
  }
  if (nvec) {
    const unsigned char* body = base + (uint64_t)h * es;
    bool flag = false;
    if constexpr (DT == SDC_F32) {
      float nf = 0.0f;
      for (uint32_t v0 = 0; v0 < nvec; v0 += kRound) {
        const uint32_t left = min(nvec - v0, kRound);
        __amdgpu_buffer_rsrc_t rs = make_rsrc(body + (uint64_t)v0 * kVecBytes, left * kVecBytes);
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const uint32_t vi = u * kBlock + t;
          v[u] = (vi < left) ? load16(rs, vi * kVecBytes) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          nf = __builtin_fmaf(__uint_as_float(v[u].x), 0.0f, nf);
          nf = __builtin_fmaf(__uint_as_float(v[u].y), 0.0f, nf);
          nf = __builtin_fmaf(__uint_as_float(v[u].z), 0.0f, nf);
          nf = __builtin_fmaf(__uint_as_float(v[u].w), 0.0f, nf);
        }
      }
      flag = __float_as_uint(nf) != 0u;
    } else {
      h2 nf = {0, 0};
      const h2 z = {0, 0};
      for (uint32_t v0 = 0; v0 < nvec; v0 += kRound) {
        const uint32_t left = min(nvec - v0, kRound);
        __amdgpu_buffer_rsrc_t rs = make_rsrc(body + (uint64_t)v0 * kVecBytes, left * kVecBytes);
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const uint32_t vi = u * kBlock + t;
          v[u] = (vi < left) ? load16(rs, vi * kVecBytes) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          nf = __builtin_elementwise_fma(as_h2(v[u].x), z, nf);
          nf = __builtin_elementwise_fma(as_h2(v[u].y), z, nf);
          nf = __builtin_elementwise_fma(as_h2(v[u].z), z, nf);
          nf = __builtin_elementwise_fma(as_h2(v[u].w), z, nf);
        }
      }
      flag = h2_bits(nf) != 0u;
    }
    if (flag) {
      for (uint32_t vi = t; vi < nvec; vi += kBlock) {
        __amdgpu_buffer_rsrc_t rs = make_rsrc(body + (uint64_t)vi * kVecBytes, kVecBytes);
        c += nonfinite_vec<DT>(load16(rs, 0));
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

__global__ void __launch_bounds__(kBlock) nonfinite_kernel(const PlanItem* __restrict__ items,
                                                           uint64_t* __restrict__ counts,
                                                           uint64_t* __restrict__ total) {
  const PlanItem it = items[blockIdx.x];
  uint32_t c;
  switch (it.dtype) {
    case SDC_F32: c = nonfinite_item<SDC_F32>(it); break;
    case SDC_BF16: c = nonfinite_item<SDC_BF16>(it); break;
    default: c = nonfinite_item<SDC_F16>(it); break;
  }
  if (threadIdx.x != 0) return;
  if (counts) {
    if (it.flags & kItemWhole) counts[it.row] = c;
    else if (c) atomicAdd(reinterpret_cast<unsigned long long*>(counts + it.row), (unsigned long long)c);
  }
  if (c) atomicAdd(reinterpret_cast<unsigned long long*>(total), (unsigned long long)c);
}

// Clears the rows that are split over several items or have no item at all
// (empty or missing tensors).  A plain fill kernel rather than a memset node,
// so the sequence stays valid under stream capture.
__global__ void __launch_bounds__(kBlock) clear_rows_kernel(const uint32_t* __restrict__ rows,
                                                            uint64_t n, sdc_row* __restrict__ out) {
  for (uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * kBlock) {
    sdc_row* r = out + rows[i];
    r->sum = 0;
    r->wsum = 0;
    r->xorsum = 0;
    r->nonfinite = 0;
  }
}

__global__ void __launch_bounds__(kBlock) clear_counts_kernel(const uint32_t* __restrict__ rows,
                                                              uint64_t n, uint64_t* __restrict__ counts,
                                                              uint64_t* __restrict__ total) {
  const uint64_t i0 = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i0 == 0) *total = 0;
  if (!counts) return;
  for (uint64_t i = i0; i < n; i += (uint64_t)gridDim.x * kBlock) counts[rows[i]] = 0;
}

// ---- host side: plan layout --------------------------------------------------
struct Layout {
  uint64_t n_items = 0, n_zero = 0, total_elems = 0, total_bytes = 0, item_bytes = 0;
  uint64_t items_off = 0, zero_off = 0, plan_bytes = 0;
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

int32_t layout_plan(const sdc_tensor* t, uint64_t n, uint64_t item_bytes, Layout* L) {
  if (n > 0 && t == nullptr) return SDC_ERR_INVALID;
  if (n >= (1ull << 32)) return SDC_ERR_RANGE;
  if (item_bytes % kVecBytes != 0 || item_bytes > kItemBytesMax) return SDC_ERR_INVALID;
  uint64_t elems = 0, bytes = 0;
  for (uint64_t k = 0; k < n; ++k) {
    if (t[k].flags != 0) return SDC_ERR_INVALID;
    const uint32_t es = element_size(t[k].dtype);
    if (es == 0) return SDC_ERR_DTYPE;
    if (t[k].ptr == nullptr || t[k].numel == 0) continue;
    if (t[k].numel >= (1ull << 62)) return SDC_ERR_RANGE;
    if (reinterpret_cast<uintptr_t>(t[k].ptr) % es != 0) return SDC_ERR_ALIGN;
    elems += t[k].numel;
    bytes += t[k].numel * es;
  }
  if (item_bytes == 0) {
    uint64_t ib = align_up(std::max<uint64_t>(bytes / kAutoTargetItems, 1), 4096);
    item_bytes = std::min(kAutoMax, std::max(kAutoMin, ib));
  }
  uint64_t items = 0, zero = 0;
  for (uint64_t k = 0; k < n; ++k) {
    if (t[k].ptr == nullptr || t[k].numel == 0) {
      zero++;
      continue;
    }
    const uint32_t es = element_size(t[k].dtype);
    uint64_t c = 0;
    split_tensor(reinterpret_cast<uintptr_t>(t[k].ptr), t[k].numel, es, item_bytes,
                 [&](uint64_t, uint64_t) { c++; });
    items += c;
    if (c > 1) zero++;
  }
  if (items > kMaxGrid) return SDC_ERR_RANGE;
  L->n_items = items;
  L->n_zero = zero;
  L->total_elems = elems;
  L->total_bytes = bytes;
  L->item_bytes = item_bytes;
  L->items_off = sizeof(PlanHeader);
  L->zero_off = L->items_off + items * sizeof(PlanItem);
  L->plan_bytes = align_up(L->zero_off + zero * sizeof(uint32_t), 256);
  return SDC_OK;
}

// Host image of the plan.  Items are ordered by their relative position in
// their tensor (then by tensor), so consecutive workgroups work on different
// tensors and the atomics of a large tensor's items are spread over the launch.
void pack_plan(const sdc_tensor* t, uint64_t n, const Layout& L, std::vector<unsigned char>& img) {
  img.assign(L.plan_bytes, 0);
  PlanHeader* hd = reinterpret_cast<PlanHeader*>(img.data());
  hd->magic = kPlanMagic;
  hd->n_tensors = n;
  hd->n_items = L.n_items;
  hd->n_zero = L.n_zero;
  hd->items_off = L.items_off;
  hd->zero_off = L.zero_off;
  hd->total_bytes = L.total_bytes;
  hd->item_bytes = L.item_bytes;
  struct Keyed {
    double key;
    PlanItem it;
  };
  std::vector<Keyed> all;
  all.reserve(L.n_items);
  uint32_t* zero = reinterpret_cast<uint32_t*>(img.data() + L.zero_off);
  uint64_t nz = 0;
  for (uint64_t k = 0; k < n; ++k) {
    if (t[k].ptr == nullptr || t[k].numel == 0) {
      zero[nz++] = (uint32_t)k;
      continue;
    }
    const uint32_t es = element_size(t[k].dtype);
    const uint64_t ptr = reinterpret_cast<uintptr_t>(t[k].ptr);
    const size_t first = all.size();
    split_tensor(ptr, t[k].numel, es, L.item_bytes, [&](uint64_t s, uint64_t len) {
      Keyed e;
      e.key = 0.0;
      e.it.addr = ptr + s * es;
      e.it.start = s;
      e.it.len = (uint32_t)len;
      e.it.row = (uint32_t)k;
      e.it.dtype = t[k].dtype;
      e.it.flags = 0;
      all.push_back(e);
    });
    const size_t cnt = all.size() - first;
    if (cnt == 1) all[first].it.flags = kItemWhole;
    else zero[nz++] = (uint32_t)k;
    for (size_t i = 0; i < cnt; ++i) all[first + i].key = (i + 0.5) / (double)cnt;
  }
  std::stable_sort(all.begin(), all.end(),
                   [](const Keyed& a, const Keyed& b) { return a.key < b.key; });
  PlanItem* items = reinterpret_cast<PlanItem*>(img.data() + L.items_off);
  for (size_t i = 0; i < all.size(); ++i) items[i] = all[i].it;
}

bool info_ok(const sdc_plan_info* h) {
  return h != nullptr && h->magic == kPlanMagic && h->n_items <= kMaxGrid &&
         h->plan_bytes >= sizeof(PlanHeader) + h->n_items * sizeof(PlanItem) + h->n_zero * 4;
}

int32_t launch_scan(const unsigned char* plan, const sdc_plan_info* h, sdc_row* out,
                    hipStream_t s) {
  const PlanItem* items = reinterpret_cast<const PlanItem*>(plan + sizeof(PlanHeader));
  const uint32_t* zero =
      reinterpret_cast<const uint32_t*>(plan + sizeof(PlanHeader) + h->n_items * sizeof(PlanItem));
  if (h->n_zero) {
    const uint64_t g = std::min<uint64_t>((h->n_zero + kBlock - 1) / kBlock, 1024);
    hipLaunchKernelGGL(clear_rows_kernel, dim3((uint32_t)g), dim3(kBlock), 0, s, zero, h->n_zero,
                       out);
    int32_t st = launch_status();
    if (st) return st;
  }
  if (h->n_items) {
    hipLaunchKernelGGL(fingerprint_kernel, dim3((uint32_t)h->n_items), dim3(kBlock), 0, s, items,
                       out);
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
  *h_bytes = L.plan_bytes;
  return SDC_OK;
}

extern "C" int32_t sdc_plan_build(const sdc_tensor* h_tensors, uint64_t n, uint64_t item_bytes,
                                  void* d_plan, uint64_t plan_bytes, sdc_plan_info* h_info,
                                  sdc_stream_t stream) {
  if (d_plan == nullptr || h_info == nullptr) return SDC_ERR_INVALID;
  Layout L;
  int32_t st = layout_plan(h_tensors, n, item_bytes, &L);
  if (st) return st;
  if (plan_bytes < L.plan_bytes) return SDC_ERR_WORKSPACE;
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
  h_info->n_zero = L.n_zero;
  h_info->total_elems = L.total_elems;
  h_info->total_bytes = L.total_bytes;
  h_info->plan_bytes = L.plan_bytes;
  h_info->item_bytes = L.item_bytes;
  return SDC_OK;
}

extern "C" int32_t sdc_fingerprint_plan(const void* d_plan, const sdc_plan_info* h_info,
                                        sdc_row* d_out, sdc_stream_t stream) {
  if (d_plan == nullptr || h_info == nullptr) return SDC_ERR_INVALID;
  if (!info_ok(h_info)) return SDC_ERR_PLAN;
  if (h_info->n_tensors > 0 && d_out == nullptr) return SDC_ERR_INVALID;
  return launch_scan(reinterpret_cast<const unsigned char*>(d_plan), h_info, d_out,
                     as_stream(stream));
}

extern "C" int32_t sdc_nonfinite(const void* d_plan, const sdc_plan_info* h_info,
                                 uint64_t* d_counts, uint64_t* d_total, sdc_stream_t stream) {
  if (d_plan == nullptr || h_info == nullptr || d_total == nullptr) return SDC_ERR_INVALID;
  if (!info_ok(h_info)) return SDC_ERR_PLAN;
  hipStream_t s = as_stream(stream);
  const unsigned char* plan = reinterpret_cast<const unsigned char*>(d_plan);
  const PlanItem* items = reinterpret_cast<const PlanItem*>(plan + sizeof(PlanHeader));
  const uint32_t* zero = reinterpret_cast<const uint32_t*>(plan + sizeof(PlanHeader) +
                                                           h_info->n_items * sizeof(PlanItem));
  const uint64_t g = std::max<uint64_t>(1, std::min<uint64_t>((h_info->n_zero + kBlock - 1) / kBlock, 1024));
  hipLaunchKernelGGL(clear_counts_kernel, dim3((uint32_t)g), dim3(kBlock), 0, s, zero,
                     h_info->n_zero, d_counts, d_total);
  int32_t st = launch_status();
  if (st) return st;
  if (h_info->n_items) {
    hipLaunchKernelGGL(nonfinite_kernel, dim3((uint32_t)h_info->n_items), dim3(kBlock), 0, s, items,
                       d_counts, d_total);
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
