// compare.hip -- comparisons of fingerprint tables on the GPU.
//
// sdc_majority_compare: strict-majority comparison of R replicas' tables
//   (AWS Machine Learning Blog, "Detecting and recovering from silent data
//   corruption on Amazon SageMaker HyperPod", section "Check 3: Weight
//   fingerprints, after the optimizer step").  One lane per tensor; the
//   candidate majority row is found with the Boyer-Moore vote and confirmed
//   by counting, which decides "more than half" exactly.  Flags and counters
//   are combined with order-independent atomics (or, min, add).
// sdc_fingerprint_diff: rows of two tables that differ (same blog, section
//   "Check 2: Ring replay, before the optimizer step": a replay is compared
//   bit for bit with the original), reported in ascending order through a
//   count / scan / write pass, with the single-bit-flip localisation.
// sdc_ring_compare / sdc_ring_localize / sdc_confirm_verdict: the ring replay
//   audit of the same section over an all-gathered [rank][own, replay] table.
#include <algorithm>
#include <cstddef>
#include <cstring>
#include <vector>

#include "sdc_internal.h"

namespace sdc {
namespace {

struct Row4 {
  uint64_t s, w, x, nf;
};

__device__ __forceinline__ Row4 load_row(const sdc_row* p) {
  const ulonglong2* q = reinterpret_cast<const ulonglong2*>(p);
  ulonglong2 a = q[0], b = q[1];
  return Row4{a.x, a.y, b.x, b.y};
}

__device__ __forceinline__ bool row_eq(const Row4& a, const Row4& b, uint32_t m) {
  return (!(m & SDC_COL_SUM) || a.s == b.s) && (!(m & SDC_COL_WSUM) || a.w == b.w) &&
         (!(m & SDC_COL_XOR) || a.x == b.x) && (!(m & SDC_COL_NONFINITE) || a.nf == b.nf);
}

bool mask_ok(uint32_t m) { return (m & SDC_COL_ALL) != 0 && (m & ~(uint32_t)SDC_COL_ALL) == 0; }

// ---- majority ----------------------------------------------------------------
// Workspace: [0, 32) counters, [32, 64) the result, [64, 64 + R) one byte per
// replica (named or not) -- result and flags are contiguous, so one copy
// brings them to the host -- then, 256-byte aligned, R 32-bit flags.
struct MajWS {
  unsigned long long n_diff, n_nomaj, first_diff, first_nomaj;
  sdc_majority res;
};
static_assert(sizeof(MajWS) == 64, "majority workspace header");

constexpr uint64_t kMajOut = offsetof(MajWS, res);  // result, then the R flag bytes
constexpr uint64_t kMajSus8 = sizeof(MajWS);
// Tables this small are compared by one workgroup in one launch (flags and
// counters in LDS); larger ones by a grid of one lane per tensor.
constexpr uint32_t kMajFusedMaxR = 1024;
constexpr uint64_t kMajFusedMaxT = 1024;

uint64_t maj_sus_off(uint32_t R) { return (kMajSus8 + R + 255) / 256 * 256; }
uint64_t maj_ws_bytes(uint32_t R) { return maj_sus_off(R) + ((uint64_t)R * 4 + 255) / 256 * 256; }

// Where the per-tensor outcome goes: device-wide atomics on the workspace, or
// LDS atomics of the one-workgroup path.  Both are order independent.
struct GlobalSink {
  MajWS* ws;
  uint32_t* sus;
  __device__ void diff(uint64_t k) {
    atomicAdd(&ws->n_diff, 1ull);
    atomicMin(&ws->first_diff, (unsigned long long)k);
  }
  __device__ void nomaj(uint64_t k) {
    atomicAdd(&ws->n_nomaj, 1ull);
    atomicMin(&ws->first_nomaj, (unsigned long long)k);
  }
  __device__ void suspect(uint32_t r) { atomicOr(&sus[r], 1u); }
};

struct LdsSink {
  unsigned long long* c;  // n_diff, n_nomaj, first_diff, first_nomaj
  uint32_t* sus;
  __device__ void diff(uint64_t k) {
    atomicAdd(&c[0], 1ull);
    atomicMin(&c[2], (unsigned long long)k);
  }
  __device__ void nomaj(uint64_t k) {
    atomicAdd(&c[1], 1ull);
    atomicMin(&c[3], (unsigned long long)k);
  }
  __device__ void suspect(uint32_t r) { atomicOr(&sus[r], 1u); }
};

// Tensor k: 0 = all R rows equal, 1 = a strict majority (the differing
// replicas are named), 2 = no strict majority.
template <class Sink>
__device__ __forceinline__ uint8_t maj_tensor(const sdc_row* __restrict__ table, uint32_t R,
                                              uint64_t T, uint64_t k, uint32_t mask, Sink& sink) {
  const Row4 r0 = load_row(table + k);
  bool differs = false;
  for (uint32_t r = 1; r < R && !differs; ++r)
    differs = !row_eq(load_row(table + (uint64_t)r * T + k), r0, mask);
  if (!differs) return 0;
  // Boyer-Moore vote: if some row is held by more than R/2 replicas it is the
  // surviving candidate; the count below confirms or rejects it.
  Row4 cand = r0;
  uint32_t votes = 1;
  for (uint32_t r = 1; r < R; ++r) {
    const Row4 v = load_row(table + (uint64_t)r * T + k);
    if (votes == 0) {
      cand = v;
      votes = 1;
    } else if (row_eq(v, cand, mask)) {
      votes++;
    } else {
      votes--;
    }
  }
  uint32_t c = 0;
  for (uint32_t r = 0; r < R; ++r) c += row_eq(load_row(table + (uint64_t)r * T + k), cand, mask);
  sink.diff(k);
  if (2ull * c > (uint64_t)R) {
    for (uint32_t r = 0; r < R; ++r)
      if (!row_eq(load_row(table + (uint64_t)r * T + k), cand, mask)) sink.suspect(r);
    return 1;
  }
  sink.nomaj(k);
  return 2;
}

// The result from the counters: with no strict majority somewhere no replica
// is named.  Executed by one workgroup.
__device__ __forceinline__ void maj_result(const unsigned long long* c, const uint32_t* sus,
                                           uint32_t R, MajWS* ws, uint8_t* sus8) {
  const bool none = c[1] != 0;
  for (uint32_t r = threadIdx.x; r < R; r += kBlock) sus8[r] = (!none && sus[r]) ? 1 : 0;
  if (threadIdx.x == 0) {
    ws->res.diverged = c[0] != 0;
    ws->res.has_majority = c[1] == 0;
    ws->res.n_diff = c[0];
    ws->res.first_diff = c[2];
    ws->res.first_no_majority = c[3];
  }
}

__global__ void __launch_bounds__(kBlock) maj_fused(const sdc_row* __restrict__ table, uint32_t R,
                                                    uint64_t T, uint32_t mask, MajWS* ws,
                                                    uint8_t* sus8, uint8_t* status) {
  __shared__ unsigned long long c[4];
  __shared__ uint32_t sus[kMajFusedMaxR];
  if (threadIdx.x == 0) {
    c[0] = 0;
    c[1] = 0;
    c[2] = ~0ull;
    c[3] = ~0ull;
  }
  for (uint32_t r = threadIdx.x; r < R; r += kBlock) sus[r] = 0;
  __syncthreads();
  LdsSink sink{c, sus};
  for (uint64_t k = threadIdx.x; k < T; k += kBlock) {
    const uint8_t st = maj_tensor(table, R, T, k, mask, sink);
    if (status) status[k] = st;
  }
  __syncthreads();
  maj_result(c, sus, R, ws, sus8);
}

__global__ void __launch_bounds__(kBlock) maj_init(MajWS* ws, uint32_t* sus, uint32_t R) {
  const uint32_t i0 = blockIdx.x * kBlock + threadIdx.x;
  if (i0 == 0) {
    ws->n_diff = 0;
    ws->n_nomaj = 0;
    ws->first_diff = ~0ull;
    ws->first_nomaj = ~0ull;
  }
  for (uint32_t r = i0; r < R; r += gridDim.x * kBlock) sus[r] = 0;
}

__global__ void __launch_bounds__(kBlock) maj_compare(const sdc_row* __restrict__ table, uint32_t R,
                                                      uint64_t T, uint32_t mask, MajWS* ws,
                                                      uint32_t* sus, uint8_t* status) {
  GlobalSink sink{ws, sus};
  for (uint64_t k = (uint64_t)blockIdx.x * kBlock + threadIdx.x; k < T;
       k += (uint64_t)gridDim.x * kBlock) {
    const uint8_t st = maj_tensor(table, R, T, k, mask, sink);
    if (status) status[k] = st;
  }
}

__global__ void __launch_bounds__(kBlock) maj_finalize(MajWS* ws, const uint32_t* sus, uint8_t* sus8,
                                                       uint32_t R) {
  const unsigned long long c[4] = {ws->n_diff, ws->n_nomaj, ws->first_diff, ws->first_nomaj};
  maj_result(c, sus, R, ws, sus8);
}

// ---- diff --------------------------------------------------------------------
constexpr uint32_t kPerLane = 4;
constexpr uint32_t kPerBlock = kBlock * kPerLane;

// Single-bit-flip localisation (see sdc_flip_hint in sdc.h).
__device__ __forceinline__ sdc_flip_hint flip_hint(const Row4& a, const Row4& b) {
  sdc_flip_hint h;
  h.index = ~0ull;
  h.bit = -1;
  h.dir = 0;
  const uint64_t dx = a.x ^ b.x;
  if (dx == 0 || (dx & (dx - 1)) != 0) return h;
  const int bit = __ffsll((long long)dx) - 1;
  const uint64_t ds = b.s - a.s;
  uint64_t dw = b.w - a.w;
  int dir;
  if (ds == dx) {
    dir = 1;
  } else if (ds == 0ull - dx) {
    dir = -1;
    dw = 0ull - dw;
  } else {
    return h;
  }
  if (dw >> 63) return h;
  const uint64_t q = dw >> bit;
  if (q == 0 || (q << bit) != dw) return h;
  h.index = q - 1;
  h.bit = bit;
  h.dir = dir;
  return h;
}

// Exclusive scan of one value per lane over the workgroup; *total gets the sum.
__device__ __forceinline__ uint32_t block_exscan(uint32_t v, uint32_t* total) {
  __shared__ uint32_t wsum[kWaves];
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_up(inc, off);
    if (lane >= (uint32_t)off) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    if ((uint32_t)i < wave) before += wsum[i];
    all += wsum[i];
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

__device__ __forceinline__ uint32_t lane_flags(const sdc_row* a, const sdc_row* b, uint64_t T,
                                               uint32_t mask, uint64_t k0) {
  uint32_t f = 0;
#pragma unroll
  for (uint32_t j = 0; j < kPerLane; ++j) {
    const uint64_t k = k0 + j;
    if (k < T && !row_eq(load_row(a + k), load_row(b + k), mask)) f |= 1u << j;
  }
  return f;
}

__global__ void __launch_bounds__(kBlock) diff_count(const sdc_row* __restrict__ a,
                                                     const sdc_row* __restrict__ b, uint64_t T,
                                                     uint32_t mask, unsigned long long* counts) {
  const uint64_t k0 = (uint64_t)blockIdx.x * kPerBlock + (uint64_t)threadIdx.x * kPerLane;
  uint32_t tot;
  block_exscan(__popc(lane_flags(a, b, T, mask, k0)), &tot);
  if (threadIdx.x == 0) counts[blockIdx.x] = tot;
}

__global__ void __launch_bounds__(kBlock) diff_scan(const unsigned long long* counts,
                                                    unsigned long long* offsets, uint64_t nb,
                                                    unsigned long long* n_diff) {
  // One workgroup; counts per block are at most kPerBlock, so 64-bit carries.
  __shared__ unsigned long long carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (uint64_t base = 0; base < nb; base += kBlock) {
    const uint64_t i = base + threadIdx.x;
    const uint32_t v = i < nb ? (uint32_t)counts[i] : 0u;
    uint32_t tot;
    const uint32_t ex = block_exscan(v, &tot);
    if (i < nb) offsets[i] = carry + ex;
    __syncthreads();
    if (threadIdx.x == 0) carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) *n_diff = carry;
}

// One differing row: its index and, when asked for, its flip localisation.
// Records are contiguous after the count, so one copy usually brings the
// whole answer to the host.
struct DiffRec {
  uint64_t index;
  sdc_flip_hint hint;
};
static_assert(sizeof(DiffRec) == 24, "diff record layout");

__device__ __forceinline__ void write_recs(const sdc_row* __restrict__ a,
                                           const sdc_row* __restrict__ b, uint64_t k0, uint32_t f,
                                           uint64_t pos, DiffRec* recs, bool hints, uint64_t cap) {
#pragma unroll
  for (uint32_t j = 0; j < kPerLane; ++j) {
    if (!(f & (1u << j))) continue;
    if (pos < cap) {
      const uint64_t k = k0 + j;
      recs[pos].index = k;
      if (hints) recs[pos].hint = flip_hint(load_row(a + k), load_row(b + k));
    }
    pos++;
  }
}

__global__ void __launch_bounds__(kBlock) diff_write(const sdc_row* __restrict__ a,
                                                     const sdc_row* __restrict__ b, uint64_t T,
                                                     uint32_t mask,
                                                     const unsigned long long* offsets,
                                                     DiffRec* recs, bool hints, uint64_t cap) {
  const uint64_t k0 = (uint64_t)blockIdx.x * kPerBlock + (uint64_t)threadIdx.x * kPerLane;
  const uint32_t f = lane_flags(a, b, T, mask, k0);
  uint32_t tot;
  const uint64_t pos = offsets[blockIdx.x] + block_exscan(__popc(f), &tot);
  write_recs(a, b, k0, f, pos, recs, hints, cap);
}

// Tables of at most one block's rows: count, offsets and records in one launch.
__global__ void __launch_bounds__(kBlock) diff_fused(const sdc_row* __restrict__ a,
                                                     const sdc_row* __restrict__ b, uint64_t T,
                                                     uint32_t mask, unsigned long long* n_diff,
                                                     DiffRec* recs, bool hints, uint64_t cap) {
  const uint64_t k0 = (uint64_t)threadIdx.x * kPerLane;
  const uint32_t f = lane_flags(a, b, T, mask, k0);
  uint32_t tot;
  const uint64_t pos = block_exscan(__popc(f), &tot);
  write_recs(a, b, k0, f, pos, recs, hints, cap);
  if (threadIdx.x == 0) *n_diff = tot;
}

// Workspace: [0, 8) the count, [16, 16 + 24 cap) the records, then the
// per-block counts and offsets of the multi-block pass.
struct DiffLayout {
  uint64_t nb, recs_off, counts_off, offsets_off, bytes;
};

// Records copied together with the count (a second copy only for more).
constexpr uint64_t kDiffInline = 16;

DiffLayout diff_layout(uint64_t T, uint64_t cap) {
  DiffLayout L;
  L.nb = (T + kPerBlock - 1) / kPerBlock;
  L.recs_off = 16;
  L.counts_off = (L.recs_off + cap * sizeof(DiffRec) + 255) / 256 * 256;
  L.offsets_off = L.counts_off + (L.nb * 8 + 255) / 256 * 256;
  L.bytes = L.offsets_off + (L.nb * 8 + 255) / 256 * 256;
  return L;
}

// ---- ring replay audit ----------------------------------------------------------
// Pair r compares the target's own result (row 0 of rank (r+offset) mod n)
// with the replayer's replay (row 1 of rank r); one workgroup per pair.
__device__ __forceinline__ uint32_t block_or(uint32_t v) {
  __shared__ uint32_t w[kWaves];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v |= __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) all |= w[i];
  return all;
}

__global__ void __launch_bounds__(kBlock) ring_compare_kernel(const uint64_t* __restrict__ table,
                                                              uint32_t n, uint64_t width,
                                                              uint32_t offset, uint8_t* flags) {
  const uint32_t r = blockIdx.x;
  const uint32_t t = (uint32_t)(((uint64_t)r + offset) % n);
  const uint64_t* own = table + ((uint64_t)t * 2 + 0) * width;
  const uint64_t* rep = table + ((uint64_t)r * 2 + 1) * width;
  uint32_t d = 0;
  for (uint64_t i = threadIdx.x; i < width; i += kBlock) d |= (own[i] != rep[i]);
  d = block_or(d);
  if (threadIdx.x == 0) flags[r] = (uint8_t)(d != 0);
}

// Equality of four vector pairs, one workgroup each: (witness, original),
// (witness, replay), (retry, original), (retry, witness).
__global__ void __launch_bounds__(kBlock) confirm_kernel(const uint64_t* __restrict__ witness,
                                                         const uint64_t* __restrict__ retry,
                                                         const uint64_t* __restrict__ original,
                                                         const uint64_t* __restrict__ replay,
                                                         uint64_t width, uint8_t* eq) {
  const uint64_t* a = blockIdx.x < 2 ? witness : retry;
  const uint64_t* b = (blockIdx.x & 1u) == 0 ? original : blockIdx.x == 1 ? replay : witness;
  uint32_t d = 0;
  for (uint64_t i = threadIdx.x; i < width; i += kBlock) d |= (a[i] != b[i]);
  d = block_or(d);
  if (threadIdx.x == 0) eq[blockIdx.x] = (uint8_t)(d == 0);
}

}  // namespace
}  // namespace sdc

using namespace sdc;

extern "C" int32_t sdc_ring_ws_bytes(uint32_t n, uint64_t* h_bytes) {
  if (h_bytes == nullptr) return SDC_ERR_INVALID;
  *h_bytes = ((uint64_t)(n < 16 ? 16 : n) + 255) / 256 * 256;
  return SDC_OK;
}

extern "C" int32_t sdc_ring_compare(const uint64_t* d_table, uint32_t n, uint64_t width,
                                    uint32_t offset, void* d_ws, uint64_t ws_bytes,
                                    uint8_t* h_mismatch, sdc_stream_t stream) {
  if (n == 0 || h_mismatch == nullptr || d_ws == nullptr || (width > 0 && d_table == nullptr))
    return SDC_ERR_INVALID;
  if (ws_bytes < n) return SDC_ERR_WORKSPACE;
  if (width >= (1ull << 56)) return SDC_ERR_RANGE;
  hipStream_t s = as_stream(stream);
  uint8_t* flags = reinterpret_cast<uint8_t*>(d_ws);
  hipLaunchKernelGGL(ring_compare_kernel, dim3(n), dim3(kBlock), 0, s, d_table, n, width, offset,
                     flags);
  int32_t st = launch_status();
  if (st) return st;
  if ((st = hip_status(hipMemcpyAsync(h_mismatch, flags, n, hipMemcpyDeviceToHost, s)))) return st;
  return hip_status(hipStreamSynchronize(s));
}

// Host decision over the mismatch flags (no HIP call): a rank in two or more
// mismatched pairs is a culprit; a mismatched pair without a culprit is
// ambiguous and goes to confirmation.
extern "C" int32_t sdc_ring_localize(const uint8_t* h_mismatch, uint32_t n, uint32_t offset,
                                     uint8_t* h_culprit, uint8_t* h_ambiguous) {
  if (n == 0 || h_mismatch == nullptr || h_culprit == nullptr || h_ambiguous == nullptr)
    return SDC_ERR_INVALID;
  std::vector<uint32_t> hits;
  try {
    hits.assign(n, 0u);
  } catch (...) {
    return SDC_ERR_RANGE;  // host allocation failed
  }
  for (uint32_t r = 0; r < n; ++r) {
    if (!h_mismatch[r]) continue;
    hits[(uint32_t)(((uint64_t)r + offset) % n)]++;
    hits[r]++;
  }
  for (uint32_t q = 0; q < n; ++q) h_culprit[q] = hits[q] >= 2;
  for (uint32_t r = 0; r < n; ++r) {
    const uint32_t t = (uint32_t)(((uint64_t)r + offset) % n);
    h_ambiguous[r] = h_mismatch[r] && !h_culprit[t] && !h_culprit[r];
  }
  return SDC_OK;
}

extern "C" int32_t sdc_confirm_verdict(const uint64_t* d_witness, const uint64_t* d_retry,
                                       const uint64_t* d_original, const uint64_t* d_replay,
                                       uint64_t width, void* d_ws, uint64_t ws_bytes,
                                       int32_t* h_verdict, sdc_stream_t stream) {
  if (h_verdict == nullptr || d_ws == nullptr ||
      (width > 0 && (!d_witness || !d_retry || !d_original || !d_replay)))
    return SDC_ERR_INVALID;
  if (ws_bytes < 16) return SDC_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  uint8_t* eq_d = reinterpret_cast<uint8_t*>(d_ws);
  hipLaunchKernelGGL(confirm_kernel, dim3(4), dim3(kBlock), 0, s, d_witness, d_retry, d_original,
                     d_replay, width, eq_d);
  int32_t st = launch_status();
  if (st) return st;
  uint8_t eq[4];
  if ((st = hip_status(hipMemcpyAsync(eq, eq_d, 4, hipMemcpyDeviceToHost, s)))) return st;
  if ((st = hip_status(hipStreamSynchronize(s)))) return st;
  const bool witness_is_original = eq[0], witness_is_replay = eq[1];
  const bool retry_is_original = eq[2], retry_is_witness = eq[3];
  // The verdict rows of [BLOG] "Decide what the alarm means", as conditions on
  // the four equalities.  The target was wrong when the witness sides with
  // the replayer (and not with the original).
  const bool target_wrong = witness_is_replay && !witness_is_original;
  if (target_wrong && retry_is_original)
    *h_verdict = SDC_VERDICT_PERSISTENT;  // reproduced its own wrong answer
  else if (target_wrong && retry_is_witness)
    *h_verdict = SDC_VERDICT_TRANSIENT;  // the retry came out right, as the witness
  else if (witness_is_original)
    *h_verdict = SDC_VERDICT_REPLAYER_WRONG;  // the witness reproduced the original
  else if (target_wrong)
    *h_verdict = SDC_VERDICT_UNCLEAR;  // the three do not line up
  else
    *h_verdict = SDC_VERDICT_UNATTRIBUTABLE;  // the witness agrees with neither side
  return SDC_OK;
}

extern "C" int32_t sdc_majority_ws_bytes(uint32_t R, uint64_t T, uint64_t* h_bytes) {
  if (h_bytes == nullptr || R == 0 || T == 0) return SDC_ERR_INVALID;
  *h_bytes = maj_ws_bytes(R);
  return SDC_OK;
}

extern "C" int32_t sdc_majority_compare(const sdc_row* d_table, uint32_t R, uint64_t T,
                                        uint32_t col_mask, void* d_ws, uint64_t ws_bytes,
                                        sdc_majority* h_res, uint8_t* h_suspect,
                                        uint8_t* d_tensor_status, sdc_stream_t stream) {
  if (d_table == nullptr || R == 0 || T == 0 || h_res == nullptr || h_suspect == nullptr ||
      d_ws == nullptr || !mask_ok(col_mask))
    return SDC_ERR_INVALID;
  if ((uint64_t)R * T / R != T || (uint64_t)R * T >= (1ull << 58)) return SDC_ERR_RANGE;
  if (ws_bytes < maj_ws_bytes(R)) return SDC_ERR_WORKSPACE;
  // host staging of the result and the flag bytes, allocated before anything is queued
  thread_local std::vector<unsigned char> stage;
  try {
    stage.resize(sizeof(sdc_majority) + R);
  } catch (...) {
    return SDC_ERR_RANGE;  // host allocation failed
  }
  hipStream_t s = as_stream(stream);
  unsigned char* base = reinterpret_cast<unsigned char*>(d_ws);
  MajWS* ws = reinterpret_cast<MajWS*>(base);
  uint8_t* sus8 = base + kMajSus8;
  uint32_t* sus = reinterpret_cast<uint32_t*>(base + maj_sus_off(R));
  int32_t st;
  if (R <= kMajFusedMaxR && T <= kMajFusedMaxT) {
    hipLaunchKernelGGL(maj_fused, dim3(1), dim3(kBlock), 0, s, d_table, R, T, col_mask, ws, sus8,
                       d_tensor_status);
    if ((st = launch_status())) return st;
  } else {
    const uint32_t gi = (uint32_t)std::min<uint64_t>((R + kBlock - 1) / kBlock, 1024);
    hipLaunchKernelGGL(maj_init, dim3(gi), dim3(kBlock), 0, s, ws, sus, R);
    if ((st = launch_status())) return st;
    const uint32_t gc = (uint32_t)std::min<uint64_t>((T + kBlock - 1) / kBlock, 4096);
    hipLaunchKernelGGL(maj_compare, dim3(gc), dim3(kBlock), 0, s, d_table, R, T, col_mask, ws, sus,
                       d_tensor_status);
    if ((st = launch_status())) return st;
    hipLaunchKernelGGL(maj_finalize, dim3(1), dim3(kBlock), 0, s, ws, sus, sus8, R);
    if ((st = launch_status())) return st;
  }
  // one copy of the result and the flag bytes, then split on the host
  if ((st = hip_status(hipMemcpyAsync(stage.data(), base + kMajOut, stage.size(),
                                      hipMemcpyDeviceToHost, s))))
    return st;
  if ((st = hip_status(hipStreamSynchronize(s)))) return st;
  std::memcpy(h_res, stage.data(), sizeof(sdc_majority));
  std::memcpy(h_suspect, stage.data() + sizeof(sdc_majority), R);
  return SDC_OK;
}

extern "C" int32_t sdc_diff_ws_bytes(uint64_t T, uint64_t idx_cap, uint64_t* h_bytes) {
  if (h_bytes == nullptr) return SDC_ERR_INVALID;
  if (T >= (1ull << 58) || idx_cap >= (1ull << 58)) return SDC_ERR_RANGE;
  *h_bytes = diff_layout(T, std::min(idx_cap, T)).bytes;  // at most T rows differ
  return SDC_OK;
}

extern "C" int32_t sdc_fingerprint_diff(const sdc_row* d_a, const sdc_row* d_b, uint64_t T,
                                        uint32_t col_mask, void* d_ws, uint64_t ws_bytes,
                                        uint64_t* h_n_diff, uint64_t* h_idx, uint64_t idx_cap,
                                        sdc_flip_hint* h_hints, sdc_stream_t stream) {
  if (h_n_diff == nullptr || !mask_ok(col_mask) || (idx_cap > 0 && h_idx == nullptr))
    return SDC_ERR_INVALID;
  if (T == 0) {
    *h_n_diff = 0;
    return SDC_OK;
  }
  if (d_a == nullptr || d_b == nullptr || d_ws == nullptr) return SDC_ERR_INVALID;
  if (T >= (1ull << 58) || idx_cap >= (1ull << 58)) return SDC_ERR_RANGE;
  const uint64_t cap = std::min(idx_cap, T);  // at most T rows differ
  const DiffLayout L = diff_layout(T, cap);
  if (ws_bytes < L.bytes) return SDC_ERR_WORKSPACE;
  if (L.nb > kMaxGrid) return SDC_ERR_RANGE;
  // host staging of the count and records, allocated before anything is queued
  thread_local std::vector<unsigned char> stage;
  try {
    stage.resize(L.recs_off + cap * sizeof(DiffRec));
  } catch (...) {
    return SDC_ERR_RANGE;  // host allocation failed
  }
  hipStream_t s = as_stream(stream);
  unsigned char* base = reinterpret_cast<unsigned char*>(d_ws);
  unsigned long long* n_diff = reinterpret_cast<unsigned long long*>(base);
  DiffRec* recs = reinterpret_cast<DiffRec*>(base + L.recs_off);
  const bool hints = h_hints != nullptr;
  int32_t st;
  if (L.nb == 1) {
    hipLaunchKernelGGL(diff_fused, dim3(1), dim3(kBlock), 0, s, d_a, d_b, T, col_mask, n_diff, recs,
                       hints, cap);
    if ((st = launch_status())) return st;
  } else {
    unsigned long long* counts = reinterpret_cast<unsigned long long*>(base + L.counts_off);
    unsigned long long* offsets = reinterpret_cast<unsigned long long*>(base + L.offsets_off);
    hipLaunchKernelGGL(diff_count, dim3((uint32_t)L.nb), dim3(kBlock), 0, s, d_a, d_b, T, col_mask,
                       counts);
    if ((st = launch_status())) return st;
    hipLaunchKernelGGL(diff_scan, dim3(1), dim3(kBlock), 0, s, counts, offsets, L.nb, n_diff);
    if ((st = launch_status())) return st;
    hipLaunchKernelGGL(diff_write, dim3((uint32_t)L.nb), dim3(kBlock), 0, s, d_a, d_b, T, col_mask,
                       offsets, recs, hints, cap);
    if ((st = launch_status())) return st;
  }
  // The count and the first records in one copy; the rest only if there are more.
  const uint64_t first = std::min(cap, kDiffInline);
  if ((st = hip_status(hipMemcpyAsync(stage.data(), base, L.recs_off + first * sizeof(DiffRec),
                                      hipMemcpyDeviceToHost, s))))
    return st;
  if ((st = hip_status(hipStreamSynchronize(s)))) return st;
  uint64_t n;
  std::memcpy(&n, stage.data(), 8);
  *h_n_diff = n;
  const uint64_t m = std::min(n, cap);
  if (m > first) {
    if ((st = hip_status(hipMemcpyAsync(stage.data() + L.recs_off + first * sizeof(DiffRec),
                                        base + L.recs_off + first * sizeof(DiffRec),
                                        (m - first) * sizeof(DiffRec), hipMemcpyDeviceToHost, s))))
      return st;
    if ((st = hip_status(hipStreamSynchronize(s)))) return st;
  }
  const DiffRec* r = reinterpret_cast<const DiffRec*>(stage.data() + L.recs_off);
  for (uint64_t i = 0; i < m; ++i) {
    h_idx[i] = r[i].index;
    if (hints) h_hints[i] = r[i].hint;
  }
  return SDC_OK;
}
