// tensor_device.h -- the scan of ONE tensor without a plan: its split into
// work items (computed from the workgroup index), the scan and merge/compare
// kernels, and their launch.  Shared by the entry points that take a
// caller workspace (tensor.hip) and the one that allocates nothing
// (noalloc.hip); each source instantiates its own copies of the kernels.
#pragma once

#include <algorithm>

#include "fingerprint_device.h"

namespace sdc {
namespace {

// The items of a single tensor follow from the workgroup index alone (the same
// split a plan makes): item 0 covers the misaligned head and the next ie
// elements, item i >= 1 the elements [h + i*ie, h + (i+1)*ie).  So the scan
// needs no plan upload and no host synchronisation.  Every item stores its
// partial row in slot i of a scratch area; one workgroup merges them.
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

// One workgroup: the tensor's row from its n partial rows; with a reference
// row, a difference under the mask adds 1 to *mismatch.
__global__ void __launch_bounds__(kBlock) merge_check_kernel(const sdc_row* __restrict__ partials,
                                                             uint32_t n, sdc_row* __restrict__ out,
                                                             const sdc_row* __restrict__ ref,
                                                             uint32_t mask,
                                                             uint32_t* __restrict__ mismatch) {
  Lane ln = merge_slots<kBlock>(partials, n, threadIdx.x);
  block_reduce(ln);
  if (threadIdx.x != 0) return;
  const sdc_row r{ln.s, ln.w, ln.x, ln.nf};
  ulonglong2* d = reinterpret_cast<ulonglong2*>(out);
  d[0] = ulonglong2{r.sum, r.wsum};
  d[1] = ulonglong2{r.xorsum, r.nonfinite};
  if (ref && rows_differ(r, *ref, mask)) atomicAdd(mismatch, 1u);
}

// Automatic item size of the single-tensor scan on a device with `cus`
// compute units.  A call scans one tensor, so the launch's start and tail
// weigh more than in a list scan.  Tensors of at least kTensorWideMin bytes
// are cut into a multiple of `cus` items (one item per CU per pass, at most
// kItemBytesMax each) and scanned in the tensor-wide shape: one workgroup per
// CU (LDS reservation), non-pipelined rounds of 8 vectors per lane.  Measured
// per call on bf16 activations (one MI355X, 256 CUs): 512 MiB 77.5 us
// (6.92 TB/s) against 82 us with ~1024 items of 512 KiB in the deep shape;
// 256 MiB 42.0 vs 44.1 us; 128 MiB 24.4 vs 26.2 us; 12 vectors per round
// 1-3 % slower, two items per CU 2-5 % slower.  Smaller tensors take about
// kTensorTargetItems items within [kAutoMin, kAutoMax] (measured on 512 MiB
// tensors in the deep shape: 64 KiB items 5.7 TB/s, 256 KiB 6.5, 512 KiB -
// 2 MiB 6.5-6.6, 4 MiB 5.6).  The split uses at most kMaxSplitCus CUs (the
// full MI355X), so workspace bounds hold on every gfx950 part.
constexpr uint64_t kMaxSplitCus = 256;
constexpr uint64_t kTensorWideMin = 128ull << 20;
constexpr uint64_t kTensorTargetItems = 1024;
typedef BodyCfg<8, false> TensorWideBody;

inline uint64_t round_4k(uint64_t b) { return (b + 4095) / 4096 * 4096; }

inline uint64_t split_cus(uint64_t cus) { return std::max<uint64_t>(1, std::min(cus, kMaxSplitCus)); }

inline uint64_t tensor_item_bytes(uint64_t bytes, uint64_t cus) {
  if (bytes >= kTensorWideMin) {
    const uint64_t c = split_cus(cus);
    const uint64_t passes = (bytes + c * kItemBytesMax - 1) / (c * kItemBytesMax);
    const uint64_t items = c * passes;
    return round_4k((bytes + items - 1) / items);  // <= kItemBytesMax, a multiple of 4 KiB
  }
  const uint64_t ib = round_4k(std::max<uint64_t>(bytes / kTensorTargetItems, 1));
  return ib < kAutoMin ? kAutoMin : (ib > kAutoMax ? kAutoMax : ib);
}

// Launch shape of the single-tensor scan: items, the split of item 0, and
// whether the items are few and large enough for the tensor-wide shape (at
// most two per CU of at least 512 KiB: what the automatic size gives tensors
// of 128 MiB - 1 GiB; larger ones, several passes of 4 MiB items, also take it).
struct TensorShape {
  uint64_t n_items, ie;
  uint32_t h, es;
  bool wide;
};

inline int32_t tensor_shape(const sdc_tensor* t, uint64_t item_bytes, uint64_t cus, TensorShape* sh) {
  if (t == nullptr) return SDC_ERR_INVALID;
  if (item_bytes % kVecBytes != 0 || item_bytes > kItemBytesMax) return SDC_ERR_INVALID;
  if ((t->flags & ~(uint32_t)SDC_FLAG_SIGNED) != 0) return SDC_ERR_INVALID;
  const uint32_t es = element_size(t->dtype);
  if (es == 0) return SDC_ERR_DTYPE;
  if (t->numel >= (1ull << 62) / es) return SDC_ERR_RANGE;  // bytes < 2^62
  const uint64_t numel = t->ptr ? t->numel : 0u;
  const uint64_t ptr = reinterpret_cast<uintptr_t>(t->ptr);
  if (ptr % es != 0) return SDC_ERR_ALIGN;
  const uint64_t ie = (item_bytes ? item_bytes : tensor_item_bytes(numel * es, cus)) / es;
  const uint64_t mis = ptr & 15u;
  const uint64_t h = mis ? std::min<uint64_t>(numel, (16u - mis) / es) : 0u;
  const uint64_t first = std::min<uint64_t>(numel, h + ie);
  sh->n_items = numel ? 1 + (numel - first + ie - 1) / ie : 0;
  if (sh->n_items > kMaxGrid) return SDC_ERR_RANGE;
  sh->ie = ie;
  sh->h = (uint32_t)h;
  sh->es = es;
  const uint64_t ib = ie * es;
  const uint64_t c = split_cus(cus);
  sh->wide = ib >= (512ull << 10) &&
             (sh->n_items <= 2 * c || (item_bytes == 0 && numel * es >= kTensorWideMin));
  return SDC_OK;
}

// Partial-row slots the scan of *t may use on any device: its item count for
// an explicit item size; with the automatic size, a bound over every CU count
// up to kMaxSplitCus (a wide split has at most c * passes + 1 <= bytes / 4 MiB
// + c + 1 items).  At least 1.
inline int32_t tensor_slots_bound(const sdc_tensor* t, uint64_t item_bytes, uint64_t* slots) {
  TensorShape sh;
  int32_t st = tensor_shape(t, item_bytes, kMaxSplitCus, &sh);
  if (st) return st;
  uint64_t n = sh.n_items;
  const uint64_t bytes = (t->ptr ? t->numel : 0u) * sh.es;
  if (item_bytes == 0 && bytes >= kTensorWideMin)
    n = std::max<uint64_t>(n, (bytes + kItemBytesMax - 1) / kItemBytesMax + kMaxSplitCus + 1);
  *slots = std::max<uint64_t>(n, 1);
  return SDC_OK;
}

// Argument checks shared by the single-tensor entry points (shape given).
inline int32_t check_tensor_call(const sdc_row* d_ref, uint32_t col_mask, const sdc_row* d_out,
                                 const uint32_t* d_mismatch) {
  if (d_out == nullptr) return SDC_ERR_INVALID;
  if (d_ref && (d_mismatch == nullptr || (col_mask & SDC_COL_ALL) == 0 ||
                (col_mask & ~(uint32_t)SDC_COL_ALL) != 0))
    return SDC_ERR_INVALID;
  return SDC_OK;
}

// Enqueues the scan (sh.n_items workgroups writing partials[0 .. n_items))
// and the merge/compare on s.
inline int32_t launch_tensor(const sdc_tensor* t, const TensorShape& sh, sdc_row* partials,
                             const sdc_row* d_ref, uint32_t col_mask, sdc_row* d_out,
                             uint32_t* d_mismatch, hipStream_t s) {
  int32_t st;
  if (sh.n_items) {
    TensorJob j;
    j.addr = reinterpret_cast<uintptr_t>(t->ptr);
    j.numel = t->numel;
    j.ie = sh.ie;
    j.h = sh.h;
    j.df = t->dtype | ((t->flags & SDC_FLAG_SIGNED) ? kItemSigned : 0u);
    j.es = sh.es;
    j.pad = 0;
    const dim3 grid((uint32_t)sh.n_items), block(kBlock);
    if (sh.wide)
      hipLaunchKernelGGL(fingerprint_tensor_kernel<TensorWideBody>, grid, block, kWideLdsBytes, s, j,
                         partials);
    else if (sh.ie * sh.es >= kDeepItemBytes)
      hipLaunchKernelGGL(fingerprint_tensor_kernel<DeepBody>, grid, block, 0, s, j, partials);
    else
      hipLaunchKernelGGL(fingerprint_tensor_kernel<DefaultBody>, grid, block, 0, s, j, partials);
    if ((st = launch_status())) return st;
  }
  hipLaunchKernelGGL(merge_check_kernel, dim3(1), dim3(kBlock), 0, s, partials,
                     (uint32_t)sh.n_items, d_out, d_ref, col_mask, d_mismatch);
  return launch_status();
}

}  // namespace
}  // namespace sdc
