// nonfinite.hip -- element-exact NaN/Inf counts per tensor over a scan plan
// (AWS Machine Learning Blog, "Detecting and recovering from silent data
// corruption on Amazon SageMaker HyperPod", section "Check 1"), for gfx950.
//
// Same items and traversal as the fingerprint scan, but only the fast
// "may hold NaN/Inf" flag is computed per lane; a lane whose flag is set
// after a round counts that round's vectors (still in registers) with the
// type's exact rule.  Raw integer tensors are never read.
#include "scan_device.h"

namespace sdc {
namespace {

// ---- NaN/Inf count only ----------------------------------------------------------
template <class Ty, int U, bool PIPE>
__device__ __forceinline__ uint32_t nonfinite_item(const PlanItem& it) {
  constexpr uint32_t es = Ty::ES;
  const uint32_t t = threadIdx.x;
  uint32_t c = 0;
  if constexpr (Ty::CHK != kChkNone) {  // raw integers are never NaN/Inf: nothing to read
    const Span sp = span_of<es>(it);
    const NfRule rule = nf_rule(it.dtype_flags & kItemDtypeMask);
    const ItemEnds<es> ends(sp, t);  // zero where the thread has none: never NaN/Inf
    if (sp.nvec) {
      const unsigned char* body = sp.base + (uint64_t)sp.h * es;
      Chk<Ty::CHK> chk(rule);
      stream_body<U, PIPE>(body, sp.nvec, [&](u32x4 v) { chk.add(v); },
                           [&](const u32x4 (&v)[U]) { count_flagged_round(chk, v, c); });
    }
    c += nf_exact(ends.head, rule) + nf_exact(ends.tail, rule);
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

template <int U, bool PIPE>
__global__ void __launch_bounds__(kBlock) nonfinite_kernel(const PlanItem* __restrict__ items,
                                                           sdc_row* __restrict__ partials,
                                                           uint64_t* __restrict__ counts,
                                                           uint64_t* __restrict__ total,
                                                           uint32_t xcds) {
  const PlanItem it = items[xcd_item(blockIdx.x, gridDim.x, xcds)];
  uint32_t c = 0;
  dispatch_type(it.dtype_flags & ~kItemSigned,
                [&](auto ty) { c = nonfinite_item<typename Unsigned<decltype(ty)>::type, U, PIPE>(it); });
  if (threadIdx.x != 0) return;
  if (counts) {
    if (it.dtype_flags & kItemWhole) counts[it.row] = c;
    else partials[it.slot].nonfinite = c;
  }
  // NaN/Inf are rare, so the total's atomics are too.
  if (c) atomicAdd(reinterpret_cast<unsigned long long*>(total), (unsigned long long)c);
}

template <class Ty, uint32_t LANES>
__device__ __forceinline__ uint32_t nonfinite_small(const PlanItem& it, uint32_t l) {
  constexpr uint32_t es = Ty::ES;
  uint32_t c = 0;
  if constexpr (Ty::CHK != kChkNone) {
    const Span sp = span_of<es>(it);
    const NfRule rule = nf_rule(it.dtype_flags & kItemDtypeMask);
    const WaveItemLoads<es, LANES> ld(sp, l);  // zero where the lane has nothing: never NaN/Inf
#pragma unroll
    for (uint32_t k = 0; k < ld.kHT; ++k) c += nf_exact(ld.head[k], rule) + nf_exact(ld.tail[k], rule);
    // the fast flag over the body vectors, and the exact count only if it is set
    Chk<Ty::CHK> chk(rule);
#pragma unroll
    for (uint32_t u = 0; u < kWaveVecs; ++u) chk.add(ld.v[u]);
    if (chk.flagged()) {
#pragma unroll
      for (uint32_t u = 0; u < kWaveVecs; ++u) c += chk.exact(ld.v[u]);
    }
  }
#pragma unroll
  for (uint32_t off = LANES / 2; off > 0; off >>= 1) c += __shfl_xor(c, off);
  return c;
}

__global__ void __launch_bounds__(kBlock) nonfinite_small_kernel(const PlanItem* __restrict__ items,
                                                                 WaveLaunch w,
                                                                 uint64_t* __restrict__ counts,
                                                                 uint64_t* __restrict__ total) {
  for_wave_item(w, [&](uint32_t i, uint32_t l, auto lanes) {
    const PlanItem it = items[i];
    uint32_t c = 0;
    dispatch_type(it.dtype_flags & ~kItemSigned, [&](auto ty) {
      c = nonfinite_small<typename Unsigned<decltype(ty)>::type, decltype(lanes)::value>(it, l);
    });
    if (l != 0) return;
    if (counts) counts[it.row] = c;
    if (c) atomicAdd(reinterpret_cast<unsigned long long*>(total), (unsigned long long)c);
  });
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
  for (uint32_t i0 = 0; i0 < sp.count; i0 += 64u * kMergeUnroll) {
    uint64_t v[kMergeUnroll];
#pragma unroll
    for (uint32_t u = 0; u < kMergeUnroll; ++u) {
      const uint32_t i = i0 + u * 64u + l;
      v[u] = (i < sp.count) ? partials[sp.first + i].nonfinite : 0u;
    }
#pragma unroll
    for (uint32_t u = 0; u < kMergeUnroll; ++u) c += v[u];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  if (l == 0) counts[sp.row] = c;
}

__global__ void clear_total_kernel(uint64_t* total) { *total = 0; }

}  // namespace
}  // namespace sdc

using namespace sdc;

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
    const WaveLaunch w = wave_launch(h_info->n_wave);
    hipLaunchKernelGGL(nonfinite_small_kernel, dim3(w.group[kWaveClasses]), dim3(kBlock), 0, s,
                       v.items + n_block, w, d_counts, d_total);
    if ((st = launch_status())) return st;
  }
  if (n_block) {
    DeviceShape dev;
    if ((st = current_device_shape(&dev))) return st;
    const dim3 grid((uint32_t)n_block), block(kBlock);
    switch (item_shape(h_info->total_bytes, h_info->n_items, kCheckDeepItemBytes)) {
      case kShapeWide:
        hipLaunchKernelGGL((nonfinite_kernel<kWideU, false>), grid, block, kWideLdsBytes, s, v.items,
                           v.partials, d_counts, d_total, dev.xcds);
        break;
      case kShapeDeep:
        hipLaunchKernelGGL((nonfinite_kernel<kCheckDeepU, true>), grid, block, 0, s, v.items,
                           v.partials, d_counts, d_total, dev.xcds);
        break;
      default:
        hipLaunchKernelGGL((nonfinite_kernel<kCheckU, true>), grid, block, 0, s, v.items, v.partials,
                           d_counts, d_total, dev.xcds);
    }
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

