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
//     U per lane in flight.  Lists of large items (>= 512 KiB on average) run
//     one workgroup per CU with 12 loads per lane per round; lists of smaller
//     items run 2-4 workgroups per CU with pipelined rounds.
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
//     result is bit-exact; no atomics).
//   * Small tensors (aligned body <= 8 KiB) are wave items instead: a group
//     of 64, 32, 16 or 8 lanes (the narrowest whose 8 vectors per lane hold
//     the body) scans one whole with all its loads in flight at once, so a
//     wave works on 1 to 8 of these latency-bound tensors together.
#include <algorithm>

#include "fingerprint_device.h"

namespace sdc {
namespace {

template <class Cfg>
__global__ void __launch_bounds__(kBlock) fingerprint_kernel(const PlanItem* __restrict__ items,
                                                             sdc_row* __restrict__ partials,
                                                             sdc_row* __restrict__ out,
                                                             uint32_t xcds) {
  const PlanItem it = items[xcd_item(blockIdx.x, gridDim.x, xcds)];
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

__global__ void __launch_bounds__(kBlock) fingerprint_small_kernel(const PlanItem* __restrict__ items,
                                                                   WaveLaunch w,
                                                                   sdc_row* __restrict__ out) {
  for_wave_item(w, [&](uint32_t i, uint32_t l, auto lanes) {
    const PlanItem it = items[i];
    Lane ln;
    dispatch_type(it.dtype_flags, [&](auto ty) {
      scan_small<decltype(ty), decltype(lanes)::value>(it, l, ln);
    });
    if (l != 0) return;
    ulonglong2* d = reinterpret_cast<ulonglong2*>(out + it.row);
    d[0] = ulonglong2{ln.s, ln.w};
    d[1] = ulonglong2{ln.x, ln.nf};
  });
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

int32_t launch_scan(const void* d_plan, const sdc_plan_info* h, sdc_row* out, hipStream_t s) {
  const PlanView v = view_of(d_plan, h);
  const uint64_t n_block = h->n_items - h->n_small;
  int32_t st;
  if (h->n_small) {
    const WaveLaunch w = wave_launch(h->n_wave);
    hipLaunchKernelGGL(fingerprint_small_kernel, dim3(w.group[kWaveClasses]), dim3(kBlock), 0, s,
                       v.items + n_block, w, out);
    if ((st = launch_status())) return st;
  }
  if (n_block) {
    DeviceShape dev;
    if ((st = current_device_shape(&dev))) return st;
    const dim3 grid((uint32_t)n_block), block(kBlock);
    switch (item_shape(h->total_bytes, h->n_items, kDeepItemBytes)) {
      case kShapeWide:
        hipLaunchKernelGGL(fingerprint_kernel<WideBody>, grid, block, kWideLdsBytes, s, v.items,
                           v.partials, out, dev.xcds);
        break;
      case kShapeDeep:
        hipLaunchKernelGGL(fingerprint_kernel<DeepBody>, grid, block, 0, s, v.items, v.partials, out,
                           dev.xcds);
        break;
      default:
        hipLaunchKernelGGL(fingerprint_kernel<DefaultBody>, grid, block, 0, s, v.items, v.partials,
                           out, dev.xcds);
    }
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

extern "C" int32_t sdc_fingerprint_ws_bytes(const sdc_tensor* h_tensors, uint64_t n,
                                            uint64_t* h_bytes) {
  return sdc_plan_bytes(h_tensors, n, 0, h_bytes);
}

extern "C" int32_t sdc_fingerprint(const sdc_tensor* h_tensors, uint64_t n, void* d_ws,
                                   uint64_t ws_bytes, sdc_row* d_out, sdc_stream_t stream) {
  sdc_plan_info info;
  int32_t st = sdc_plan_build(h_tensors, n, 0, d_ws, ws_bytes, &info, stream);
  if (st) return st;
  return sdc_fingerprint_plan(d_ws, &info, d_out, stream);
}
