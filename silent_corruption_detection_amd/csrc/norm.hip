// norm.hip -- per-tensor squared norms over a scan plan, the norm form of
// the NaN/Inf check (AWS Machine Learning Blog, "Detecting and recovering
// from silent data corruption on Amazon SageMaker HyperPod", section
// "Check 1"), for gfx950.
#include "scan_device.h"

namespace sdc {
namespace {

// ---- squared norm (the norm-based check) --------------------------------------------
// Element values decoded exactly (every format here converts to double without
// rounding), squared and summed in double in a fixed order: per lane, a
// workgroup item's body vectors in index order and then its head and tail
// element, a wave item's head and tail elements and then its body vectors;
// then fixed shuffle / LDS trees, partial slots in slot order, and one
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

template <class Dt, int U, bool PIPE>
__device__ __forceinline__ double sq_item(const PlanItem& it) {
  constexpr uint32_t DT = Dt::DTYPE, es = dt_size<DT>();
  const Span sp = span_of<es>(it);
  const uint32_t t = threadIdx.x;
  const ItemEnds<es> ends(sp, t);  // zero where the thread has none: fma(0, 0, acc) is acc
  double acc = 0.0;
  // lane t adds its vectors t, t + 256, t + 512, ... in that order, whatever
  // the round depth and pipelining, then its head and its tail element
  if (sp.nvec)
    stream_body<U, PIPE>(sp.base + (uint64_t)sp.h * es, sp.nvec,
                         [&](u32x4 v) { acc = sq_vec<DT>(v, acc); });
  const double y = value_of<DT>(ends.head), z = value_of<DT>(ends.tail);
  acc = __builtin_fma(y, y, acc);
  acc = __builtin_fma(z, z, acc);
  return acc;
}

template <int U, bool PIPE>
__global__ void __launch_bounds__(kBlock) sqnorm_kernel(const PlanItem* __restrict__ items,
                                                        sdc_row* __restrict__ partials,
                                                        double* __restrict__ sq,
                                                        uint32_t xcds) {
  const PlanItem it = items[xcd_item(blockIdx.x, gridDim.x, xcds)];
  double acc = 0.0;
  dispatch_dtype(it.dtype_flags, [&](auto dt) { acc = sq_item<decltype(dt), U, PIPE>(it); });
  acc = block_sum_d(acc);
  if (threadIdx.x != 0) return;
  if (it.dtype_flags & kItemWhole) sq[it.row] = acc;
  else partials[it.slot].sum = (uint64_t)__double_as_longlong(acc);
}

template <class Dt, uint32_t LANES>
__device__ __forceinline__ double sq_small(const PlanItem& it, uint32_t l) {
  constexpr uint32_t DT = Dt::DTYPE, es = dt_size<DT>();
  const Span sp = span_of<es>(it);
  // zero where the lane has nothing: fma(0, 0, acc) is acc exactly
  const WaveItemLoads<es, LANES> ld(sp, l);
  double acc = 0.0;
#pragma unroll
  for (uint32_t k = 0; k < ld.kHT; ++k) {
    const double y = value_of<DT>(ld.head[k]), z = value_of<DT>(ld.tail[k]);
    acc = __builtin_fma(y, y, acc);
    acc = __builtin_fma(z, z, acc);
  }
#pragma unroll
  for (uint32_t u = 0; u < kWaveVecs; ++u) acc = sq_vec<DT>(ld.v[u], acc);
#pragma unroll
  for (uint32_t off = LANES / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  return acc;
}

__global__ void __launch_bounds__(kBlock) sqnorm_small_kernel(const PlanItem* __restrict__ items,
                                                              WaveLaunch w, double* __restrict__ sq) {
  for_wave_item(w, [&](uint32_t i, uint32_t l, auto lanes) {
    const PlanItem it = items[i];
    double acc = 0.0;
    dispatch_dtype(it.dtype_flags, [&](auto dt) {
      acc = sq_small<decltype(dt), decltype(lanes)::value>(it, l);
    });
    if (l == 0) sq[it.row] = acc;
  });
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
  for (uint32_t i0 = 0; i0 < sp.count; i0 += 64u * kMergeUnroll) {
    double v[kMergeUnroll];
#pragma unroll
    for (uint32_t u = 0; u < kMergeUnroll; ++u) {
      const uint32_t i = i0 + u * 64u + l;
      v[u] = (i < sp.count) ? __longlong_as_double((long long)partials[sp.first + i].sum) : 0.0;
    }
#pragma unroll
    for (uint32_t u = 0; u < kMergeUnroll; ++u) acc += v[u];
  }
  acc = wave_sum_d(acc);
  if (l == 0) sq[sp.row] = acc;
}

// Total over all tensors in a fixed order, and the decision: the squared sum
// rounded to fp32 is not finite.
// Sum of src[0..n) in a fixed order: thread t adds entries t, t + 256, ...,
// then the fixed workgroup tree.
__device__ __forceinline__ double ordered_sum(const double* __restrict__ src, uint64_t n) {
  double acc = 0.0;
  for (uint64_t k = threadIdx.x; k < n; k += kBlock) acc += src[k];
  return block_sum_d(acc);
}

// Chunk c of the tensors' squared sums (kSqChunk tensors) -> chunks[c].
__global__ void __launch_bounds__(kBlock) sq_chunk_kernel(const double* __restrict__ sq, uint64_t n,
                                                          double* __restrict__ chunks) {
  const uint64_t first = (uint64_t)blockIdx.x * kSqChunk;
  const double acc = ordered_sum(sq + first, min(n - first, kSqChunk));
  if (threadIdx.x == 0) chunks[blockIdx.x] = acc;
}

// The total from the tensors' sums (one chunk) or from the chunk sums, and
// the decision: the squared sum rounded to fp32 is not finite.
__global__ void __launch_bounds__(kBlock) sq_total_kernel(const double* __restrict__ src, uint64_t n,
                                                          double* __restrict__ total,
                                                          uint32_t* __restrict__ flag) {
  const double acc = ordered_sum(src, n);
  if (threadIdx.x == 0) {
    *total = acc;
    if (flag) *flag = !__builtin_isfinite((float)acc);
  }
}

}  // namespace
}  // namespace sdc

using namespace sdc;

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
    const WaveLaunch w = wave_launch(h_info->n_wave);
    hipLaunchKernelGGL(sqnorm_small_kernel, dim3(w.group[kWaveClasses]), dim3(kBlock), 0, s,
                       v.items + n_block, w, d_sq);
    if ((st = launch_status())) return st;
  }
  if (n_block) {
    DeviceShape dev;
    if ((st = current_device_shape(&dev))) return st;
    const dim3 grid((uint32_t)n_block), block(kBlock);
    switch (item_shape(h_info->total_bytes, h_info->n_items, kCheckDeepItemBytes)) {
      case kShapeWide:
        hipLaunchKernelGGL((sqnorm_kernel<kWideU, false>), grid, block, kWideLdsBytes, s, v.items,
                           v.partials, d_sq, dev.xcds);
        break;
      case kShapeDeep:
        hipLaunchKernelGGL((sqnorm_kernel<kCheckDeepU, true>), grid, block, 0, s, v.items, v.partials,
                           d_sq, dev.xcds);
        break;
      default:
        hipLaunchKernelGGL((sqnorm_kernel<kCheckU, true>), grid, block, 0, s, v.items, v.partials,
                           d_sq, dev.xcds);
    }
    if ((st = launch_status())) return st;
  }
  if (h_info->n_split) {
    hipLaunchKernelGGL(merge_sq_kernel, dim3((uint32_t)((h_info->n_split + kWaves - 1) / kWaves)),
                       dim3(kBlock), 0, s, v.split, (uint32_t)h_info->n_split, v.partials, d_sq);
    if ((st = launch_status())) return st;
  }
  // The total in a fixed order: over the tensors directly when they fit one
  // chunk, else over the chunk sums (the order depends on the plan only).
  const uint64_t n_chunks = (h_info->n_tensors + kSqChunk - 1) / kSqChunk;
  if (n_chunks > 1) {
    hipLaunchKernelGGL(sq_chunk_kernel, dim3((uint32_t)n_chunks), dim3(kBlock), 0, s, d_sq,
                       h_info->n_tensors, v.chunks);
    if ((st = launch_status())) return st;
    hipLaunchKernelGGL(sq_total_kernel, dim3(1), dim3(kBlock), 0, s, v.chunks, n_chunks, d_total,
                       d_flag);
  } else {
    hipLaunchKernelGGL(sq_total_kernel, dim3(1), dim3(kBlock), 0, s, d_sq, h_info->n_tensors,
                       d_total, d_flag);
  }
  return launch_status();
}
