// Internal definitions of libsdc.so: device plan layout, launch constants and
// error plumbing.  Not part of the public ABI (that is include/sdc.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdc.h"

namespace sdc {

// Workgroup size of every scan kernel: 4 waves of 64 lanes.
constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
// Bytes of one coalesced vector load per lane.
constexpr uint32_t kVecBytes = 16;
// Largest work item.  Bounds the per-lane 32-bit accumulators of the 16-bit
// path: with U-way unrolling a lane sees at most kItemBytesMax / (16 * 256)
// = 1024 vectors of 8 elements, so sum_x < 2^29 and sum_(k x) < 2^31.
constexpr uint64_t kItemBytesMax = 4ull << 20;
// Automatic item size: aim at this many items, within [kAutoMin, kAutoMax].
constexpr uint64_t kAutoTargetItems = 16384;
constexpr uint64_t kAutoMin = 16ull << 10;
constexpr uint64_t kAutoMax = 1ull << 20;
constexpr uint64_t kMaxGrid = 0x7FFFFFFFull;

constexpr uint64_t kPlanMagic = 0x31766E6163534453ull;  // "SDScanv1", little-endian

// Item flags.
constexpr uint32_t kItemWhole = 1u;  // the item is the whole tensor: plain store, no clearing

// Device plan: [PlanHeader][PlanItem x n_items][uint32 row x n_zero].
struct PlanHeader {
  uint64_t magic;
  uint64_t n_tensors;
  uint64_t n_items;
  uint64_t n_zero;
  uint64_t items_off;
  uint64_t zero_off;
  uint64_t total_bytes;
  uint64_t item_bytes;
};
static_assert(sizeof(PlanHeader) == 64, "plan header layout");

// One work item: a contiguous element range of one tensor, scanned by one
// workgroup.  Self-contained so a workgroup needs a single scalar load.
struct PlanItem {
  uint64_t addr;   // device address of the item's first element
  uint64_t start;  // index of that element within its tensor
  uint32_t len;    // elements in the item
  uint32_t row;    // output row (tensor index in the list)
  uint32_t dtype;  // SDC_F32 / SDC_BF16 / SDC_F16
  uint32_t flags;  // kItemWhole
};
static_assert(sizeof(PlanItem) == 32, "plan item layout");

inline uint32_t element_size(uint32_t dtype) {
  return dtype == SDC_F32 ? 4u : (dtype == SDC_BF16 || dtype == SDC_F16) ? 2u : 0u;
}

// Thread-local record of the last failing HIP call.
void set_hip_error(hipError_t e);

inline int32_t hip_status(hipError_t e) {
  if (e == hipSuccess) return SDC_OK;
  set_hip_error(e);
  return SDC_ERR_HIP;
}

// Status of the kernels just enqueued (launch-configuration errors).
inline int32_t launch_status() { return hip_status(hipGetLastError()); }

inline hipStream_t as_stream(sdc_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace sdc
