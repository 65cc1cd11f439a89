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
constexpr uint64_t kAutoTargetItems = 65536;
constexpr uint64_t kAutoMin = 64ull << 10;
constexpr uint64_t kAutoMax = 1ull << 20;
constexpr uint64_t kMaxGrid = 0x7FFFFFFFull;

constexpr uint64_t kPlanMagic = 0x31766E6163534453ull;  // "SDScanv1", little-endian

// Wave items: a tensor whose aligned body is at most kWaveVecs vectors per
// lane of one wave (64 x 8 x 16 B = 8 KiB) is scanned whole by one wave, with
// every load of a lane issued at once and a wave-only reduction.
constexpr uint32_t kWaveVecs = 8;
constexpr uint32_t kWaveBodyVecs = 64 * kWaveVecs;

// Item flag: the item is the whole tensor, so it stores the tensor's row.
constexpr uint32_t kItemWhole = 1u << 8;
constexpr uint32_t kItemDtypeMask = 0xFFu;

// Device plan, all offsets from the plan's base:
//   [PlanHeader]
//   [PlanItem   x n_items]   n_items - n_small workgroup items, then n_small
//                            wave items
//   [PlanSplit  x n_split]   tensors not covered by exactly one item
//   (pad to 256)
//   [sdc_row    x n_slots]   partial rows of the items of split tensors
// The partial rows are scratch written by every scan with this plan.
struct PlanHeader {
  uint64_t magic;
  uint64_t n_tensors;
  uint64_t n_items;
  uint64_t n_split;
  uint64_t n_slots;
  uint64_t total_bytes;
  uint64_t item_bytes;
  uint64_t n_small;
};
static_assert(sizeof(PlanHeader) == 64, "plan header layout");

// One work item: a contiguous element range of one tensor, scanned by one
// workgroup.  Self-contained so a workgroup needs a single scalar load.
struct PlanItem {
  uint64_t addr;         // device address of the item's first element
  uint64_t start;        // index of that element within its tensor
  uint32_t len;          // elements in the item
  uint32_t row;          // output row (tensor index in the list)
  uint32_t slot;         // partial-row slot (split tensors only)
  uint32_t dtype_flags;  // SDC_F32 / SDC_BF16 / SDC_F16 | kItemWhole
};
static_assert(sizeof(PlanItem) == 32, "plan item layout");

// A tensor whose row is merged from `count` partial rows starting at slot
// `first` (count 0: a missing or empty tensor, row all zero).
struct PlanSplit {
  uint32_t row;
  uint32_t first;
  uint32_t count;
  uint32_t pad;
};
static_assert(sizeof(PlanSplit) == 16, "plan split layout");

struct PlanOffsets {
  uint64_t items, split, partials, end;
};

inline PlanOffsets plan_offsets(uint64_t n_items, uint64_t n_split, uint64_t n_slots) {
  PlanOffsets o;
  o.items = sizeof(PlanHeader);
  o.split = o.items + n_items * sizeof(PlanItem);
  o.partials = (o.split + n_split * sizeof(PlanSplit) + 255) / 256 * 256;
  o.end = o.partials + n_slots * sizeof(sdc_row);
  return o;
}

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
