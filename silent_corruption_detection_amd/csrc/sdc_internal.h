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
// Largest work item.  Bounds the per-lane 32-bit accumulators of the 1- and
// 2-byte paths: a lane sees at most kItemBytesMax / (16 * 256) = 1024 vectors,
// so for 16-bit elements |sum x| < 2^29 and |sum k x| < 2^31, for bytes
// sum x < 2^23 and sum k x < 2^25.
constexpr uint64_t kItemBytesMax = 4ull << 20;
// Automatic item size of a list scan: the largest power of two in
// [kAutoMin, kAutoMax] whose split still gives at least kAutoMinItems work
// items (else kAutoMin).  Large items split fewer tensors (fewer workgroups
// and partial rows to merge); enough items keep every CU busy to the end.
// Measured per list (ms): 3 x 100k small tensors 64 KiB-class 0.83 vs 1 MiB
// 0.785; 0.96B fp32 gradients 116 KiB 1.148 vs 128 KiB 1.086 vs 1 MiB 1.187;
// the 70B bf16 list flat within 1 % from 256 KiB to 1 MiB.
constexpr uint64_t kAutoMinItems = 49152;
constexpr uint64_t kAutoMin = 64ull << 10;
constexpr uint64_t kAutoMax = 1ull << 20;
constexpr uint64_t kMaxGrid = 0x7FFFFFFFull;

constexpr uint64_t kPlanMagic = 0x31766E6163534453ull;  // "SDScanv1", little-endian

// Wave items: small tensors scanned whole by a group of 64 >> c lanes of a
// wave (class c = 0..3: 64, 32, 16 or 8 lanes), kWaveVecs vectors per lane,
// every load of a lane issued at once, and a reduction within the group.
// Class c takes bodies of at most (64 >> c) x 8 vectors (8, 4, 2, 1 KiB) and
// puts 1 << c tensors in a wave: small tensors are latency-bound, so narrower
// groups keep more loads in flight at the same register cost.
constexpr uint32_t kWaveVecs = 8;
constexpr uint32_t kWaveClasses = 4;
constexpr uint32_t class_lanes(uint32_t c) { return 64u >> c; }
constexpr uint32_t class_body_vecs(uint32_t c) { return class_lanes(c) * kWaveVecs; }

// Item flags: the item is the whole tensor, so it stores the tensor's row;
// the tensor's 2-/4-byte patterns are sign-extended (SDC_FLAG_SIGNED).
constexpr uint32_t kItemWhole = 1u << 8;
constexpr uint32_t kItemSigned = 1u << 9;
constexpr uint32_t kItemDtypeMask = 0xFFu;

// Device plan, all offsets from the plan's base:
//   [PlanHeader]
//   [PlanItem   x n_items]   n_items - n_small workgroup items, then the
//                            n_small wave items, class 0 to 3 (n_wave[c]
//                            each)
//   [PlanSplit  x n_split]   tensors not covered by exactly one item
//   (pad to 256)
//   [sdc_row    x n_slots]   partial rows of the items of split tensors
//   [double     x ceil(n_tensors / kSqChunk)]   chunk sums of the squared norm
// The partial rows and chunk sums are scratch written by the scans.
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
  uint32_t dtype_flags;  // SDC_* element type | kItemWhole | kItemSigned
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

// Tensors per partial sum of the ordered squared-norm total.
constexpr uint64_t kSqChunk = 4096;

struct PlanOffsets {
  uint64_t items, split, partials, chunks, end;
};

inline PlanOffsets plan_offsets(uint64_t n_items, uint64_t n_split, uint64_t n_slots,
                                uint64_t n_tensors) {
  PlanOffsets o;
  o.items = sizeof(PlanHeader);
  o.split = o.items + n_items * sizeof(PlanItem);
  o.partials = (o.split + n_split * sizeof(PlanSplit) + 255) / 256 * 256;
  o.chunks = o.partials + n_slots * sizeof(sdc_row);
  o.end = o.chunks + (n_tensors + kSqChunk - 1) / kSqChunk * sizeof(double);
  return o;
}

inline uint32_t element_size(uint32_t dtype) {
  switch (dtype) {
    case SDC_F32: case SDC_U32: return 4;
    case SDC_BF16: case SDC_F16: case SDC_U16: return 2;
    case SDC_F64: case SDC_U64: return 8;
    case SDC_U8: case SDC_FP8_E4M3: case SDC_FP8_E5M2: case SDC_FP8_E4M3FNUZ:
    case SDC_FP8_E5M2FNUZ: return 1;
    default: return 0;
  }
}

// Shape of the device a call runs on (csrc/device.cpp): its compute units and
// XCDs.  Work splits that aim at "one item per CU" use `cus`; the list scans'
// workgroup-to-item map uses `xcds`.  gfx950 XCDs hold kCusPerXcd active CUs.
constexpr uint32_t kCusPerXcd = 32;
struct DeviceShape {
  uint32_t cus, xcds;
};
uint32_t xcds_of(uint32_t cus);
// Shape of the calling thread's current device (queried once per device).
int32_t current_device_shape(DeviceShape* out);

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

// Host-side check that a plan info describes a plan image, and views of the
// image's parts.
inline bool info_ok(const sdc_plan_info* h) {
  if (h == nullptr || h->magic != kPlanMagic || h->n_items > kMaxGrid ||
      h->n_split > h->n_tensors || h->n_small > h->n_items)
    return false;
  uint64_t w = 0;
  for (uint32_t c = 0; c < kWaveClasses; ++c) w += h->n_wave[c];
  if (w != h->n_small) return false;
  return h->plan_bytes >= plan_offsets(h->n_items, h->n_split, h->n_slots, h->n_tensors).end;
}

struct PlanView {
  const PlanItem* items;
  const PlanSplit* split;
  sdc_row* partials;
  double* chunks;
};

inline PlanView view_of(const void* d_plan, const sdc_plan_info* h) {
  unsigned char* base = reinterpret_cast<unsigned char*>(const_cast<void*>(d_plan));
  const PlanOffsets o = plan_offsets(h->n_items, h->n_split, h->n_slots, h->n_tensors);
  return PlanView{reinterpret_cast<const PlanItem*>(base + o.items),
                  reinterpret_cast<const PlanSplit*>(base + o.split),
                  reinterpret_cast<sdc_row*>(base + o.partials),
                  reinterpret_cast<double*>(base + o.chunks)};
}


}  // namespace sdc
