// plan.cpp -- host side of the scan plan: splitting a tensor list into
// self-contained work items (workgroup items, then wave items by class), the
// split-tensor table and partial-row slots, and the one host-to-device copy.
#include <algorithm>
#include <cstring>
#include <vector>

#include "sdc_internal.h"

namespace sdc {
namespace {

// ---- host side: plan layout --------------------------------------------------
struct Layout {
  uint64_t n_items = 0, n_small = 0, n_split = 0, n_slots = 0, total_elems = 0, total_bytes = 0;
  uint64_t n_wave[kWaveClasses] = {0, 0, 0, 0};
  uint64_t item_bytes = 0;
  PlanOffsets off{};
};

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

uint64_t items_of(uint64_t ptr, uint64_t numel, uint32_t es, uint64_t item_bytes) {
  const uint64_t mis = ptr & 15u;
  const uint64_t h = mis ? std::min<uint64_t>(numel, (16u - mis) / es) : 0u;
  const uint64_t ie = item_bytes / es;
  const uint64_t first = std::min<uint64_t>(numel, h + ie);
  return 1 + (numel - first + ie - 1) / ie;
}

bool has_data(const sdc_tensor& t) { return t.ptr != nullptr && t.numel != 0; }

// Wave-item class of a tensor: -1 = workgroup item(s); c = 0..3 = scanned
// whole by 64 >> c lanes.  A wave item is a single item anyway, and its
// aligned body fits the group's kWaveVecs vectors per lane (the narrowest
// group that fits).
constexpr int kClassBlock = -1;

int wave_class(uint64_t ptr, uint64_t numel, uint32_t es, uint64_t item_bytes) {
  if (items_of(ptr, numel, es, item_bytes) != 1) return kClassBlock;
  const uint64_t mis = ptr & 15u;
  const uint64_t h = mis ? std::min<uint64_t>(numel, (16u - mis) / es) : 0u;
  const uint64_t body = (numel - h) * es / kVecBytes;
  for (int c = kWaveClasses - 1; c >= 0; --c)
    if (body <= class_body_vecs((uint32_t)c)) return c;
  return kClassBlock;
}

int32_t layout_plan(const sdc_tensor* t, uint64_t n, uint64_t item_bytes, Layout* L) {
  if (n > 0 && t == nullptr) return SDC_ERR_INVALID;
  if (n >= (1ull << 31)) return SDC_ERR_RANGE;
  if (item_bytes % kVecBytes != 0 || item_bytes > kItemBytesMax) return SDC_ERR_INVALID;
  uint64_t elems = 0, bytes = 0;
  for (uint64_t k = 0; k < n; ++k) {
    if ((t[k].flags & ~(uint32_t)SDC_FLAG_SIGNED) != 0) return SDC_ERR_INVALID;
    const uint32_t es = element_size(t[k].dtype);
    if (es == 0) return SDC_ERR_DTYPE;
    if (!has_data(t[k])) continue;
    if (t[k].numel >= (1ull << 62) / es) return SDC_ERR_RANGE;  // bytes < 2^62: no overflow below
    if (reinterpret_cast<uintptr_t>(t[k].ptr) % es != 0) return SDC_ERR_ALIGN;
    elems += t[k].numel;
    bytes += t[k].numel * es;
  }
  if (item_bytes == 0) {
    // items per candidate size kAutoMax >> c, counted in one pass
    constexpr int kCand = 5;  // 1 MiB .. 64 KiB
    static_assert((kAutoMax >> (kCand - 1)) == kAutoMin, "candidate sizes");
    uint64_t cnt[kCand] = {0, 0, 0, 0, 0};
    for (uint64_t k = 0; k < n; ++k) {
      if (!has_data(t[k])) continue;
      const uint64_t ptr = reinterpret_cast<uintptr_t>(t[k].ptr);
      const uint32_t es = element_size(t[k].dtype);
      for (int c = 0; c < kCand; ++c)  // saturating: each term is below 2^62
        cnt[c] = std::min<uint64_t>(cnt[c] + items_of(ptr, t[k].numel, es, kAutoMax >> c), 1ull << 62);
    }
    item_bytes = kAutoMin;
    for (int c = 0; c < kCand; ++c)
      if (cnt[c] >= kAutoMinItems) {
        item_bytes = kAutoMax >> c;
        break;
      }
  }
  uint64_t items = 0, small = 0, split = 0, slots = 0;
  uint64_t nw[kWaveClasses] = {0, 0, 0, 0};
  for (uint64_t k = 0; k < n; ++k) {
    if (!has_data(t[k])) {
      split++;
      continue;
    }
    const uint64_t ptr = reinterpret_cast<uintptr_t>(t[k].ptr);
    const uint32_t es = element_size(t[k].dtype);
    const uint64_t c = items_of(ptr, t[k].numel, es, item_bytes);
    items += c;
    if (items > kMaxGrid) return SDC_ERR_RANGE;  // before the running sum could wrap
    const int wc = wave_class(ptr, t[k].numel, es, item_bytes);
    if (wc != kClassBlock) {
      small++;
      nw[wc]++;
    }
    if (c > 1) {
      split++;
      slots += c;
    }
  }
  if (items > kMaxGrid || slots >= (1ull << 32)) return SDC_ERR_RANGE;
  L->n_items = items;
  L->n_small = small;
  for (uint32_t c = 0; c < kWaveClasses; ++c) L->n_wave[c] = nw[c];
  L->n_split = split;
  L->n_slots = slots;
  L->total_elems = elems;
  L->total_bytes = bytes;
  L->item_bytes = item_bytes;
  L->off = plan_offsets(items, split, slots, n);
  return SDC_OK;
}

// Host image of the plan (the partial-row slots are left uninitialised).
// Workgroup items come first, then wave items; each group is in list order
// and in address order within a tensor.
void pack_plan(const sdc_tensor* t, uint64_t n, const Layout& L, std::vector<unsigned char>& img) {
  img.assign(L.off.partials, 0);
  PlanHeader* hd = reinterpret_cast<PlanHeader*>(img.data());
  hd->magic = kPlanMagic;
  hd->n_tensors = n;
  hd->n_items = L.n_items;
  hd->n_split = L.n_split;
  hd->n_slots = L.n_slots;
  hd->total_bytes = L.total_bytes;
  hd->item_bytes = L.item_bytes;
  hd->n_small = L.n_small;
  PlanItem* items = reinterpret_cast<PlanItem*>(img.data() + L.off.items);
  PlanSplit* split = reinterpret_cast<PlanSplit*>(img.data() + L.off.split);
  // next free index of the workgroup items and of each wave-item class
  uint64_t ni = 0, ns = 0, slot = 0;
  uint64_t wi[kWaveClasses + 1];
  wi[0] = L.n_items - L.n_small;
  for (uint32_t c = 0; c < kWaveClasses; ++c) wi[c + 1] = wi[c] + L.n_wave[c];
  const uint64_t class_start[kWaveClasses + 1] = {wi[0], wi[1], wi[2], wi[3], wi[4]};
  for (uint64_t k = 0; k < n; ++k) {
    if (!has_data(t[k])) {
      split[ns++] = PlanSplit{(uint32_t)k, 0u, 0u, 0u};
      continue;
    }
    const uint32_t es = element_size(t[k].dtype);
    const uint64_t ptr = reinterpret_cast<uintptr_t>(t[k].ptr);
    const uint64_t c = items_of(ptr, t[k].numel, es, L.item_bytes);
    const uint32_t whole = (c == 1) ? kItemWhole : 0u;
    const int wc = wave_class(ptr, t[k].numel, es, L.item_bytes);
    if (c > 1) split[ns++] = PlanSplit{(uint32_t)k, (uint32_t)slot, (uint32_t)c, 0u};
    split_tensor(ptr, t[k].numel, es, L.item_bytes, [&](uint64_t s, uint64_t len) {
      PlanItem& it = items[wc == kClassBlock ? ni++ : wi[wc]++];
      it.addr = ptr + s * es;
      it.start = s;
      it.len = (uint32_t)len;
      it.row = (uint32_t)k;
      it.slot = whole ? 0u : (uint32_t)slot++;
      it.dtype_flags = t[k].dtype | whole | ((t[k].flags & SDC_FLAG_SIGNED) ? kItemSigned : 0u);
    });
  }
  // Each group of wave items ordered by element type: the lanes of a wave
  // then mostly take the same path through the type dispatch instead of one
  // after the other.
  const auto by_type = [](const PlanItem& a, const PlanItem& b) {
    return (a.dtype_flags & (kItemDtypeMask | kItemSigned)) <
           (b.dtype_flags & (kItemDtypeMask | kItemSigned));
  };
  for (uint32_t c = 0; c < kWaveClasses; ++c)
    std::stable_sort(items + class_start[c], items + class_start[c + 1], by_type);
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
  *h_bytes = L.off.end;
  return SDC_OK;
}

extern "C" int32_t sdc_plan_build(const sdc_tensor* h_tensors, uint64_t n, uint64_t item_bytes,
                                  void* d_plan, uint64_t plan_bytes, sdc_plan_info* h_info,
                                  sdc_stream_t stream) {
  if (d_plan == nullptr || h_info == nullptr) return SDC_ERR_INVALID;
  Layout L;
  int32_t st = layout_plan(h_tensors, n, item_bytes, &L);
  if (st) return st;
  if (plan_bytes < L.off.end) return SDC_ERR_WORKSPACE;
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
  h_info->n_small = L.n_small;
  for (uint32_t c = 0; c < kWaveClasses; ++c) h_info->n_wave[c] = L.n_wave[c];
  h_info->n_split = L.n_split;
  h_info->n_slots = L.n_slots;
  h_info->total_elems = L.total_elems;
  h_info->total_bytes = L.total_bytes;
  h_info->plan_bytes = L.off.end;
  h_info->item_bytes = L.item_bytes;
  return SDC_OK;
}

extern "C" int32_t sdc_plan_pack_host(const sdc_tensor* h_tensors, uint64_t n, uint64_t item_bytes,
                                      void* h_plan, uint64_t plan_bytes, sdc_plan_info* h_info) {
  if (h_plan == nullptr || h_info == nullptr) return SDC_ERR_INVALID;
  Layout L;
  int32_t st = layout_plan(h_tensors, n, item_bytes, &L);
  if (st) return st;
  if (plan_bytes < L.off.partials) return SDC_ERR_WORKSPACE;
  std::vector<unsigned char> img;
  try {
    pack_plan(h_tensors, n, L, img);
  } catch (...) {
    return SDC_ERR_RANGE;
  }
  std::memcpy(h_plan, img.data(), img.size());
  h_info->magic = kPlanMagic;
  h_info->n_tensors = n;
  h_info->n_items = L.n_items;
  h_info->n_small = L.n_small;
  for (uint32_t c = 0; c < kWaveClasses; ++c) h_info->n_wave[c] = L.n_wave[c];
  h_info->n_split = L.n_split;
  h_info->n_slots = L.n_slots;
  h_info->total_elems = L.total_elems;
  h_info->total_bytes = L.total_bytes;
  h_info->plan_bytes = L.off.end;
  h_info->item_bytes = L.item_bytes;
  return SDC_OK;
}

