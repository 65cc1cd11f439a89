// tensor.hip -- the fingerprint of ONE tensor without a plan, with an
// on-device compare against a stored row: the recompute check of the AEGIS
// review page ("Safeguarding LLM Training at Scale"), section "core method",
// item 4 (fingerprints of an original and of its deterministic
// recomputation, compared bit for bit), for gfx950.  The partial rows of the
// tensor's work items live in a caller workspace.
#include "tensor_device.h"

using namespace sdc;

extern "C" int32_t sdc_tensor_ws_bytes(const sdc_tensor* h_tensor, uint64_t item_bytes,
                                       uint64_t* h_bytes) {
  if (h_bytes == nullptr) return SDC_ERR_INVALID;
  uint64_t slots = 0;
  const int32_t st = tensor_slots_bound(h_tensor, item_bytes, &slots);
  if (st) return st;
  *h_bytes = slots * sizeof(sdc_row);
  return SDC_OK;
}

extern "C" int32_t sdc_tensor_split_host(const sdc_tensor* h_tensor, uint64_t item_bytes,
                                         uint32_t cu_count, uint64_t* h_n_items,
                                         uint64_t* h_item_bytes) {
  if (h_n_items == nullptr || h_item_bytes == nullptr || cu_count == 0) return SDC_ERR_INVALID;
  TensorShape sh;
  const int32_t st = tensor_shape(h_tensor, item_bytes, cu_count, &sh);
  if (st) return st;
  *h_n_items = sh.n_items;
  *h_item_bytes = sh.ie * sh.es;
  return SDC_OK;
}

extern "C" int32_t sdc_fingerprint_tensor(const sdc_tensor* h_tensor, uint64_t item_bytes, void* d_ws,
                                          uint64_t ws_bytes, const sdc_row* d_ref, uint32_t col_mask,
                                          sdc_row* d_out, uint32_t* d_mismatch, sdc_stream_t stream) {
  TensorShape sh;
  int32_t st = tensor_shape(h_tensor, item_bytes, kMaxSplitCus, &sh);  // argument checks first
  if (st) return st;
  if ((st = check_tensor_call(d_ref, col_mask, d_out, d_mismatch))) return st;
  if (d_ws == nullptr) return SDC_ERR_INVALID;
  DeviceShape dev;
  if ((st = current_device_shape(&dev))) return st;
  if ((st = tensor_shape(h_tensor, item_bytes, dev.cus, &sh))) return st;
  if (ws_bytes < std::max<uint64_t>(sh.n_items, 1) * sizeof(sdc_row)) return SDC_ERR_WORKSPACE;
  return launch_tensor(h_tensor, sh, reinterpret_cast<sdc_row*>(d_ws), d_ref, col_mask, d_out,
                       d_mismatch, as_stream(stream));
}
