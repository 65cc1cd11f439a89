// noalloc.hip -- sdc_fingerprint_tensor_noalloc: the single-tensor scan of
// sdc_fingerprint_tensor (tensor_device.h) for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The partial rows of the tensor's work items go to a
// static device array instead of a caller workspace; nothing is allocated.
#include <mutex>

#include "tensor_device.h"

// Partial-row scratch of the scans made through this entry point: one array
// per GPU (every device the library runs on holds its copy until the process
// ends).  Each call's items write their slots before its merge reads them, so
// nothing needs clearing between calls; calls that overlap in time on one GPU
// share it and race.
constexpr uint64_t kScratchRows = 8192;  // 256 KiB of sdc_row
static __device__ __align__(256) sdc_row scratch[kScratchRows];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
sdc_row* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch`, per device

// Device address of this device's `scratch`, looked up once per device with
// that device current.  (The array's name in host code is a host-side handle,
// not a device address: only this pointer may reach a kernel.)
int32_t scratch_of_current_device(sdc_row** out) {
  int dev = 0;
  int32_t st = sdc::hip_status(hipGetDevice(&dev));
  if (st) return st;
  if (dev < 0 || dev >= kMaxScratchDevices) return SDC_ERR_RANGE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if ((st = sdc::hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))))) return st;
    if (p == nullptr) return SDC_ERR_HIP;
    g_scratch_ptr[dev] = reinterpret_cast<sdc_row*>(p);
  }
  *out = g_scratch_ptr[dev];
  return SDC_OK;
}

}  // namespace

using namespace sdc;

extern "C" int32_t sdc_fingerprint_tensor_noalloc(const sdc_tensor* h_tensor, uint64_t item_bytes,
                                                  const sdc_row* d_ref, uint32_t col_mask,
                                                  sdc_row* d_out, uint32_t* d_mismatch,
                                                  sdc_stream_t stream) {
  uint64_t slots = 0;  // argument checks, and the size limit on any device, before any HIP call
  int32_t st = tensor_slots_bound(h_tensor, item_bytes, &slots);
  if (st) return st;
  if ((st = check_tensor_call(d_ref, col_mask, d_out, d_mismatch))) return st;
  if (slots > kScratchRows) return SDC_ERR_RANGE;
  DeviceShape dev;
  if ((st = current_device_shape(&dev))) return st;
  TensorShape sh;
  if ((st = tensor_shape(h_tensor, item_bytes, dev.cus, &sh))) return st;
  if (sh.n_items > kScratchRows) return SDC_ERR_RANGE;  // cannot happen: slots bounds it
  sdc_row* rows = nullptr;
  if ((st = scratch_of_current_device(&rows))) return st;
  return launch_tensor(h_tensor, sh, rows, d_ref, col_mask, d_out, d_mismatch, as_stream(stream));
}
