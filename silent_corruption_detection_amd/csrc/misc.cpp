// misc.cpp -- status strings, last HIP error, ABI version.
#include "sdc_internal.h"

namespace sdc {
namespace {
thread_local int32_t g_last_hip_error = 0;
}
void set_hip_error(hipError_t e) { g_last_hip_error = (int32_t)e; }
}  // namespace sdc

extern "C" const char* sdc_status_string(int32_t status) {
  switch (status) {
    case SDC_OK: return "ok";
    case SDC_ERR_INVALID: return "invalid argument";
    case SDC_ERR_DTYPE: return "unknown element type";
    case SDC_ERR_ALIGN: return "tensor pointer not aligned to its element size";
    case SDC_ERR_WORKSPACE: return "plan or workspace buffer too small";
    case SDC_ERR_HIP: return "HIP runtime call failed";
    case SDC_ERR_PLAN: return "plan info does not describe a plan";
    case SDC_ERR_RANGE: return "size out of supported range";
    default: return "unknown status";
  }
}

extern "C" int32_t sdc_last_hip_error(void) { return sdc::g_last_hip_error; }

extern "C" uint32_t sdc_abi_version(void) { return SDC_ABI_VERSION; }
