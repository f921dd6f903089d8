// ABI plumbing: status strings, the thread-local error message, launch checks
// and the workspace fill kernel.
#include "common.hpp"

#include <cstring>

namespace dlc {

static thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DLC_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return DLC_OK;
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (; i < n; i += stride) p[i] = v;
}

int fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return DLC_OK;
  int64_t blocks = ceil_div(n, 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, p, v, n);
  return check_launch("fill");
}

}  // namespace dlc

extern "C" {

int dlc_abi_version(void) { return DLC_ABI_VERSION; }

const char* dlc_status_str(int status) {
  switch (status) {
    case DLC_OK: return "DLC_OK";
    case DLC_E_INVAL: return "DLC_E_INVAL";
    case DLC_E_DTYPE: return "DLC_E_DTYPE";
    case DLC_E_SHAPE: return "DLC_E_SHAPE";
    case DLC_E_WORKSPACE: return "DLC_E_WORKSPACE";
    case DLC_E_HIP: return "DLC_E_HIP";
    case DLC_E_UNSUPPORTED: return "DLC_E_UNSUPPORTED";
    default: return "DLC_E_UNKNOWN";
  }
}

const char* dlc_last_error(void) { return dlc::g_last_error; }

}  // extern "C"
