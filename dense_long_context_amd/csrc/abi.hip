// ABI plumbing: status strings, the thread-local error message, launch checks
// and the workspace fill kernel.
#include "common.hpp"

#include <algorithm>
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

constexpr int kStages = 7;
static thread_local hipEvent_t g_armed[kStages][2] = {};

StageTimer::StageTimer(int stage, hipStream_t s) : stage_(stage), s_(s) {
  if (g_armed[stage_][0]) (void)hipEventRecord(g_armed[stage_][0], s_);
}

StageTimer::~StageTimer() {
  if (g_armed[stage_][1]) (void)hipEventRecord(g_armed[stage_][1], s_);
  g_armed[stage_][0] = g_armed[stage_][1] = nullptr;
}

__global__ void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (; i < n; i += stride) dst[i] = src[i];
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

int dlc_timing_arm(int stage, void* ev_begin, void* ev_end) {
  DLC_REQUIRE(stage >= 1 && stage < dlc::kStages, DLC_E_INVAL, "dlc_timing_arm: unknown stage %d", stage);
  dlc::g_armed[stage][0] = reinterpret_cast<hipEvent_t>(ev_begin);
  dlc::g_armed[stage][1] = reinterpret_cast<hipEvent_t>(ev_end);
  return DLC_OK;
}

int dlc_copy(void* dst, const void* src, size_t bytes, void* stream) {
  using namespace dlc;
  DLC_REQUIRE(dst && src, DLC_E_INVAL, "dlc_copy: NULL pointer");
  DLC_REQUIRE(bytes % 16 == 0 && aligned(dst, 16) && aligned(src, 16), DLC_E_INVAL,
              "dlc_copy: size and pointers must be 16-byte multiples");
  const int64_t n = int64_t(bytes / 16);
  if (n == 0) return DLC_OK;
  const int64_t blocks = std::min<int64_t>(ceil_div(n, 256), 256 * 32);
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
  return check_launch("dlc_copy");
}

}  // extern "C"
