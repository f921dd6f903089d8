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

constexpr int kStages = 8;
static thread_local hipEvent_t g_armed[kStages][2] = {};
static thread_local int g_depth[kStages] = {};

// Timers of one stage may nest (a call that runs the stage range by range
// times the whole of it): only the outermost records its events.
StageTimer::StageTimer(int stage, hipStream_t s) : stage_(stage), s_(s) {
  if (g_depth[stage_]++ == 0 && g_armed[stage_][0]) (void)hipEventRecord(g_armed[stage_][0], s_);
}

StageTimer::~StageTimer() {
  if (--g_depth[stage_] > 0) return;
  if (g_armed[stage_][1]) (void)hipEventRecord(g_armed[stage_][1], s_);
  g_armed[stage_][0] = g_armed[stage_][1] = nullptr;
}

bool take_stage_events(int stage, hipEvent_t* begin, hipEvent_t* end) {
  *begin = *end = nullptr;
  if (g_depth[stage] > 0 || !g_armed[stage][0] || !g_armed[stage][1]) return false;
  *begin = g_armed[stage][0];
  *end = g_armed[stage][1];
  g_armed[stage][0] = g_armed[stage][1] = nullptr;
  return true;
}

// Bandwidth reference: one 16-byte nontemporal load and store per thread and
// pass, a block per 4 KB, enough blocks to cover the buffer in one pass up to
// 2^20 blocks (then grid-strided).  Swept on a 1 GiB copy (loads in flight
// per thread 1, 2, 4, 8, 16; 1024 to 262144 blocks; plain or nontemporal
// accesses) this simplest form was the fastest: 6.5 TB/s of read + write
// bytes, against 5.4 for eight loads a thread on 2048 blocks.
constexpr int64_t kCopyMaxBlocks = int64_t(1) << 20;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Read-only bandwidth references, one per load form; nothing is written, and
// the counters of each calibrate the read counters of the kernels that load
// the same way.  Direct-to-LDS form (the FP4 indexer's key stream): each wave
// moves 1 KB per global_load_lds_dwordx4 straight into LDS (no register
// write), up to eight in flight in a ring of 1 KB slots, and every 1 KB of
// the source is loaded once.
__global__ void __launch_bounds__(256) read_lds_kernel(const unsigned char* src, int64_t n_kb) {
  constexpr int kSlots = 8;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[4][kSlots][1024];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lds = (uint32_t)(uintptr_t)DLC_LDS(&ring[wave][0][0]);
  const int64_t stride = int64_t(gridDim.x) * 4;
  int k = 0;
  for (int64_t i = int64_t(blockIdx.x) * 4 + wave; i < n_kb; i += stride, ++k) {
    if (k >= kSlots) wait_vm<kSlots - 1>();  // the load that last used this slot has landed
    dma_row(src + i * 1024, uint32_t(lane) * 16u, lds + uint32_t(k % kSlots) * 1024u);
  }
  wait_vm<0>();
}

// Register form in the bf16 indexer's MFMA operand pattern: the source is
// 16-row tiles of 256-byte rows; for each of its tiles (tiles interleaved
// over the grid's waves) lane l loads the 16 bytes at row l%16, byte
// 64*kt + 16*(l/16), for kt = 0..3, so one instruction covers 64 bytes of
// each of 16 rows.  The loaded words are folded together and handed to an
// empty asm statement, which keeps the loads without storing anything.
__global__ void __launch_bounds__(256) read_tiles_kernel(const unsigned char* src, int64_t n_tiles) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t stride = int64_t(gridDim.x) * 4;
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll 3
  for (int64_t t = int64_t(blockIdx.x) * 4 + wave; t < n_tiles; t += stride) {
    const unsigned char* row = src + (t * 16 + r16) * 256 + 16 * g;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) acc ^= *reinterpret_cast<const u32x4*>(row + 64 * kt);
  }
  asm volatile("" ::"v"(acc.x), "v"(acc.y), "v"(acc.z), "v"(acc.w));
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
  const int64_t blocks = std::min<int64_t>(ceil_div(n, 256), kCopyMaxBlocks);
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
  return check_launch("dlc_copy");
}

int dlc_read(const void* src, size_t bytes, int form, void* stream) {
  using namespace dlc;
  DLC_REQUIRE(src, DLC_E_INVAL, "dlc_read: NULL pointer");
  DLC_REQUIRE(form == DLC_READ_LDS || form == DLC_READ_TILES, DLC_E_INVAL, "dlc_read: unknown form %d", form);
  const size_t unit = form == DLC_READ_LDS ? 1024 : 4096;
  DLC_REQUIRE(bytes % unit == 0 && aligned(src, 16), DLC_E_INVAL,
              "dlc_read: size must be a multiple of %zu and the pointer 16-byte aligned", unit);
  const int64_t n = int64_t(bytes / unit);
  if (n == 0) return DLC_OK;
  hipEvent_t evb, eve;
  take_stage_events(DLC_STAGE_READ, &evb, &eve);
  if (form == DLC_READ_LDS) {
    const int64_t blocks = std::min<int64_t>(ceil_div(n, 4 * 32), 2048);
    hipExtLaunchKernelGGL(read_lds_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream), evb, eve, 0u,
                          static_cast<const unsigned char*>(src), n);
  } else {
    const int64_t blocks = std::min<int64_t>(ceil_div(n, 4), 768);
    hipExtLaunchKernelGGL(read_tiles_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream), evb, eve, 0u,
                          static_cast<const unsigned char*>(src), n);
  }
  return check_launch("dlc_read");
}

}  // extern "C"
