// Shared device helpers and host-side validation for the gfx950 kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "dlc.h"

namespace dlc {

// ----------------------------------------------------------------------------
// host side: error reporting
// ----------------------------------------------------------------------------

int fail(int status, const char* fmt, ...);       // records a thread-local message
int check_launch(const char* what);               // DLC_OK or DLC_E_HIP after a launch

#define DLC_REQUIRE(cond, status, ...) \
  do {                                 \
    if (!(cond)) return ::dlc::fail((status), __VA_ARGS__); \
  } while (0)

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ----------------------------------------------------------------------------
// device side: number formats
// ----------------------------------------------------------------------------

typedef uint16_t bf16_raw;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// fp32 -> bf16, round to nearest, ties to even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <typename T> struct Fmt;
template <> struct Fmt<float> {
  static constexpr int kVec = 4;  // elements per 16-byte load
  __device__ static float load(const float* p) { return *p; }
  __device__ static void store(float* p, float v) { *p = v; }
  __device__ static void load_vec(const float* p, float* v) {
    float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
  __device__ static void store_vec(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct Fmt<bf16_raw> {
  static constexpr int kVec = 8;
  __device__ static float load(const bf16_raw* p) { return bf16_to_f32(*p); }
  __device__ static void store(bf16_raw* p, float v) { *p = f32_to_bf16(v); }
  __device__ static void load_vec(const bf16_raw* p, float* v) {
    uint4 x = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static void store_vec(bf16_raw* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = uint32_t(f32_to_bf16(v[2 * i])) | (uint32_t(f32_to_bf16(v[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// Order-preserving map of an fp32 score to uint32: a larger score gives a
// larger key, and -0.0 maps to the key of +0.0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Reductions over the four 16-lane rows of a wave (lanes l%16 + 16*r,
// r = 0..3): v_permlane16_swap / v_permlane32_swap exchange whole rows between
// two copies of the value, so combining the two results pairs every lane with
// its partner 16 (then 32) lanes away.  Plain VALU, unlike ds_bpermute, which
// queues behind LDS reads.  The sum adds (row0 + row1) + (row2 + row3).
// Inclusive prefix sum over the 64 lanes of a wave in six DPP adds: row_shr
// 1, 2, 4, 8 within each 16-lane row, then row_bcast:15 (row r's last lane
// into row r+1, rows 1 and 3) and row_bcast:31 (lane 31 into rows 2 and 3).
// Lanes without a source add the old value 0.  The whole wave must be active.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x111, 0xf, 0xf, false));  // row_shr:1
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x112, 0xf, 0xf, false));  // row_shr:2
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x114, 0xf, 0xf, false));  // row_shr:4
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x118, 0xf, 0xf, false));  // row_shr:8
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x142, 0xa, 0xf, false));  // row_bcast:15
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x143, 0xc, 0xf, false));  // row_bcast:31
  return v;
}
// the wave's total of an inclusive scan (lane 63)
__device__ __forceinline__ uint32_t wave_total(uint32_t incl) {
  return uint32_t(__builtin_amdgcn_readlane(int(incl), 63));
}

__device__ __forceinline__ float rows4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// LDS pointer of a __shared__ object (address space 3)
#define DLC_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// One direct global->LDS load (global_load_lds_dwordx4): every active lane i
// moves the 16 bytes at base + lane_off to LDS byte address lds_addr + 16*i.
// base and lds_addr are wave-uniform (SGPRs), lane_off a per-lane unsigned
// byte offset.  Issued through asm so the compiler does not fold it into its
// own wait bookkeeping (it would drain every load in flight before each LDS
// read); the caller waits for it with an explicit s_waitcnt vmcnt.  The
// instruction writes no VGPR.
__device__ __forceinline__ void dma_row(const void* base, uint32_t lane_off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(lane_off), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}

// The same with 4 bytes per lane (global_load_lds_dword): active lane i moves
// the dword at base + lane_off to LDS byte address lds_addr + 4*i.
__device__ __forceinline__ void dma_dword(const void* base, uint32_t lane_off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(lane_off), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Values that cross workgroups within one kernel are written and read with
// agent-scope atomic accesses, which this chip performs at the point of
// coherence of all its L2 caches (global_store / global_load with sc1): once
// a wave's stores have completed (vmcnt 0), another workgroup's atomic loads
// see them, with no L2 write-back or invalidation, whichever XCD it runs on.
template <typename T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup barrier that waits only for LDS and scalar-memory operations:
// __syncthreads would also drain every vector-memory load in flight (the
// direct global->LDS loads of the next tiles).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left at their maxima
  __builtin_amdgcn_s_barrier();
}

// Records the caller's armed events around a stage's launches (see
// dlc_timing_arm); a no-op unless armed.
class StageTimer {
 public:
  StageTimer(int stage, hipStream_t s);
  ~StageTimer();
 private:
  int stage_;
  hipStream_t s_;
};

// For a stage that is a single kernel launch: hands over the armed events of
// `stage` (and disarms it) so that the caller binds them to that kernel's own
// dispatch (hipExtLaunchKernelGGL).  They then time the kernel alone, where
// events recorded around the launch also take in its dispatch latency.
// Returns false, events null, when the stage is not armed or one of its
// timers is open.
bool take_stage_events(int stage, hipEvent_t* begin, hipEvent_t* end);

// fill kernel: clears workspace on the stream (no memset nodes, so the calls
// stay safe to capture in a graph)
__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n);
int fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s);

}  // namespace dlc
