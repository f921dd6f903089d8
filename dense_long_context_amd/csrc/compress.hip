// Token-level KV compressor: CSA (overlapping 2m windows) and HCA (m' windows).
//
// "DeepSeek-V4 Hybrid Attention: CSA and HCA from Scratch", §4-§5 (CSA) and
// §10 (HCA): every output column is its own softmax-weighted pooling of the
// window's rows.  A thread owns one (entry, group of columns) - a group is one
// 16-byte vector (8 bf16 or 4 fp32 columns) on the fast path and one column on
// the generic path - or, for calls with few entries, one slice of that pair's
// window rows.  Consecutive threads take consecutive column groups of the same
// rows, so a wave reads whole row segments, and each stream row is read once
// per entry that uses it.  The window is consumed in chunks of kChunk rows with
// an online softmax: all loads of a chunk are in flight together, the running
// max moves once per chunk, and the pass costs one exp per logit plus one per
// chunk, with no second pass over Z.
#include "pool_math.hpp"

namespace dlc {

namespace {

constexpr int kChunk = kPoolChunk;
// CSA entries per thread on the full-pass path (a window of 2m rows is only
// two chunks: one entry alone is too little work for a wave's start-up)
#ifndef DLC_POOL_EPT
#define DLC_POOL_EPT 2
#endif
constexpr int64_t kEntriesPerThread = DLC_POOL_EPT;
#ifndef DLC_NT_ENTRIES
#define DLC_NT_ENTRIES 1
#endif
constexpr bool kNtEntries = DLC_NT_ENTRIES != 0;
typedef unsigned int u32x4_pool __attribute__((ext_vector_type(4)));

struct PoolArgs {
  const void* Z[2];      // [0]: a-stream (HCA: its only stream), [1]: b-stream
  const void* C[2];
  const float* bias[2];  // [rows][c] fp32 or nullptr
  int64_t ld, batch_stride;
  int64_t c, m;          // width, window rows per segment (m or m')
  int64_t i_begin, n_entries;
  int64_t col_groups;
  int64_t ept;           // entries per thread (R = 1 path): consecutive entries, folded in turn
  void* out;
  int64_t cap;
};

template <typename T, int VEC>
__device__ __forceinline__ void load_cols(const T* p, int64_t j0, int64_t c, float* v) {
  if constexpr (VEC == 1) {
    v[0] = Fmt<T>::load(p + j0);
  } else {
    Fmt<T>::load_vec(p + j0, v);
  }
}

template <int VEC>
__device__ __forceinline__ void load_bias(const float* bias, int64_t r, int64_t c, int64_t j0, float* v) {
  if (bias == nullptr) {
#pragma unroll
    for (int u = 0; u < VEC; ++u) v[u] = 0.f;
  } else {
#pragma unroll
    for (int u = 0; u < VEC; ++u) v[u] = bias[r * c + j0 + u];
  }
}

// Window row rho of entry i: rho < m is row m*i + rho of the a-streams (bias
// row rho), m <= rho < 2m is row m*(i-1) + rho - m of the b-streams (bias row
// rho - m).  The window is cut into chunks of kChunk rows.  A chunk's partial
// softmax state is (max, sum, acc) with its weights taken against its own max;
// all its loads are in flight together, so a chunk costs one memory round trip.
template <typename T, int VEC>
__device__ __forceinline__ void chunk_partial(const PoolArgs& a, int64_t boff, int64_t i, int r0, int r1,
                                              int64_t j0, float* mx, float* sum, float* acc) {
  float l[kChunk][VEC], cv[kChunk][VEC];
#pragma unroll
  for (int rr = 0; rr < kChunk; ++rr) {
    const int rho = r0 + rr;
    if (rho < r1) {
      const int seg = rho >= a.m ? 1 : 0;
      const int64_t rb = seg ? rho - a.m : rho;  // row within the block (bias row)
      const int64_t row = a.m * (i - seg) + rb;
      const T* Z = static_cast<const T*>(a.Z[seg]) + boff + row * a.ld;
      const T* C = static_cast<const T*>(a.C[seg]) + boff + row * a.ld;
      float bv[VEC];
      load_cols<T, VEC>(Z, j0, a.c, l[rr]);
      load_cols<T, VEC>(C, j0, a.c, cv[rr]);
      load_bias<VEC>(a.bias[seg], rb, a.c, j0, bv);
#pragma unroll
      for (int u = 0; u < VEC; ++u) l[rr][u] = pool_logit(l[rr][u], bv[u]);
    }
  }
  chunk_fold<VEC>(l, cv, r1 - r0, mx, sum, acc);
}

// The entry's value is the left-to-right fold of its chunk partials.
// R = 1: a thread owns one (entry, column group) and folds its chunks in turn.
// R > 1 (calls with few entries): R adjacent lanes share one (entry, column
// group), lane q computes chunk q, and lane 0 folds them in order through lane
// shuffles - the same fold, so an entry has the same bits whichever way it was
// computed (an incremental decode call reproduces the full pass exactly).
// Thread t = ((e * col_groups + g) * R + q); consecutive column groups of the
// same rows sit in consecutive lanes, so a wave reads whole row segments.
template <typename T, int VEC, bool OVERLAP, int R>
__global__ void __launch_bounds__(256) pool_kernel(PoolArgs a) {
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t boff = int64_t(blockIdx.y) * a.batch_stride;
  auto store = [&](int64_t i, int64_t j0, const float* acc, const float* sum) {
    float o[VEC];
#pragma unroll
    for (int u = 0; u < VEC; ++u) o[u] = pool_value(acc[u], sum[u]);
    T* out = static_cast<T*>(a.out) + (int64_t(blockIdx.y) * a.cap + i) * a.c + j0;
    if constexpr (VEC == 1) {
      Fmt<T>::store(out, o[0]);
    } else if constexpr (kNtEntries) {
      // the entries are read by later calls only: nontemporal stores keep
      // them out of the L2 that the stream passes through
      alignas(16) T tmp[16 / sizeof(T)];
      Fmt<T>::store_vec(tmp, o);
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4_pool*>(tmp), reinterpret_cast<u32x4_pool*>(out));
    } else {
      Fmt<T>::store_vec(out, o);
    }
  };
  if constexpr (R == 1) {
    // thread (entry group, column group): entries ept*g .. ept*g + ept-1 in
    // turn (a wave still covers one entry's column groups at a time)
    const int64_t groups = ceil_div(a.n_entries, a.ept);
    if (t >= groups * a.col_groups) return;
    const int64_t eg = t / a.col_groups;
    const int64_t j0 = (t - eg * a.col_groups) * VEC;
    for (int64_t e = eg * a.ept; e < min(a.n_entries, (eg + 1) * a.ept); ++e) {
      const int64_t i = a.i_begin + e;
      const int rows = int((OVERLAP && i > 0) ? 2 * a.m : a.m);  // i = 0 has no b-rows
      float mx[VEC], sum[VEC], acc[VEC];
#pragma unroll
      for (int u = 0; u < VEC; ++u) { mx[u] = -INFINITY; sum[u] = 0.f; acc[u] = 0.f; }
      for (int r0 = 0; r0 < rows; r0 += kChunk) {
        float pm[VEC], ps[VEC], pa[VEC];
        chunk_partial<T, VEC>(a, boff, i, r0, min(rows, r0 + kChunk), j0, pm, ps, pa);
        merge_state<VEC>(mx, sum, acc, pm, ps, pa);
      }
      store(i, j0, acc, sum);
    }
  } else {
    const int q = int(t % R);
    const int64_t eg = t / R;
    const bool live = eg < a.n_entries * a.col_groups;
    const int64_t e = live ? eg / a.col_groups : 0;
    const int64_t j0 = (eg - e * a.col_groups) * VEC;
    const int64_t i = a.i_begin + e;
    const int rows = int((OVERLAP && i > 0) ? 2 * a.m : a.m);  // i = 0 has no b-rows
    float mx[VEC], sum[VEC], acc[VEC];
    {
      float pm[VEC], ps[VEC], pa[VEC];
      const int r0 = q * kChunk;
      if (live && r0 < rows) {
        chunk_partial<T, VEC>(a, boff, i, r0, min(rows, r0 + kChunk), j0, pm, ps, pa);
      } else {
#pragma unroll
        for (int u = 0; u < VEC; ++u) { pm[u] = -INFINITY; ps[u] = 0.f; pa[u] = 0.f; }
      }
#pragma unroll
      for (int u = 0; u < VEC; ++u) { mx[u] = -INFINITY; sum[u] = 0.f; acc[u] = 0.f; }
      const int base = int(threadIdx.x & 63) & ~(R - 1);  // lane of chunk 0
#pragma unroll 1
      for (int k = 0; k < R; ++k) {
        float km[VEC], ks[VEC], ka[VEC];
#pragma unroll
        for (int u = 0; u < VEC; ++u) {
          km[u] = __shfl(pm[u], base + k);
          ks[u] = __shfl(ps[u], base + k);
          ka[u] = __shfl(pa[u], base + k);
        }
        merge_state<VEC>(mx, sum, acc, km, ks, ka);
      }
    }
    if (!live || q != 0) return;
    store(i, j0, acc, sum);
  }
}

template <typename T, int VEC, int R>
int launch_pool_r(PoolArgs a, bool overlap, int64_t B, hipStream_t s) {
  a.ept = R == 1 && overlap ? kEntriesPerThread : 1;
  const int64_t threads = (R == 1 ? ceil_div(a.n_entries, a.ept) : a.n_entries) * a.col_groups * R;
  const int64_t blocks = ceil_div(threads, 256);
  DLC_REQUIRE(blocks < (int64_t(1) << 31) && B <= 65535, DLC_E_UNSUPPORTED, "compress: grid too large");
  dim3 grid{(unsigned)blocks, (unsigned)B, 1u};
  StageTimer timer(DLC_STAGE_COMPRESS, s);
  if (overlap)
    hipLaunchKernelGGL((pool_kernel<T, VEC, true, R>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((pool_kernel<T, VEC, false, R>), grid, dim3(256), 0, s, a);
  return check_launch("compress");
}

// fewer than this many (entry, column group) pairs over all sequences: split rows
constexpr int64_t kSmallLaunch = 1 << 16;

template <typename T, int VEC>
int launch_pool(PoolArgs a, bool overlap, int64_t B, hipStream_t s) {
  // a few entries: one lane per chunk of window rows, if the window has at most 32 chunks
  const int64_t chunks = ceil_div((overlap ? 2 : 1) * a.m, int64_t(kChunk));
  if (a.n_entries * a.col_groups * B < kSmallLaunch && chunks <= 32) {
    if (chunks <= 2) return launch_pool_r<T, VEC, 2>(a, overlap, B, s);
    if (chunks <= 4) return launch_pool_r<T, VEC, 4>(a, overlap, B, s);
    if (chunks <= 8) return launch_pool_r<T, VEC, 8>(a, overlap, B, s);
    if (chunks <= 16) return launch_pool_r<T, VEC, 16>(a, overlap, B, s);
    return launch_pool_r<T, VEC, 32>(a, overlap, B, s);
  }
  return launch_pool_r<T, VEC, 1>(a, overlap, B, s);
}

int pool_dispatch(const char* name, int dtype, int64_t B, int64_t n, int64_t c, int64_t m,
                  const void* Z0, const void* Z1, const void* C0, const void* C1, int64_t ld,
                  int64_t batch_stride, const float* b0, const float* b1, int64_t i_begin,
                  int64_t i_end, void* out, int64_t cap, bool overlap, void* stream) {
  DLC_REQUIRE(dtype == DLC_F32 || dtype == DLC_BF16, DLC_E_DTYPE, "%s: unsupported dtype %d", name, dtype);
  DLC_REQUIRE(B >= 1 && n >= 0 && c >= 1 && m >= 1, DLC_E_INVAL,
              "%s: need B >= 1, n >= 0, c >= 1, m >= 1 (got B=%lld n=%lld c=%lld m=%lld)", name,
              (long long)B, (long long)n, (long long)c, (long long)m);
  DLC_REQUIRE(Z0 && C0 && out && (!overlap || (Z1 && C1)), DLC_E_INVAL, "%s: NULL stream or output", name);
  DLC_REQUIRE(ld >= c, DLC_E_SHAPE, "%s: ld (%lld) < c (%lld)", name, (long long)ld, (long long)c);
  DLC_REQUIRE(B == 1 || n == 0 || batch_stride >= (n - 1) * ld + c, DLC_E_SHAPE,
              "%s: batch_stride %lld overlaps rows of the next sequence", name, (long long)batch_stride);
  DLC_REQUIRE(0 <= i_begin && i_begin <= i_end && i_end <= n / m, DLC_E_SHAPE,
              "%s: need 0 <= i_begin <= i_end <= n/m (got %lld, %lld, n/m=%lld)", name,
              (long long)i_begin, (long long)i_end, (long long)(n / m));
  DLC_REQUIRE(cap >= i_end, DLC_E_SHAPE, "%s: cap %lld < i_end %lld", name, (long long)cap, (long long)i_end);
  if (i_end == i_begin) return DLC_OK;

  PoolArgs a{};
  a.Z[0] = Z0; a.Z[1] = Z1; a.C[0] = C0; a.C[1] = C1;
  a.bias[0] = b0; a.bias[1] = b1;
  a.ld = ld; a.batch_stride = batch_stride; a.c = c; a.m = m;
  a.i_begin = i_begin; a.n_entries = i_end - i_begin; a.out = out; a.cap = cap;
  hipStream_t s = as_stream(stream);

  const size_t esz = dtype == DLC_BF16 ? 2 : 4;
  const int vec = dtype == DLC_BF16 ? 8 : 4;
  bool vec_ok = (c % vec == 0) && (ld % vec == 0) && (B == 1 || batch_stride % vec == 0);
  for (const void* p : {Z0, C0, (const void*)out}) vec_ok = vec_ok && aligned(p, 16);
  if (overlap) vec_ok = vec_ok && aligned(Z1, 16) && aligned(C1, 16);
  (void)esz;
  if (vec_ok) {
    a.col_groups = c / vec;
    return dtype == DLC_BF16 ? launch_pool<bf16_raw, 8>(a, overlap, B, s)
                             : launch_pool<float, 4>(a, overlap, B, s);
  }
  a.col_groups = c;
  return dtype == DLC_BF16 ? launch_pool<bf16_raw, 1>(a, overlap, B, s)
                           : launch_pool<float, 1>(a, overlap, B, s);
}

}  // namespace
}  // namespace dlc

extern "C" {

int csa_compress(int dtype, int64_t B, int64_t n, int64_t c, int64_t m, const void* Za, const void* Zb,
                 const void* Ca, const void* Cb, int64_t ld, int64_t batch_stride, const float* Ba,
                 const float* Bb, int64_t i_begin, int64_t i_end, void* Ccomp, int64_t cap, void* stream) {
  return dlc::pool_dispatch("csa_compress", dtype, B, n, c, m, Za, Zb, Ca, Cb, ld, batch_stride, Ba, Bb,
                            i_begin, i_end, Ccomp, cap, true, stream);
}

int hca_compress(int dtype, int64_t B, int64_t n, int64_t c, int64_t m_prime, const void* Z, const void* C,
                 int64_t ld, int64_t batch_stride, const float* Bias, int64_t i_begin, int64_t i_end,
                 void* Chca, int64_t cap, void* stream) {
  return dlc::pool_dispatch("hca_compress", dtype, B, n, c, m_prime, Z, nullptr, C, nullptr, ld,
                            batch_stride, Bias, nullptr, i_begin, i_end, Chca, cap, false, stream);
}

}  // extern "C"
