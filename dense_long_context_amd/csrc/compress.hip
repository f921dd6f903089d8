// Token-level KV compressor: CSA (overlapping 2m windows) and HCA (m' windows).
//
// "DeepSeek-V4 Hybrid Attention: CSA and HCA from Scratch", §4-§5 (CSA) and
// §10 (HCA): every output column is its own softmax-weighted pooling of the
// window's rows.  One thread owns one (entry, group of columns); a group is
// one 16-byte vector (8 bf16 or 4 fp32 columns) on the fast path and one
// column on the generic path.  Each stream row is read exactly once per entry
// that uses it, with consecutive threads on consecutive columns, so a wave
// reads whole rows.  The window is consumed in chunks of kChunk rows with an
// online softmax: the running max moves once per chunk, so the pass costs one
// exp per logit plus one per chunk, with no second pass over Z.
#include "common.hpp"

namespace dlc {

namespace {

constexpr int kChunk = 8;
constexpr float kLog2e = 1.4426950408889634f;

struct PoolArgs {
  const void* Z[2];      // [0]: a-stream (HCA: its only stream), [1]: b-stream
  const void* C[2];
  const float* bias[2];  // [rows][c] fp32 or nullptr
  int64_t ld, batch_stride;
  int64_t c, m;          // width, window rows per segment (m or m')
  int64_t i_begin, n_entries;
  int64_t col_groups;
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

// One window segment: rows row0 .. row0+m-1 of (Z, C) with bias rows 0 .. m-1.
template <typename T, int VEC>
__device__ __forceinline__ void pool_segment(const T* Z, const T* C, const float* bias, int64_t row0,
                                             const PoolArgs& a, int64_t j0, float* mx, float* sum,
                                             float* acc) {
  for (int64_t r0 = 0; r0 < a.m; r0 += kChunk) {
    float l[kChunk][VEC];
    const int rows = int(a.m - r0 < kChunk ? a.m - r0 : kChunk);
#pragma unroll
    for (int rr = 0; rr < kChunk; ++rr) {
      if (rr < rows) {
        float z[VEC], bv[VEC];
        load_cols<T, VEC>(Z + (row0 + r0 + rr) * a.ld, j0, a.c, z);
        load_bias<VEC>(bias, r0 + rr, a.c, j0, bv);
#pragma unroll
        for (int u = 0; u < VEC; ++u) l[rr][u] = (z[u] + bv[u]) * kLog2e;
      }
    }
    // move the running max once for the whole chunk
#pragma unroll
    for (int u = 0; u < VEC; ++u) {
      float cm = mx[u];
#pragma unroll
      for (int rr = 0; rr < kChunk; ++rr)
        if (rr < rows) cm = fmaxf(cm, l[rr][u]);
      if (cm > mx[u]) {
        const float f = (mx[u] == -INFINITY) ? 0.f : exp2f(mx[u] - cm);
        sum[u] *= f;
        acc[u] *= f;
        mx[u] = cm;
      }
    }
#pragma unroll
    for (int rr = 0; rr < kChunk; ++rr) {
      if (rr < rows) {
        float cv[VEC];
        load_cols<T, VEC>(C + (row0 + r0 + rr) * a.ld, j0, a.c, cv);
#pragma unroll
        for (int u = 0; u < VEC; ++u) {
          const float w = (l[rr][u] == -INFINITY) ? 0.f : exp2f(l[rr][u] - mx[u]);
          sum[u] += w;
          acc[u] = fmaf(w, cv[u], acc[u]);
        }
      }
    }
  }
}

template <typename T, int VEC, bool OVERLAP>
__global__ void __launch_bounds__(256) pool_kernel(PoolArgs a) {
  const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (tid >= a.n_entries * a.col_groups) return;
  const int64_t e = tid / a.col_groups;
  const int64_t j0 = (tid - e * a.col_groups) * VEC;
  const int64_t i = a.i_begin + e;
  const int64_t boff = int64_t(blockIdx.y) * a.batch_stride;

  float mx[VEC], sum[VEC], acc[VEC];
#pragma unroll
  for (int u = 0; u < VEC; ++u) { mx[u] = -INFINITY; sum[u] = 0.f; acc[u] = 0.f; }

  pool_segment<T, VEC>(static_cast<const T*>(a.Z[0]) + boff, static_cast<const T*>(a.C[0]) + boff,
                       a.bias[0], a.m * i, a, j0, mx, sum, acc);
  if (OVERLAP && i > 0)
    pool_segment<T, VEC>(static_cast<const T*>(a.Z[1]) + boff, static_cast<const T*>(a.C[1]) + boff,
                         a.bias[1], a.m * (i - 1), a, j0, mx, sum, acc);

  float o[VEC];
#pragma unroll
  for (int u = 0; u < VEC; ++u) o[u] = acc[u] / sum[u];
  T* out = static_cast<T*>(a.out) + (int64_t(blockIdx.y) * a.cap + i) * a.c + j0;
  if constexpr (VEC == 1) {
    Fmt<T>::store(out, o[0]);
  } else {
    Fmt<T>::store_vec(out, o);
  }
}

template <typename T, int VEC>
int launch_pool(PoolArgs a, bool overlap, int64_t B, hipStream_t s) {
  const int64_t threads = a.n_entries * a.col_groups;
  const int64_t blocks = ceil_div(threads, 256);
  DLC_REQUIRE(blocks < (int64_t(1) << 31) && B <= 65535, DLC_E_UNSUPPORTED, "compress: grid too large");
  dim3 grid{(unsigned)blocks, (unsigned)B, 1u};
  StageTimer timer(DLC_STAGE_COMPRESS, s);
  if (overlap)
    hipLaunchKernelGGL((pool_kernel<T, VEC, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((pool_kernel<T, VEC, false>), grid, dim3(256), 0, s, a);
  return check_launch("compress");
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
