// Dense token projections: out[M][N] = A[M][K] . W[K][N], W given as Wt[N][K].
//
// "DeepSeek-V4 Hybrid Attention: CSA and HCA from Scratch", §3 (C^a = H W^{aKV}
// and the other stream projections), §6.1-6.3 and §8 (c^Q, q^I, w^I, q).
//
// bf16 path: one 128x128 output tile per workgroup, the tile product of
// gemm128.hpp (v_mfma_f32_32x32x16_bf16, fp32 accumulation).  Other dtypes and
// shapes use a VALU kernel.
#include "gemm128.hpp"

namespace dlc {
namespace {

struct ProjArgs {
  const void* A;
  const void* W;
  void* out;
  int64_t M, N, K, lda, ldw, ldo;
  int out_bf16;
};

template <typename T>
__global__ void __launch_bounds__(256) project_valu_kernel(ProjArgs a) {
  const int64_t n = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t mrow = blockIdx.y;
  if (n >= a.N) return;
  const T* A = static_cast<const T*>(a.A) + mrow * a.lda;
  const T* W = static_cast<const T*>(a.W) + n * a.ldw;
  float acc = 0.f;
  for (int64_t k = 0; k < a.K; ++k) acc = fmaf(Fmt<T>::load(A + k), Fmt<T>::load(W + k), acc);
  if (a.out_bf16)
    Fmt<bf16_raw>::store(static_cast<bf16_raw*>(a.out) + mrow * a.ldo + n, acc);
  else
    static_cast<float*>(a.out)[mrow * a.ldo + n] = acc;
}

constexpr int TM = kGemmTile, TN = kGemmTile;

__global__ void __launch_bounds__(256) project_mfma_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) GemmSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  // XCD-aware order: consecutive workgroups share the same A rows
  const int64_t tiles_n = ceil_div(a.N, TN);
  const int64_t m0 = (int64_t(blockIdx.x) / tiles_n) * TM;
  const int64_t n0 = (int64_t(blockIdx.x) % tiles_n) * TN;
  const bf16_raw* A = static_cast<const bf16_raw*>(a.A);
  const bf16_raw* W = static_cast<const bf16_raw*>(a.W);
  const bf16_raw* arow[2];
  const bf16_raw* brow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = (tid + 256 * i) >> 2;
    arow[i] = m0 + row < a.M ? A + (m0 + row) * a.lda : nullptr;
    brow[i] = n0 + row < a.N ? W + (n0 + row) * a.ldw : nullptr;
  }
  f32x16 acc[2][2];
  gemm128(sm, arow, brow, a.K, acc);
  // D: lane holds column l32, rows 8*(r/4) + 4*g2 + r%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t gn = n0 + wn * 64 + j * 32 + l32;
      if (gn >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t gm = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * g2 + (r & 3);
        if (gm < a.M) {
          if (a.out_bf16)
            static_cast<bf16_raw*>(a.out)[gm * a.ldo + gn] = f32_to_bf16(acc[i][j][r]);
          else
            static_cast<float*>(a.out)[gm * a.ldo + gn] = acc[i][j][r];
        }
      }
    }
}

}  // namespace
}  // namespace dlc

extern "C" int dlc_project(int dtype, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* Wt,
                           int64_t ldw, void* out, int64_t ldo, int out_dtype, void* stream) {
  using namespace dlc;
  DLC_REQUIRE(dtype == DLC_F32 || dtype == DLC_BF16, DLC_E_DTYPE, "dlc_project: unsupported dtype %d", dtype);
  DLC_REQUIRE(out_dtype == DLC_F32 || out_dtype == dtype, DLC_E_DTYPE,
              "dlc_project: out_dtype must be DLC_F32 or the input dtype");
  DLC_REQUIRE(M >= 0 && N >= 0 && K >= 1, DLC_E_INVAL, "dlc_project: need M, N >= 0 and K >= 1");
  DLC_REQUIRE(lda >= K && ldw >= K && ldo >= N, DLC_E_SHAPE, "dlc_project: leading dimensions too small");
  DLC_REQUIRE(A && Wt && out, DLC_E_INVAL, "dlc_project: NULL argument");
  if (M == 0 || N == 0) return DLC_OK;
  ProjArgs a{A, Wt, out, M, N, K, lda, ldw, ldo, out_dtype == DLC_BF16};
  hipStream_t s = as_stream(stream);
  const bool mfma = dtype == DLC_BF16 && K % 8 == 0 && lda % 8 == 0 && ldw % 8 == 0 && aligned(A, 16) &&
                    aligned(Wt, 16);
  if (mfma) {
    const int64_t tiles = ceil_div(M, TM) * ceil_div(N, TN);
    DLC_REQUIRE(tiles < (int64_t(1) << 31), DLC_E_UNSUPPORTED, "dlc_project: too many tiles");
    hipLaunchKernelGGL(project_mfma_kernel, dim3((unsigned)tiles), dim3(256), 0, s, a);
  } else {
    DLC_REQUIRE(M <= 65535, DLC_E_UNSUPPORTED, "dlc_project: M > 65535 on the VALU path");
    dim3 grid{(unsigned)ceil_div(N, 256), (unsigned)M, 1u};
    if (dtype == DLC_BF16)
      hipLaunchKernelGGL(project_valu_kernel<bf16_raw>, grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(project_valu_kernel<float>, grid, dim3(256), 0, s, a);
  }
  return check_launch("dlc_project");
}
