// The 128x128 bf16 tile product shared by dlc_project and the fused
// projection + pooling calls ("DeepSeek-V4 Hybrid Attention: CSA and HCA from
// Scratch", §3: every stream is a row of H times a weight matrix).
//
// A workgroup of 4 waves (2x2, 64x64 each) computes D[128][128] =
// A[128 rows][K] . B[128 rows][K]^T with v_mfma_f32_32x32x16_bf16 and fp32
// accumulation; K is consumed in 32-deep steps staged through LDS with padded
// rows, the next step's global loads in flight during the current step's
// MFMAs.  Both operands are K-contiguous rows given by pointer (nullptr: a
// zero row), so global loads are whole 16-byte vectors.  Every output element
// goes through the same MFMA sequence whichever tile computes it, so callers
// that cut rows differently get the same bits.
#pragma once
#include "common.hpp"

namespace dlc {

constexpr int kGemmTile = 128, kGemmTK = 32;
constexpr int kGemmLRow = kGemmTK + 8;  // padded LDS row (bf16): 80 bytes

struct GemmSmem {
  bf16_raw sA[2][kGemmTile * kGemmLRow];
  bf16_raw sB[2][kGemmTile * kGemmLRow];
};

// Thread tid stages rows (tid + 256*i) >> 2, i < 2, of both operands: the
// caller passes those rows' pointers (arow[i], brow[i], or nullptr).
// D layout on return: wave (wm, wn) = (wave >> 1, wave & 1), acc[i][j] is the
// 32x32 block at rows wm*64 + i*32, columns wn*64 + j*32; lane l holds column
// l%32 and rows 8*(r/4) + 4*(l/32) + r%4 of element r.
__device__ __forceinline__ void gemm128(GemmSmem& sm, const bf16_raw* const (&arow)[2],
                                        const bf16_raw* const (&brow)[2], int64_t K, f32x16 (&acc)[2][2]) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  uint4 ra[2], rb[2];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kc = ((tid + 256 * i) & 3) * 8;
      const int64_t gk = k0 + kc;
      ra[i] = (arow[i] && gk < K) ? *reinterpret_cast<const uint4*>(arow[i] + gk) : make_uint4(0, 0, 0, 0);
      rb[i] = (brow[i] && gk < K) ? *reinterpret_cast<const uint4*>(brow[i] + gk) : make_uint4(0, 0, 0, 0);
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = tid + 256 * i;
      const int row = v >> 2, kc = (v & 3) * 8;
      *reinterpret_cast<uint4*>(&sm.sA[buf][row * kGemmLRow + kc]) = ra[i];
      *reinterpret_cast<uint4*>(&sm.sB[buf][row * kGemmLRow + kc]) = rb[i];
    }
  };
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int64_t nk = ceil_div(K, kGemmTK);
  gload(0);
  swrite(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = int(kt & 1);
    if (kt + 1 < nk) gload((kt + 1) * kGemmTK);
#pragma unroll
    for (int ks = 0; ks < kGemmTK / 16; ++ks) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&sm.sA[buf][(wm * 64 + i * 32 + l32) * kGemmLRow + ks * 16 + g2 * 8]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(&sm.sB[buf][(wn * 64 + j * 32 + l32) * kGemmLRow + ks * 16 + g2 * 8]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) swrite(buf ^ 1);
    __syncthreads();
  }
}

}  // namespace dlc
