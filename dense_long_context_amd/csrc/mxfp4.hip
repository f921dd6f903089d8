// MXFP4 row quantizer: the FP4 indexer's key cache.
//
// "DeepSeek-V4 Hybrid Attention: CSA and HCA from Scratch", §6.4 and §12: the
// indexer's q . K products run in FP4.  The format (OCP MXFP4: E2M1 codes on
// a power-of-two scale per 32 elements) is the reading encoded in mxfp4.hpp.
// Each thread encodes one 32-element block; a row of width c^I yields c^I/2
// code bytes and c^I/32 scale bytes.  Keys are quantized once, when their
// compressed entry is written (a whole cache at set-up, one entry per m
// tokens in decode).
#include "mxfp4.hpp"

namespace dlc {
namespace {

template <typename T>
__global__ void __launch_bounds__(256) mxfp4_quantize_kernel(const T* src, int64_t src_bstride, int64_t rows,
                                                             int64_t width, uint8_t* codes, int64_t codes_bstride,
                                                             uint8_t* scales, int64_t scales_bstride,
                                                             int64_t blocks_per_batch) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t b = blockIdx.y;
  if (i >= blocks_per_batch) return;
  const int64_t bpr = width / 32;
  const int64_t r = i / bpr, j = i % bpr;
  float v[32];
  load32<T>(src + b * src_bstride + r * width + j * 32, v);
  uint32_t e8m0;
  const uint4 c = mxfp4_encode32(v, e8m0);
  *reinterpret_cast<uint4*>(codes + b * codes_bstride + r * (width / 2) + j * 16) = c;
  scales[b * scales_bstride + r * bpr + j] = uint8_t(e8m0);
}

}  // namespace
}  // namespace dlc

extern "C" int mxfp4_quantize(int dtype, int64_t B, int64_t rows, int64_t width, const void* src,
                              int64_t src_bstride, uint8_t* codes, int64_t codes_bstride, uint8_t* scales,
                              int64_t scales_bstride, void* stream) {
  using namespace dlc;
  DLC_REQUIRE(dtype == DLC_F32 || dtype == DLC_BF16, DLC_E_DTYPE, "mxfp4_quantize: unsupported dtype %d", dtype);
  DLC_REQUIRE(B >= 1 && rows >= 0 && width >= 32 && width % 32 == 0, DLC_E_SHAPE,
              "mxfp4_quantize: need B >= 1, rows >= 0 and width a positive multiple of 32");
  if (rows == 0) return DLC_OK;
  DLC_REQUIRE(src && codes && scales, DLC_E_INVAL, "mxfp4_quantize: NULL argument");
  DLC_REQUIRE(src_bstride >= rows * width && codes_bstride >= rows * width / 2 && scales_bstride >= rows * width / 32,
              DLC_E_SHAPE, "mxfp4_quantize: a batch stride is smaller than its rows");
  DLC_REQUIRE(aligned(src, 16) && aligned(codes, 16) && src_bstride % 8 == 0 && codes_bstride % 16 == 0,
              DLC_E_INVAL, "mxfp4_quantize: src and codes (and their batch strides) must be 16-byte aligned");
  DLC_REQUIRE(B <= 65535, DLC_E_UNSUPPORTED, "mxfp4_quantize: B > 65535");
  const int64_t blocks = rows * (width / 32);
  DLC_REQUIRE(ceil_div(blocks, 256) < (int64_t(1) << 31), DLC_E_UNSUPPORTED, "mxfp4_quantize: too many rows");
  hipStream_t s = as_stream(stream);
  dim3 grid{(unsigned)ceil_div(blocks, 256), (unsigned)B, 1u};
  if (dtype == DLC_BF16)
    hipLaunchKernelGGL(mxfp4_quantize_kernel<bf16_raw>, grid, dim3(256), 0, s, static_cast<const bf16_raw*>(src),
                       src_bstride, rows, width, codes, codes_bstride, scales, scales_bstride, blocks);
  else
    hipLaunchKernelGGL(mxfp4_quantize_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(src),
                       src_bstride, rows, width, codes, codes_bstride, scales, scales_bstride, blocks);
  return check_launch("mxfp4_quantize");
}
