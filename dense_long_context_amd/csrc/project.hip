// Dense token projections: out[M][N] = A[M][K] . W[K][N], W given as Wt[N][K].
//
// "DeepSeek-V4 Hybrid Attention: CSA and HCA from Scratch", §3 (C^a = H W^{aKV}
// and the other stream projections), §6.1-6.3 and §8 (c^Q, q^I, w^I, q).
//
// bf16 path: one 128x128 output tile per workgroup, the tile product of
// gemm128.hpp (v_mfma_f32_32x32x16_bf16, fp32 accumulation).  At M <= 16 rows
// (a decode step's tokens) the weights dominate the traffic and a 128-row
// tile would leave most of the chip idle, so project_rows_kernel streams the
// weight rows instead.  Other dtypes and shapes use a VALU kernel.
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

// Row-vector path (M <= 16): a wave computes D[16 n][16 m] = Wt[n0 .. n0+15][K]
// . A[M rows][K]^T with v_mfma_f32_16x16x32_bf16, the weight rows as the A
// operand.  In each 32-deep step s, lane l loads 16 bytes of weight row
// n0 + l%16 and of activation row l%16 (zero from row M on) at k = 32s +
// 8(l/16): one load instruction reads 64 contiguous bytes of 16 weight rows.
// A column tile's steps are split over KW waves of one workgroup (wave w:
// steps w, w + KW, ... of the workgroup's k-slice) and, with a workspace,
// over S workgroups (blockIdx.y: k-slice y of S).  The wave sums meet in LDS
// and are added in wave order; the slice sums go to the workspace, and the
// last workgroup of a tile to arrive adds them in slice order.  So the bits
// do not depend on timing.  Steps past K are masked.
constexpr int kRowsWaves = 16, kRowsMaxM = 16;

struct RowsSplit {
  uint32_t* cnt;   // [NT] arrival counters, zero between calls
  float* part;     // [NT][S][64 lanes][4] slice sums in the D fragment layout
  int64_t S, kss;  // slices per tile; k-steps per slice
};

template <int KW, bool SPLIT>
__global__ void __launch_bounds__(64 * kRowsWaves) __attribute__((amdgpu_waves_per_eu(1, 4)))
project_rows_kernel(ProjArgs a, RowsSplit sp) {
  constexpr int TPW = kRowsWaves / KW, U = 8;  // column tiles per workgroup; steps in flight
  __shared__ f32x4 red[KW > 1 ? 64 * kRowsWaves : 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i16 = lane & 15, g = lane >> 4;
  const int kw = wave % KW;
  const int64_t tile = int64_t(blockIdx.x) * TPW + wave / KW, n0 = tile * 16;
  const int64_t K = a.K, KS = ceil_div(K, 32);
  const int64_t ks0 = SPLIT ? int64_t(blockIdx.y) * sp.kss : 0;
  const int64_t ks1 = SPLIT ? std::min(KS, ks0 + sp.kss) : KS;
  const bf16_raw* wp = static_cast<const bf16_raw*>(a.W) + std::min<int64_t>(n0 + i16, a.N - 1) * a.ldw;
  const bf16_raw* ap = static_cast<const bf16_raw*>(a.A) + std::min<int64_t>(i16, a.M - 1) * a.lda;
  const bool mrow = i16 < a.M;
  // the wave's steps j = 0 .. nst-1 are k-steps ks0 + kw + j*KW; unit u of
  // group i is step i*U + u, and its registers are refilled with step
  // (i+1)*U + u as soon as its MFMA has read them.  Inside the loop every
  // load is unconditional (past the wave's steps from a clamped address,
  // masked), so the compiler keeps all U steps in flight across iterations;
  // the last group is peeled and loads nothing more.
  const int64_t span = ks1 - ks0;
  const int64_t nst = span > kw ? ceil_div(span - kw, int64_t(KW)) : 0;
  const int64_t ng = ceil_div(nst, int64_t(U));
  uint4 wv[U], av[U];
  bool in[U];
  auto load = [&](int64_t j, int u) {  // K % 8 == 0: a lane's eight elements are all in or all out
    const int64_t k = 32 * (ks0 + kw + j * KW) + 8 * g;
    in[u] = j < nst && k < K;
    const int64_t kc = in[u] ? k : K - 8;
    wv[u] = *reinterpret_cast<const uint4*>(wp + kc);
    av[u] = *reinterpret_cast<const uint4*>(ap + kc);
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto mfma = [&](int u) {
    const uint4 z = make_uint4(0, 0, 0, 0);
    const uint4 w = in[u] ? wv[u] : z;
    const uint4 x = in[u] && mrow ? av[u] : z;
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), __builtin_bit_cast(bf16x8, x), acc,
                                                  0, 0, 0);
  };
  // (the empty asm statements with a memory clobber keep the compiler from
  // merging a step's loads from both loop entries into one load at the loop
  // head, which would leave nothing in flight across iterations)
  if (ng > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      in[u] = false;
      if (u < nst) load(u, u);  // uniform: a wave with fewer steps loads no more than it has
    }
    asm volatile("" ::: "memory");
    for (int64_t i = 0; i + 1 < ng; ++i) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        mfma(u);
        load((i + 1) * U + u, u);
        asm volatile("" ::: "memory");
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) mfma(u);
  }
  if constexpr (KW > 1) {
    red[tid] = acc;
    __syncthreads();
    if (kw != 0) return;
    for (int w = 1; w < KW; ++w) {
      const f32x4 v = red[tid + 64 * w];
      acc[0] += v[0]; acc[1] += v[1]; acc[2] += v[2]; acc[3] += v[3];
    }
  }
  if constexpr (SPLIT) {
    if (n0 >= a.N) return;  // a tile past N (last workgroup): no counter
    float* mine = sp.part + ((tile * sp.S + blockIdx.y) * 64 + lane) * 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) st_agent(mine + r, acc[r]);
    wait_vm<0>();  // the slice sum is visible before the arrival
    uint32_t prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(sp.cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __shfl(prev, 0);
    if (prev != uint32_t(sp.S - 1)) return;
    // the slice sums in slice order; the tile's slots and counter are left
    // zero, so that the next call, whatever its shape, finds the workspace
    // as the first one did
    float* all = sp.part + (tile * sp.S * 64 + lane) * 4;
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t y = 0; y < sp.S; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] += ld_agent(all + y * 256 + r);
    for (int64_t y = 0; y < sp.S; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) st_agent(all + y * 256 + r, 0.f);
    if (lane == 0) st_agent(sp.cnt + tile, 0u);
  }
  // D: lane l holds rows n0 + 4(l/16) + r of column m = l%16
  if (!mrow) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t n = n0 + 4 * g + r;
    if (n < a.N) {
      if (a.out_bf16)
        static_cast<bf16_raw*>(a.out)[i16 * a.ldo + n] = f32_to_bf16(acc[r]);
      else
        static_cast<float*>(a.out)[i16 * a.ldo + n] = acc[r];
    }
  }
}

// The row path's plan: waves per column tile inside a workgroup (doubled
// while the grid is under one workgroup per CU and every wave keeps four
// steps at least), then, with a workspace, k-slices over workgroups (doubled
// while the grid is under 256 workgroups and every wave keeps a step).
struct RowsPlan {
  int kw;
  int64_t blocks, S, kss, NT;
};
RowsPlan rows_plan(int64_t N, int64_t K, bool split) {
  RowsPlan p{1, 0, 1, 0, ceil_div(N, int64_t(16))};
  const int64_t KS = ceil_div(K, int64_t(32));
  while (p.kw < kRowsWaves && ceil_div(p.NT, int64_t(kRowsWaves / p.kw)) < 256 && KS >= 4 * p.kw) p.kw *= 2;
  p.blocks = ceil_div(p.NT, int64_t(kRowsWaves / p.kw));
  if (split)
    while (p.blocks * p.S < 256 && ceil_div(KS, 2 * p.S) >= p.kw) p.S *= 2;
  p.kss = ceil_div(KS, p.S);
  p.S = ceil_div(KS, p.kss);
  return p;
}
size_t rows_ws_bytes(const RowsPlan& p) {
  return p.S > 1 ? align_up(size_t(p.NT) * 4, 256) + size_t(p.NT) * size_t(p.S) * 64 * 16 : 0;
}

}  // namespace
}  // namespace dlc

extern "C" size_t dlc_project_ws(int dtype, int64_t M, int64_t N, int64_t K) {
  using namespace dlc;
  if (dtype != DLC_BF16 || M < 1 || M > kRowsMaxM || N < 1 || K < 1) return 0;
  return rows_ws_bytes(rows_plan(N, K, true));
}

extern "C" int dlc_project(int dtype, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* Wt,
                           int64_t ldw, void* out, int64_t ldo, int out_dtype, void* ws, size_t ws_bytes,
                           void* stream) {
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
  if (mfma && M <= kRowsMaxM) {
    const RowsPlan full = rows_plan(N, K, true);
    const size_t need = rows_ws_bytes(full);
    DLC_REQUIRE(!ws || ws_bytes >= need, DLC_E_WORKSPACE, "dlc_project: workspace of %zu bytes, %zu needed",
                ws_bytes, need);
    const bool split = ws && need > 0;
    const RowsPlan p = split ? full : rows_plan(N, K, false);
    DLC_REQUIRE(p.blocks < (int64_t(1) << 31), DLC_E_UNSUPPORTED, "dlc_project: too many column tiles");
    RowsSplit sp{nullptr, nullptr, p.S, p.kss};
    if (split) {
      sp.cnt = static_cast<uint32_t*>(ws);
      sp.part = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(size_t(p.NT) * 4, 256));
    }
    const dim3 grid{(unsigned)p.blocks, (unsigned)p.S, 1u}, block{64u * kRowsWaves, 1u, 1u};
#define DLC_ROWS(kw_)                                                                    \
  if (p.kw == kw_) {                                                                     \
    if (split) hipLaunchKernelGGL((project_rows_kernel<kw_, true>), grid, block, 0, s, a, sp);  \
    else hipLaunchKernelGGL((project_rows_kernel<kw_, false>), grid, block, 0, s, a, sp);       \
  }
    DLC_ROWS(1) DLC_ROWS(2) DLC_ROWS(4) DLC_ROWS(8) DLC_ROWS(16)
#undef DLC_ROWS
  } else if (mfma) {
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
