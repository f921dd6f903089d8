// The compressor's stream projections and its pooling in one pass.
//
// "DeepSeek-V4 Hybrid Attention: CSA and HCA from Scratch", §3 (the streams
// Z^a, Z^b, C^a, C^b are the token rows of H times four weight matrices),
// §4-§5 (CSA: an entry pools the 2m rows of two adjacent blocks) and §10
// (HCA: an entry pools the m' rows of one block).
//
// A workgroup computes one 128-row x 128-column tile of the streams with the
// tile product of dlc_project (gemm128.hpp) and pools it in its epilogue, so
// the projected streams never reach HBM: the tile's columns are one group of
// channels of every stream the pooling needs (CSA: 32 channels each of Z^a,
// Z^b, C^a, C^b; HCA: 64 channels each of Z, C).  Each stream value is rounded
// to the storage type exactly as dlc_project stores it, put in LDS, and the
// compressor's chunked fold (pool_math.hpp) runs over it: the entries equal
// those of dlc_project followed by csa_compress / hca_compress, bit for bit.
//
// Rows.  HCA (m' | 128): tile t holds the 128/m' blocks of entries
// E0 .. E0 + 128/m' - 1, E0 = i_begin + t*128/m'.  CSA (m | 128): entry e
// needs blocks e (Z^a, C^a) and e-1 (Z^b, C^b), so tile t holds the 128/m
// blocks E0-1 .. E0+128/m-2 and completes the 128/m - 1 entries E0 .. with
// E0 = i_begin + t*(128/m - 1); consecutive tiles share one block, whose m
// rows are projected twice.  Rows before 0 or past n project to nothing
// (zero rows) and are never pooled.
#include "gemm128.hpp"
#include "pool_math.hpp"

namespace dlc {
namespace {

struct FusedArgs {
  const bf16_raw* H;        // [B] x [n][d] hidden rows: row r of sequence b at H + b*h_bstride + r*ldh
  int64_t ldh, h_bstride;
  const bf16_raw* W[4];     // per stream [c][ldw] (W transposed: channel j is row j); CSA: Za, Zb, Ca, Cb; HCA: Z, C
  int64_t ldw;
  const float* bias[2];     // [m][c] fp32 or nullptr; CSA: Ba, Bb; HCA: Bias
  int64_t n, d, c, m;
  int64_t i_begin, n_entries, ept;  // entries per tile
  bf16_raw* out;            // [B][cap][c]
  int64_t cap;
};

constexpr int kTileLds = kGemmTile * kGemmTile * 2;  // the bf16 stream tile of the epilogue

// One (row tile, channel group) of one sequence per workgroup.  OVERLAP: CSA (four
// streams of 32 channels), else HCA (two streams of 64 channels).
template <bool OVERLAP>
__global__ void __launch_bounds__(256) project_pool_kernel(FusedArgs a) {
  constexpr int NS = OVERLAP ? 4 : 2, CH = kGemmTile / NS;  // streams, channels per stream in the tile
  static_assert(sizeof(GemmSmem) >= kTileLds, "the stream tile reuses the operand buffers");
  __shared__ __attribute__((aligned(16))) GemmSmem sm;
  bf16_raw* tile = reinterpret_cast<bf16_raw*>(&sm);  // [128 rows][128 columns] after the product
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  // consecutive workgroups take the channel groups of one row tile, so the
  // hidden rows they share are fetched once while they are in the caches
  const int64_t groups = a.c / CH;
  const int64_t t = blockIdx.x / groups, grp = blockIdx.x % groups, b = blockIdx.y;
  const int64_t E0 = a.i_begin + t * a.ept;
  const int64_t row0 = OVERLAP ? a.m * (E0 - 1) : a.m * E0;  // stream row of tile row 0
  const bf16_raw* Hb = a.H + b * a.h_bstride;
  const bf16_raw* arow[2];
  const bf16_raw* brow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (tid + 256 * i) >> 2;
    const int64_t row = row0 + r;
    arow[i] = (row >= 0 && row < a.n) ? Hb + row * a.ldh : nullptr;
    brow[i] = a.W[r / CH] + (grp * CH + r % CH) * a.ldw;
  }
  f32x16 acc[2][2];
  gemm128(sm, arow, brow, a.d, acc);

  // the stream tile, rounded as dlc_project stores it (the product's last
  // barrier has released the operand buffers)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * g2 + (r & 3);
        const int col = wn * 64 + j * 32 + l32;
        tile[row * kGemmTile + col] = f32_to_bf16(acc[i][j][r]);
      }
  __syncthreads();

  auto value = [&](int row, int col) { return Fmt<bf16_raw>::load(tile + row * kGemmTile + col); };
  const int64_t n_here = min(a.ept, a.n_entries - t * a.ept);
  if constexpr (OVERLAP) {
    // thread (entry slot es, channel ch): the entries es, es+8, ...; window row
    // rho < m is tile row m*jb + rho of Z^a / C^a (bias row rho), m <= rho < 2m
    // tile row m*(jb-1) + rho - m of Z^b / C^b, where jb = e - E0 + 1 is the
    // entry's own block in the tile
    const int ch = tid & 31, es = tid >> 5;
    const int64_t gch = grp * CH + ch;
    for (int64_t el = es; el < n_here; el += 8) {
      const int64_t e = E0 + el;
      const int jb = int(el) + 1;
      const int rows = int(e > 0 ? 2 * a.m : a.m);  // entry 0 has no b-rows
      float mx[1] = {-INFINITY}, sum[1] = {0.f}, ac[1] = {0.f};
      for (int r0 = 0; r0 < rows; r0 += kPoolChunk) {
        const int nr = min(rows - r0, kPoolChunk);
        float l[kPoolChunk][1], cv[kPoolChunk][1];
#pragma unroll
        for (int rr = 0; rr < kPoolChunk; ++rr) {
          if (rr < nr) {
            const int rho = r0 + rr;
            const int seg = rho >= a.m ? 1 : 0;
            const int rb = seg ? rho - int(a.m) : rho;
            const int trow = int(a.m) * (jb - seg) + rb;
            const float* bias = a.bias[seg];
            const float bv = bias ? bias[rb * a.c + gch] : 0.f;
            l[rr][0] = pool_logit(value(trow, seg * CH + ch), bv);
            cv[rr][0] = value(trow, (2 + seg) * CH + ch);
          }
        }
        float pm[1], ps[1], pa[1];
        chunk_fold<1>(l, cv, nr, pm, ps, pa);
        merge_state<1>(mx, sum, ac, pm, ps, pa);
      }
      Fmt<bf16_raw>::store(a.out + (b * a.cap + e) * a.c + gch, pool_value(ac[0], sum[0]));
    }
  } else {
    // HCA: Q lanes per (entry, channel), lane q taking chunks q, q+Q, ...;
    // the first lane folds the chunk states in order through shuffles (the
    // fold of the compressor, whichever lanes computed the chunks)
    constexpr int Q = 4;  // lanes per output
    const int nch = int(ceil_div(a.m, kPoolChunk));
    const int q = tid & (Q - 1);
    const int64_t outputs = n_here * CH;
    for (int64_t o0 = 0; o0 < outputs; o0 += 256 / Q) {
      const int64_t o = o0 + (tid >> 2);
      const bool live = o < outputs;
      const int el = live ? int(o / CH) : 0, ch = int(o % CH);
      const int64_t gch = grp * CH + ch;
      float mx[1] = {-INFINITY}, sum[1] = {0.f}, ac[1] = {0.f};
      const int base = lane & ~(Q - 1);
#pragma unroll 1
      for (int k0 = 0; k0 < nch; k0 += Q) {
        // chunk k0 + q on this lane, then chunks k0 .. k0+Q-1 folded in order
        float pm = -INFINITY, ps = 0.f, pa = 0.f;
        const int ck = k0 + q;
        if (live && ck < nch) {
          const int r0 = ck * kPoolChunk, nr = min(int(a.m) - r0, kPoolChunk);
          float l[kPoolChunk][1], cv[kPoolChunk][1];
#pragma unroll
          for (int rr = 0; rr < kPoolChunk; ++rr) {
            if (rr < nr) {
              const int rho = r0 + rr;
              const int trow = int(a.m) * el + rho;
              const float bv = a.bias[0] ? a.bias[0][rho * a.c + gch] : 0.f;
              l[rr][0] = pool_logit(value(trow, ch), bv);
              cv[rr][0] = value(trow, CH + ch);
            }
          }
          chunk_fold<1>(l, cv, nr, &pm, &ps, &pa);
        }
#pragma unroll
        for (int qq = 0; qq < Q; ++qq) {
          const float km = __shfl(pm, base + qq), ks = __shfl(ps, base + qq), ka = __shfl(pa, base + qq);
          if (k0 + qq < nch) merge_state<1>(mx, sum, ac, &km, &ks, &ka);
        }
      }
      if (live && q == 0) Fmt<bf16_raw>::store(a.out + (b * a.cap + E0 + el) * a.c + gch, pool_value(ac[0], sum[0]));
    }
  }
}

int fused_dispatch(const char* name, int dtype, int64_t B, int64_t n, int64_t d, int64_t c, int64_t m,
                   const void* H, int64_t ldh, int64_t h_bstride, const void* const* W, int nw, int64_t ldw,
                   const float* b0, const float* b1, int64_t i_begin, int64_t i_end, void* out, int64_t cap,
                   bool overlap, void* stream) {
  DLC_REQUIRE(dtype == DLC_BF16, DLC_E_UNSUPPORTED, "%s: only DLC_BF16 (got dtype %d)", name, dtype);
  DLC_REQUIRE(B >= 1 && n >= 0 && d >= 1 && c >= 1 && m >= 1, DLC_E_INVAL,
              "%s: need B, d, c, m >= 1 and n >= 0", name);
  DLC_REQUIRE(H && out, DLC_E_INVAL, "%s: NULL H or output", name);
  for (int s = 0; s < nw; ++s) DLC_REQUIRE(W[s] != nullptr, DLC_E_INVAL, "%s: NULL weight", name);
  const int ch = overlap ? 32 : 64;
  DLC_REQUIRE(c % ch == 0, DLC_E_UNSUPPORTED, "%s: c=%lld is not a multiple of %d", name, (long long)c, ch);
  DLC_REQUIRE(kGemmTile % m == 0 && (!overlap || m < kGemmTile), DLC_E_UNSUPPORTED,
              "%s: the ratio %lld must divide %d%s", name, (long long)m, kGemmTile, overlap ? " (and be below it)" : "");
  DLC_REQUIRE(d % 8 == 0 && ldh % 8 == 0 && ldw % 8 == 0 && (B == 1 || h_bstride % 8 == 0) && aligned(H, 16),
              DLC_E_UNSUPPORTED, "%s: d, ldh, ldw and the batch stride must be multiples of 8, H 16-byte aligned",
              name);
  for (int s = 0; s < nw; ++s)
    DLC_REQUIRE(aligned(W[s], 16), DLC_E_UNSUPPORTED, "%s: weights must be 16-byte aligned", name);
  DLC_REQUIRE(ldh >= d && ldw >= d, DLC_E_SHAPE, "%s: ldh and ldw must be >= d", name);
  DLC_REQUIRE(B == 1 || n == 0 || h_bstride >= (n - 1) * ldh + d, DLC_E_SHAPE,
              "%s: batch stride overlaps rows of the next sequence", name);
  DLC_REQUIRE(0 <= i_begin && i_begin <= i_end && i_end <= n / m, DLC_E_SHAPE,
              "%s: need 0 <= i_begin <= i_end <= n/m (got %lld, %lld, n/m=%lld)", name, (long long)i_begin,
              (long long)i_end, (long long)(n / m));
  DLC_REQUIRE(cap >= i_end, DLC_E_SHAPE, "%s: cap %lld < i_end %lld", name, (long long)cap, (long long)i_end);
  if (i_end == i_begin) return DLC_OK;

  FusedArgs a{};
  a.H = static_cast<const bf16_raw*>(H);
  a.ldh = ldh;
  a.h_bstride = h_bstride;
  for (int s = 0; s < nw; ++s) a.W[s] = static_cast<const bf16_raw*>(W[s]);
  a.ldw = ldw;
  a.bias[0] = b0;
  a.bias[1] = b1;
  a.n = n; a.d = d; a.c = c; a.m = m;
  a.i_begin = i_begin;
  a.n_entries = i_end - i_begin;
  a.ept = overlap ? kGemmTile / m - 1 : kGemmTile / m;
  a.out = static_cast<bf16_raw*>(out);
  a.cap = cap;
  const int64_t tiles = ceil_div(a.n_entries, a.ept);
  DLC_REQUIRE(tiles * (c / ch) < (int64_t(1) << 31) && B <= 65535, DLC_E_UNSUPPORTED, "%s: grid too large", name);
  hipStream_t s = as_stream(stream);
  const dim3 grid{(unsigned)(tiles * (c / ch)), (unsigned)B, 1u};
  StageTimer timer(DLC_STAGE_COMPRESS, s);
  if (overlap)
    hipLaunchKernelGGL(project_pool_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(project_pool_kernel<false>, grid, dim3(256), 0, s, a);
  return check_launch(name);
}

}  // namespace
}  // namespace dlc

extern "C" {

int csa_project_compress(int dtype, int64_t B, int64_t n, int64_t d, int64_t c, int64_t m, const void* H,
                         int64_t ldh, int64_t h_bstride, const void* WtZa, const void* WtZb, const void* WtCa,
                         const void* WtCb, int64_t ldw, const float* Ba, const float* Bb, int64_t i_begin,
                         int64_t i_end, void* Ccomp, int64_t cap, void* stream) {
  const void* W[4] = {WtZa, WtZb, WtCa, WtCb};
  return dlc::fused_dispatch("csa_project_compress", dtype, B, n, d, c, m, H, ldh, h_bstride, W, 4, ldw, Ba, Bb,
                             i_begin, i_end, Ccomp, cap, true, stream);
}

int hca_project_compress(int dtype, int64_t B, int64_t n, int64_t d, int64_t c, int64_t m_prime, const void* H,
                         int64_t ldh, int64_t h_bstride, const void* WtZ, const void* WtC, int64_t ldw,
                         const float* Bias, int64_t i_begin, int64_t i_end, void* Chca, int64_t cap, void* stream) {
  const void* W[2] = {WtZ, WtC};
  return dlc::fused_dispatch("hca_project_compress", dtype, B, n, d, c, m_prime, H, ldh, h_bstride, W, 2, ldw, Bias,
                             nullptr, i_begin, i_end, Chca, cap, false, stream);
}

}  // extern "C"
