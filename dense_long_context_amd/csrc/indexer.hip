// Lightning indexer and exact top-k over the CSA cache.
//
// "DeepSeek-V4 Hybrid Attention: CSA and HCA from Scratch", §6.4 (score
// I[s] = sum_h w[h] * ReLU(q[h] . K[s])) and §7 (keep the k largest over the
// visible entries s < floor(t/m)).
//
// Pipeline per call (all on the caller's stream):
//   1. clear      zero the first-digit histograms and the counters
//   2. scores     one pass over K^I: for bf16 with c^I % 32 == 0 the heads x keys
//                 product runs on MFMA (v_mfma_f32_16x16x32_bf16) with the
//                 queries held in registers; otherwise a VALU kernel.  Each
//                 workgroup also builds an LDS histogram of the top 11 bits of
//                 the order-preserving score key and adds its non-zero bins to
//                 the query's histogram.
//   3. filter     every workgroup finds the threshold bin T from that
//                 histogram, appends entries above T to the selected list and
//                 entries in T to the candidate list (wave-aggregated atomics).
//   4. finish     one workgroup per query resolves the candidates with radix
//                 passes over the remaining key bits and then the index (ties
//                 go to the smaller index), sorts the k_eff winners ascending in
//                 LDS and writes idx / count.
#include "common.hpp"

namespace dlc {
namespace {

constexpr int kBins = 2048;      // first digit: top 11 bits of the key
constexpr int kShift1 = 21;
constexpr int kMaxK = 8192;

struct IdxArgs {
  const void* qI;      // [BQ][n_hI][cI]
  const float* wI;     // [BQ][n_hI]
  const void* KI;      // [B][cap][cI]
  const int64_t* t;    // [BQ]
  int64_t n_q, n_hI, cI, m, k, cap, t_max;
  float* scores;       // [BQ][score_ld]
  int64_t score_ld;
  uint32_t* hist;      // [BQ][kBins]
  uint32_t* cnt;       // [BQ][4]: selected, candidates
  int32_t* sel;        // [BQ][k]
  int32_t* cand;       // [BQ][cap]
  int32_t* idx;        // [BQ][k]
  int32_t* count;      // [BQ]
  int64_t keys_per_wg; // scores / filter chunk
};

__device__ __forceinline__ int64_t visible(const IdxArgs& a, int64_t bq) {
  int64_t t = a.t[bq];
  t = t < 0 ? 0 : (t > a.t_max ? a.t_max : t);
  int64_t v = t / a.m;
  return v < a.cap ? v : a.cap;
}

__device__ __forceinline__ float canon_zero(float s) { return s == 0.f ? 0.f : s; }

// LDS histogram of the first digit -> the query's global histogram
__device__ __forceinline__ void flush_hist(uint32_t* lds, uint32_t* global) {
  __syncthreads();
  for (int b = threadIdx.x; b < kBins; b += blockDim.x) {
    const uint32_t v = lds[b];
    if (v) atomicAdd(global + b, v);
  }
}

// ---------------------------------------------------------------- scores (VALU)

template <typename T>
__global__ void __launch_bounds__(256) scores_valu_kernel(IdxArgs a) {
  extern __shared__ float smem[];
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem);
  float* q = smem + kBins;                // [n_hI][cI]
  float* w = q + a.n_hI * a.cI;           // [n_hI]
  const int64_t bq = blockIdx.y;
  const int64_t nvis = visible(a, bq);
  const int64_t s0 = int64_t(blockIdx.x) * a.keys_per_wg;
  if (s0 >= nvis) return;
  const int64_t s1 = min(nvis, s0 + a.keys_per_wg);

  for (int i = threadIdx.x; i < kBins; i += blockDim.x) hist[i] = 0;
  const T* qg = static_cast<const T*>(a.qI) + bq * a.n_hI * a.cI;
  for (int64_t i = threadIdx.x; i < a.n_hI * a.cI; i += blockDim.x) q[i] = Fmt<T>::load(qg + i);
  for (int64_t i = threadIdx.x; i < a.n_hI; i += blockDim.x) w[i] = a.wI[bq * a.n_hI + i];
  __syncthreads();

  const int64_t b = bq / a.n_q;
  const T* K = static_cast<const T*>(a.KI) + b * a.cap * a.cI;
  for (int64_t s = s0 + threadIdx.x; s < s1; s += blockDim.x) {
    const T* ks = K + s * a.cI;
    float score = 0.f;
    for (int64_t h = 0; h < a.n_hI; ++h) {
      float dot = 0.f;
      for (int64_t d = 0; d < a.cI; ++d) dot = fmaf(q[h * a.cI + d], Fmt<T>::load(ks + d), dot);
      score = fmaf(w[h], fmaxf(dot, 0.f), score);
    }
    score = canon_zero(score);
    a.scores[bq * a.score_ld + s] = score;
    atomicAdd(&hist[order_key(score) >> kShift1], 1u);
  }
  flush_hist(hist, a.hist + bq * kBins);
}

// ---------------------------------------------------------------- scores (MFMA)
//
// One wave scores 16 keys per step: D[16 heads][16 keys] += Q[16 heads][32 dims]
// x K^T[32 dims][16 keys] for every head tile and 32-dim step.  Lane l holds
// head/key l%16 of the A/B operands and dims 8*(l/16) .. +7 of each 32-dim
// step; the result holds key l%16 and heads 4*(l/16) .. +3.  The head sum is
// finished with two cross-lane adds.  Queries stay in registers for the whole
// pass; keys stream from HBM, the next tile's loads in flight while the
// current tile is multiplied.

template <int HT, int KT>
__global__ void __launch_bounds__(256) scores_mfma_kernel(IdxArgs a) {
  __shared__ uint32_t hist[kBins];
  const int64_t bq = blockIdx.y;
  const int64_t nvis = visible(a, bq);
  const int64_t s0 = int64_t(blockIdx.x) * a.keys_per_wg;
  if (s0 >= nvis) return;
  const int64_t s1 = min(nvis, s0 + a.keys_per_wg);
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) hist[i] = 0;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int cI = KT * 32;

  // queries: A operand, rows = heads
  bf16x8 qf[HT][KT];
  const bf16_raw* qg = static_cast<const bf16_raw*>(a.qI) + bq * a.n_hI * cI;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int h = ht * 16 + r16;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (h < a.n_hI) v = *reinterpret_cast<const uint4*>(qg + h * cI + kt * 32 + g * 8);
      qf[ht][kt] = __builtin_bit_cast(bf16x8, v);
    }
  }
  float wv[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = ht * 16 + g * 4 + r;
      wv[ht][r] = h < a.n_hI ? a.wI[bq * a.n_hI + h] : 0.f;
    }
  __syncthreads();

  const int64_t b = bq / a.n_q;
  const bf16_raw* K = static_cast<const bf16_raw*>(a.KI) + b * a.cap * cI;
  const int64_t ntiles = (s1 - s0 + 15) / 16;
  int64_t tile = wave;
  uint4 cur[KT], nxt[KT];
  auto load_tile = [&](int64_t tl, uint4* dst) {
    int64_t row = s0 + tl * 16 + r16;
    row = row < s1 ? row : s1 - 1;  // rows past the end repeat the last visible row
    const bf16_raw* p = K + row * cI + g * 8;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) dst[kt] = *reinterpret_cast<const uint4*>(p + kt * 32);
  };
  if (tile < ntiles) load_tile(tile, cur);
  for (; tile < ntiles; tile += 4) {
    if (tile + 4 < ntiles) load_tile(tile + 4, nxt);
    f32x4 acc[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const bf16x8 kb = __builtin_bit_cast(bf16x8, cur[kt]);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ht][kt], kb, acc[ht], 0, 0, 0);
    }
    float part = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int r = 0; r < 4; ++r) part = fmaf(wv[ht][r], fmaxf(acc[ht][r], 0.f), part);
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    const int64_t s = s0 + tile * 16 + r16;
    if (g == 0 && s < s1) {
      const float score = canon_zero(part);
      a.scores[bq * a.score_ld + s] = score;
      atomicAdd(&hist[order_key(score) >> kShift1], 1u);
    }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) cur[kt] = nxt[kt];
  }
  flush_hist(hist, a.hist + bq * kBins);
}

// ---------------------------------------------------------------- threshold

// Finds the bin T with above(T) < need <= above(T) + h[T], where above(T)
// counts the entries in bins > T.  Every thread of the block gets (T, above).
// h is an LDS array of nbins (a multiple of blockDim.x); scratch holds
// blockDim.x + 2 words.
__device__ void find_threshold(const uint32_t* h, int nbins, uint32_t need, uint32_t* scratch,
                               int* T_out, uint32_t* above_out) {
  const int per = nbins / blockDim.x;
  const int lo = threadIdx.x * per;
  uint32_t mine = 0;
  for (int i = 0; i < per; ++i) mine += h[lo + i];
  scratch[threadIdx.x] = mine;
  if (threadIdx.x == 0) {  // defaults if no bin qualifies (inconsistent counts)
    scratch[blockDim.x] = 0;
    scratch[blockDim.x + 1] = 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // suffix scan from the top thread down; blockDim.x <= 1024 so this is short
    uint32_t run = 0;
    for (int i = blockDim.x - 1; i >= 0; --i) {
      const uint32_t v = scratch[i];
      scratch[i] = run;  // entries in bins owned by higher threads
      run += v;
    }
  }
  __syncthreads();
  uint32_t run = scratch[threadIdx.x];
  __syncthreads();
  for (int i = per - 1; i >= 0; --i) {
    const uint32_t v = h[lo + i];
    if (run < need && run + v >= need) {
      scratch[blockDim.x] = uint32_t(lo + i);
      scratch[blockDim.x + 1] = run;
    }
    run += v;
  }
  __syncthreads();
  *T_out = int(scratch[blockDim.x]);
  *above_out = scratch[blockDim.x + 1];
  __syncthreads();
}

// wave-aggregated append of `pred` entries to list[cnt] (slots past `limit` are dropped)
__device__ __forceinline__ void wave_append(bool pred, int32_t value, uint32_t* counter, int32_t* list,
                                            uint32_t limit) {
  const uint64_t mask = __ballot(pred);
  if (mask == 0) return;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)mask) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, uint32_t(__popcll(mask)));
  base = __shfl(base, leader);
  const uint32_t pos = base + uint32_t(__popcll(mask & ((uint64_t(1) << lane) - 1)));
  if (pred && pos < limit) list[pos] = value;
}

__global__ void __launch_bounds__(256) filter_kernel(IdxArgs a) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t scratch[256 + 2];
  const int64_t bq = blockIdx.y;
  const int64_t nvis = visible(a, bq);
  const int64_t keff = min(a.k, nvis);
  const int64_t s0 = int64_t(blockIdx.x) * a.keys_per_wg;
  if (keff == nvis || s0 >= nvis) return;  // keep-all and empty chunks need no filtering
  const int64_t s1 = min(nvis, s0 + a.keys_per_wg);
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) h[i] = a.hist[bq * kBins + i];
  __syncthreads();
  int T;
  uint32_t above;
  find_threshold(h, kBins, uint32_t(keff), scratch, &T, &above);

  const float* sc = a.scores + bq * a.score_ld;
  // whole waves iterate together so the ballots see every lane
  for (int64_t base = s0; base < s1; base += blockDim.x) {
    const int64_t s = base + threadIdx.x;
    int d = -1;
    if (s < s1) d = int(order_key(sc[s]) >> kShift1);
    wave_append(d > T, int32_t(s), a.cnt + bq * 4 + 0, a.sel + bq * a.k, uint32_t(a.k));
    wave_append(d == T, int32_t(s), a.cnt + bq * 4 + 1, a.cand + bq * a.cap, uint32_t(a.cap));
  }
}

// ---------------------------------------------------------------- finish

// radix passes over the candidates' composite key: the low 21 bits of the score
// key (the top 11 bits are T for all of them), then the bit-inverted index
constexpr int kPasses = 5;
__constant__ int kPassShift[kPasses] = {42, 32, 21, 10, 0};
__constant__ int kPassBits[kPasses] = {11, 10, 11, 11, 10};

__device__ __forceinline__ uint64_t cand_key(const float* sc, int32_t s) {
  const uint64_t key = order_key(sc[s]) & 0x1fffffu;
  return (key << 32) | uint64_t(0xffffffffu - uint32_t(s));
}

__global__ void __launch_bounds__(1024) finish_kernel(IdxArgs a) {
  extern __shared__ uint32_t fsm[];
  uint32_t* h = fsm;                                    // kBins
  uint32_t* scratch = h + kBins;                         // 1024 + 2
  uint32_t* nsel_lds = scratch + 1024 + 2;               // 1
  int32_t* buf = reinterpret_cast<int32_t*>(nsel_lds + 2);  // pow2 >= keff
  const int64_t bq = blockIdx.x;
  const int64_t nvis = visible(a, bq);
  const int64_t keff = min(a.k, nvis);
  int32_t* out = a.idx + bq * a.k;
  if (threadIdx.x == 0) a.count[bq] = int32_t(keff);
  if (keff == nvis) {
    for (int64_t j = threadIdx.x; j < a.k; j += blockDim.x) out[j] = j < nvis ? int32_t(j) : -1;
    return;
  }
  const uint32_t n_sel = min(a.cnt[bq * 4 + 0], uint32_t(keff));
  const uint32_t n_cand = min(a.cnt[bq * 4 + 1], uint32_t(a.cap));
  const int32_t* sel = a.sel + bq * a.k;
  const int32_t* cand = a.cand + bq * a.cap;
  const float* sc = a.scores + bq * a.score_ld;
  int P = 1;
  while (P < keff) P <<= 1;
  for (int j = threadIdx.x; j < P; j += blockDim.x) buf[j] = j < int(n_sel) ? sel[j] : 0x7fffffff;
  if (threadIdx.x == 0) *nsel_lds = n_sel;
  __syncthreads();

  uint32_t need = uint32_t(keff) - n_sel;
  uint64_t pval = 0, pmask = 0;
  for (int pass = 0; pass < kPasses && need > 0; ++pass) {
    const int shift = kPassShift[pass], bits = kPassBits[pass];
    const uint32_t dmask = (1u << bits) - 1u;
    const int nb = 1 << bits;
    for (int i = threadIdx.x; i < kBins; i += blockDim.x) h[i] = 0;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < n_cand; i += blockDim.x) {
      const uint64_t ck = cand_key(sc, cand[i]);
      if ((ck & pmask) == pval) atomicAdd(&h[(ck >> shift) & dmask], 1u);
    }
    __syncthreads();
    int D;
    uint32_t above;
    find_threshold(h, nb < 1024 ? 1024 : nb, need, scratch, &D, &above);
    const bool take_all = (above + h[D] == need);
    // select every candidate with a larger digit (and, if the bin D is exactly what
    // is still needed, the whole bin D as well)
    for (uint32_t i = threadIdx.x; i < n_cand; i += blockDim.x) {
      const int32_t s = cand[i];
      const uint64_t ck = cand_key(sc, s);
      if ((ck & pmask) == pval) {
        const uint32_t dg = uint32_t(ck >> shift) & dmask;
        if (dg > uint32_t(D) || (take_all && dg == uint32_t(D))) {
          const uint32_t pos = atomicAdd(nsel_lds, 1u);
          if (pos < uint32_t(P)) buf[pos] = s;
        }
      }
    }
    __syncthreads();
    need = take_all ? 0 : need - above;
    pval |= uint64_t(D) << shift;
    pmask |= uint64_t(dmask) << shift;
  }
  __syncthreads();

  // bitonic sort of buf[0 .. P) ascending (padding INT_MAX sinks to the end)
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < P / 2; i += blockDim.x) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const bool asc = (lo & size) == 0;
        const int32_t x = buf[lo], y = buf[hi];
        if ((x > y) == asc) { buf[lo] = y; buf[hi] = x; }
      }
      __syncthreads();
    }
  }
  for (int64_t j = threadIdx.x; j < a.k; j += blockDim.x) out[j] = j < keff ? buf[j] : -1;
}

// ---------------------------------------------------------------- host

struct WsLayout {
  size_t scores, hist, cnt, sel, cand, total;
};

WsLayout ws_layout(int64_t B, int64_t n_q, int64_t cap, int64_t k, bool own_scores) {
  const size_t BQ = size_t(B) * size_t(n_q);
  WsLayout L{};
  size_t off = 0;
  L.hist = off;  off = align_up(off + BQ * kBins * 4, 256);
  L.cnt = off;   off = align_up(off + BQ * 4 * 4, 256);
  L.sel = off;   off = align_up(off + BQ * size_t(k) * 4, 256);
  L.cand = off;  off = align_up(off + BQ * size_t(cap) * 4, 256);
  L.scores = off;
  if (own_scores) off = align_up(off + BQ * size_t(cap) * 4, 256);
  L.total = off;
  return L;
}

}  // namespace
}  // namespace dlc

extern "C" {

size_t csa_index_topk_ws(int64_t B, int64_t n_q, int64_t cap, int64_t k) {
  if (B < 1 || n_q < 1 || cap < 0 || k < 1) return 0;
  return dlc::ws_layout(B, n_q, cap, k, true).total;
}

int csa_index_topk(int dtype, int64_t B, int64_t n_q, int64_t n_hI, int64_t cI, int64_t m, int64_t k,
                   const void* qI, const float* wI, const void* KI, int64_t cap, const int64_t* t,
                   int64_t t_max, int32_t* idx, int32_t* count, float* scores, void* ws, size_t ws_bytes,
                   void* stream) {
  using namespace dlc;
  DLC_REQUIRE(dtype == DLC_F32 || dtype == DLC_BF16, DLC_E_DTYPE, "csa_index_topk: unsupported dtype %d", dtype);
  DLC_REQUIRE(B >= 1 && n_q >= 1 && n_hI >= 1 && cI >= 1 && m >= 1 && cap >= 0 && t_max >= 0, DLC_E_INVAL,
              "csa_index_topk: need B, n_q, n_hI, cI, m >= 1 and cap, t_max >= 0");
  DLC_REQUIRE(k >= 1 && k <= kMaxK, DLC_E_UNSUPPORTED, "csa_index_topk: k=%lld outside [1, %d]", (long long)k, kMaxK);
  const bool mfma_shape = dtype == DLC_BF16 && (cI == 32 || cI == 64 || cI == 128 || cI == 256) && n_hI <= 64;
  DLC_REQUIRE(mfma_shape || n_hI * cI <= 8192, DLC_E_UNSUPPORTED,
              "csa_index_topk: n_hI*cI=%lld > 8192 outside the MFMA shapes", (long long)(n_hI * cI));
  DLC_REQUIRE(t_max / m <= cap, DLC_E_SHAPE, "csa_index_topk: floor(t_max/m)=%lld exceeds cap=%lld",
              (long long)(t_max / m), (long long)cap);
  DLC_REQUIRE(cap < (int64_t(1) << 31), DLC_E_UNSUPPORTED, "csa_index_topk: cap must be < 2^31");
  DLC_REQUIRE(qI && wI && t && idx && count && (KI || cap == 0), DLC_E_INVAL, "csa_index_topk: NULL argument");
  const WsLayout L = ws_layout(B, n_q, cap, k, scores == nullptr);
  DLC_REQUIRE(ws != nullptr && ws_bytes >= L.total, DLC_E_WORKSPACE,
              "csa_index_topk: workspace of %zu bytes needed, %zu given", L.total, ws_bytes);
  DLC_REQUIRE(aligned(ws, 256), DLC_E_WORKSPACE, "csa_index_topk: workspace must be 256-byte aligned");
  DLC_REQUIRE(B * n_q <= 65535, DLC_E_UNSUPPORTED, "csa_index_topk: B*n_q > 65535");

  hipStream_t s = as_stream(stream);
  char* w = static_cast<char*>(ws);
  IdxArgs a{};
  a.qI = qI; a.wI = wI; a.KI = KI; a.t = t;
  a.n_q = n_q; a.n_hI = n_hI; a.cI = cI; a.m = m; a.k = k; a.cap = cap; a.t_max = t_max;
  a.scores = scores ? scores : reinterpret_cast<float*>(w + L.scores);
  a.score_ld = cap;
  a.hist = reinterpret_cast<uint32_t*>(w + L.hist);
  a.cnt = reinterpret_cast<uint32_t*>(w + L.cnt);
  a.sel = reinterpret_cast<int32_t*>(w + L.sel);
  a.cand = reinterpret_cast<int32_t*>(w + L.cand);
  a.idx = idx; a.count = count;
  const int64_t BQ = B * n_q;

  // hist and cnt are adjacent: one clear covers both
  int rc = fill_u32(a.hist, 0, int64_t((L.sel - L.hist) / 4), s);
  if (rc) return rc;

  const int64_t vis_max = t_max / m;
  if (vis_max > 0) {
    const bool mfma = mfma_shape && aligned(qI, 16) && aligned(KI, 16);
    DLC_REQUIRE(mfma || n_hI * cI <= 8192, DLC_E_UNSUPPORTED, "csa_index_topk: MFMA shape needs 16-byte alignment");
    // aim for about 1024 workgroups in flight over the whole batch
    const int64_t tiles = ceil_div(vis_max, 16) * BQ;
    int64_t tiles_per_wave = tiles / (1024 * 4);
    tiles_per_wave = tiles_per_wave < 1 ? 1 : (tiles_per_wave > 16 ? 16 : tiles_per_wave);
    a.keys_per_wg = tiles_per_wave * 4 * 16;
    const int64_t nchunks = ceil_div(vis_max, a.keys_per_wg);
    dim3 grid{(unsigned)nchunks, (unsigned)BQ, 1u};
    {
    StageTimer timer(DLC_STAGE_INDEX_SCORES, s);
    if (mfma) {
      const int HT = int(ceil_div(n_hI, 16)), KT = int(cI / 32);
#define DLC_SCORES(ht, kt) \
  if (HT == ht && KT == kt) hipLaunchKernelGGL((scores_mfma_kernel<ht, kt>), grid, dim3(256), 0, s, a);
      DLC_SCORES(1, 1) DLC_SCORES(1, 2) DLC_SCORES(1, 4) DLC_SCORES(1, 8)
      DLC_SCORES(2, 1) DLC_SCORES(2, 2) DLC_SCORES(2, 4) DLC_SCORES(2, 8)
      DLC_SCORES(3, 1) DLC_SCORES(3, 2) DLC_SCORES(3, 4) DLC_SCORES(3, 8)
      DLC_SCORES(4, 1) DLC_SCORES(4, 2) DLC_SCORES(4, 4) DLC_SCORES(4, 8)
#undef DLC_SCORES
    } else {
      const size_t smem = (kBins + n_hI * cI + n_hI) * 4;
      if (dtype == DLC_BF16)
        hipLaunchKernelGGL((scores_valu_kernel<bf16_raw>), grid, dim3(256), smem, s, a);
      else
        hipLaunchKernelGGL((scores_valu_kernel<float>), grid, dim3(256), smem, s, a);
    }
    }
    if ((rc = check_launch("csa_index_topk/scores"))) return rc;
  }
  StageTimer timer(DLC_STAGE_TOPK_SELECT, s);
  if (vis_max > 0) {
    const int64_t nchunks = ceil_div(vis_max, a.keys_per_wg);
    dim3 grid{(unsigned)nchunks, (unsigned)BQ, 1u};
    hipLaunchKernelGGL(filter_kernel, grid, dim3(256), 0, s, a);
    if ((rc = check_launch("csa_index_topk/filter"))) return rc;
  }
  int P = 1;
  while (P < k) P <<= 1;
  const size_t fsmem = (kBins + 1024 + 4) * 4 + size_t(P) * 4;
  hipLaunchKernelGGL(finish_kernel, dim3((unsigned)BQ), dim3(1024), fsmem, s, a);
  return check_launch("csa_index_topk/finish");
}

}  // extern "C"
