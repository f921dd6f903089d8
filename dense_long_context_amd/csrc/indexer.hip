// Lightning indexer and exact top-k over the CSA cache.
//
// "DeepSeek-V4 Hybrid Attention: CSA and HCA from Scratch", §6.4 (score
// I[s] = sum_h w[h] * ReLU(q[h] . K[s])) and §7 (keep the k largest over the
// visible entries s < floor(t/m)).
//
// Pipeline per call (all on the caller's stream):
//   1. clear      zero the two digit histograms of every query
//   2. scores     one pass over K^I: for bf16 with c^I % 32 == 0 the heads x keys
//                 product runs on MFMA (v_mfma_f32_16x16x32_bf16) with the
//                 queries held in registers; otherwise a VALU kernel; with
//                 MXFP4 operands (csa_index_topk_fp4, §6.4's FP4 indexer) on
//                 the block-scaled v_mfma_scale_f32_16x16x128_f8f6f4.  Each
//                 workgroup also builds an LDS histogram of the top 11 bits of
//                 the order-preserving score key and adds its non-zero bins to
//                 the query's histogram.
//   3. filter     every workgroup finds the threshold bin T from that
//                 histogram and writes its chunk's entries above T (selected)
//                 and in T (candidates, with their keys) to the chunk's own
//                 segments in index order; the candidates' next 11 key bits go
//                 into the query's second histogram.
//   4. finish     one workgroup per query gathers the chunk lists, resolves the
//                 candidates by radix passes over the remaining key bits and
//                 then the index (ties go to the smaller index), starting from
//                 the second histogram, and merges the two ascending lists into
//                 idx / count.
#include "common.hpp"
#include "mxfp4.hpp"

namespace dlc {
namespace {

constexpr int kBins = 2048;      // first digit: top 11 bits of the key
constexpr int kShift1 = 21;
constexpr int kMaxK = 8192;
#ifndef DLC_PREFILL_NB
#define DLC_PREFILL_NB 2  // stages of the prefill scores kernel's query ring
#endif
#ifndef DLC_PREFILL_HPS
#define DLC_PREFILL_HPS 2  // heads per stage of that ring
#endif

struct IdxArgs {
  const void* qI;      // [BQ][n_hI][cI]
  const float* wI;     // [BQ][n_hI]
  const void* KI;      // [B][cap][cI] (FP4: [B][cap][cI/2] code bytes)
  const uint8_t* k_scale;  // FP4: [B][cap][cI/32] E8M0 scale bytes
  const uint8_t* q_code;   // FP4: [BQ][n_hI][cI/2] query code bytes
  const uint8_t* q_scale;  // FP4: [BQ][n_hI][cI/32] query scale bytes
  const int64_t* t;    // [BQ]
  int64_t n_q, n_hI, cI, m, k, cap, t_max;
  float* scores;       // [BQ][score_ld]
  int64_t score_ld;
  uint32_t* hist;      // [BQ][kBins] first-digit histogram (top 11 key bits)
  uint32_t* hist2;     // [BQ][kBins] second digit (key bits 20..10) of the entries in bin T
  uint32_t* ccnt;      // [BQ][max_chunks][2] per-chunk counts: selected, candidates
  int32_t* sel;        // [BQ][cap] chunk c's selected entries start at c*keys_per_wg
  int32_t* cand;       // [BQ][cap] chunk c's candidates start at c*keys_per_wg
  uint32_t* cand_kseg; // [BQ][cap] their score keys, same positions
  int32_t* cand_idx;   // [BQ][cap] compacted candidates when they overflow LDS
  uint32_t* cand_key;  // [BQ][cap] their score keys
  int32_t* idx;        // [BQ][k]
  int32_t* count;      // [BQ]
  int64_t keys_per_wg; // scores / filter chunk
  int64_t max_chunks;
};

__device__ __forceinline__ int64_t visible(const IdxArgs& a, int64_t bq) {
  int64_t t = a.t[bq];
  t = t < 0 ? 0 : (t > a.t_max ? a.t_max : t);
  int64_t v = t / a.m;
  return v < a.cap ? v : a.cap;
}

__device__ __forceinline__ float canon_zero(float s) { return s == 0.f ? 0.f : s; }

// ReLU of an MFMA result in one instruction: v_med3_f32(x, 0, 3e38) is x for
// 0 <= x <= 3e38 and 0 below (a signed zero may come out as -0, which the
// final canon_zero maps to +0).  fmaxf(x, 0), or a median with +inf (which
// the compiler folds into that max), costs two: the compiler first
// canonicalises x for the IEEE max.
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 3.0e38f); }

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
// x K^T[32 dims][16 keys] (v_mfma_f32_16x16x32_bf16) for every head tile and
// 32-dim step.  Lane l holds head/key l%16 of the A/B operands and dims
// 8*(l/16) .. +7 of each 32-dim step; the result holds key l%16 and heads
// 4*(l/16) .. +3, and the head sum is finished with two cross-lane adds.
// Queries stay in registers for the whole pass; they arrive once per
// workgroup, wave w moving heads 16w .. 16w+15 into the last stage of its
// ring, from where every wave reads its operands.  Key tiles (16 keys,
// 16*2*c^I bytes) arrive by direct global->LDS loads, one instruction moving
// 1 KB of consecutive rows, so HBM sees whole lines.  Each wave streams its
// own tiles through a ring of NS LDS stages, and only it reads them, so the
// loop has no barrier.  A tile's operands are read into registers first and
// its stage refilled right away, so NS tiles are in flight during the
// compute.  Within a row, 16-byte chunk c is stored at slot
// c ^ (row % chunks): the 16 rows that one ds_read_b128 pass reads at the
// same chunk then fall on distinct banks (64 banks of 4 bytes).
// The scores of kScoreBuf tiles collect in LDS and go out together: vmcnt
// counts stores too, so a store per tile between the tile loads would make
// every wait for a tile also wait for part of the next one.

constexpr int kScoreBuf = 32;  // tiles whose scores a wave collects before storing them

template <int HT, int KT, int NS>
__global__ void __launch_bounds__(256) scores_mfma_kernel(IdxArgs a) {
  constexpr int ROWB = KT * 64;     // bytes per key row (2 * c^I)
  constexpr int CPR = KT * 4;       // 16-byte chunks per row
  constexpr int TILEB = 16 * ROWB;  // one tile: 16 keys
  constexpr int RPI = 1024 / ROWB;  // rows per 1 KB load (KT loads per tile)
  static_assert(RPI * KT == 16, "tile geometry");
  static_assert(HT <= 4, "one 16-head block of queries per wave");
  __shared__ uint32_t hist[kBins];
  __shared__ __attribute__((aligned(1024))) unsigned char sK[4][NS][TILEB];
  __shared__ float sS[4][kScoreBuf * 16];
  const int64_t bq = blockIdx.y;
  const int64_t s0 = int64_t(blockIdx.x) * a.keys_per_wg;
  // The grid covers floor(t_max/m) <= cap entries, so rows below s1l exist
  // whatever this query's t: the first tiles go out by that bound, before
  // t has been read (rows past the query's own visible end are loaded and
  // scored but neither stored nor counted).
  const int64_t s1l = min(min(a.t_max / a.m, a.cap), s0 + a.keys_per_wg);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int cI = KT * 32;

  const int64_t b = bq / a.n_q;
  const bf16_raw* K = static_cast<const bf16_raw*>(a.KI) + b * a.cap * cI;
  // this wave's tiles: wave, wave+4, ... (the four waves stream one region together)
  auto tiles_of_wave = [&](int64_t end) {
    const int64_t nt = (end - s0 + 15) / 16;
    return nt > wave ? (nt - wave + 3) / 4 : int64_t(0);
  };
  // load j of a tile: lane -> row rho = j*RPI + lane/CPR, slot lane%CPR, which
  // holds chunk slot ^ (rho % CPR) of that row; rows past s1l repeat row
  // s1l - 1
  auto issue = [&](int64_t it, int st) {
    const int64_t row0 = s0 + (wave + 4 * it) * 16;  // < s1l
    const bf16_raw* base = K + row0 * cI;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const int rho = j * RPI + lane / CPR;
      const int chunk = (lane % CPR) ^ (rho % CPR);
      const int64_t row = min(row0 + rho, s1l - 1);
      const uint32_t off = uint32_t((row - row0) * ROWB + chunk * 16);
      const uint32_t lds = (uint32_t)(uintptr_t)DLC_LDS(&sK[wave][st][0]) + uint32_t(j * 1024);
      dma_row(base, off, lds);
    }
  };
  // queries: wave w < HT moves heads 16w .. 16w+15 (rows past n_hI repeat
  // head n_hI-1) into the last stage of its ring, rows in order
  if (wave < HT) {
    const bf16_raw* qg = static_cast<const bf16_raw*>(a.qI) + bq * a.n_hI * cI;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const int h = min(wave * 16 + j * RPI + lane / CPR, int(a.n_hI) - 1);
      const uint32_t off = uint32_t(h * ROWB + (lane % CPR) * 16);
      const uint32_t lds = (uint32_t)(uintptr_t)DLC_LDS(&sK[wave][NS - 1][0]) + uint32_t(j * 1024);
      dma_row(qg, off, lds);
    }
  }
  {
    const int64_t first = tiles_of_wave(s1l);
#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
      if (p < first) issue(p, p);
  }
  const int64_t nvis = visible(a, bq);
  if (s0 >= nvis) {  // nothing of this chunk is visible to the query (the whole workgroup)
    wait_vm<0>();
    return;
  }
  const int64_t s1 = min(nvis, s0 + a.keys_per_wg);
  const int64_t my_tiles = tiles_of_wave(s1);  // <= the tiles issued by s1l
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) hist[i] = 0;
  float wv[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = ht * 16 + g * 4 + r;
      wv[ht][r] = h < a.n_hI ? a.wI[bq * a.n_hI + h] : 0.f;
    }
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int r = 0; r < 4; ++r) asm volatile("" ::"v"(wv[ht][r]));
  wait_vm<0>();     // the query block and the first tiles
  __syncthreads();  // every wave's query rows landed; hist cleared
  // A operand, rows = heads: head ht*16 + r16 from wave ht's block; heads past
  // n_hI are zeroed (their weight is 0 too)
  bf16x8 qf[HT][KT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const bool pad = ht * 16 + r16 >= a.n_hI;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const uint4 v = *reinterpret_cast<const uint4*>(&sK[ht][NS - 1][r16 * ROWB + kt * 64 + g * 16]);
      qf[ht][kt] = __builtin_bit_cast(bf16x8, pad ? make_uint4(0, 0, 0, 0) : v);
    }
  }
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) asm volatile("" ::"v"(qf[ht][kt]));
  __syncthreads();  // every wave holds its operands: the last stages may take tiles
  if (NS - 1 < my_tiles) issue(NS - 1, NS - 1);

  for (int64_t it = 0; it < my_tiles; ++it) {
    const int st = int(it % NS);
    // tiles it+1 .. it+NS-1 (those that exist) were issued after tile it;
    // tile it has landed once at most their loads are outstanding (tiles
    // issued by s1l past my_tiles only make the wait longer)
    const int64_t rest = my_tiles - 1 - it;
    const int after = rest < NS - 1 ? int(rest) : NS - 1;
    static_assert(NS == 4, "the waits below enumerate three tiles in flight");
    if (after == 3) wait_vm<3 * KT>();
    else if (after == 2) wait_vm<2 * KT>();
    else if (after == 1) wait_vm<KT>();
    else wait_vm<0>();
    asm volatile("" ::: "memory");
    // the tile's operands into registers; the stage then takes tile it+NS,
    // so NS tiles stay in flight while this one is computed
    const unsigned char* tile = &sK[wave][st][0];
    bf16x8 kb[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int slot = (4 * kt + g) ^ (r16 % CPR);
      kb[kt] = *reinterpret_cast<const bf16x8*>(tile + r16 * ROWB + slot * 16);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the reads are done
    asm volatile("" ::: "memory");
    if (it + NS < my_tiles) issue(it + NS, st);
    f32x4 acc[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ht][kt], kb[kt], acc[ht], 0, 0, 0);
    // four independent partial sums (one per head row of the lane), then a tree
    float ps[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ps[r] = wv[0][r] * relu(acc[0][r]);
#pragma unroll
      for (int ht = 1; ht < HT; ++ht) ps[r] = fmaf(wv[ht][r], relu(acc[ht][r]), ps[r]);
    }
    const float part = rows4_sum((ps[0] + ps[1]) + (ps[2] + ps[3]));
    const int64_t s = s0 + (wave + 4 * it) * 16 + r16;
    const int slot = int(it % kScoreBuf);
    if (g == 0) {
      const float score = canon_zero(part);
      sS[wave][slot * 16 + r16] = score;
      if (s < s1) atomicAdd(&hist[order_key(score) >> kShift1], 1u);
    }
    if (slot == kScoreBuf - 1 || it + 1 == my_tiles) {
      // the wave's buffered tiles it-slot .. it, 16 scores each (the LDS
      // accesses of one wave run in order)
      asm volatile("" ::: "memory");
      const int64_t t0 = it - slot;
#pragma unroll
      for (int q = 0; q < kScoreBuf / 4; ++q) {
        const int idx = q * 64 + lane, tl = idx >> 4;
        const int64_t sk = s0 + (wave + 4 * (t0 + tl)) * 16 + (idx & 15);
        if (tl <= slot && sk < s1) a.scores[bq * a.score_ld + sk] = sS[wave][idx];
      }
      asm volatile("" ::: "memory");
    }
  }
  wait_vm<0>();  // tiles issued by s1l that no iteration waited for
  flush_hist(hist, a.hist + bq * kBins);
}

// ---------------------------------------------------------------- scores (FP4)
//
// MXFP4 operands on v_mfma_scale_f32_16x16x128_f8f6f4: D[16 heads][16 keys]
// += Q[16 heads][128 dims] x K^T[128 dims][16 keys], each operand carrying one
// E8M0 scale per 32 dims, so every product is exact and only the fp32 sums
// round.  Lane l supplies head/key l%16 and the 32-dim block l/16 of each
// 128-dim step: 16 code bytes and one scale byte.  The streaming is that of
// the bf16 kernel: a 16-key tile (16 code rows of c^I/2 bytes, then their 16
// scale rows of c^I/32 bytes) arrives by direct global->LDS loads into the
// wave's own ring of NS stages, NS-1 tiles in flight, no barrier.  Within a
// code row, 16-byte chunk c sits at slot c ^ ((row / RPB) % CPR) (RPB rows
// per 256 bytes, CPR chunks per row), so the 16 rows of one ds_read_b128
// pass fall on distinct banks.  The queries arrive quantized
// (mxfp4_quantize, run on them just before).  Result layout, head sum and
// the buffered score stores as in the bf16 kernel.

typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int CI, int NS, int NW>
__global__ void __launch_bounds__(64 * NW) scores_fp4_kernel(IdxArgs a) {
  constexpr int KB = CI / 32;               // scale bytes (32-dim blocks) per row
  constexpr int ROWB = CI / 2;              // code bytes per row
  constexpr int CPR = ROWB / 16;            // 16-byte chunks per code row
  constexpr int RPB = 256 / ROWB;           // code rows per 256 bytes (the bank width)
  constexpr int NJ = CI / 128;              // 128-dim MFMA steps = 1 KB code loads per tile
  constexpr int CODEB = 16 * ROWB;          // code bytes of a tile
  constexpr int STB = CODEB + 16 * KB;      // stage: codes, then scales
  constexpr int SLANES = 16 * KB / 4;       // lanes of the scale load (4 bytes each)
  constexpr int HT = 4;                     // head tiles: up to 64 heads
  static_assert(CI == 128 || CI == 256, "c^I");
  __shared__ uint32_t hist[kBins];
  __shared__ __attribute__((aligned(16))) unsigned char sK[NW][NS][STB];
  __shared__ float sS[NW][kScoreBuf * 16];
  const int64_t bq = blockIdx.y;
  const int64_t s0 = int64_t(blockIdx.x) * a.keys_per_wg;
  // rows below s1l exist whatever this query's t (as in the bf16 kernel):
  // the first tiles go out before t has been read
  const int64_t s1l = min(min(a.t_max / a.m, a.cap), s0 + a.keys_per_wg);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t b = bq / a.n_q;
  const uint8_t* Kc = static_cast<const uint8_t*>(a.KI) + b * a.cap * ROWB;
  const uint8_t* Ks = a.k_scale + b * a.cap * KB;
  auto tiles_of_wave = [&](int64_t end) {
    const int64_t nt = (end - s0 + 15) / 16;
    return nt > wave ? (nt - wave + NW - 1) / NW : int64_t(0);
  };
  // tile it of this wave: rows row0 .. row0+15 (rows past s1l repeat row s1l - 1)
  auto issue = [&](int64_t it, int st) {
    const int64_t row0 = s0 + (wave + NW * it) * 16;  // < s1l
    const uint32_t lds = (uint32_t)(uintptr_t)DLC_LDS(&sK[wave][st][0]);
#pragma unroll
    for (int q = 0; q < NJ; ++q) {
      const int pos = q * 1024 + 16 * lane;
      const int rho = pos / ROWB, slot = (pos % ROWB) / 16;
      const int chunk = slot ^ ((rho / RPB) % CPR);
      const int64_t row = min(row0 + rho, s1l - 1);
      dma_row(Kc + row0 * ROWB, uint32_t((row - row0) * ROWB + chunk * 16), lds + uint32_t(q * 1024));
    }
    if (lane < SLANES) {
      const int rho = 4 * lane / KB;
      const int64_t row = min(row0 + rho, s1l - 1);
      dma_dword(Ks + row0 * KB, uint32_t((row - row0) * KB + (4 * lane) % KB), lds + uint32_t(CODEB));
    }
  };
  {
    const int64_t first = tiles_of_wave(s1l);
#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
      if (p < first) issue(p, p);
  }
  const int64_t nvis = visible(a, bq);
  if (s0 >= nvis) {  // nothing of this chunk is visible to the query (the whole workgroup)
    wait_vm<0>();
    return;
  }
  const int64_t s1 = min(nvis, s0 + a.keys_per_wg);  // this query's end of the chunk
  const int64_t my_tiles = tiles_of_wave(s1);         // <= the tiles issued by s1l
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) hist[i] = 0;

  // queries (A operand, rows = heads): head ht*16 + r16, block 4j + g; heads
  // past n_hI take zero codes (their weight is 0 too)
  i32x8 qa[HT][NJ];
  int qs[HT][NJ];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int h = ht * 16 + r16;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int blk = 4 * j + g;
      uint4 c = make_uint4(0, 0, 0, 0);
      int e8 = 127;
      if (h < a.n_hI) {
        c = *reinterpret_cast<const uint4*>(a.q_code + (bq * a.n_hI + h) * ROWB + blk * 16);
        e8 = a.q_scale[(bq * a.n_hI + h) * KB + blk];
      }
      qa[ht][j] = i32x8{int(c.x), int(c.y), int(c.z), int(c.w), 0, 0, 0, 0};
      qs[ht][j] = e8;
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
  // wait for the query and weight loads (and with them the first tiles) here:
  // a wait for them inside the loop would drain the tile loads in flight
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
    for (int r = 0; r < 4; ++r) asm volatile("" ::"v"(wv[ht][r]));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      asm volatile("" ::"v"(qa[ht][j][0]), "v"(qa[ht][j][1]), "v"(qa[ht][j][2]), "v"(qa[ht][j][3]), "v"(qs[ht][j]));
  }
  __syncthreads();  // hist cleared

  constexpr int LPT = NJ + 1;  // loads per tile and lane (the scale load counts for every lane)
  for (int64_t it = 0; it < my_tiles; ++it) {
    const int st = int(it % NS);
    const int64_t nxt = it + NS - 1;
    int after;  // tiles issued after tile it
    if (nxt < my_tiles) {
      issue(nxt, int(nxt % NS));
      after = NS - 1;
    } else {
      after = int(my_tiles - 1 - it);
    }
    if (after >= NS - 1) wait_vm<(NS - 1) * LPT>();
    else if (after == 2) wait_vm<2 * LPT>();
    else if (after == 1) wait_vm<LPT>();
    else wait_vm<0>();
    asm volatile("" ::: "memory");
    const unsigned char* tile = &sK[wave][st][0];
    f32x4 acc[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int blk = 4 * j + g;
      const int slot = blk ^ ((r16 / RPB) % CPR);
      const uint4 k4 = *reinterpret_cast<const uint4*>(tile + r16 * ROWB + slot * 16);
      const int ksc = tile[CODEB + r16 * KB + blk];
      const i32x8 kb = i32x8{int(k4.x), int(k4.y), int(k4.z), int(k4.w), 0, 0, 0, 0};
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        acc[ht] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[ht][j], kb, acc[ht], 4, 4, 0, qs[ht][j], 0,
                                                                   ksc);
    }
    // four independent partial sums (one per head row of the lane), then a tree
    float ps[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ps[r] = wv[0][r] * relu(acc[0][r]);
#pragma unroll
      for (int ht = 1; ht < HT; ++ht) ps[r] = fmaf(wv[ht][r], relu(acc[ht][r]), ps[r]);
    }
    const float part = rows4_sum((ps[0] + ps[1]) + (ps[2] + ps[3]));
    const int64_t s = s0 + (wave + NW * it) * 16 + r16;
    const int slot = int(it % kScoreBuf);
    if (g == 0) {
      const float score = canon_zero(part);
      sS[wave][slot * 16 + r16] = score;
      if (s < s1) atomicAdd(&hist[order_key(score) >> kShift1], 1u);
    }
    if (slot == kScoreBuf - 1 || it + 1 == my_tiles) {
      asm volatile("" ::: "memory");
      const int64_t t0 = it - slot;
#pragma unroll
      for (int q = 0; q < kScoreBuf / 4; ++q) {
        const int idx = q * 64 + lane, tl = idx >> 4;
        const int64_t sk = s0 + (wave + NW * (t0 + tl)) * 16 + (idx & 15);
        if (tl <= slot && sk < s1) a.scores[bq * a.score_ld + sk] = sS[wave][idx];
      }
      asm volatile("" ::: "memory");
    }
  }
  wait_vm<0>();  // tiles issued by s1l that no iteration waited for
  flush_hist(hist, a.hist + bq * kBins);
}

// The FP4 call's preparation in one launch: blocks below fill_blocks clear
// the histograms; the others quantize the queries, one 32-element block per
// thread, with the encoding of mxfp4_quantize (codes [rows][c^I/2], scales
// [rows][c^I/32]).
template <typename T>
__global__ void __launch_bounds__(256) prep_fp4_kernel(uint32_t* hist, int64_t nhist, int fill_blocks, const T* q,
                                                       int64_t qblocks, int64_t bpr, uint8_t* codes,
                                                       uint8_t* scales) {
  if (int(blockIdx.x) < fill_blocks) {
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < nhist; i += int64_t(fill_blocks) * 256) hist[i] = 0;
    return;
  }
  const int64_t i = int64_t(blockIdx.x - fill_blocks) * 256 + threadIdx.x;
  if (i >= qblocks) return;
  const int64_t r = i / bpr, j = i % bpr;
  float v[32];
  load32<T>(q + (r * bpr + j) * 32, v);
  uint32_t e8;
  const uint4 c = mxfp4_encode32(v, e8);
  *reinterpret_cast<uint4*>(codes + (r * bpr + j) * 16) = c;
  scales[r * bpr + j] = uint8_t(e8);
}

// ---------------------------------------------------------------- scores (prefill)
//
// Many queries of one sequence (a prefill chunk; [Scratch] §6.4's cost
// paragraph: the indexer's term is quadratic in n).  Keys are now reused
// across queries, so the product is a real GEMM: a workgroup scores a tile
// of TQ = 64 queries x TK = 256 keys, looping over the heads:
//   S_h[32 queries][32 keys] = Q_h[32][16] . K^T[16][32]  (v_mfma_f32_32x32x16_bf16,
//   which on this part issues at about 1.7x the rate of the 16x16x32 form)
//   score[q][s] += w[q][h] * ReLU(S_h[q][s])
// Wave w owns queries 32*(w/4) .. +31 and keys 64*(w%4) .. +63 of the tile.
// Its K^T operands (64 keys x 128 dims, 64 VGPRs) stay in registers for all
// heads; each head's 64 x 128 query tile arrives by direct global->LDS loads
// two heads at a time into a double buffer of 32 KB stages, one barrier per
// stage; an odd head count is padded with a zero-weight copy of the last
// head.  The ReLU-and-weight epilogue of each
// head runs behind the next head's MFMAs.
// Within a query row, 16-byte chunk c sits at slot c ^ (row % 16), so the 16
// rows of one ds_read_b128 pass fall on distinct banks.  Only visible
// entries are written; hist_kernel then builds the first-digit histogram
// from the scores.  Grid: (key tiles, query tiles, B), key tiles fastest, so
// the workgroups resident on an XCD share one query tile in its L2.

template <int CI>
__global__ void __launch_bounds__(512) scores_prefill_kernel(IdxArgs a) {
  constexpr int KS = CI / 16;           // 16-dim steps of v_mfma_f32_32x32x16_bf16
  constexpr int TQ = 64, TK = 256, NW = 8, NB = DLC_PREFILL_NB;
  constexpr int QROWB = CI * 2;         // bytes of one query-head row
  constexpr int QTILEB = TQ * QROWB;    // one head's query tile
  constexpr int CPR = QROWB / 16;       // 16-byte chunks per row
  constexpr int ROWS_PER_LOAD = 1024 / QROWB;
  constexpr int LOADS_PER_HEAD = QTILEB / 1024 / NW;  // per wave
  constexpr int HPS = DLC_PREFILL_HPS;                 // heads per stage (even)
  constexpr int LPS = HPS * LOADS_PER_HEAD;           // per wave and stage
  static_assert(CPR == 16 && LOADS_PER_HEAD >= 1, "tile geometry for c^I = 128");
  static_assert(HPS % 2 == 0 && HPS <= 64, "heads per stage");
  __shared__ __attribute__((aligned(1024))) unsigned char sQ[NB][HPS][QTILEB];
  __shared__ float sW[64 + HPS][TQ];    // w[h][q]; rows n_hI .. stay 0 (head counts not a multiple of HPS)
  __shared__ int64_t sVis[TQ];
  __shared__ int64_t sMax;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, hi = lane >> 5;
  const int64_t b = blockIdx.z;
  const int64_t q0 = int64_t(blockIdx.y) * TQ;
  const int64_t k0 = int64_t(blockIdx.x) * TK;
  const int nq = int(min(int64_t(TQ), a.n_q - q0));
  const int n_hI = int(a.n_hI);
  const int ngroups = (n_hI + HPS - 1) / HPS;  // heads go in groups of HPS; a short last group is padded
                                               // with zero-weight copies of the last head
  if (tid == 0) sMax = 0;
  __syncthreads();
  if (tid < TQ) {
    const int64_t v = tid < nq ? visible(a, b * a.n_q + q0 + tid) : 0;
    sVis[tid] = v;
    atomicMax(reinterpret_cast<unsigned long long*>(&sMax), (unsigned long long)v);
  }
  for (int i = tid; i < TQ * (64 + HPS); i += NW * 64) {
    const int h = i / TQ, q = i % TQ;
    sW[h][q] = (q < nq && h < n_hI) ? a.wI[(b * a.n_q + q0 + q) * n_hI + h] : 0.f;
  }
  __syncthreads();
  if (k0 >= sMax) return;  // no query of the tile sees these keys

  // the query tiles of head group p -> stage p % NB: load j of a wave covers
  // rows ROWS_PER_LOAD*(wave*LOADS_PER_HEAD + j) ..; rows past the tile's
  // queries repeat its last query, a head past n_hI repeats the last head
  const bf16_raw* qbase = static_cast<const bf16_raw*>(a.qI) + (b * a.n_q + q0) * n_hI * CI;
  const uint32_t lds0 = (uint32_t)(uintptr_t)DLC_LDS(&sQ[0][0][0]);
  auto issue = [&](int p) {
#pragma unroll
    for (int u = 0; u < HPS; ++u) {
      const bf16_raw* base = qbase + min(HPS * p + u, n_hI - 1) * CI;
#pragma unroll
      for (int j = 0; j < LOADS_PER_HEAD; ++j) {
        const int ld = wave * LOADS_PER_HEAD + j;
        const int row = ld * ROWS_PER_LOAD + lane / CPR;
        const int chunk = (lane % CPR) ^ (row % CPR);
        const int qr = min(row, nq - 1);
        const uint32_t off = uint32_t(qr * n_hI * QROWB + chunk * 16);
        dma_row(base, off, lds0 + uint32_t(((p % NB) * HPS + u) * QTILEB + ld * 1024));
      }
    }
  };
  const int npre = min(NB - 1, ngroups);
  for (int p = 0; p < npre; ++p) issue(p);

  // K^T operands (B, 16 dims x 32 keys per step) of this wave: key
  // k0 + 64*(wave%4) + 32*j + r32, dims 16*ks + 8*hi .. +7
  const bf16_raw* Kb = static_cast<const bf16_raw*>(a.KI) + b * a.cap * CI;
  bf16x8 kf[2][KS];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t key = min(k0 + 64 * (wave & 3) + 32 * j + r32, a.cap - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[j][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Kb + key * CI + 16 * ks + 8 * hi));
  }
  // wait for the key operands (and the first query tiles) once, outside the head loop
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(kf[j][ks]));

  f32x16 sc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[j][r] = 0.f;
  const int qw = 32 * (wave >> 2);  // the wave's first query row in the tile
  const int qrow = qw + r32;        // the query row this lane supplies to the A operand

  // one head's S^T tiles, and its epilogue: score += w[q][h] * ReLU(S_h)
  auto head_mfma = [&](const unsigned char* tile, f32x16 (&S)[2]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int slot = (2 * ks + hi) ^ (qrow % CPR);
      const bf16x8 qa = *reinterpret_cast<const bf16x8*>(tile + qrow * QROWB + slot * 16);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        S[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[j][ks], ks == 0 ? f32x16{} : S[j], 0, 0, 0);
    }
  };
  // S[j] lane: key 32j + r32 of the wave's keys, queries qw + 8(r/4) + 4hi + r%4
  auto head_epilogue = [&](int h, const f32x16 (&S)[2]) {
    const float* wrow = &sW[h][qw + 4 * hi];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const float4 w = *reinterpret_cast<const float4*>(wrow + 8 * r4);
      const float wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < 2; ++j) sc[j][4 * r4 + e] = fmaf(wv[e], relu(S[j][4 * r4 + e]), sc[j][4 * r4 + e]);
    }
  };
  // heads in groups of HPS (one barrier per group); the epilogue of each
  // head runs behind the next head's MFMAs
  f32x16 Sa[2], Sb[2];
  for (int p = 0; p < ngroups; ++p) {
    const int after = min(NB - 2, ngroups - 1 - p);  // groups issued after group p
    if (after >= 2) wait_vm<2 * LPS>();
    else if (after == 1) wait_vm<LPS>();
    else wait_vm<0>();
    lds_barrier();  // every wave is past group p-1: its stage takes group p+NB-1
    if (p + NB - 1 < ngroups) issue(p + NB - 1);
#pragma unroll
    for (int u = 0; u < HPS; u += 2) {
      const int h = HPS * p + u;
      head_mfma(&sQ[p % NB][u][0], Sa);
      if (h > 0) head_epilogue(h - 1, Sb);
      head_mfma(&sQ[p % NB][u + 1][0], Sb);
      head_epilogue(h, Sa);
    }
  }
  if (ngroups > 0) head_epilogue(HPS * ngroups - 1, Sb);
  // visible entries only
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int qr = qw + 8 * (r >> 2) + 4 * hi + (r & 3);
    if (qr >= nq) continue;
    const int64_t nv = sVis[qr];
    float* out = a.scores + (b * a.n_q + q0 + qr) * a.score_ld;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t key = k0 + 64 * (wave & 3) + 32 * j + r32;
      if (key < nv) out[key] = canon_zero(sc[j][r]);
    }
  }
}

// The same query tiling with MXFP4 operands (csa_index_topk_fp4 at many
// queries): S_h[32 q][32 keys] on v_mfma_scale_f32_32x32x64_f8f6f4, lane l
// supplying row/column l%32 and the 32-dim block l/32 of a 64-dim step (16
// code bytes and its E8M0 scale byte).  The wave's key operands (64 keys x
// c^I: codes and scales) stay in registers; HPS heads' query codes (64 rows
// of c^I/2 bytes, chunk c at slot c ^ ((row/4) % 4)) and scales arrive per
// stage by direct global->LDS loads, double-buffered.

template <int CI>
__global__ void __launch_bounds__(512) scores_prefill_fp4_kernel(IdxArgs a) {
  constexpr int KB = CI / 32;           // scale bytes (32-dim blocks) per row
  constexpr int ROWB = CI / 2;          // code bytes per row
  constexpr int CPR = ROWB / 16;        // 16-byte chunks per code row
  constexpr int NJ = CI / 64;           // 64-dim MFMA steps
  constexpr int TQ = 64, TK = 256, NW = 8, NB = 2, HPS = 8;
  constexpr int QCODEB = TQ * ROWB;     // one head's query codes (4 KB at c^I = 128)
  constexpr int QSCB = TQ * KB;         // its scales (256 B)
  constexpr int HEADB = QCODEB + QSCB;
  constexpr int CODE_LOADS = QCODEB / 1024;  // 1 KB loads per head
  static_assert(CI == 128 && CPR == 4 && KB == 4, "tile geometry for c^I = 128");
  static_assert(HPS * (CODE_LOADS + 1) == 5 * NW, "one stage is five loads per wave");
  __shared__ __attribute__((aligned(1024))) unsigned char sQ[NB][HPS][HEADB];
  __shared__ float sW[64 + HPS][TQ];
  __shared__ int64_t sVis[TQ];
  __shared__ int64_t sMax;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, hi = lane >> 5;
  const int64_t b = blockIdx.z;
  const int64_t q0 = int64_t(blockIdx.y) * TQ;
  const int64_t k0 = int64_t(blockIdx.x) * TK;
  const int nq = int(min(int64_t(TQ), a.n_q - q0));
  const int n_hI = int(a.n_hI);
  const int ngroups = (n_hI + HPS - 1) / HPS;
  if (tid == 0) sMax = 0;
  __syncthreads();
  if (tid < TQ) {
    const int64_t v = tid < nq ? visible(a, b * a.n_q + q0 + tid) : 0;
    sVis[tid] = v;
    atomicMax(reinterpret_cast<unsigned long long*>(&sMax), (unsigned long long)v);
  }
  for (int i = tid; i < TQ * (64 + HPS); i += NW * 64) {
    const int h = i / TQ, q = i % TQ;
    sW[h][q] = (q < nq && h < n_hI) ? a.wI[(b * a.n_q + q0 + q) * n_hI + h] : 0.f;
  }
  __syncthreads();
  if (k0 >= sMax) return;

  // stage p holds heads HPS*p .. +HPS-1 (a head past n_hI repeats the last
  // head, at zero weight); load u of wave w: head (5w+u)/5 ... laid out as
  // HPS*(CODE_LOADS+1) loads spread over the waves, each either 1 KB of codes
  // (16 query rows) or the head's 64 scale dwords
  const uint8_t* qc = a.q_code + (b * a.n_q + q0) * n_hI * ROWB;
  const uint8_t* qs = a.q_scale + (b * a.n_q + q0) * n_hI * KB;
  const uint32_t lds0 = (uint32_t)(uintptr_t)DLC_LDS(&sQ[0][0][0]);
  auto issue = [&](int p) {
#pragma unroll
    for (int u = 0; u < 5; ++u) {
      const int ld = wave * 5 + u;                       // 0 .. HPS*(CODE_LOADS+1)-1
      const int hh = ld / (CODE_LOADS + 1), part = ld % (CODE_LOADS + 1);
      const int h = min(HPS * p + hh, n_hI - 1);
      const uint32_t dst = lds0 + uint32_t(((p % NB) * HPS + hh) * HEADB);
      if (part < CODE_LOADS) {
        const int row = part * 16 + lane / CPR;
        const int chunk = (lane % CPR) ^ ((row >> 2) & 3);
        const int qr = min(row, nq - 1);
        dma_row(qc + h * ROWB, uint32_t(qr * n_hI * ROWB + chunk * 16), dst + uint32_t(part * 1024));
      } else {
        const int qr = min(lane, nq - 1);
        dma_dword(qs + h * KB, uint32_t(qr * n_hI * KB), dst + uint32_t(QCODEB));
      }
    }
  };
  const int npre = min(NB - 1, ngroups);
  for (int p = 0; p < npre; ++p) issue(p);

  // K^T operands: key k0 + 64*(wave%4) + 32*j + r32, block 2*ks + hi
  const uint8_t* Kc = static_cast<const uint8_t*>(a.KI) + b * a.cap * ROWB;
  const uint8_t* Ks = a.k_scale + b * a.cap * KB;
  i32x8 kf[2][NJ];
  int ksc[2][NJ];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t key = min(k0 + 64 * (wave & 3) + 32 * j + r32, a.cap - 1);
#pragma unroll
    for (int ks = 0; ks < NJ; ++ks) {
      const uint4 c = *reinterpret_cast<const uint4*>(Kc + key * ROWB + (2 * ks + hi) * 16);
      kf[j][ks] = i32x8{int(c.x), int(c.y), int(c.z), int(c.w), 0, 0, 0, 0};
      ksc[j][ks] = Ks[key * KB + 2 * ks + hi];
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int ks = 0; ks < NJ; ++ks)
      asm volatile("" ::"v"(kf[j][ks][0]), "v"(kf[j][ks][1]), "v"(kf[j][ks][2]), "v"(kf[j][ks][3]),
                   "v"(ksc[j][ks]));

  f32x16 sc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[j][r] = 0.f;
  const int qw = 32 * (wave >> 2);
  const int qrow = qw + r32;

  auto head_mfma = [&](const unsigned char* hb, f32x16 (&S)[2]) {
#pragma unroll
    for (int ks = 0; ks < NJ; ++ks) {
      const int slot = (2 * ks + hi) ^ ((qrow >> 2) & 3);
      const uint4 c = *reinterpret_cast<const uint4*>(hb + qrow * ROWB + slot * 16);
      const int qsc = hb[QCODEB + qrow * KB + 2 * ks + hi];
      const i32x8 qa = i32x8{int(c.x), int(c.y), int(c.z), int(c.w), 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 2; ++j)
        S[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, kf[j][ks], ks == 0 ? f32x16{} : S[j], 4, 4, 0,
                                                                qsc, 0, ksc[j][ks]);
    }
  };
  auto head_epilogue = [&](int h, const f32x16 (&S)[2]) {
    const float* wrow = &sW[h][qw + 4 * hi];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const float4 w = *reinterpret_cast<const float4*>(wrow + 8 * r4);
      const float wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < 2; ++j) sc[j][4 * r4 + e] = fmaf(wv[e], relu(S[j][4 * r4 + e]), sc[j][4 * r4 + e]);
    }
  };
  f32x16 Sa[2], Sb[2];
  for (int p = 0; p < ngroups; ++p) {
    if (p + 1 < ngroups) wait_vm<5>(); else wait_vm<0>();
    lds_barrier();
    if (p + NB - 1 < ngroups) issue(p + NB - 1);
#pragma unroll 1
    for (int u = 0; u < HPS; u += 2) {
      const int h = HPS * p + u;
      head_mfma(&sQ[p % NB][u][0], Sa);
      if (h > 0) head_epilogue(h - 1, Sb);
      head_mfma(&sQ[p % NB][u + 1][0], Sb);
      head_epilogue(h, Sa);
    }
  }
  if (ngroups > 0) head_epilogue(HPS * ngroups - 1, Sb);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int qr = qw + 8 * (r >> 2) + 4 * hi + (r & 3);
    if (qr >= nq) continue;
    const int64_t nv = sVis[qr];
    float* out = a.scores + (b * a.n_q + q0 + qr) * a.score_ld;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t key = k0 + 64 * (wave & 3) + 32 * j + r32;
      if (key < nv) out[key] = canon_zero(sc[j][r]);
    }
  }
}

// first-digit histogram of the scores, chunk by chunk (the prefill path; the
// other scores kernels build it as they go)
__global__ void __launch_bounds__(256) hist_kernel(IdxArgs a) {
  __shared__ uint32_t hist[kBins];
  const int64_t bq = blockIdx.y;
  const int64_t nvis = visible(a, bq);
  const int64_t s0 = int64_t(blockIdx.x) * a.keys_per_wg;
  if (s0 >= nvis) return;
  const int64_t s1 = min(nvis, s0 + a.keys_per_wg);
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  const float* sc = a.scores + bq * a.score_ld;
  // 16 scores a thread per round (four 16-byte loads in flight together;
  // one at a time, the loop was load-latency bound); the scalar head and
  // tail of a misaligned or ragged chunk one by one
  auto count = [&](float x) { atomicAdd(&hist[order_key(x) >> kShift1], 1u); };
  // first 16-byte aligned score at or after s0
  int64_t a0 = s0 + int64_t(((16u - uint32_t(reinterpret_cast<uintptr_t>(sc + s0) & 15u)) & 15u) / 4u);
  if (a0 > s1) a0 = s1;
  for (int64_t s = s0 + threadIdx.x; s < a0; s += blockDim.x) count(sc[s]);
  const int64_t nv4 = (s1 - a0) / 4;
  const float4* p4 = reinterpret_cast<const float4*>(sc + a0);
  for (int64_t v0 = threadIdx.x; v0 < nv4; v0 += 4 * blockDim.x) {
    float4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t v = v0 + u * blockDim.x;
      x[u] = p4[v < nv4 ? v : nv4 - 1];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (v0 + u * blockDim.x < nv4) {
        count(x[u].x);
        count(x[u].y);
        count(x[u].z);
        count(x[u].w);
      }
    }
  }
  for (int64_t s = a0 + nv4 * 4 + threadIdx.x; s < s1; s += blockDim.x) count(sc[s]);
  flush_hist(hist, a.hist + bq * kBins);
}

// ---------------------------------------------------------------- threshold

// Finds the bin T with above(T) < need <= above(T) + h[T], where above(T)
// counts the entries in bins > T.  Every thread of the block gets (T, above).
// h is an LDS array of nbins (a multiple of blockDim.x, blockDim.x a multiple
// of 64 and at most 1024); scratch holds 16 + 2 words.  Each thread owns a
// run of nbins/blockDim.x bins; a suffix scan of the per-thread totals (wave
// shuffles, then the wave totals) locates the one thread whose run crosses
// `need`, and that thread walks its own bins.
__device__ void find_threshold(const uint32_t* h, int nbins, uint32_t need, uint32_t* scratch,
                               int* T_out, uint32_t* above_out) {
  const int per = nbins / blockDim.x;
  const int lo = threadIdx.x * per;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  uint32_t mine = 0;
  for (int i = 0; i < per; ++i) mine += h[lo + i];
  // inclusive suffix sum within the wave (this lane and those above it)
  const uint32_t pre = wave_incl_scan(mine);
  const uint32_t suf = wave_total(pre) - pre + mine;
  if (lane == 0) scratch[wave] = suf;  // the wave's total
  if (threadIdx.x == 0) {              // defaults if no bin qualifies (inconsistent counts)
    scratch[16] = 0;
    scratch[17] = 0;
  }
  __syncthreads();
  uint32_t higher = 0;
  for (int w = wave + 1; w < nwaves; ++w) higher += scratch[w];
  uint32_t run = higher + suf - mine;  // entries in bins owned by higher threads
  if (run < need && run + mine >= need) {
    for (int i = per - 1; i >= 0; --i) {
      const uint32_t v = h[lo + i];
      if (run < need && run + v >= need) {
        scratch[16] = uint32_t(lo + i);
        scratch[17] = run;
      }
      run += v;
    }
  }
  __syncthreads();
  *T_out = int(scratch[16]);
  *above_out = scratch[17];
  __syncthreads();
}

// The same search over a histogram the threads hold in registers: thread i
// owns bins PER*i .. PER*i + PER-1, given in v (nbins = PER * blockDim.x).
template <int PER>
__device__ void find_threshold_regs(const uint32_t (&v)[PER], uint32_t need, uint32_t* scratch, int* T_out,
                                    uint32_t* above_out) {
  const int lo = threadIdx.x * PER;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) mine += v[i];
  const uint32_t pre = wave_incl_scan(mine);
  const uint32_t suf = wave_total(pre) - pre + mine;
  if (lane == 0) scratch[wave] = suf;
  if (threadIdx.x == 0) {
    scratch[16] = 0;
    scratch[17] = 0;
  }
  __syncthreads();
  uint32_t higher = 0;
  for (int w = wave + 1; w < nwaves; ++w) higher += scratch[w];
  uint32_t run = higher + suf - mine;
  if (run < need && run + mine >= need) {
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      if (run < need && run + v[i] >= need) {
        scratch[16] = uint32_t(lo + i);
        scratch[17] = run;
      }
      run += v[i];
    }
  }
  __syncthreads();
  *T_out = int(scratch[16]);
  *above_out = scratch[17];
  __syncthreads();
}

// Ordered compaction helper: returns this thread's position among the threads
// of the block with pred set (in thread order) and, through *total, their
// count.  wtot holds blockDim.x/64 words.  Ends with the block synchronised.
__device__ __forceinline__ uint32_t block_rank(bool pred, uint32_t* wtot, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const uint64_t mask = __ballot(pred);
  if (lane == 0) wtot[wave] = uint32_t(__popcll(mask));
  __syncthreads();
  uint32_t before = 0, all = 0;
  for (int w = 0; w < nwaves; ++w) {
    const uint32_t x = wtot[w];
    before += w < wave ? x : 0u;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + uint32_t(__popcll(mask & ((uint64_t(1) << lane) - 1)));
}

// Block-wide exclusive scan of one value per thread (blockDim.x = 256);
// returns the block total.  wsum holds 4 words.  Ends synchronised.
__device__ __forceinline__ uint32_t scan256(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x = wsum[w];
    before += w < wave ? x : 0u;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// Every workgroup recomputes the threshold bin T of its query from the
// first-digit histogram, then splits its own chunk of keys into "above T"
// (selected for sure) and "in T" (candidates, stored with their keys).  Thread
// j takes entries 4j .. 4j+3 of each 1024-entry batch, so one scan of packed
// counts orders both lists by index.  Both lists go to the chunk's own
// segment and the two counts to the chunk's own slot: no global atomics for
// the lists, and the result does not depend on scheduling.  The candidates'
// second digit (key bits 20..10) is counted into the query's second
// histogram, which is the first radix pass of the finish.
__global__ void __launch_bounds__(256) filter_kernel(IdxArgs a) {
  static_assert(kBins == 8 * 256, "filter_kernel: eight first-digit bins per thread");
  __shared__ uint32_t h2[kBins];
  __shared__ uint32_t scratch[18];
  __shared__ uint32_t wsum[4];
  const int64_t bq = blockIdx.y;
  const int64_t nvis = visible(a, bq);
  const int64_t keff = min(a.k, nvis);
  const int64_t s0 = int64_t(blockIdx.x) * a.keys_per_wg;
  if (keff == nvis || s0 >= nvis) return;  // keep-all and empty chunks need no filtering
  const int64_t s1 = min(nvis, s0 + a.keys_per_wg);
  const float* sc = a.scores + bq * a.score_ld;
  // the first batches of scores are in flight while the threshold is found
  auto load4 = [&](int64_t base, float* v) {
    const int64_t s = base + 4 * threadIdx.x;
    if (s + 3 < s1 && (reinterpret_cast<uintptr_t>(sc + s) & 15) == 0) {
      const float4 x = *reinterpret_cast<const float4*>(sc + s);
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = s + e < s1 ? sc[s + e] : 0.f;
    }
  };
  // a ring of FD batches in registers: batch i+FD is loaded as batch i is
  // used (one batch at a time, the loop was load-latency bound)
  constexpr int FD = 4;
  float vb[FD][4];
#pragma unroll
  for (int d = 0; d < FD; ++d) load4(s0 + int64_t(d) * 4 * blockDim.x, vb[d]);
  // thread j holds first-digit bins 8j .. 8j+7 (two 16-byte loads)
  uint32_t hv[8];
  {
    const uint4* hp = reinterpret_cast<const uint4*>(a.hist + bq * kBins) + 2 * threadIdx.x;
    const uint4 x = hp[0], y = hp[1];
    hv[0] = x.x; hv[1] = x.y; hv[2] = x.z; hv[3] = x.w;
    hv[4] = y.x; hv[5] = y.y; hv[6] = y.z; hv[7] = y.w;
  }
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) h2[i] = 0;
  int T;
  uint32_t above;
  find_threshold_regs<8>(hv, uint32_t(keff), scratch, &T, &above);  // also orders the h2 clear

  int32_t* sel = a.sel + bq * a.cap + s0;
  int32_t* cand = a.cand + bq * a.cap + s0;
  uint32_t* ckey = a.cand_kseg + bq * a.cap + s0;
  uint32_t nsel = 0, ncand = 0;
  const int64_t step = 4 * int64_t(blockDim.x);
  for (int64_t round = s0; round < s1; round += FD * step) {
#pragma unroll
    for (int dd = 0; dd < FD; ++dd) {
      const int64_t base = round + dd * step;
      if (base >= s1) break;  // uniform
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = vb[dd][e];
      load4(base + FD * step, vb[dd]);  // past s1: zeros, no access
      const int64_t sb = base + 4 * threadIdx.x;
      uint32_t key[4], packed = 0;
      int d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        key[e] = order_key(v[e]);
        d[e] = sb + e < s1 ? int(key[e] >> kShift1) : -1;
        packed += d[e] > T ? 1u : 0u;
        packed += d[e] == T ? 0x10000u : 0u;
      }
      uint32_t tot;
      const uint32_t ex = scan256(packed, wsum, &tot);
      uint32_t ps = nsel + (ex & 0xffffu), pc = ncand + (ex >> 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (d[e] > T) sel[ps++] = int32_t(sb + e);
        if (d[e] == T) {
          cand[pc] = int32_t(sb + e);
          ckey[pc] = key[e];
          ++pc;
          atomicAdd(&h2[(key[e] >> 10) & 0x7ffu], 1u);
        }
      }
      nsel += tot & 0xffffu;
      ncand += tot >> 16;
    }
  }
  flush_hist(h2, a.hist2 + bq * kBins);
  if (threadIdx.x == 0) {
    a.ccnt[(bq * a.max_chunks + blockIdx.x) * 2 + 0] = nsel;
    a.ccnt[(bq * a.max_chunks + blockIdx.x) * 2 + 1] = ncand;
  }
}

// ---------------------------------------------------------------- finish

constexpr int kMaxChunks = 4096;
constexpr int kLdsCand = 4096;

// radix passes over the candidates' composite key: the low 21 bits of the score
// key (the top 11 bits are T for all of them), then the bit-inverted index
constexpr int kPasses = 5;
__device__ __forceinline__ int pass_shift(int p) { return p == 0 ? 42 : p == 1 ? 32 : p == 2 ? 21 : p == 3 ? 10 : 0; }
__device__ __forceinline__ int pass_bits(int p) { return (p == 1 || p == 4) ? 10 : 11; }

__device__ __forceinline__ uint64_t cand_key(uint32_t key, int32_t s) {
  return (uint64_t(key & 0x1fffffu) << 32) | uint64_t(0xffffffffu - uint32_t(s));
}

// Block-wide exclusive scans of two arrays v[0 .. n) and w[0 .. n) in place;
// the totals come back through tv and tw.  Thread j owns the runs at
// [j*per, (j+1)*per), per = ceil(n / blockDim.x); wsum holds 2*blockDim.x/64
// words.  Ends synchronised.
__device__ void block_exclusive_scan2(uint32_t* v, uint32_t* w, int n, uint32_t* wsum, uint32_t* tv,
                                      uint32_t* tw) {
  const int per = (n + int(blockDim.x) - 1) / int(blockDim.x);
  const int lo = threadIdx.x * per, hi = min(n, lo + per);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  uint32_t mv = 0, mw = 0;
  for (int i = lo; i < hi; ++i) {
    mv += v[i];
    mw += w[i];
  }
  const uint32_t iv = wave_incl_scan(mv), iw = wave_incl_scan(mw);
  if (lane == 63) {
    wsum[wave] = iv;
    wsum[nwaves + wave] = iw;
  }
  __syncthreads();
  uint32_t bv = 0, bw = 0, sv = 0, sw = 0;
  for (int k = 0; k < nwaves; ++k) {
    const uint32_t x = wsum[k], y = wsum[nwaves + k];
    if (k < wave) {
      bv += x;
      bw += y;
    }
    sv += x;
    sw += y;
  }
  uint32_t rv = bv + iv - mv, rw = bw + iw - mw;
  for (int i = lo; i < hi; ++i) {
    const uint32_t x = v[i], y = w[i];
    v[i] = rv;
    w[i] = rw;
    rv += x;
    rw += y;
  }
  __syncthreads();
  *tv = sv;
  *tw = sw;
}

// number of entries of the ascending list l[0 .. n) that are < x
__device__ __forceinline__ uint32_t lower_bound(const int32_t* l, uint32_t n, int32_t x) {
  uint32_t lo = 0, hi = n;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (l[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// One workgroup per query.  The "above T" lists of all chunks, in chunk order,
// form one ascending list; radix passes over the candidates find the exact
// k_eff-th composite key; the candidates at or above it are compacted in
// order into a second ascending list; the two lists are merged by rank.
__global__ void __launch_bounds__(1024) finish_kernel(IdxArgs a) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t scratch[18];
  __shared__ uint32_t wsum[32];
  __shared__ uint32_t off_sel[kMaxChunks], off_cand[kMaxChunks];
  __shared__ int32_t lsel[kMaxK], lc2[kMaxK];
  __shared__ int32_t lc_idx[kLdsCand];
  __shared__ uint32_t lc_key[kLdsCand];
  const int64_t bq = blockIdx.x;
  const int64_t nvis = visible(a, bq);
  const int64_t keff = min(a.k, nvis);
  int32_t* out = a.idx + bq * a.k;
  if (threadIdx.x == 0) a.count[bq] = int32_t(keff);
  if (keff == nvis) {
    for (int64_t j = threadIdx.x; j < a.k; j += blockDim.x) out[j] = j < nvis ? int32_t(j) : -1;
    return;
  }
  const int nch = int(ceil_div(nvis, a.keys_per_wg));
  const uint2* cc = reinterpret_cast<const uint2*>(a.ccnt + bq * a.max_chunks * 2);
  // the chunk counts and the candidates' first composite digit (counted by
  // the filter; pass 0 below) load together
  static_assert(kBins % 2 == 0, "bins in pairs");
  const uint2* h2g = reinterpret_cast<const uint2*>(a.hist2 + bq * kBins);
  for (int i = threadIdx.x; i < kBins / 2 || i < nch; i += blockDim.x) {
    uint2 x = make_uint2(0, 0), y = make_uint2(0, 0);
    if (i < nch) x = cc[i];
    if (i < kBins / 2) y = h2g[i];
    if (i < nch) {
      off_sel[i] = x.x;
      off_cand[i] = x.y;
    }
    if (i < kBins / 2) {
      h[2 * i] = y.x;
      h[2 * i + 1] = y.y;
    }
  }
  __syncthreads();
  uint32_t tsel, tcand;
  block_exclusive_scan2(off_sel, off_cand, nch, wsum, &tsel, &tcand);
  const uint32_t n_sel = min(tsel, uint32_t(keff));
  const uint32_t n_cand = min(tcand, uint32_t(nvis));
  const bool in_lds = n_cand <= uint32_t(kLdsCand);
  int32_t* cidx = in_lds ? lc_idx : a.cand_idx + bq * a.cap;
  uint32_t* ckey = in_lds ? lc_key : a.cand_key + bq * a.cap;
  // gather the chunks' lists: every thread takes independent entries and finds
  // its chunk by binary search over the exclusive offsets
  auto chunk_of = [&](const uint32_t* off, uint32_t i) {
    int lo = 0, hi = nch - 1;  // largest c with off[c] <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  // both lists in one sweep, four entries of each per thread per round, all
  // their loads in flight together
  constexpr int G = 4;
  const uint32_t n_both = n_sel > n_cand ? n_sel : n_cand;
  for (uint32_t i0 = threadIdx.x; i0 < n_both; i0 += G * blockDim.x) {
    int32_t vs[G], vi[G];
    uint32_t vk[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const uint32_t i = i0 + u * blockDim.x;
      if (i < n_sel) {
        const int c = chunk_of(off_sel, i);
        vs[u] = a.sel[bq * a.cap + int64_t(c) * a.keys_per_wg + (i - off_sel[c])];
      }
      if (i < n_cand) {
        const int c = chunk_of(off_cand, i);
        const int64_t at = bq * a.cap + int64_t(c) * a.keys_per_wg + (i - off_cand[c]);
        vi[u] = a.cand[at];
        vk[u] = a.cand_kseg[at];
      }
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const uint32_t i = i0 + u * blockDim.x;
      if (i < n_sel) lsel[i] = vs[u];
      if (i < n_cand) {
        cidx[i] = vi[u];
        ckey[i] = vk[u];
      }
    }
  }
  __threadfence_block();
  __syncthreads();

  // the exact threshold: after the passes, the selected candidates are those
  // whose composite key is >= thr
  uint32_t need = uint32_t(keff) - n_sel;
  uint64_t pval = 0, pmask = 0;
  for (int pass = 0; pass < kPasses; ++pass) {
    const int shift = pass_shift(pass), bits = pass_bits(pass);
    const uint32_t dmask = (1u << bits) - 1u;
    const int nb = 1 << bits;
    if (pass == 0) {
      // the filter already counted the candidates' first composite digit (h,
      // loaded with the chunk counts)
    } else {
      for (int i = threadIdx.x; i < kBins; i += blockDim.x) h[i] = 0;
      __syncthreads();
      for (uint32_t i = threadIdx.x; i < n_cand; i += blockDim.x) {
        const uint64_t ck = cand_key(ckey[i], cidx[i]);
        if ((ck & pmask) == pval) atomicAdd(&h[(ck >> shift) & dmask], 1u);
      }
      __syncthreads();
    }
    int D;
    uint32_t above;
    find_threshold(h, nb < 1024 ? 1024 : nb, need, scratch, &D, &above);
    const bool take_all = (above + h[D] == need);
    pval |= uint64_t(D) << shift;
    pmask |= uint64_t(dmask) << shift;
    if (take_all) break;
    need -= above;
  }
  const uint64_t thr = pval;

  // ordered compaction of the selected candidates
  uint32_t n2 = 0;
  for (uint32_t base = 0; base < n_cand; base += blockDim.x) {
    const uint32_t i = base + threadIdx.x;
    const bool take = i < n_cand && cand_key(ckey[i], cidx[i]) >= thr;
    uint32_t tot;
    const uint32_t r = block_rank(take, wsum, &tot);
    if (take && n2 + r < uint32_t(kMaxK)) lc2[n2 + r] = cidx[i];
    n2 += tot;
  }
  n2 = min(n2, uint32_t(keff) - n_sel);
  // merge two ascending lists by rank
  for (uint32_t i = threadIdx.x; i < n_sel; i += blockDim.x) {
    const int32_t x = lsel[i];
    out[i + lower_bound(lc2, n2, x)] = x;
  }
  for (uint32_t j = threadIdx.x; j < n2; j += blockDim.x) {
    const int32_t y = lc2[j];
    out[j + lower_bound(lsel, n_sel, y)] = y;
  }
  for (int64_t j = n_sel + n2 + threadIdx.x; j < a.k; j += blockDim.x) out[j] = -1;
}

// ---------------------------------------------------------------- host

struct WsLayout {
  size_t scores, hist, ccnt, sel, cand, cand_kseg, cand_idx, cand_key, total;
};

// keys per scores/filter workgroup: a multiple of 64 chosen so that the whole
// batch takes about kScoreWorkgroups workgroups - the number that are resident
// at once (2 per CU for the scores kernel, whose key stages take 64 KB of
// LDS), so there is no partial second round - and at most kMaxChunks chunks
// per query
#ifndef DLC_SCORES_WGS
#define DLC_SCORES_WGS 512
#endif
constexpr int64_t kScoreWorkgroups = DLC_SCORES_WGS;
// query-tiled (prefill) calls: the chunks of the histogram and filter
// kernels, sized for eight 256-thread workgroups per CU
constexpr int64_t kSelectWorkgroups = 2048;
// queries per sequence from which the indexer runs query-tiled (prefill)
#ifndef DLC_PREFILL_MIN_Q
#define DLC_PREFILL_MIN_Q 64
#endif
constexpr int64_t kPrefillMinQueries = DLC_PREFILL_MIN_Q;
#ifndef DLC_FP4_NS
#define DLC_FP4_NS 4  // LDS stages per wave in the FP4 scores kernel (NS-1 tiles in flight)
#endif
#ifndef DLC_FP4_NW
#define DLC_FP4_NW 8  // waves per workgroup of the FP4 scores kernel
#endif
// wgs: the workgroups the batch should take (kScoreWorkgroups for the
// decode scores kernel, which shares its chunks with the selection;
// kSelectWorkgroups when only the histogram and filter kernels use them)
int64_t keys_per_wg(int64_t BQ, int64_t vis_max, int64_t wgs = kScoreWorkgroups) {
  const int64_t vis = vis_max > 0 ? vis_max : 1;
  int64_t kpw = ceil_div(ceil_div(vis * BQ, wgs), 64) * 64;
  kpw = kpw < 64 ? 64 : kpw;
  const int64_t floor_kpw = ceil_div(ceil_div(vis, kMaxChunks), 64) * 64;
  return kpw > floor_kpw ? kpw : floor_kpw;
}

WsLayout ws_layout(int64_t B, int64_t n_q, int64_t cap, int64_t k, bool own_scores) {
  const size_t BQ = size_t(B) * size_t(n_q);
  (void)k;
  WsLayout L{};
  size_t off = 0;
  L.hist = off;      off = align_up(off + BQ * kBins * 2 * 4, 256);  // hist, then hist2
  L.ccnt = off;      off = align_up(off + BQ * kMaxChunks * 2 * 4, 256);
  L.sel = off;       off = align_up(off + BQ * size_t(cap) * 4, 256);
  L.cand = off;      off = align_up(off + BQ * size_t(cap) * 4, 256);
  L.cand_kseg = off; off = align_up(off + BQ * size_t(cap) * 4, 256);
  L.cand_idx = off;  off = align_up(off + BQ * size_t(cap) * 4, 256);
  L.cand_key = off;  off = align_up(off + BQ * size_t(cap) * 4, 256);
  L.scores = off;
  if (own_scores) off = align_up(off + BQ * size_t(cap) * 4, 256);
  L.total = off;
  return L;
}

// IdxArgs pointers into the workspace
void bind_ws(IdxArgs& a, const WsLayout& L, void* ws, float* scores, int64_t BQ, int64_t cap) {
  char* w = static_cast<char*>(ws);
  a.scores = scores ? scores : reinterpret_cast<float*>(w + L.scores);
  a.score_ld = cap;
  a.hist = reinterpret_cast<uint32_t*>(w + L.hist);
  a.hist2 = a.hist + size_t(BQ) * kBins;
  a.ccnt = reinterpret_cast<uint32_t*>(w + L.ccnt);
  a.sel = reinterpret_cast<int32_t*>(w + L.sel);
  a.cand = reinterpret_cast<int32_t*>(w + L.cand);
  a.cand_kseg = reinterpret_cast<uint32_t*>(w + L.cand_kseg);
  a.cand_idx = reinterpret_cast<int32_t*>(w + L.cand_idx);
  a.cand_key = reinterpret_cast<uint32_t*>(w + L.cand_key);
  a.max_chunks = kMaxChunks;
}

// threshold/filter and finish: scores (and the first histogram) -> idx, count
int select_topk(IdxArgs& a, int64_t BQ, int64_t vis_max, hipStream_t s) {
  int rc;
  StageTimer timer(DLC_STAGE_TOPK_SELECT, s);
  if (vis_max > 0) {
    const int64_t nchunks = ceil_div(vis_max, a.keys_per_wg);
    dim3 grid{(unsigned)nchunks, (unsigned)BQ, 1u};
    hipLaunchKernelGGL(filter_kernel, grid, dim3(256), 0, s, a);
    if ((rc = check_launch("csa_index_topk/filter"))) return rc;
  }
  if (vis_max == 0) a.keys_per_wg = 64;
  hipLaunchKernelGGL(finish_kernel, dim3((unsigned)BQ), dim3(1024), 0, s, a);
  return check_launch("csa_index_topk/finish");
}

// the FP4 call's workspace: the common layout, then the quantized queries
struct Fp4Ws {
  size_t code, scale, total;
};
Fp4Ws fp4_query_off(int64_t B, int64_t n_q, int64_t cap, int64_t k, int64_t n_hI, int64_t cI) {
  const size_t rows = size_t(B) * size_t(n_q) * size_t(n_hI);
  Fp4Ws w{};
  w.code = ws_layout(B, n_q, cap, k, true).total;
  w.scale = align_up(w.code + rows * size_t(cI / 2), 256);
  w.total = align_up(w.scale + rows * size_t(cI / 32), 256);
  return w;
}

}  // namespace
}  // namespace dlc

extern "C" {

size_t csa_index_topk_ws(int64_t B, int64_t n_q, int64_t cap, int64_t k) {
  if (B < 1 || n_q < 1 || cap < 0 || k < 1) return 0;
  return dlc::ws_layout(B, n_q, cap, k, true).total;
}

size_t csa_index_topk_fp4_ws(int64_t B, int64_t n_q, int64_t n_hI, int64_t cI, int64_t cap, int64_t k) {
  if (B < 1 || n_q < 1 || n_hI < 1 || cI < 32 || cap < 0 || k < 1) return 0;
  return dlc::fp4_query_off(B, n_q, cap, k, n_hI, cI).total;
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
  IdxArgs a{};
  a.qI = qI; a.wI = wI; a.KI = KI; a.t = t;
  a.n_q = n_q; a.n_hI = n_hI; a.cI = cI; a.m = m; a.k = k; a.cap = cap; a.t_max = t_max;
  const int64_t BQ = B * n_q;
  bind_ws(a, L, ws, scores, BQ, cap);
  a.idx = idx; a.count = count;

  int rc = fill_u32(a.hist, 0, int64_t(BQ * kBins * 2), s);
  if (rc) return rc;

  const int64_t vis_max = t_max / m;
  if (vis_max > 0) {
    const bool mfma = mfma_shape && aligned(qI, 16) && aligned(KI, 16);
    DLC_REQUIRE(mfma || n_hI * cI <= 8192, DLC_E_UNSUPPORTED, "csa_index_topk: MFMA shape needs 16-byte alignment");
    const bool prefill = mfma && cI == 128 && n_q >= kPrefillMinQueries;
    a.keys_per_wg = keys_per_wg(BQ, vis_max, prefill ? kSelectWorkgroups : kScoreWorkgroups);
    const int64_t nchunks = ceil_div(vis_max, a.keys_per_wg);
    dim3 grid{(unsigned)nchunks, (unsigned)BQ, 1u};
    {
    StageTimer timer(DLC_STAGE_INDEX_SCORES, s);
    if (prefill) {
      dim3 pgrid{(unsigned)ceil_div(vis_max, 256), (unsigned)ceil_div(n_q, 64), (unsigned)B};
      hipLaunchKernelGGL((scores_prefill_kernel<128>), pgrid, dim3(512), 0, s, a);
    } else if (mfma) {
      const int HT = int(ceil_div(n_hI, 16)), KT = int(cI / 32);
#define DLC_SCORES(ht, kt) \
  if (HT == ht && KT == kt) hipLaunchKernelGGL((scores_mfma_kernel<ht, kt, 4>), grid, dim3(256), 0, s, a);
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
    if (prefill) {  // the first-digit histogram, which the other scores kernels build as they go
      hipLaunchKernelGGL(hist_kernel, grid, dim3(256), 0, s, a);
      if ((rc = check_launch("csa_index_topk/hist"))) return rc;
    }
  }
  return select_topk(a, BQ, vis_max, s);
}

int csa_index_topk_fp4(int dtype, int64_t B, int64_t n_q, int64_t n_hI, int64_t cI, int64_t m, int64_t k,
                       const void* qI, const float* wI, const uint8_t* KIc, const uint8_t* KIs, int64_t cap,
                       const int64_t* t, int64_t t_max, int32_t* idx, int32_t* count, float* scores, void* ws,
                       size_t ws_bytes, void* stream) {
  using namespace dlc;
  DLC_REQUIRE(dtype == DLC_F32 || dtype == DLC_BF16, DLC_E_DTYPE, "csa_index_topk_fp4: unsupported dtype %d", dtype);
  DLC_REQUIRE(B >= 1 && n_q >= 1 && n_hI >= 1 && m >= 1 && cap >= 0 && t_max >= 0, DLC_E_INVAL,
              "csa_index_topk_fp4: need B, n_q, n_hI, m >= 1 and cap, t_max >= 0");
  DLC_REQUIRE(cI == 128 || cI == 256, DLC_E_UNSUPPORTED, "csa_index_topk_fp4: cI=%lld not in {128, 256}",
              (long long)cI);
  DLC_REQUIRE(n_hI <= 64, DLC_E_UNSUPPORTED, "csa_index_topk_fp4: n_hI=%lld > 64", (long long)n_hI);
  DLC_REQUIRE(k >= 1 && k <= kMaxK, DLC_E_UNSUPPORTED, "csa_index_topk_fp4: k=%lld outside [1, %d]", (long long)k,
              kMaxK);
  DLC_REQUIRE(t_max / m <= cap, DLC_E_SHAPE, "csa_index_topk_fp4: floor(t_max/m)=%lld exceeds cap=%lld",
              (long long)(t_max / m), (long long)cap);
  DLC_REQUIRE(cap < (int64_t(1) << 31), DLC_E_UNSUPPORTED, "csa_index_topk_fp4: cap must be < 2^31");
  DLC_REQUIRE(qI && wI && t && idx && count && ((KIc && KIs) || cap == 0), DLC_E_INVAL,
              "csa_index_topk_fp4: NULL argument");
  DLC_REQUIRE(aligned(qI, 16) && (cap == 0 || aligned(KIc, 16)), DLC_E_INVAL,
              "csa_index_topk_fp4: qI and KIc must be 16-byte aligned");
  const WsLayout L = ws_layout(B, n_q, cap, k, true);
  const Fp4Ws W = fp4_query_off(B, n_q, cap, k, n_hI, cI);
  DLC_REQUIRE(ws != nullptr && ws_bytes >= W.total, DLC_E_WORKSPACE,
              "csa_index_topk_fp4: workspace of %zu bytes needed, %zu given", W.total, ws_bytes);
  DLC_REQUIRE(aligned(ws, 256), DLC_E_WORKSPACE, "csa_index_topk_fp4: workspace must be 256-byte aligned");
  DLC_REQUIRE(B * n_q <= 65535, DLC_E_UNSUPPORTED, "csa_index_topk_fp4: B*n_q > 65535");

  hipStream_t s = as_stream(stream);
  IdxArgs a{};
  a.qI = qI; a.wI = wI; a.KI = KIc; a.k_scale = KIs; a.t = t;
  a.n_q = n_q; a.n_hI = n_hI; a.cI = cI; a.m = m; a.k = k; a.cap = cap; a.t_max = t_max;
  const int64_t BQ = B * n_q;
  bind_ws(a, L, ws, scores, BQ, cap);
  a.idx = idx; a.count = count;
  uint8_t* qc = static_cast<uint8_t*>(ws) + W.code;
  uint8_t* qsc = static_cast<uint8_t*>(ws) + W.scale;
  a.q_code = qc; a.q_scale = qsc;

  int rc;
  const int64_t vis_max = t_max / m;
  if (vis_max > 0) {  // histograms cleared and queries quantized by one launch
    const int64_t nhist = BQ * kBins * 2, qblocks = BQ * n_hI * (cI / 32);
    const int fill_blocks = int(std::min<int64_t>(ceil_div(nhist, 1024), 256));
    const dim3 pgrid{unsigned(fill_blocks + ceil_div(qblocks, 256)), 1u, 1u};
    if (dtype == DLC_BF16)
      hipLaunchKernelGGL(prep_fp4_kernel<bf16_raw>, pgrid, dim3(256), 0, s, a.hist, nhist, fill_blocks,
                         static_cast<const bf16_raw*>(qI), qblocks, cI / 32, qc, qsc);
    else
      hipLaunchKernelGGL(prep_fp4_kernel<float>, pgrid, dim3(256), 0, s, a.hist, nhist, fill_blocks,
                         static_cast<const float*>(qI), qblocks, cI / 32, qc, qsc);
    if ((rc = check_launch("csa_index_topk_fp4/prep"))) return rc;
    const bool prefill = cI == 128 && n_q >= kPrefillMinQueries;
    a.keys_per_wg = keys_per_wg(BQ, vis_max, prefill ? kSelectWorkgroups : kScoreWorkgroups);
    dim3 grid{(unsigned)ceil_div(vis_max, a.keys_per_wg), (unsigned)BQ, 1u};
    StageTimer timer(DLC_STAGE_INDEX_SCORES, s);
    if (prefill) {
      dim3 pgrid{(unsigned)ceil_div(vis_max, 256), (unsigned)ceil_div(n_q, 64), (unsigned)B};
      hipLaunchKernelGGL((scores_prefill_fp4_kernel<128>), pgrid, dim3(512), 0, s, a);
    }
    if (!prefill && cI == 128)
      hipLaunchKernelGGL((scores_fp4_kernel<128, DLC_FP4_NS, DLC_FP4_NW>), grid, dim3(64 * DLC_FP4_NW), 0, s, a);
    if (!prefill && cI == 256)
      hipLaunchKernelGGL((scores_fp4_kernel<256, DLC_FP4_NS, DLC_FP4_NW>), grid, dim3(64 * DLC_FP4_NW), 0, s, a);
    if ((rc = check_launch("csa_index_topk_fp4/scores"))) return rc;
    if (prefill) {
      hipLaunchKernelGGL(hist_kernel, grid, dim3(256), 0, s, a);
      if ((rc = check_launch("csa_index_topk_fp4/hist"))) return rc;
    }
  } else if ((rc = fill_u32(a.hist, 0, int64_t(BQ * kBins * 2), s))) {
    return rc;
  }
  return select_topk(a, BQ, vis_max, s);
}

}  // extern "C"
