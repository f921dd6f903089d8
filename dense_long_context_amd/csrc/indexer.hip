// Lightning indexer and exact top-k over the CSA cache.
//
// "DeepSeek-V4 Hybrid Attention: CSA and HCA from Scratch", §6.4 (score
// I[s] = sum_h w[h] * ReLU(q[h] . K[s])) and §7 (keep the k largest over the
// visible entries s < floor(t/m)).
//
// Pipeline per call (all on the caller's stream):
//   1. scores     one pass over K^I: for bf16 with c^I % 32 == 0 the heads x keys
//                 product runs on MFMA (v_mfma_f32_16x16x32_bf16) with the
//                 queries held in registers; otherwise a VALU kernel; with
//                 MXFP4 operands (csa_index_topk_fp4, §6.4's FP4 indexer) on
//                 the block-scaled v_mfma_scale_f32_16x16x128_f8f6f4.  Each
//                 workgroup also builds an LDS histogram of the top 11 bits of
//                 the order-preserving score key and adds its non-zero bins to
//                 the query's histogram (which the previous call's selection
//                 left at zero).
//   2. select     every workgroup finds the threshold bin T from that
//                 histogram and writes its chunk's entries above T (selected)
//                 and in T (candidates, with their keys) to the chunk's own
//                 segments in index order; the candidates' next 11 key bits go
//                 into the query's second histogram.  The last workgroup of a
//                 query resolves the candidates by radix passes over the
//                 remaining key bits and then the index (ties go to the
//                 smaller index), starting from the second histogram, and
//                 writes the selected and chosen entries to their slots of
//                 idx in ascending order.
#include "common.hpp"
#include "mxfp4.hpp"

namespace dlc {
namespace {

constexpr int kBins = 2048;      // first digit: top 11 bits of the key
constexpr int kShift1 = 21;
constexpr int kMaxK = 8192;
constexpr int kTicketStride = 32;  // words between the queries' arrival counters (one 128-byte line each)
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
  uint32_t* cand_srk;  // [BQ][cap] selected entries of the chunk before each candidate, same positions
  uint32_t* ticket;    // [BQ][kTicketStride] selection workgroups of the query that have finished
  int32_t* cand_idx;   // [BQ][cap] the query's candidates gathered, when they overflow LDS
  uint32_t* cand_key;  // [BQ][cap] their score keys
  uint32_t* cand_srk2; // [BQ][cap] their selected-entry counts
  int32_t* chosen;     // [BQ][k] the chosen candidates, when they overflow LDS
  int32_t* idx;        // [BQ][k]
  int32_t* count;      // [BQ]
  int64_t keys_per_wg; // scores / filter chunk
  int64_t max_chunks;
  // a range of the cache (the streaming prefill): entries key_begin ..
  // key_begin + cap - 1 of every sequence, KI (and k_scale) pointing at
  // entry key_begin of sequence 0, sequences key_bstride entries apart;
  // entry numbers inside the kernels are relative to key_begin
  int64_t key_begin, key_bstride;
};

// entries of the range visible to query bq: s < floor(t/m), from key_begin
__device__ __forceinline__ int64_t visible(const IdxArgs& a, int64_t bq) {
  int64_t t = a.t[bq];
  t = t < 0 ? 0 : (t > a.t_max ? a.t_max : t);
  int64_t v = t / a.m - a.key_begin;
  v = v < 0 ? 0 : v;
  return v < a.cap ? v : a.cap;
}

// the range's entries visible to the query with the largest t (t_max)
__device__ __forceinline__ int64_t visible_max(const IdxArgs& a) {
  const int64_t v = a.t_max / a.m - a.key_begin;
  return v < 0 ? 0 : (v < a.cap ? v : a.cap);
}

__device__ __forceinline__ float canon_zero(float s) { return s == 0.f ? 0.f : s; }

// the score behind an order_key (zeros come back as +0)
__device__ __forceinline__ float key_score(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

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

// The selection kernel that follows a scores kernel needs the query's second
// histogram and arrival counter at zero: the first workgroup of each query
// in the scores kernel clears them.
__device__ __forceinline__ void clear_select_state(const IdxArgs& a, int64_t bq) {
  if (blockIdx.x != 0) return;
  uint4* h2 = reinterpret_cast<uint4*>(a.hist2 + bq * kBins);
  for (int i = threadIdx.x; i < kBins / 4; i += blockDim.x) h2[i] = make_uint4(0, 0, 0, 0);
  if (threadIdx.x == 0) a.ticket[bq * kTicketStride] = 0;
}

// ---------------------------------------------------------------- scores (VALU)

template <typename T>
__global__ void __launch_bounds__(256) scores_valu_kernel(IdxArgs a) {
  extern __shared__ float smem[];
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem);
  float* q = smem + kBins;                // [n_hI][cI]
  float* w = q + a.n_hI * a.cI;           // [n_hI]
  const int64_t bq = blockIdx.y;
  clear_select_state(a, bq);
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
  const T* K = static_cast<const T*>(a.KI) + b * a.key_bstride * a.cI;
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
// Queries stay in registers for the whole pass.

#ifndef DLC_SCORES_U
#define DLC_SCORES_U 3  // key tiles in flight per wave in the register-load scores kernel
#endif
#ifndef DLC_SCORES_OCC
#define DLC_SCORES_OCC 3  // waves per SIMD the register-load scores kernel is compiled for
#endif
#ifndef DLC_SCORES_RWGS
#define DLC_SCORES_RWGS 768  // its workgroups per call (three per CU, one round)
#endif

// Scores a decode scores wave keeps in LDS while it streams keys, written
// out after its last tile: interleaving the score stores with the key stream
// costs the stream more than the same stores issued together at the end.
// Waves with more tiles store each tile's scores as they come.
#ifndef DLC_SCORE_STAGE_TILES
#define DLC_SCORE_STAGE_TILES 64
#endif
constexpr int kStageTiles = DLC_SCORE_STAGE_TILES;

// the staged scores of a wave (lane group g takes tiles g, g+4, ...)
__device__ __forceinline__ void store_staged(float* srow, const float (*st)[16], int64_t my_tiles, int64_t first,
                                             int64_t step, int64_t nvis, int lane) {
  const int r16 = lane & 15, g = lane >> 4;
  for (int64_t i = g; i < my_tiles; i += 4) {
    const int64_t s = (first + i * step) * 16 + r16;
    if (s < nvis) srow[s] = st[i][r16];
  }
}

// The bf16 kernel loads the key operands straight into registers: each
// lane loads, per 16-key tile, the four 16-byte pieces of its key row that
// its K^T operand needs (row r16 of the tile, bytes 64*kt + 16*g), so one
// load instruction covers 64 bytes of 16 rows and the tile never passes
// through LDS (on this part the register form streams faster than the
// direct-to-LDS one).  The G = gridDim.x workgroups of a query take its tiles
// interleaved, wave v of workgroup x taking tiles (it*G + x)*4 + v, so at any
// moment the whole grid reads one narrow window of each key cache, as a
// grid-strided copy does, rather than G far-apart streams.  Each wave keeps
// U tiles in flight (U * 16 VGPRs): the loop is unrolled by U so each tile's
// registers are named statically, a tile's registers are refilled with the
// wave's tile U steps on as soon as its MFMAs have read them, and every load
// is unconditional (rows clamp to the last row any query of the batch sees)
// with no early exit inside a group of U, so every path into the loop head
// carries the same loads in flight and the waits before each tile count only
// the tiles behind it.  Queries arrive through LDS once per workgroup; each
// tile's 16 scores go out as one 64-byte store.  Registers: the query block
// takes 4*HT*KT VGPRs and the tiles in flight 4*U*KT; c^I = 256 (KT = 8)
// keeps two tiles in flight at two waves per SIMD, the narrower rows three
// at DLC_SCORES_OCC waves per SIMD.
template <int HT, int KT, int U>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KT >= 8 ? 2 : DLC_SCORES_OCC)))
scores_reg_kernel(IdxArgs a) {
  constexpr int ROWB = KT * 64;     // bytes per key row (2 * c^I)
  constexpr int CPR = KT * 4;       // 16-byte chunks per row
  constexpr int RPI = 1024 / ROWB;  // rows per 1 KB query load
  static_assert(RPI * KT == 16, "tile geometry");
  static_assert(HT <= 4, "one 16-head block of queries per staging wave");
  __shared__ uint32_t hist[kBins];
  __shared__ __attribute__((aligned(1024))) unsigned char sQ[HT][16 * ROWB];
  __shared__ float sS[4][kStageTiles][16];
  const int64_t bq = blockIdx.y;
  clear_select_state(a, bq);
  const int64_t vmax = visible_max(a);  // rows below vmax exist whatever this query's t

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int cI = KT * 32;
  const int64_t step = int64_t(gridDim.x) * 4;      // tiles between a wave's consecutive tiles
  const int64_t first = int64_t(blockIdx.x) * 4 + wave;

  const int64_t b = bq / a.n_q;
  const bf16_raw* K = static_cast<const bf16_raw*>(a.KI) + b * a.key_bstride * cI;
  // this lane's pieces of the wave's tile it
  auto load = [&](int64_t it, uint4 (&dst)[KT]) {
    const int64_t row = min((first + it * step) * 16 + r16, vmax - 1);
    const bf16_raw* p = K + row * cI + 8 * g;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) dst[kt] = *reinterpret_cast<const uint4*>(p + 32 * kt);
  };
  // queries: wave w < HT moves heads 16w .. 16w+15 (rows past n_hI repeat
  // head n_hI-1) into its block of sQ, rows in order
  if (wave < HT) {
    const bf16_raw* qg = static_cast<const bf16_raw*>(a.qI) + bq * a.n_hI * cI;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const int h = min(wave * 16 + j * RPI + lane / CPR, int(a.n_hI) - 1);
      const uint32_t off = uint32_t(h * ROWB + (lane % CPR) * 16);
      const uint32_t lds = (uint32_t)(uintptr_t)DLC_LDS(&sQ[wave][0]) + uint32_t(j * 1024);
      dma_row(qg, off, lds);
    }
  }
  uint4 kb[U][KT];
#pragma unroll
  for (int u = 0; u < U; ++u) load(u, kb[u]);
  const int64_t nvis = visible(a, bq);
  const int64_t n_tiles = (nvis + 15) / 16;
  if (int64_t(blockIdx.x) * 64 >= nvis) {  // no wave of this workgroup has a visible tile
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }
  const int64_t my_tiles = n_tiles > first ? (n_tiles - first + step - 1) / step : 0;
  const bool staged = my_tiles <= kStageTiles;  // wave-uniform
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) hist[i] = 0;
  float wv[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = ht * 16 + g * 4 + r;
      wv[ht][r] = h < a.n_hI ? a.wI[bq * a.n_hI + h] : 0.f;
    }
  wait_vm<0>();     // the query block (and the first tiles)
  __syncthreads();  // every wave's query rows landed; hist cleared
  bf16x8 qf[HT][KT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const bool pad = ht * 16 + r16 >= a.n_hI;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const uint4 v = *reinterpret_cast<const uint4*>(&sQ[ht][r16 * ROWB + kt * 64 + g * 16]);
      qf[ht][kt] = __builtin_bit_cast(bf16x8, pad ? make_uint4(0, 0, 0, 0) : v);
    }
  }
  float* srow = a.scores + bq * a.score_ld;

  // whole groups of U tiles: the up to U-1 tiles past my_tiles in the last
  // group lie at or past nvis, so their stores and counts are masked off
  for (int64_t it0 = 0; it0 < my_tiles; it0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t it = it0 + u;
      f32x4 acc[HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (it < my_tiles) {  // the last group's tiles past my_tiles are loaded, not computed
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
            acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ht][kt], __builtin_bit_cast(bf16x8, kb[u][kt]),
                                                              acc[ht], 0, 0, 0);
      }
      load(it + U, kb[u]);
      float ps[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ps[r] = wv[0][r] * relu(acc[0][r]);
#pragma unroll
        for (int ht = 1; ht < HT; ++ht) ps[r] = fmaf(wv[ht][r], relu(acc[ht][r]), ps[r]);
      }
      const float part = rows4_sum((ps[0] + ps[1]) + (ps[2] + ps[3]));
      const int64_t s = (first + it * step) * 16 + r16;
      if (g == 0 && s < nvis) {
        const float score = canon_zero(part);
        if (staged) sS[wave][it][r16] = score;
        else srow[s] = score;
        atomicAdd(&hist[order_key(score) >> kShift1], 1u);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the tiles loaded past the end
  if (staged) store_staged(srow, sS[wave], my_tiles, first, step, nvis, lane);
  flush_hist(hist, a.hist + bq * kBins);
}

// ---------------------------------------------------------------- scores (FP4)
//
// MXFP4 operands on v_mfma_scale_f32_16x16x128_f8f6f4: D[16 heads][16 keys]
// += Q[16 heads][128 dims] x K^T[128 dims][16 keys], each operand carrying one
// E8M0 scale per 32 dims, so every product is exact and only the fp32 sums
// round.  Lane l supplies head/key l%16 and the 32-dim block l/16 of each
// 128-dim step: 16 code bytes and one scale byte.  The queries arrive
// quantized (prep_fp4_kernel, run on them just before).  Result layout and
// head sum as in the bf16 kernel.

typedef int i32x8 __attribute__((ext_vector_type(8)));

// The decode kernel loads the key operands straight into registers, in the
// bf16 register kernel's scheme (tiles interleaved over
// the G workgroups of a query, U tiles in flight per wave, every load
// unconditional with rows clamped to the last row the batch may see, whole
// groups of U tiles).  A 16-key tile is 16 code rows of c^I/2 bytes, and
// lane l's operand for 128-dim step j is the 16 bytes of row l%16 at
// 16*(4j + l/16): at c^I = 128 one 16-byte load per lane reads the whole
// 1 KB tile.  Its scale byte (row l%16, block 4j + l/16) comes from one
// 4-byte load of the row's scales.  Tiles are small (1 KB at c^I = 128), so
// three in flight per wave, at 768 workgroups, is the measured best: more
// tiles a wave or more workgroups leave each wave too few tiles for its
// start-up and its last, partly wasted group.
template <int CI, int U>
__global__ void __launch_bounds__(256) scores_fp4_reg_kernel(IdxArgs a) {
  constexpr int KB = CI / 32;    // scale bytes (32-dim blocks) per row
  constexpr int ROWB = CI / 2;   // code bytes per row
  constexpr int NJ = CI / 128;   // 128-dim MFMA steps
  constexpr int HT = 4;          // head tiles: up to 64 heads
  static_assert(CI == 128 || CI == 256, "c^I");
  __shared__ uint32_t hist[kBins];
  __shared__ float sS[4][kStageTiles][16];
  const int64_t bq = blockIdx.y;
  clear_select_state(a, bq);
  const int64_t vmax = visible_max(a);  // rows below vmax exist whatever this query's t

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t step = int64_t(gridDim.x) * 4;
  const int64_t first = int64_t(blockIdx.x) * 4 + wave;
  const int64_t b = bq / a.n_q;
  const uint8_t* Kc = static_cast<const uint8_t*>(a.KI) + b * a.key_bstride * ROWB;
  const uint8_t* Ks = a.k_scale + b * a.key_bstride * KB;
  // codes of step j, and the 4-byte word holding the row's scales of blocks
  // 4j .. 4j+3 (this lane's is byte g of it; Ks is 4-byte aligned)
  auto load = [&](int64_t it, uint4 (&kc)[NJ], uint32_t (&ks)[NJ]) {
    const int64_t row = min((first + it * step) * 16 + r16, vmax - 1);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      kc[j] = *reinterpret_cast<const uint4*>(Kc + row * ROWB + (4 * j + g) * 16);
      ks[j] = *reinterpret_cast<const uint32_t*>(Ks + row * KB + 4 * j);
    }
  };
  uint4 kc[U][NJ];
  uint32_t ksc[U][NJ];
#pragma unroll
  for (int u = 0; u < U; ++u) load(u, kc[u], ksc[u]);
  const int64_t nvis = visible(a, bq);
  const int64_t n_tiles = (nvis + 15) / 16;
  if (int64_t(blockIdx.x) * 64 >= nvis) {  // no wave of this workgroup has a visible tile
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }
  const int64_t my_tiles = n_tiles > first ? (n_tiles - first + step - 1) / step : 0;
  const bool staged = my_tiles <= kStageTiles;  // wave-uniform
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) hist[i] = 0;
  // queries (A operand, rows = heads): head ht*16 + r16, block 4j + g; heads
  // past n_hI take zero codes (their weight is 0 too)
  i32x8 qa[HT][NJ];
  int qs[HT][NJ];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int h = min(ht * 16 + r16, int(a.n_hI) - 1);
    const bool pad = ht * 16 + r16 >= a.n_hI;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int blk = 4 * j + g;
      const uint4 c = *reinterpret_cast<const uint4*>(a.q_code + (bq * a.n_hI + h) * ROWB + blk * 16);
      const int e8 = a.q_scale[(bq * a.n_hI + h) * KB + blk];
      qa[ht][j] = pad ? i32x8{0, 0, 0, 0, 0, 0, 0, 0} : i32x8{int(c.x), int(c.y), int(c.z), int(c.w), 0, 0, 0, 0};
      qs[ht][j] = pad ? 127 : e8;
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
  wait_vm<0>();     // the query, the weights and the first tiles
  __syncthreads();  // hist cleared
  float* srow = a.scores + bq * a.score_ld;

  // whole groups of U tiles: the tiles past my_tiles in the last group lie at
  // or past nvis, so their stores and counts are masked off
  for (int64_t it0 = 0; it0 < my_tiles; it0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t it = it0 + u;
      f32x4 acc[HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const i32x8 kb = i32x8{int(kc[u][j].x), int(kc[u][j].y), int(kc[u][j].z), int(kc[u][j].w), 0, 0, 0, 0};
        // byte g of the scale word, taken apart only here: the empty asm keeps
        // the compiler from doing it (and so waiting for every tile in
        // flight) at the loop head
        uint32_t w = ksc[u][j];
        asm volatile("" : "+v"(w));
        const int sc = int((w >> (8 * g)) & 0xffu);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          acc[ht] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[ht][j], kb, acc[ht], 4, 4, 0, qs[ht][j], 0, sc);
      }
      load(it + U, kc[u], ksc[u]);
      float ps[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ps[r] = wv[0][r] * relu(acc[0][r]);
#pragma unroll
        for (int ht = 1; ht < HT; ++ht) ps[r] = fmaf(wv[ht][r], relu(acc[ht][r]), ps[r]);
      }
      const float part = rows4_sum((ps[0] + ps[1]) + (ps[2] + ps[3]));
      const int64_t s = (first + it * step) * 16 + r16;
      if (g == 0 && s < nvis) {
        const float score = canon_zero(part);
        if (staged) sS[wave][it][r16] = score;
        else srow[s] = score;
        atomicAdd(&hist[order_key(score) >> kShift1], 1u);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the tiles loaded past the end
  if (staged) store_staged(srow, sS[wave], my_tiles, first, step, nvis, lane);
  flush_hist(hist, a.hist + bq * kBins);
}

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
  const bf16_raw* Kb = static_cast<const bf16_raw*>(a.KI) + b * a.key_bstride * CI;
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
  const uint8_t* Kc = static_cast<const uint8_t*>(a.KI) + b * a.key_bstride * ROWB;
  const uint8_t* Ks = a.k_scale + b * a.key_bstride * KB;
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
  clear_select_state(a, bq);
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
// counts the entries in bins > T, over a histogram the threads hold in
// registers: thread i owns bins PER*i .. PER*i + PER-1, given in v (nbins =
// PER * blockDim.x, blockDim.x a multiple of 64 and at most 1024).  Every
// thread gets (T, above), h[T] and, in *total_out, the sum of all bins.
// scratch holds 16 + 3 words.  A suffix scan of the per-thread totals (within the
// wave, then over the wave totals) locates the one thread whose run crosses
// `need`, and that thread walks its own bins.
template <int PER>
__device__ void find_threshold_regs(const uint32_t (&v)[PER], uint32_t need, uint32_t* scratch, int* T_out,
                                    uint32_t* above_out, uint32_t* total_out, uint32_t* count_out = nullptr) {
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
    scratch[18] = 0;
  }
  __syncthreads();
  uint32_t higher = 0, all = 0;
  for (int w = 0; w < nwaves; ++w) {
    const uint32_t x = scratch[w];
    higher += w > wave ? x : 0u;
    all += x;
  }
  *total_out = all;
  uint32_t run = higher + suf - mine;
  if (run < need && run + mine >= need) {
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      if (run < need && run + v[i] >= need) {
        scratch[16] = uint32_t(lo + i);
        scratch[17] = run;
        scratch[18] = v[i];
      }
      run += v[i];
    }
  }
  __syncthreads();
  *T_out = int(scratch[16]);
  if (count_out) *count_out = scratch[18];
  *above_out = scratch[17];
  __syncthreads();
}

// Block-wide exclusive scan of one value per thread (NW waves); returns the
// block total.  wsum holds NW words.  Ends synchronised.
template <int NW>
__device__ __forceinline__ uint32_t scan_block(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t x = wsum[w];
    before += w < wave ? x : 0u;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// ---------------------------------------------------------------- selection
//
// One kernel after the scores: a workgroup per chunk of keys_per_wg entries
// filters its chunk, and the last workgroup of a query to finish resolves
// the query's threshold exactly and writes idx / count.
//
// Filter (every workgroup).  The threshold bin T of the query comes from the
// first-digit histogram: above(T) < k_eff <= above(T) + h[T].  The chunk's
// entries above T (selected for sure) and in T (candidates, stored with
// their keys and with the number of the chunk's selected entries before
// them) go to the chunk's own segments in index order: thread j takes
// entries 4j .. 4j+3 of each batch of 4*kSelThreads, so one scan of packed
// counts orders both lists.  The candidates' second digit (key bits 20..10) is
// counted into the query's second histogram.
//
// Finish (the last workgroup of the query; an arrival counter per query,
// cleared by the scores kernel of the same call).  After the exclusive scans
// of the chunk counts, radix passes over the candidates' composite key (the
// low 21 key bits, then the bit-inverted index) find the exact k_eff-th
// entry, starting from the second histogram.  The chosen candidates are
// those at or above it, and their output slots follow from the counts:
// chosen candidate j (in index order) goes to j + (selected entries before
// its chunk) + (selected entries of its chunk before it); selected entry i
// goes to i + (chosen candidates below it), a binary search over the chosen
// list.  The finishing workgroup then clears the query's first-digit
// histogram, so that the next call's scores kernel finds it zero.  A
// histogram that did not start at zero (a workspace that no call of the
// library has cleared) shows as a bin above the visible count or a total
// other than it; the filter then counts the query's scores again itself.
constexpr int kMaxChunks = 1024;  // chunks per query (keys_per_wg keeps to it)
constexpr int kFinCand = 4096;    // candidates the finishing workgroup holds in LDS (more: the workspace)
constexpr int kFinChosen = 2048;  // chosen candidates it holds in LDS (more: the workspace)
constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kBpt = kBins / kSelThreads;  // first-digit bins per thread

// radix passes over the candidates' composite key: the low 21 bits of the score
// key (the top 11 bits are T for all of them), then the bit-inverted index
constexpr int kPasses = 5;
__device__ __forceinline__ int pass_shift(int p) { return p == 0 ? 42 : p == 1 ? 32 : p == 2 ? 21 : p == 3 ? 10 : 0; }
__device__ __forceinline__ int pass_bits(int p) { return (p == 1 || p == 4) ? 10 : 11; }

__device__ __forceinline__ uint64_t cand_key(uint32_t key, int32_t s) {
  return (uint64_t(key & 0x1fffffu) << 32) | uint64_t(0xffffffffu - uint32_t(s));
}

// Exclusive scans of v[0 .. n) and w[0 .. n) in place (kSelThreads threads);
// the totals come back through tv and tw.  Thread j owns the run [j*per,
// (j+1)*per), per = ceil(n / kSelThreads); wsum holds 2*kSelWaves words.
// Ends synchronised.
__device__ void scan_runs2(uint32_t* v, uint32_t* w, int n, uint32_t* wsum, uint32_t* tv, uint32_t* tw) {
  const int per = (n + kSelThreads - 1) / kSelThreads;
  const int lo = threadIdx.x * per, hi = min(n, lo + per);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t mv = 0, mw = 0;
  for (int i = lo; i < hi; ++i) {
    mv += v[i];
    mw += w[i];
  }
  const uint32_t iv = wave_incl_scan(mv), iw = wave_incl_scan(mw);
  if (lane == 63) {
    wsum[wave] = iv;
    wsum[kSelWaves + wave] = iw;
  }
  __syncthreads();
  uint32_t bv = 0, bw = 0, sv = 0, sw = 0;
#pragma unroll
  for (int k = 0; k < kSelWaves; ++k) {
    const uint32_t x = wsum[k], y = wsum[kSelWaves + k];
    bv += k < wave ? x : 0u;
    bw += k < wave ? y : 0u;
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

// Binary searches of G keys at once: the same number of halving steps for
// every key and lane (n is uniform), so the G reads of a step are in flight
// together.
// r[u] = the number of entries of the ascending list l[0 .. n) below x[u]
template <int G>
__device__ __forceinline__ void lower_bounds(const int32_t* l, uint32_t n, const int32_t (&x)[G], uint32_t (&r)[G]) {
  uint32_t base[G];
#pragma unroll
  for (int u = 0; u < G; ++u) base[u] = 0;
  uint32_t len = n;
  while (len > 1) {
    const uint32_t half = len >> 1;
#pragma unroll
    for (int u = 0; u < G; ++u) base[u] = l[base[u] + half] < x[u] ? base[u] + half : base[u];
    len -= half;
  }
#pragma unroll
  for (int u = 0; u < G; ++u) r[u] = base[u] + ((n > 0 && l[base[u]] < x[u]) ? 1u : 0u);
}
// c[u] = the largest chunk c < n with off[c] <= i[u] (off ascending, off[0] = 0)
template <int G>
__device__ __forceinline__ void chunks_of(const uint32_t* off, int n, const uint32_t (&i)[G], int (&c)[G]) {
#pragma unroll
  for (int u = 0; u < G; ++u) c[u] = 0;
  int len = n;
  while (len > 1) {
    const int half = len >> 1;
#pragma unroll
    for (int u = 0; u < G; ++u) c[u] = off[c[u] + half] <= i[u] ? c[u] + half : c[u];
    len -= half;
  }
}

// thresholds over an LDS histogram of PER*kSelThreads bins; *count gets h[T] (read
// before the search's last barrier, so h may be overwritten after it)
template <int PER>
__device__ __forceinline__ void find_in_lds(const uint32_t* h, uint32_t need, uint32_t* scratch, int* T,
                                            uint32_t* above, uint32_t* count) {
  uint32_t v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = h[PER * threadIdx.x + i];
  uint32_t total;
  find_threshold_regs<PER>(v, need, scratch, T, above, &total, count);
}

// Values that cross workgroups inside the selection kernel (the chunk lists,
// counts and the second histogram) are written and read with the
// agent-scope accesses of st_agent / ld_agent.

struct FinishLds {
  uint32_t off_sel[kMaxChunks], off_cand[kMaxChunks];
  int32_t c_idx[kFinCand];
  uint32_t c_key[kFinCand], c_srk[kFinCand];
  int32_t chosen[kFinChosen];
};

__device__ void finish_query(const IdxArgs& a, int64_t bq, int64_t nvis, int64_t keff, uint32_t* h, FinishLds& L,
                             uint32_t* scratch, uint32_t* wsum) {
  const int tid = threadIdx.x;
  const int64_t kpw = a.keys_per_wg;
  const int nch = int(ceil_div(nvis, kpw));
  int32_t* out = a.idx + bq * a.k;
  // the chunk counts and the candidates' second digit (pass 0 below)
  const uint32_t* cc = a.ccnt + bq * a.max_chunks * 2;
  const uint32_t* h2g = a.hist2 + bq * kBins;
  {
    uint32_t y[kBpt];
#pragma unroll
    for (int u = 0; u < kBpt; ++u) y[u] = ld_agent(h2g + tid + u * kSelThreads);
    for (int i = tid; i < nch; i += kSelThreads) {
      L.off_sel[i] = ld_agent(cc + 2 * i);
      L.off_cand[i] = ld_agent(cc + 2 * i + 1);
    }
#pragma unroll
    for (int u = 0; u < kBpt; ++u) h[tid + u * kSelThreads] = y[u];
  }
  __syncthreads();
  uint32_t tsel, tcand;
  scan_runs2(L.off_sel, L.off_cand, nch, wsum, &tsel, &tcand);
  const uint32_t n_sel = min(tsel, uint32_t(keff));
  const uint32_t n_cand = min(tcand, uint32_t(nvis));
  const uint32_t need0 = uint32_t(keff) - n_sel;
  const bool cand_lds = n_cand <= uint32_t(kFinCand);
  int32_t* ci = cand_lds ? L.c_idx : a.cand_idx + bq * a.cap;
  uint32_t* ck = cand_lds ? L.c_key : a.cand_key + bq * a.cap;
  uint32_t* cs = cand_lds ? L.c_srk : a.cand_srk2 + bq * a.cap;
  int32_t* chosen = need0 <= uint32_t(kFinChosen) ? L.chosen : a.chosen + bq * a.k;
  const int32_t* selg = a.sel + bq * a.cap;
  const int64_t cbase = bq * a.cap;

  // the first 1024 selected entries, loaded with the candidates
  constexpr int G = 4;
  int32_t sv[G];
  {
    uint32_t si[G];
    int sc[G];
#pragma unroll
    for (int u = 0; u < G; ++u) si[u] = tid + u * kSelThreads;
    chunks_of<G>(L.off_sel, nch, si, sc);
#pragma unroll
    for (int u = 0; u < G; ++u)
      sv[u] = si[u] < n_sel ? ld_agent(selg + int64_t(sc[u]) * kpw + (si[u] - L.off_sel[sc[u]])) : 0;
  }
  // eight candidates a thread per round, their loads in flight together
  constexpr int GC = 8;
  for (uint32_t i0 = tid; i0 < n_cand; i0 += GC * kSelThreads) {
    int32_t vi[GC];
    uint32_t vk[GC], vs[GC], ii[GC];
    int cc[GC];
#pragma unroll
    for (int u = 0; u < GC; ++u) ii[u] = i0 + u * kSelThreads;
    chunks_of<GC>(L.off_cand, nch, ii, cc);
#pragma unroll
    for (int u = 0; u < GC; ++u) {
      if (ii[u] < n_cand) {
        const int64_t at = cbase + int64_t(cc[u]) * kpw + (ii[u] - L.off_cand[cc[u]]);
        vi[u] = ld_agent(a.cand + at);
        vk[u] = ld_agent(a.cand_kseg + at);
        vs[u] = ld_agent(a.cand_srk + at);
      }
    }
#pragma unroll
    for (int u = 0; u < GC; ++u) {
      const uint32_t i = i0 + u * kSelThreads;
      if (i < n_cand) {
        ci[i] = vi[u];
        ck[i] = vk[u];
        cs[i] = vs[u];
      }
    }
  }
  __threadfence_block();
  __syncthreads();

  // the exact threshold: the chosen candidates are those whose composite key
  // is >= thr
  uint32_t need = need0;
  uint64_t pval = 0, pmask = 0;
  for (int pass = 0; pass < kPasses && need > 0; ++pass) {
    const int shift = pass_shift(pass), bits = pass_bits(pass);
    const uint32_t dmask = (1u << bits) - 1u;
    if (pass > 0) {
      for (int i = tid; i < kBins; i += kSelThreads) h[i] = 0;
      __syncthreads();
      for (uint32_t i = tid; i < n_cand; i += kSelThreads) {
        const uint64_t key = cand_key(ck[i], ci[i]);
        if ((key & pmask) == pval) atomicAdd(&h[(key >> shift) & dmask], 1u);
      }
      __syncthreads();
    }
    int D;
    uint32_t above, hD;
    if (bits == 11) find_in_lds<kBpt>(h, need, scratch, &D, &above, &hD);
    else find_in_lds<kBpt / 2>(h, need, scratch, &D, &above, &hD);
    const bool take_all = above + hD == need;
    pval |= uint64_t(D) << shift;
    pmask |= uint64_t(dmask) << shift;
    if (take_all) break;
    need -= above;
  }
  const uint64_t thr = pval;
  // need0 == 0: no candidate is chosen (thr stays above every key)
  const bool none = need0 == 0;

  // chosen candidates in index order: thread j counts its run, one scan
  // gives the ranks; each goes straight to its output slot
  {
    const uint32_t per = (n_cand + kSelThreads - 1) / kSelThreads;
    const uint32_t lo = tid * per, hi = min(n_cand, lo + per);
    uint32_t mine = 0;
    if (!none)
      for (uint32_t i = lo; i < hi; ++i) mine += cand_key(ck[i], ci[i]) >= thr ? 1u : 0u;
    uint32_t tot;
    uint32_t j = scan_block<kSelWaves>(mine, wsum, &tot);
    if (!none) {
      for (uint32_t i = lo; i < hi; ++i) {
        if (cand_key(ck[i], ci[i]) < thr) continue;
        if (j < need0) {
          const int32_t y = ci[i];
          const int c = int(uint32_t(y) / uint32_t(kpw));
          chosen[j] = y;
          out[j + L.off_sel[c] + cs[i]] = y;
        }
        ++j;
      }
    }
  }
  __threadfence_block();
  __syncthreads();
  const uint32_t n2 = need0;
  // selected entries: slot i + (chosen entries below)
  {
    uint32_t r[G];
    lower_bounds<G>(chosen, n2, sv, r);
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const uint32_t i = tid + u * kSelThreads;
      if (i < n_sel) out[i + r[u]] = sv[u];
    }
  }
  for (uint32_t i0 = tid + G * kSelThreads; i0 < n_sel; i0 += G * kSelThreads) {
    uint32_t si[G], r[G];
    int sc[G];
    int32_t x[G];
#pragma unroll
    for (int u = 0; u < G; ++u) si[u] = i0 + u * kSelThreads;
    chunks_of<G>(L.off_sel, nch, si, sc);
#pragma unroll
    for (int u = 0; u < G; ++u)
      x[u] = si[u] < n_sel ? ld_agent(selg + int64_t(sc[u]) * kpw + (si[u] - L.off_sel[sc[u]])) : 0;
    lower_bounds<G>(chosen, n2, x, r);
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (si[u] < n_sel) out[si[u] + r[u]] = x[u];
  }
  for (int64_t j = keff + tid; j < a.k; j += kSelThreads) out[j] = -1;
  if (tid == 0) a.count[bq] = int32_t(keff);
  // the first-digit histogram back to zero for the next call
  uint4* hg = reinterpret_cast<uint4*>(a.hist + bq * kBins);
  for (int i = tid; i < kBins / 4; i += kSelThreads) hg[i] = make_uint4(0, 0, 0, 0);
}

__global__ void __launch_bounds__(kSelThreads) select_kernel(IdxArgs a) {
  static_assert(kBins == kBpt * kSelThreads && kBpt % 4 == 0, "select_kernel: whole 16-byte runs of bins per thread");
  __shared__ uint32_t h2[kBins];
  __shared__ uint32_t scratch[19];
  __shared__ uint32_t wsum[2 * kSelWaves];
  __shared__ uint32_t s_last;
  __shared__ FinishLds L;
  const int tid = threadIdx.x;
  const int64_t bq = blockIdx.y;
  const int64_t nvis = visible(a, bq);
  const int64_t keff = min(a.k, nvis);
  const int64_t s0 = int64_t(blockIdx.x) * a.keys_per_wg;
  if (keff == nvis) {  // keep all (or nothing visible): the first workgroup writes the result
    if (blockIdx.x == 0) {
      int32_t* out = a.idx + bq * a.k;
      for (int64_t j = tid; j < a.k; j += kSelThreads) out[j] = j < nvis ? int32_t(j) : -1;
      if (tid == 0) a.count[bq] = int32_t(keff);
      uint4* hg = reinterpret_cast<uint4*>(a.hist + bq * kBins);
      for (int i = tid; i < kBins / 4; i += kSelThreads) hg[i] = make_uint4(0, 0, 0, 0);
    }
    return;
  }
  if (s0 >= nvis) return;
  const int64_t s1 = min(nvis, s0 + a.keys_per_wg);
  const float* sc = a.scores + bq * a.score_ld;
  // the first batches of scores are in flight while the threshold is found
  auto load4 = [&](int64_t base, float* v) {
    const int64_t s = base + 4 * tid;
    if (s + 3 < s1 && (reinterpret_cast<uintptr_t>(sc + s) & 15) == 0) {
      const float4 x = *reinterpret_cast<const float4*>(sc + s);
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = s + e < s1 ? sc[s + e] : 0.f;
    }
  };
  // a ring of FD batches in registers: batch i+FD is loaded as batch i is used
  constexpr int FD = 2;
  float vb[FD][4];
#pragma unroll
  for (int d = 0; d < FD; ++d) load4(s0 + int64_t(d) * 4 * kSelThreads, vb[d]);
  // thread j holds first-digit bins kBpt*j .. kBpt*j + kBpt-1 (16-byte loads)
  uint32_t hv[kBpt];
  {
    const uint4* hp = reinterpret_cast<const uint4*>(a.hist + bq * kBins) + (kBpt / 4) * tid;
#pragma unroll
    for (int q = 0; q < kBpt / 4; ++q) {
      const uint4 x = hp[q];
      hv[4 * q] = x.x; hv[4 * q + 1] = x.y; hv[4 * q + 2] = x.z; hv[4 * q + 3] = x.w;
    }
  }
  for (int i = tid; i < kBins; i += kSelThreads) h2[i] = 0;
  int T;
  uint32_t above, total;
  bool over = false;
#pragma unroll
  for (int e = 0; e < kBpt; ++e) over = over || hv[e] > uint32_t(nvis);
  over = __syncthreads_or(over);
  find_threshold_regs<kBpt>(hv, uint32_t(keff), scratch, &T, &above, &total);  // also orders the h2 clear
  if (over || total != uint32_t(nvis)) {
    // the histogram did not start at zero (no bin of a clean one exceeds the
    // visible count, and the bins sum to it): count the query's scores again
    for (int64_t s = tid; s < nvis; s += kSelThreads) atomicAdd(&h2[order_key(sc[s]) >> kShift1], 1u);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kBpt; ++e) hv[e] = h2[kBpt * tid + e];
    __syncthreads();
    for (int i = tid; i < kBins; i += kSelThreads) h2[i] = 0;
    find_threshold_regs<kBpt>(hv, uint32_t(keff), scratch, &T, &above, &total);
  }

  int32_t* sel = a.sel + bq * a.cap + s0;
  int32_t* cand = a.cand + bq * a.cap + s0;
  uint32_t* ckey = a.cand_kseg + bq * a.cap + s0;
  uint32_t* csrk = a.cand_srk + bq * a.cap + s0;
  uint32_t nsel = 0, ncand = 0;
  const int64_t step = 4 * int64_t(kSelThreads);
  for (int64_t round = s0; round < s1; round += FD * step) {
#pragma unroll
    for (int dd = 0; dd < FD; ++dd) {
      const int64_t base = round + dd * step;
      if (base >= s1) break;  // uniform
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = vb[dd][e];
      load4(base + FD * step, vb[dd]);  // past s1: zeros, no access
      const int64_t sb = base + 4 * tid;
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
      const uint32_t ex = scan_block<kSelWaves>(packed, wsum, &tot);
      uint32_t ps = nsel + (ex & 0xffffu), pc = ncand + (ex >> 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (d[e] > T) st_agent(sel + ps++, int32_t(sb + e));
        if (d[e] == T) {
          st_agent(cand + pc, int32_t(sb + e));
          st_agent(ckey + pc, key[e]);
          st_agent(csrk + pc, ps);  // the chunk's selected entries before this one
          ++pc;
          atomicAdd(&h2[(key[e] >> 10) & 0x7ffu], 1u);
        }
      }
      nsel += tot & 0xffffu;
      ncand += tot >> 16;
    }
  }
  flush_hist(h2, a.hist2 + bq * kBins);
  if (tid == 0) {
    st_agent(a.ccnt + (bq * a.max_chunks + blockIdx.x) * 2 + 0, nsel);
    st_agent(a.ccnt + (bq * a.max_chunks + blockIdx.x) * 2 + 1, ncand);
  }
  // arrive once every wave's lists, counts and histogram adds have completed
  // (agent-scope stores and atomics: complete means visible to every
  // workgroup); the last workgroup of the query finishes it
  wait_vm<0>();
  __syncthreads();
  if (tid == 0) {
    const uint32_t nch = uint32_t(ceil_div(nvis, a.keys_per_wg));
    s_last = __hip_atomic_fetch_add(&a.ticket[bq * kTicketStride], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nch - 1 ? 1u
                                                                                                         : 0u;
  }
  __syncthreads();
  if (s_last == 0) return;
  finish_query(a, bq, nvis, keff, h2, L, scratch, wsum);
}

// no entry is visible to any query (floor(t_max/m) = 0)
__global__ void __launch_bounds__(256) select_none_kernel(int32_t* idx, int32_t* count, int64_t BQ, int64_t k) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < BQ * k) idx[i] = -1;
  if (i < BQ) count[i] = 0;
}

// ---------------------------------------------------------------- merge (streaming prefill)
//
// Query-tiled calls run the cache in ranges of kStreamKeys entries, so the
// workspace holds one range's scores and lists, not the whole cache's.  Each
// range gets its own top-k by the kernels above (entry numbers relative to
// the range); this kernel folds it into the query's running top-k: the k
// best of (running, range) under the selection's order (score descending,
// then index ascending) are the k best of the union, since every entry left
// out of either part has k better ones in that part.  One workgroup per
// query: the candidates (running entries first, then the range's, so in
// ascending index order) are staged in LDS, radix passes over the composite
// key (score key, then the bit-inverted index) find the k_eff-th, and the
// chosen ones are written in index order with their scores.
struct MergeArgs {
  const int32_t* in_idx;   // [BQ][k] running top-k (entry numbers), or nullptr before the first range
  const float* in_sc;      // [BQ][k] their scores
  const int32_t* in_cnt;   // [BQ]
  const int32_t* part_idx; // [BQ][k] the range's top-k, relative to key_begin
  const int32_t* part_cnt; // [BQ]
  const float* part_sc;    // the range's scores, row bq at part_sc + bq*score_ld, relative entries
  int64_t score_ld, key_begin, k;
  int32_t* out_idx;        // [BQ][k], -1 after the count
  float* out_sc;           // [BQ][k] or nullptr (the last range)
  int32_t* out_cnt;        // [BQ]
};

__global__ void __launch_bounds__(256) merge_topk_kernel(MergeArgs a) {
  extern __shared__ uint32_t mlds[];  // [2k] entries, then [2k] score keys
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t scratch[19];
  __shared__ uint32_t wsum[4];
  const int tid = threadIdx.x;
  const int64_t bq = blockIdx.x, k = a.k;
  int32_t* ent = reinterpret_cast<int32_t*>(mlds);
  uint32_t* key = mlds + 2 * k;
  const int64_t n_in = a.in_idx ? min(max(int64_t(a.in_cnt[bq]), int64_t(0)), k) : 0;
  const int64_t n_p = min(max(int64_t(a.part_cnt[bq]), int64_t(0)), k);
  const uint32_t n = uint32_t(n_in + n_p), keff = uint32_t(min(int64_t(n), k));
  for (uint32_t j = tid; j < n; j += 256) {
    int32_t e;
    float sc;
    if (j < n_in) {
      e = a.in_idx[bq * k + j];
      sc = a.in_sc[bq * k + j];
    } else {
      const int32_t r = a.part_idx[bq * k + (j - n_in)];
      e = int32_t(a.key_begin + r);
      sc = a.part_sc[bq * a.score_ld + r];
    }
    ent[j] = e;
    key[j] = order_key(sc);
  }
  __syncthreads();
  auto composite = [&](uint32_t j) { return (uint64_t(key[j]) << 32) | uint64_t(0xffffffffu - uint32_t(ent[j])); };
  // the exact k_eff-th composite key (all are distinct), when some are left out
  uint64_t thr = 0;
  if (n > keff) {
    uint32_t need = keff;
    uint64_t pval = 0, pmask = 0;
    for (int pass = 0; pass < 6 && need > 0; ++pass) {
      const int shift = pass == 0 ? 53 : pass == 1 ? 42 : pass == 2 ? 32 : pass == 3 ? 21 : pass == 4 ? 10 : 0;
      const int bits = (pass == 2 || pass == 5) ? 10 : 11;
      const uint32_t dmask = (1u << bits) - 1u;
      for (int i = tid; i < kBins; i += 256) h[i] = 0;
      __syncthreads();
      for (uint32_t j = tid; j < n; j += 256) {
        const uint64_t c = composite(j);
        if ((c & pmask) == pval) atomicAdd(&h[(c >> shift) & dmask], 1u);
      }
      __syncthreads();
      uint32_t v[8], above, hD, total;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = h[8 * tid + i];
      int D;
      find_threshold_regs<8>(v, need, scratch, &D, &above, &total, &hD);
      pval |= uint64_t(D) << shift;
      pmask |= uint64_t(dmask) << shift;
      if (above + hD == need) break;
      need -= above;
    }
    thr = pval;
  }
  // chosen candidates in index order: thread j counts its run, one scan ranks them
  const uint32_t per = (n + 255) / 256;
  const uint32_t lo = tid * per, hi = min(n, lo + per);
  uint32_t mine = 0;
  for (uint32_t j = lo; j < hi; ++j) mine += composite(j) >= thr ? 1u : 0u;
  uint32_t tot;
  uint32_t r = scan_block<4>(mine, wsum, &tot);
  for (uint32_t j = lo; j < hi; ++j) {
    if (composite(j) < thr) continue;
    if (r < keff) {
      a.out_idx[bq * k + r] = ent[j];
      if (a.out_sc) a.out_sc[bq * k + r] = key_score(key[j]);
    }
    ++r;
  }
  for (int64_t j = keff + tid; j < k; j += 256) a.out_idx[bq * k + j] = -1;
  if (tid == 0) a.out_cnt[bq] = int32_t(keff);
}

// ---------------------------------------------------------------- host

struct WsLayout {
  size_t scores, hist, ccnt, sel, cand, cand_kseg, cand_srk, cand_idx, cand_key, cand_srk2, chosen, total;
};

// keys per workgroup of the VALU scores kernel: a multiple of 64 chosen so
// that the whole batch takes about kScoreWorkgroups workgroups, and at most
// kMaxChunks chunks per query.  The MFMA scores kernels size their own grids
// (kScoreRegWorkgroups, kFp4RegWorkgroups: tiles interleaved over the
// workgroups of a query), and the selection its own chunks
// (kSelectDecodeWorkgroups).
#ifndef DLC_SCORES_WGS
#define DLC_SCORES_WGS 512
#endif
constexpr int64_t kScoreWorkgroups = DLC_SCORES_WGS;
constexpr int64_t kScoreRegWorkgroups = DLC_SCORES_RWGS;
// query-tiled (prefill) calls: the chunks of the histogram and filter
// kernels, sized for eight 256-thread workgroups per CU
constexpr int64_t kSelectWorkgroups = 2048;
// per-query (decode) calls: the chunks of the selection kernel, which need
// not be the scores kernel's.  Fewer, longer chunks leave the workgroup that
// finishes a query fewer chunk lists to walk.
#ifndef DLC_SELECT_WGS
#define DLC_SELECT_WGS 256
#endif
constexpr int64_t kSelectDecodeWorkgroups = DLC_SELECT_WGS;
// queries per sequence from which the indexer runs query-tiled (prefill)
#ifndef DLC_PREFILL_MIN_Q
#define DLC_PREFILL_MIN_Q 64
#endif
constexpr int64_t kPrefillMinQueries = DLC_PREFILL_MIN_Q;
#ifndef DLC_FP4_U
#define DLC_FP4_U 3  // key tiles in flight per wave in the FP4 register-load kernel
#endif
#ifndef DLC_FP4_RWGS
#define DLC_FP4_RWGS 768  // its workgroups per call
#endif
constexpr int64_t kFp4RegWorkgroups = DLC_FP4_RWGS;
// wgs: the workgroups the batch should take (kScoreWorkgroups for the VALU
// scores kernel, kSelectDecodeWorkgroups for the decode selection,
// kSelectWorkgroups for the query-tiled histogram and filter kernels)
int64_t keys_per_wg(int64_t BQ, int64_t vis_max, int64_t wgs = kScoreWorkgroups) {
  const int64_t vis = vis_max > 0 ? vis_max : 1;
  int64_t kpw = ceil_div(ceil_div(vis * BQ, wgs), 64) * 64;
  kpw = kpw < 64 ? 64 : kpw;
  const int64_t floor_kpw = ceil_div(ceil_div(vis, kMaxChunks), 64) * 64;  // at most kMaxChunks chunks
  return kpw > floor_kpw ? kpw : floor_kpw;
}

WsLayout ws_layout(int64_t B, int64_t n_q, int64_t cap, int64_t k, bool own_scores) {
  const size_t BQ = size_t(B) * size_t(n_q);
  WsLayout L{};
  size_t off = 0;
  L.hist = off;      off = align_up(off + BQ * (kBins * 2 + kTicketStride) * 4, 256);  // hist, hist2, tickets
  L.ccnt = off;      off = align_up(off + BQ * kMaxChunks * 2 * 4, 256);
  L.sel = off;       off = align_up(off + BQ * size_t(cap) * 4, 256);
  L.cand = off;      off = align_up(off + BQ * size_t(cap) * 4, 256);
  L.cand_kseg = off; off = align_up(off + BQ * size_t(cap) * 4, 256);
  L.cand_srk = off;  off = align_up(off + BQ * size_t(cap) * 4, 256);
  L.cand_idx = off;  off = align_up(off + BQ * size_t(cap) * 4, 256);
  L.cand_key = off;  off = align_up(off + BQ * size_t(cap) * 4, 256);
  L.cand_srk2 = off; off = align_up(off + BQ * size_t(cap) * 4, 256);
  L.chosen = off;    off = align_up(off + BQ * size_t(k) * 4, 256);
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
  a.ticket = a.hist2 + size_t(BQ) * kBins;
  a.ccnt = reinterpret_cast<uint32_t*>(w + L.ccnt);
  a.sel = reinterpret_cast<int32_t*>(w + L.sel);
  a.cand = reinterpret_cast<int32_t*>(w + L.cand);
  a.cand_kseg = reinterpret_cast<uint32_t*>(w + L.cand_kseg);
  a.cand_srk = reinterpret_cast<uint32_t*>(w + L.cand_srk);
  a.cand_idx = reinterpret_cast<int32_t*>(w + L.cand_idx);
  a.cand_key = reinterpret_cast<uint32_t*>(w + L.cand_key);
  a.cand_srk2 = reinterpret_cast<uint32_t*>(w + L.cand_srk2);
  a.chosen = reinterpret_cast<int32_t*>(w + L.chosen);
  a.max_chunks = kMaxChunks;
}

// the selection: scores (and the first histogram) -> idx, count
int select_topk(IdxArgs& a, int64_t BQ, int64_t vis_max, hipStream_t s) {
  StageTimer timer(DLC_STAGE_TOPK_SELECT, s);
  if (vis_max == 0) {
    hipLaunchKernelGGL(select_none_kernel, dim3((unsigned)ceil_div(BQ * a.k, 256)), dim3(256), 0, s, a.idx, a.count,
                       BQ, a.k);
    return check_launch("csa_index_topk/select");
  }
  const int64_t nchunks = ceil_div(vis_max, a.keys_per_wg);
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)nchunks, (unsigned)BQ, 1u), dim3(kSelThreads), 0, s, a);
  return check_launch("csa_index_topk/select");
}

// Query-tiled calls (n_q >= kPrefillMinQueries) run the cache in ranges of
// kStreamKeys entries and fold each range's top-k into a running one
// (merge_topk_kernel), so their workspace grows with n_q, not with n_q * cap.
#ifndef DLC_STREAM_KEYS
#define DLC_STREAM_KEYS 32768
#endif
constexpr int64_t kStreamKeys = DLC_STREAM_KEYS;
bool streaming(int64_t n_q) { return n_q >= kPrefillMinQueries; }

// a call's workspace: the arrays of one range (of the whole cache when not
// streaming), then the two running top-k buffers and the range's top-k
struct CallWs {
  WsLayout L;
  int64_t range;
  size_t run_idx[2], run_sc[2], run_cnt[2], part_idx, part_cnt, total;
};
CallWs call_ws(int64_t B, int64_t n_q, int64_t cap, int64_t k, bool own_scores) {
  CallWs w{};
  const size_t BQ = size_t(B) * size_t(n_q);
  w.range = streaming(n_q) ? std::min(cap, kStreamKeys) : cap;
  w.L = ws_layout(B, n_q, w.range, k, own_scores);
  size_t off = w.L.total;
  if (streaming(n_q)) {
    for (int i = 0; i < 2; ++i) {
      w.run_idx[i] = off; off = align_up(off + BQ * size_t(k) * 4, 256);
      w.run_sc[i] = off;  off = align_up(off + BQ * size_t(k) * 4, 256);
      w.run_cnt[i] = off; off = align_up(off + BQ * 4, 256);
    }
    w.part_idx = off; off = align_up(off + BQ * size_t(k) * 4, 256);
    w.part_cnt = off; off = align_up(off + BQ * 4, 256);
  }
  w.total = off;
  return w;
}

// the FP4 call's workspace: the common layout, then the quantized queries
struct Fp4Ws {
  size_t code, scale, total;
};
Fp4Ws fp4_query_off(int64_t B, int64_t n_q, int64_t cap, int64_t k, int64_t n_hI, int64_t cI) {
  const size_t rows = size_t(B) * size_t(n_q) * size_t(n_hI);
  Fp4Ws w{};
  w.code = call_ws(B, n_q, cap, k, true).total;
  w.scale = align_up(w.code + rows * size_t(cI / 2), 256);
  w.total = align_up(w.scale + rows * size_t(cI / 32), 256);
  return w;
}

// entries of the range a.key_begin .. a.key_begin + a.cap - 1 visible to the
// query with the largest t
int64_t host_visible_max(const IdxArgs& a) {
  const int64_t v = a.t_max / a.m - a.key_begin;
  return v < 0 ? 0 : (v < a.cap ? v : a.cap);
}

// The call over the whole cache, or range by range.  a carries the inputs;
// range(a) runs scores and selection over the range set in a (key_begin,
// cap, KI, k_scale, scores, idx, count); key_row / scale_row are the bytes
// of one cache entry (and of its scales).
template <typename Range>
int run_call(IdxArgs& a, const CallWs& w, void* ws, float* scores, int64_t BQ, int64_t cap, int32_t* idx,
             int32_t* count, size_t key_row, size_t scale_row, hipStream_t s, Range range) {
  const void* KI0 = a.KI;
  const uint8_t* KS0 = a.k_scale;
  a.key_bstride = cap;
  if (!streaming(a.n_q)) {
    a.key_begin = 0;
    a.cap = cap;
    bind_ws(a, w.L, ws, scores, BQ, cap);
    a.idx = idx;
    a.count = count;
    return range(a);
  }
  const int64_t vis_total = std::min(a.t_max / a.m, cap);
  if (vis_total == 0) {
    a.idx = idx;
    a.count = count;
    return select_topk(a, BQ, 0, s);
  }
  char* wb = static_cast<char*>(ws);
  const size_t mlds = size_t(2) * size_t(a.k) * 8;
  if (mlds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&merge_topk_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(mlds));
    if (e != hipSuccess) return fail(DLC_E_HIP, "csa_index_topk: hipFuncSetAttribute: %s", hipGetErrorString(e));
  }
  int cur = 0, rc;
  // the scores stage of a streaming call is the whole indexer: every range's
  // scores, selection and merge
  StageTimer timer(DLC_STAGE_INDEX_SCORES, s);
  for (int64_t r0 = 0; r0 < vis_total; r0 += w.range) {
    a.key_begin = r0;
    a.cap = std::min(w.range, cap - r0);
    a.KI = static_cast<const char*>(KI0) + size_t(r0) * key_row;
    if (KS0) a.k_scale = KS0 + size_t(r0) * scale_row;
    bind_ws(a, w.L, ws, scores ? scores + r0 : nullptr, BQ, w.range);
    if (scores) a.score_ld = cap;
    a.idx = reinterpret_cast<int32_t*>(wb + w.part_idx);
    a.count = reinterpret_cast<int32_t*>(wb + w.part_cnt);
    if ((rc = range(a))) return rc;
    const bool last = r0 + w.range >= vis_total;
    MergeArgs m{};
    if (r0 > 0) {
      m.in_idx = reinterpret_cast<const int32_t*>(wb + w.run_idx[cur]);
      m.in_sc = reinterpret_cast<const float*>(wb + w.run_sc[cur]);
      m.in_cnt = reinterpret_cast<const int32_t*>(wb + w.run_cnt[cur]);
    }
    m.part_idx = a.idx;
    m.part_cnt = a.count;
    m.part_sc = a.scores;
    m.score_ld = a.score_ld;
    m.key_begin = r0;
    m.k = a.k;
    m.out_idx = last ? idx : reinterpret_cast<int32_t*>(wb + w.run_idx[cur ^ 1]);
    m.out_sc = last ? nullptr : reinterpret_cast<float*>(wb + w.run_sc[cur ^ 1]);
    m.out_cnt = last ? count : reinterpret_cast<int32_t*>(wb + w.run_cnt[cur ^ 1]);
    {
      StageTimer timer(DLC_STAGE_TOPK_SELECT, s);
      hipLaunchKernelGGL(merge_topk_kernel, dim3((unsigned)BQ), dim3(256), mlds, s, m);
    }
    if ((rc = check_launch("csa_index_topk/merge"))) return rc;
    cur ^= 1;
  }
  return DLC_OK;
}

}  // namespace
}  // namespace dlc

extern "C" {

size_t csa_index_topk_ws(int64_t B, int64_t n_q, int64_t cap, int64_t k) {
  if (B < 1 || n_q < 1 || cap < 0 || k < 1) return 0;
  return dlc::call_ws(B, n_q, cap, k, true).total;
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
  const CallWs W = call_ws(B, n_q, cap, k, scores == nullptr);
  DLC_REQUIRE(ws != nullptr && ws_bytes >= W.total, DLC_E_WORKSPACE,
              "csa_index_topk: workspace of %zu bytes needed, %zu given", W.total, ws_bytes);
  DLC_REQUIRE(aligned(ws, 256), DLC_E_WORKSPACE, "csa_index_topk: workspace must be 256-byte aligned");
  DLC_REQUIRE(B * n_q <= 65535, DLC_E_UNSUPPORTED, "csa_index_topk: B*n_q > 65535");
  const bool mfma = mfma_shape && aligned(qI, 16) && (cap == 0 || aligned(KI, 16));
  DLC_REQUIRE(mfma || n_hI * cI <= 8192, DLC_E_UNSUPPORTED, "csa_index_topk: MFMA shape needs 16-byte alignment");

  hipStream_t s = as_stream(stream);
  IdxArgs a{};
  a.qI = qI; a.wI = wI; a.KI = KI; a.t = t;
  a.n_q = n_q; a.n_hI = n_hI; a.cI = cI; a.m = m; a.k = k; a.t_max = t_max;
  const int64_t BQ = B * n_q;
  const size_t esz = dtype == DLC_BF16 ? 2 : 4;
  const bool prefill = mfma && cI == 128 && n_q >= kPrefillMinQueries;
  auto range = [&](IdxArgs& r) -> int {
    int rc;
    const int64_t vis_max = host_visible_max(r);
    if (vis_max > 0) {
      r.keys_per_wg = keys_per_wg(BQ, vis_max, prefill ? kSelectWorkgroups : kScoreWorkgroups);
      const int64_t nchunks = ceil_div(vis_max, r.keys_per_wg);
      dim3 grid{(unsigned)nchunks, (unsigned)BQ, 1u};
      {
      // the decode scores kernel is one launch: the armed events go on its dispatch
      hipEvent_t evb = nullptr, eve = nullptr;
      if (!prefill && mfma) take_stage_events(DLC_STAGE_INDEX_SCORES, &evb, &eve);
      StageTimer timer(DLC_STAGE_INDEX_SCORES, s);
      if (prefill) {
        dim3 pgrid{(unsigned)ceil_div(vis_max, 256), (unsigned)ceil_div(n_q, 64), (unsigned)B};
        hipLaunchKernelGGL((scores_prefill_kernel<128>), pgrid, dim3(512), 0, s, r);
      } else if (mfma) {
        const int HT = int(ceil_div(n_hI, 16)), KT = int(cI / 32);
        // G workgroups per query, about kScoreRegWorkgroups in all, 64 keys each at least
        const IdxArgs& rs = r;
        const int64_t G = std::max<int64_t>(1, std::min(ceil_div(kScoreRegWorkgroups, BQ), ceil_div(vis_max, 64)));
        const dim3 sgrid{(unsigned)G, (unsigned)BQ, 1u};
#define DLC_SCORES(ht, kt) \
  if (HT == ht && KT == kt)                                                                              \
    hipExtLaunchKernelGGL((scores_reg_kernel<ht, kt, kt >= 8 ? 2 : DLC_SCORES_U>), sgrid, dim3(256), 0, s, evb, \
                          eve, 0u, rs);
        DLC_SCORES(1, 1) DLC_SCORES(1, 2) DLC_SCORES(1, 4) DLC_SCORES(1, 8)
        DLC_SCORES(2, 1) DLC_SCORES(2, 2) DLC_SCORES(2, 4) DLC_SCORES(2, 8)
        DLC_SCORES(3, 1) DLC_SCORES(3, 2) DLC_SCORES(3, 4) DLC_SCORES(3, 8)
        DLC_SCORES(4, 1) DLC_SCORES(4, 2) DLC_SCORES(4, 4) DLC_SCORES(4, 8)
#undef DLC_SCORES
      } else {
        const size_t smem = (kBins + n_hI * cI + n_hI) * 4;
        if (dtype == DLC_BF16)
          hipLaunchKernelGGL((scores_valu_kernel<bf16_raw>), grid, dim3(256), smem, s, r);
        else
          hipLaunchKernelGGL((scores_valu_kernel<float>), grid, dim3(256), smem, s, r);
      }
      }
      if ((rc = check_launch("csa_index_topk/scores"))) return rc;
      if (prefill) {  // the first-digit histogram, which the other scores kernels build as they go
        hipLaunchKernelGGL(hist_kernel, grid, dim3(256), 0, s, r);
        if ((rc = check_launch("csa_index_topk/hist"))) return rc;
      }
    }
    if (vis_max > 0 && !prefill) r.keys_per_wg = keys_per_wg(BQ, vis_max, kSelectDecodeWorkgroups);
    return select_topk(r, BQ, vis_max, s);
  };
  return run_call(a, W, ws, scores, BQ, cap, idx, count, size_t(cI) * esz, 0, s, range);
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
  DLC_REQUIRE(aligned(qI, 16) && (cap == 0 || (aligned(KIc, 16) && aligned(KIs, 4))), DLC_E_INVAL,
              "csa_index_topk_fp4: qI and KIc must be 16-byte aligned, KIs 4-byte aligned");
  const CallWs CW = call_ws(B, n_q, cap, k, true);
  const Fp4Ws W = fp4_query_off(B, n_q, cap, k, n_hI, cI);
  DLC_REQUIRE(ws != nullptr && ws_bytes >= W.total, DLC_E_WORKSPACE,
              "csa_index_topk_fp4: workspace of %zu bytes needed, %zu given", W.total, ws_bytes);
  DLC_REQUIRE(aligned(ws, 256), DLC_E_WORKSPACE, "csa_index_topk_fp4: workspace must be 256-byte aligned");
  DLC_REQUIRE(B * n_q <= 65535, DLC_E_UNSUPPORTED, "csa_index_topk_fp4: B*n_q > 65535");

  hipStream_t s = as_stream(stream);
  IdxArgs a{};
  a.qI = qI; a.wI = wI; a.KI = KIc; a.k_scale = KIs; a.t = t;
  a.n_q = n_q; a.n_hI = n_hI; a.cI = cI; a.m = m; a.k = k; a.t_max = t_max;
  const int64_t BQ = B * n_q;
  uint8_t* qc = static_cast<uint8_t*>(ws) + W.code;
  uint8_t* qsc = static_cast<uint8_t*>(ws) + W.scale;
  a.q_code = qc; a.q_scale = qsc;

  int rc;
  if (t_max / m > 0) {  // histograms and tickets cleared and queries quantized by one launch
    uint32_t* hist = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + CW.L.hist);
    const int64_t nhist = BQ * (kBins * 2 + kTicketStride), qblocks = BQ * n_hI * (cI / 32);
    const int fill_blocks = int(std::min<int64_t>(ceil_div(nhist, 1024), 256));
    const dim3 pgrid{unsigned(fill_blocks + ceil_div(qblocks, 256)), 1u, 1u};
    if (dtype == DLC_BF16)
      hipLaunchKernelGGL(prep_fp4_kernel<bf16_raw>, pgrid, dim3(256), 0, s, hist, nhist, fill_blocks,
                         static_cast<const bf16_raw*>(qI), qblocks, cI / 32, qc, qsc);
    else
      hipLaunchKernelGGL(prep_fp4_kernel<float>, pgrid, dim3(256), 0, s, hist, nhist, fill_blocks,
                         static_cast<const float*>(qI), qblocks, cI / 32, qc, qsc);
    if ((rc = check_launch("csa_index_topk_fp4/prep"))) return rc;
  }
  const bool prefill = cI == 128 && n_q >= kPrefillMinQueries;
  auto range = [&](IdxArgs& r) -> int {
    int rc2;
    const int64_t vis_max = host_visible_max(r);
    if (vis_max > 0) {
      r.keys_per_wg = keys_per_wg(BQ, vis_max, prefill ? kSelectWorkgroups : kScoreWorkgroups);
      dim3 grid{(unsigned)ceil_div(vis_max, r.keys_per_wg), (unsigned)BQ, 1u};
      {
      hipEvent_t evb = nullptr, eve = nullptr;
      if (!prefill && (cI == 128 || cI == 256)) take_stage_events(DLC_STAGE_INDEX_SCORES, &evb, &eve);
      StageTimer timer(DLC_STAGE_INDEX_SCORES, s);
      if (prefill) {
        dim3 pgrid{(unsigned)ceil_div(vis_max, 256), (unsigned)ceil_div(n_q, 64), (unsigned)B};
        hipLaunchKernelGGL((scores_prefill_fp4_kernel<128>), pgrid, dim3(512), 0, s, r);
      }
      // the register-load kernel on its own grid, as the bf16 one
      const int64_t G = std::max<int64_t>(1, std::min(ceil_div(kFp4RegWorkgroups, BQ), ceil_div(vis_max, 64)));
      const dim3 sgrid{(unsigned)G, (unsigned)BQ, 1u};
      if (!prefill && cI == 128)
        hipExtLaunchKernelGGL((scores_fp4_reg_kernel<128, DLC_FP4_U>), sgrid, dim3(256), 0, s, evb, eve, 0u, r);
      if (!prefill && cI == 256)
        hipExtLaunchKernelGGL((scores_fp4_reg_kernel<256, DLC_FP4_U>), sgrid, dim3(256), 0, s, evb, eve, 0u, r);
      }
      if ((rc2 = check_launch("csa_index_topk_fp4/scores"))) return rc2;
      if (prefill) {
        hipLaunchKernelGGL(hist_kernel, grid, dim3(256), 0, s, r);
        if ((rc2 = check_launch("csa_index_topk_fp4/hist"))) return rc2;
      }
    }
    if (vis_max > 0 && !prefill) r.keys_per_wg = keys_per_wg(BQ, vis_max, kSelectDecodeWorkgroups);
    return select_topk(r, BQ, vis_max, s);
  };
  return run_call(a, CW, ws, scores, BQ, cap, idx, count, size_t(cI / 2), size_t(cI / 32), s, range);
}

}  // extern "C"
