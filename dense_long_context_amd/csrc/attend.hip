// Shared-KV multi-query attention over compressed entries.
//
// "DeepSeek-V4 Hybrid Attention: CSA and HCA from Scratch": §8 (CSA core
// attention over the top-k set: key = value = the compressed entry, logits
// q.C/sqrt(c)) and §10-§11 (HCA: the same attention over every visible entry).
//
// Flash-decoding split-K: the key range of a query is cut into splits; each
// workgroup runs an online softmax over its split and writes a normalised
// partial output plus its log-sum-exp; a combine kernel merges the splits
// exactly (o = sum_j e^{lse_j - lse} o_j, lse = log sum_j e^{lse_j}).
//
// MFMA paths (bf16).  A workgroup is 8 waves and covers 128 heads; all heads
// share each key row, so a 32-key tile is staged once in LDS, row-major for
// Q.K^T and read transposed for P.V.
//  * c in {128, 256} (attend_mfma_kernel): wave w owns heads 32*(w/2) .. +31
//    and half w%2 of the c dimensions, with v_mfma_f32_32x32x16_bf16:
//      S^T[32 keys][32 heads] = K[32 keys][half] . Q^T[half][32 heads]
//      (the two halves' partial S^T are swapped through LDS and added)
//      O[32 heads][half]     += P[32 heads][32 keys] . V[32 keys][half]
//    The S^T accumulator already holds, per lane, the 16 keys of one head
//    that the P operand needs, so P never goes through memory.  Tiles are
//    double-buffered.
//  * c = 512 (attend512_kernel): 16 heads per wave over all 512 dims, a
//    four-buffer tile ring with P.V of one tile interleaved with Q.K^T of the
//    next, and bf16 split-K partials written in MFMA fragment order
//    (described at the kernel, merged by combine_frag_kernel).  A workgroup
//    is 8 waves (128 heads), or 4 waves (64 heads) when the minimum split
//    length leaves the 128-head grid under half the target.  Over dense keys
//    (HCA) the 8-wave kernel runs in its HD form: the softmax stays per head,
//    P is exchanged through LDS and each wave owns a 64-dim slice of O for
//    every head, so the LDS reads per tile drop from 64 KB to 44 KB a wave.
// The VALU path covers fp32 and other shapes.
#include "common.hpp"

#include <mutex>

namespace dlc {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// split policy: aim for kTargetWorkgroups workgroups, but give every split at
// least kMinKeysPerSplit keys (the partial output of a split costs as much
// traffic as 2*heads/keys of its key reads)
#ifndef DLC_ATTEND_TARGET_WGS
#define DLC_ATTEND_TARGET_WGS 256
#endif
#ifndef DLC_ATTEND_MIN_KEYS
#define DLC_ATTEND_MIN_KEYS 64
#endif
constexpr int kMinKeysPerSplit = DLC_ATTEND_MIN_KEYS;
// split-K partial outputs of the c = 512 MFMA path in bf16 (halves their
// write and the combine's read; the final output and lse stay fp32)
#ifndef DLC_BF16_PARTIALS
#define DLC_BF16_PARTIALS 1
#endif
constexpr bool kBf16Partials = DLC_BF16_PARTIALS != 0;
constexpr int kTargetWorkgroups = DLC_ATTEND_TARGET_WGS;
// the HD form of the c = 512 kernel for dense keys (eight waves; with the
// window's ring arithmetic it would spill a register), for splits of at
// least kHdMinKeys keys: its two extra barriers and the per-tile flag reads
// are a fixed cost that a short (decode) split does not win back
#ifndef DLC_ATTEND_HD
#define DLC_ATTEND_HD 1
#endif
constexpr bool kHeadsDims = DLC_ATTEND_HD != 0;
#ifndef DLC_HD_MIN_KEYS
#define DLC_HD_MIN_KEYS 1024
#endif
constexpr int64_t kHdMinKeys = DLC_HD_MIN_KEYS;



// which keys a query attends to
constexpr int kDense = 0;   // entries s < min(floor(t/m'), cap)            (HCA)
constexpr int kGather = 1;  // entries idx[0 .. count-1]                     (CSA)
constexpr int kWindow = 2;  // tokens max(0, t-n_win+1) .. t of a ring of n_win rows

struct AttArgs {
  const void* q;        // [BQ][n_h][c]
  const void* kv;       // [B][cap][c]; window: the ring of cap rows
  const int32_t* idx;   // gather: [BQ][k]
  const int32_t* count; // gather: [BQ]
  const int64_t* t;     // dense, window: [BQ]
  int64_t n_q, n_h, c, cap, k, m_prime, t_max;
  int64_t n_win;        // window: tokens per window (<= cap)
  // optional sliding-window tail after the mode's own keys (the joined forms of
  // csa_attend / hca_attend): tokens max(0,t-win_n+1) .. t of the ring win
  const void* win;      // [B][win_ring][c] or nullptr
  int64_t win_ring, win_n, win_tmax;
  const int64_t* win_t; // [BQ]
  int64_t splits, keys_per_split, head_groups;
  float scale_log2;
  float* o;             // [BQ][splits][n_h][c] (splits == 1: the final output)
  bf16_raw* ob;         // c = 512 MFMA path with partials: [BQ][splits][n_h][c] bf16 (o unused)
  float* lse;           // [BQ][splits][n_h] (may be nullptr when splits == 1)
};

template <int MODE>
__device__ __forceinline__ int64_t n_keys(const AttArgs& a, int64_t bq) {
  if constexpr (MODE == kGather) {
    int64_t n = a.count[bq];
    return n < 0 ? 0 : (n > a.k ? a.k : n);
  } else {
    int64_t t = a.t[bq];
    t = t < 0 ? 0 : (t > a.t_max ? a.t_max : t);
    if constexpr (MODE == kWindow) {
      return t + 1 < a.n_win ? t + 1 : a.n_win;
    } else {
      const int64_t v = t / a.m_prime;
      return v < a.cap ? v : a.cap;
    }
  }
}

// row of the j-th key of query bq, or -1 if that key is masked (j >= lim);
// nk is the query's key count (n_keys)
template <int MODE>
__device__ __forceinline__ int64_t key_row(const AttArgs& a, int64_t bq, int64_t j, int64_t lim, int64_t nk) {
  if (j >= lim) return -1;
  if constexpr (MODE == kGather) {
    const int64_t r = a.idx[bq * a.k + j];
    return (r >= 0 && r < a.cap) ? r : -1;
  } else if constexpr (MODE == kWindow) {
    int64_t t = a.t[bq];
    t = t < 0 ? 0 : (t > a.t_max ? a.t_max : t);
    return (t - nk + 1 + j) % a.cap;  // token position modulo the ring size
  } else {
    return j;
  }
}

// keys of the sliding-window tail of query bq (0 without one)
__device__ __forceinline__ int64_t n_win_keys(const AttArgs& a, int64_t bq) {
  if (a.win == nullptr) return 0;
  int64_t t = a.win_t[bq];
  t = t < 0 ? 0 : (t > a.win_tmax ? a.win_tmax : t);
  return t + 1 < a.win_n ? t + 1 : a.win_n;
}

// Encoded source of key j of query bq (j < lim, else -1): r >= 0 is row r of
// the mode's cache, -2 - r is row r of the window ring, -1 a masked key.  nkm
// is the count of the mode's own keys, which come first.
template <int MODE>
__device__ __forceinline__ int64_t key_code(const AttArgs& a, int64_t bq, int64_t j, int64_t lim, int64_t nkm) {
  if (j >= lim) return -1;
  if (j < nkm) return key_row<MODE>(a, bq, j, nkm, nkm);
  int64_t t = a.win_t[bq];
  t = t < 0 ? 0 : (t > a.win_tmax ? a.win_tmax : t);
  const int64_t nkw = t + 1 < a.win_n ? t + 1 : a.win_n;
  return -2 - (t - nkw + 1 + (j - nkm)) % a.win_ring;
}

template <typename T>
__device__ __forceinline__ const T* key_ptr(const AttArgs& a, int64_t b, int64_t code) {
  if (code >= 0) return static_cast<const T*>(a.kv) + (b * a.cap + code) * a.c;
  if (code <= -2) return static_cast<const T*>(a.win) + (b * a.win_ring + (-2 - code)) * a.c;
  return nullptr;
}

// ------------------------------------------------------------------ VALU path

template <typename T, int MODE, int MAXD>
__global__ void __launch_bounds__(64) attend_valu_kernel(AttArgs a) {
  const int64_t split = blockIdx.x, h = blockIdx.y, bq = blockIdx.z;
  const int lane = threadIdx.x;
  const int64_t b = bq / a.n_q;
  const int64_t nkm = n_keys<MODE>(a, bq);
  const int64_t nk = nkm + n_win_keys(a, bq);
  const int64_t k0 = split * a.keys_per_split;
  const int64_t k1 = min(nk, k0 + a.keys_per_split);
  const T* q = static_cast<const T*>(a.q) + (bq * a.n_h + h) * a.c;

  float qv[MAXD], acc[MAXD];
#pragma unroll
  for (int u = 0; u < MAXD; ++u) {
    const int64_t d = lane + 64 * u;
    qv[u] = d < a.c ? Fmt<T>::load(q + d) : 0.f;
    acc[u] = 0.f;
  }
  float mrun = -INFINITY, lrun = 0.f;
  for (int64_t j = k0; j < k1; ++j) {
    const T* row = key_ptr<T>(a, b, key_code<MODE>(a, bq, j, nk, nkm));
    if (row == nullptr) continue;
    float cv[MAXD];
    float dot = 0.f;
#pragma unroll
    for (int u = 0; u < MAXD; ++u) {
      const int64_t d = lane + 64 * u;
      cv[u] = d < a.c ? Fmt<T>::load(row + d) : 0.f;
      dot = fmaf(qv[u], cv[u], dot);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
    const float x = dot * a.scale_log2;
    const float mnew = fmaxf(mrun, x);
    const float alpha = exp2f(mrun - mnew);  // mrun = -inf gives 0
    const float p = exp2f(x - mnew);
    lrun = lrun * alpha + p;
#pragma unroll
    for (int u = 0; u < MAXD; ++u) acc[u] = fmaf(p, cv[u], acc[u] * alpha);
    mrun = mnew;
  }
  const int64_t slot = (bq * a.splits + split) * a.n_h + h;
  const float inv = lrun > 0.f ? 1.f / lrun : 0.f;
#pragma unroll
  for (int u = 0; u < MAXD; ++u) {
    const int64_t d = lane + 64 * u;
    if (d < a.c) a.o[slot * a.c + d] = acc[u] * inv;
  }
  if (lane == 0 && a.lse) a.lse[slot] = lrun > 0.f ? (mrun + log2f(lrun)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ MFMA path

template <int CD, int MODE>
__global__ void __launch_bounds__(512) attend_mfma_kernel(AttArgs a) {
  constexpr int HALF = CD / 2;
  constexpr int KSH = HALF / 16;  // 16-dim Q.K^T steps in one half of c
  constexpr int NTH = HALF / 32;  // 32-dim P.V output tiles in one half of c
  constexpr int KROW = CD + 8;    // padded row of the row-major key tile (bf16)
  constexpr int VROW = 36;        // padded row of the transposed tile (32 keys + pad)
  constexpr int UNITS = CD;       // staging units: 8 key-quads x CD/8 dim groups
  constexpr int UPT = (UNITS + 511) / 512;
  __shared__ __attribute__((aligned(16))) bf16_raw sK[2][32 * KROW];
  __shared__ __attribute__((aligned(16))) bf16_raw sV[2][CD * VROW];
  __shared__ int32_t sValid[2][32];
  // partial-S^T exchange (8 waves x 16 regs x 64 lanes fp32): inside the key
  // buffer just consumed when it is large enough (c = 512), else its own array
  constexpr bool kXInK = 8 * 16 * 64 * 4 <= 32 * KROW * 2;
  __shared__ float sX[kXInK ? 1 : 8 * 16 * 64];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int hp = wave >> 1, dh = wave & 1;  // head slice of 32, half of c
  const int64_t bq = blockIdx.y;
  const int64_t split = blockIdx.x / a.head_groups;
  const int64_t hg = blockIdx.x - split * a.head_groups;
  const int64_t b = bq / a.n_q;
  const int64_t nkm = n_keys<MODE>(a, bq);
  const int64_t nk = nkm + n_win_keys(a, bq);
  const int64_t k0 = split * a.keys_per_split;
  const int64_t k1 = min(nk, k0 + a.keys_per_split);
  const int64_t hbase = hg * 128 + hp * 32;  // first head of this wave
  const bool active = hbase < a.n_h;

  // Q^T operand over this wave's half of c: lane holds head hbase + l32,
  // dims dh*HALF + ks*16 + g2*8 .. +7
  bf16x8 qf[KSH];
  {
    const int64_t h = hbase + l32;
    const bf16_raw* qp =
        static_cast<const bf16_raw*>(a.q) + (bq * a.n_h + (h < a.n_h ? h : 0)) * CD + dh * HALF + g2 * 8;
#pragma unroll
    for (int ks = 0; ks < KSH; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (h < a.n_h) v = *reinterpret_cast<const uint4*>(qp + ks * 16);
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 o[NTH];
#pragma unroll
  for (int nt = 0; nt < NTH; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[nt][r] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;  // for head hbase + l32

  // staging: unit u -> key quad kq (keys 4kq .. 4kq+3) and 8-dim group dg;
  // consecutive threads take consecutive 16-byte pieces of the same rows
  uint4 stg[UPT][4];
  uint32_t stv[UPT];  // bit j: key 4kq+j is valid
  auto gload = [&](int64_t kbase) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + 512 * i;
      if (u < UNITS) {
        const int kq = u / (CD / 8), dg = u % (CD / 8);
        stv[i] = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16_raw* row = key_ptr<bf16_raw>(a, b, key_code<MODE>(a, bq, kbase + 4 * kq + j, k1, nkm));
          stv[i] |= uint32_t(row != nullptr) << j;
          stg[i][j] = row ? *reinterpret_cast<const uint4*>(row + dg * 8) : make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + 512 * i;
      if (u < UNITS) {
        const int kq = u / (CD / 8), dg = u % (CD / 8);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint4*>(&sK[buf][(4 * kq + j) * KROW + dg * 8]) = stg[i][j];
        // transpose: for each of the 8 dims, the 4 keys' values side by side
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&stg[i][0]);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&stg[i][1]);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&stg[i][2]);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&stg[i][3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // dims 2e (low halves) and 2e+1 (high halves)
          const uint32_t lo01 = (w0[e] & 0xffffu) | (w1[e] << 16);
          const uint32_t lo23 = (w2[e] & 0xffffu) | (w3[e] << 16);
          const uint32_t hi01 = (w0[e] >> 16) | (w1[e] & 0xffff0000u);
          const uint32_t hi23 = (w2[e] >> 16) | (w3[e] & 0xffff0000u);
          *reinterpret_cast<uint2*>(&sV[buf][(dg * 8 + 2 * e) * VROW + 4 * kq]) = make_uint2(lo01, lo23);
          *reinterpret_cast<uint2*>(&sV[buf][(dg * 8 + 2 * e + 1) * VROW + 4 * kq]) = make_uint2(hi01, hi23);
        }
        if (dg == 0)
#pragma unroll
          for (int j = 0; j < 4; ++j) sValid[buf][4 * kq + j] = (stv[i] >> j) & 1;
      }
    }
  };

  const int64_t ntile = k1 > k0 ? (k1 - k0 + 31) / 32 : 0;
  if (ntile > 0) {
    gload(k0);
    swrite(0);
  }
  __syncthreads();
  for (int64_t it = 0; it < ntile; ++it) {
    const int buf = int(it & 1);
    if (it + 1 < ntile) gload(k0 + (it + 1) * 32);
    // partial S^T over this wave's half of c
    f32x16 sx;
#pragma unroll
    for (int r = 0; r < 16; ++r) sx[r] = 0.f;
    if (active) {
      const bf16_raw* krow = &sK[buf][l32 * KROW + dh * HALF + g2 * 8];
      // one LDS fragment in flight ahead of each MFMA; the compiler barrier keeps
      // the scheduler from hoisting every fragment load (and its registers) up front
      bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow);
#pragma unroll
      for (int ks = 0; ks < KSH; ++ks) {
        bf16x8 kn = ka;
        if (ks + 1 < KSH) kn = *reinterpret_cast<const bf16x8*>(krow + (ks + 1) * 16);
        sx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], sx, 0, 0, 0);
        ka = kn;
        asm volatile("" ::: "memory");
      }
    }
    __syncthreads();  // every wave is done with sK[buf]: reuse it for the exchange
    float* xch = kXInK ? reinterpret_cast<float*>(&sK[buf][0]) : sX;
    if (active) {
#pragma unroll
      for (int r = 0; r < 16; ++r) xch[(wave * 16 + r) * 64 + lane] = sx[r];
    }
    __syncthreads();
    if (active) {
      // full S^T = both halves; lane holds head l32, keys kr(r) = 8*(r/4) + 4*g2 + r%4
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float other = xch[((wave ^ 1) * 16 + r) * 64 + lane];
        const float full = dh == 0 ? sx[r] + other : other + sx[r];
        const int kr = 8 * (r >> 2) + 4 * g2 + (r & 3);
        sx[r] = sValid[buf][kr] ? full * a.scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, sx[r]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      // Lazy running max: it moves only when a logit exceeds it by more than 8
      // (a factor 256), so the O rescale is rare; p stays below 2^8 either way
      // and the result is the same softmax.
      const bool move = tmax > mrun + 8.f;
      if (__any(move)) {
        const float mnew = move ? tmax : mrun;
        const float alpha = mrun == -INFINITY ? 0.f : exp2f(mrun - mnew);
        lrun *= alpha;
        mrun = mnew;
        // O rows are heads 8*(r/4) + 4*g2 + r%4: fetch their factors
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float al = __shfl(alpha, 8 * (r >> 2) + 4 * g2 + (r & 3));
#pragma unroll
          for (int nt = 0; nt < NTH; ++nt) o[nt][r] *= al;
        }
      }
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sx[r] = sx[r] == -INFINITY ? 0.f : exp2f(sx[r] - mrun);
        psum += sx[r];
      }
      psum += __shfl_xor(psum, 32);
      lrun += psum;
      bf16x8 pa[2];
#pragma unroll
      for (int uu = 0; uu < 2; ++uu)
#pragma unroll
        for (int e = 0; e < 8; ++e) pa[uu][e] = (__bf16)sx[8 * uu + e];
      // P . V over this wave's half of c: B operand lane holds dim
      // dh*HALF + nt*32 + l32 and keys 16u + 8*(e/4) + 4*g2 + e%4
      auto vfrag = [&](int f) {
        const bf16_raw* vrow = &sV[buf][(dh * HALF + (f >> 1) * 32 + l32) * VROW + 4 * g2 + 16 * (f & 1)];
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
        return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      };
      bf16x8 vb = vfrag(0);
#pragma unroll
      for (int f = 0; f < 2 * NTH; ++f) {
        bf16x8 vn = vb;
        if (f + 1 < 2 * NTH) vn = vfrag(f + 1);
        o[f >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[f & 1], vb, o[f >> 1], 0, 0, 0);
        vb = vn;
        asm volatile("" ::: "memory");
      }
    }
    if (it + 1 < ntile) swrite(buf ^ 1);
    __syncthreads();
  }

  if (!active) return;
  // normalise and write: lane holds dims dh*HALF + nt*32 + l32 of heads 8*(r/4) + 4*g2 + r%4
  const int64_t slot0 = (bq * a.splits + split) * a.n_h;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int hr = 8 * (r >> 2) + 4 * g2 + (r & 3);
    const float l = __shfl(lrun, hr);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t h = hbase + hr;
    if (h < a.n_h) {
      float* op = a.o + (slot0 + h) * CD + dh * HALF + l32;
#pragma unroll
      for (int nt = 0; nt < NTH; ++nt) op[nt * 32] = o[nt][r] * inv;
    }
  }
  if (dh == 0 && g2 == 0 && a.lse && hbase + l32 < a.n_h)
    a.lse[slot0 + hbase + l32] = lrun > 0.f ? (mrun + log2f(lrun)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ shared by the c = 512 kernel

__device__ __align__(16) bf16_raw g_zero_row[512];  // masked keys load this row

constexpr int kTileBytes = 34816;   // 32 rows of 1 KB at the offsets of h16_row_off, rounded up to 1 KB
constexpr int kMaxGatherKeys = 2048;  // keys per split whose rows sit in LDS
typedef short s16x4 __attribute__((ext_vector_type(4)));

// One 16-byte piece of a bf16 split partial.  The partials are read once,
// by the combine kernel (on any XCD), so they are written as nontemporal
// stores rather than left as dirty lines in this XCD's L2 for the write-back
// at the kernel's end.
#ifndef DLC_COMBINE8
#define DLC_COMBINE8 1
#endif
constexpr bool kCombine8 = DLC_COMBINE8 != 0;  // more than 32 splits: eight waves a store
#ifndef DLC_NT_PARTIALS
#define DLC_NT_PARTIALS 1
#endif
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_partial(bf16_raw* p, const bf16x8& v) {
  if constexpr (DLC_NT_PARTIALS != 0)
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_nt, v), reinterpret_cast<u32x4_nt*>(p));
  else
    *reinterpret_cast<bf16x8*>(p) = v;
}

// ------------------------------------------------------------------ MFMA path, c = 512, 16 heads per wave
//
// Eight waves, each owning 16 heads over all 512 dims, so no partial S^T is
// exchanged and no softmax is computed twice.  Per 32-key tile and wave:
//   S^T[16 keys][16 heads] = K[16 keys][32 dims] . Q^T[32 dims][16 heads]
//     (v_mfma_f32_16x16x32_bf16, two 16-key halves x 16 dim steps),
//   O[16 heads][16 dims] += P[16 heads][32 keys] . K[32 keys][16 dims]
//     (32 output tiles).
// Q (64 VGPRs) and O (128) stay in registers at two waves per SIMD.  The S^T
// accumulator of lane l holds head l%16 and keys 4*(l/16) .. +3 of each half,
// which is exactly the A operand P needs (its k-slots relabelled to those
// keys); the B operand reads the same keys through ds_read_b64_tr_b16.
//
// Pipeline: tiles arrive by direct global->LDS loads (dma_row) into a ring of
// four buffers, three tiles ahead.  Step i runs O += P_i . V_i interleaved
// with S^T_{i+1} = K_{i+1} . Q^T (four MFMAs per 32-dim step, every LDS
// operand read one step before its MFMA), then the softmax of tile i+1; the
// per-head max and sum use row swaps (v_permlane16/32_swap) rather than LDS
// permutes, which would queue behind the tile reads.
//
// LDS row layout of this kernel: row r starts at 1024*r + d(r) with
// d(r) = 256*(r/8) + 32*(r%8) + 16*((r/8)%2), so that
//  * the 16 rows of a ds_read_b128 pass (Q.K^T A operand) start on 16
//    distinct 4-bank groups, and
//  * the 8 rows x 32 bytes of a ds_read_b64_tr_b16 pass (P.V B operand,
//    32 lanes) fall on 8 disjoint 8-bank groups.

__device__ __forceinline__ constexpr int h16_row_off(int r) {
  return 1024 * r + 256 * (r >> 3) + 32 * (r & 7) + 16 * ((r >> 3) & 1);
}
static_assert(h16_row_off(31) + 1024 <= kTileBytes, "tile layout");

// HD (heads / dims) form, eight waves: S^T and the softmax stay per head
// (wave w, heads 16w .. 16w+15), but the P.V product is split by output
// dims: wave w owns O[all 128 heads][dims 64w .. 64w+63].  Each wave puts its
// P fragment (16 bytes per lane, already in the A-operand layout) into LDS
// and every wave reads the eight fragments back, so per tile and wave the
// LDS delivers the 32 KB key tile once (for S^T), a 4 KB slice of it (V)
// and 8 KB of P, instead of the whole tile twice.  A running max that moves
// is published as per-head factors alpha with a flag per wave; the owners of
// the O slices apply them before adding the tile.  Double-buffered P,
// alpha and flags need no barrier beyond the one per tile.
template <int MODE, int NW, bool HD = false>  // NW waves: 16*NW heads per workgroup
__global__ void __launch_bounds__(64 * NW) attend512_kernel(AttArgs a) {
  constexpr int CD = 512, KS = 16, NT = 32;  // 32-dim Q.K^T steps; 16-dim output tiles
  constexpr int NST = 4, RPW = 32 / NW, HPG = 16 * NW;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(!HD || (NW == 8 && MODE != kGather), "the HD form: eight waves, no gather list (LDS)");
  __shared__ __attribute__((aligned(1024))) unsigned char sK[NST * kTileBytes];
  __shared__ int32_t sRow[MODE == kGather ? kMaxGatherKeys : 1];
  constexpr int PB = HD ? 2 : 1;
  __shared__ __attribute__((aligned(16))) bf16x8 sP[PB][HD ? 8 : 1][64];  // [buffer][head block][lane]
  __shared__ __attribute__((aligned(16))) float sAlpha[PB][HD ? 128 : 4];
  __shared__ __attribute__((aligned(16))) int32_t sMove[PB][8];
  __shared__ __attribute__((aligned(16))) float sL[HD ? 128 : 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4, i16 = lane & 15;
  const int64_t bq = blockIdx.y;
  // block x -> (split, head group hg).  With several head groups and at
  // least 8 splits, x = 8 * (chunk * head_groups + hg) + xcd runs split
  // 8 * chunk + xcd (the grid rounded to whole chunks), so the head groups
  // of a split are dispatched to one XCD and share its L2; otherwise x =
  // split * head_groups + hg (with one head group, consecutive splits go to
  // consecutive XCDs)
  int64_t hg, split;
  if (a.head_groups > 1 && a.splits >= 8) {
    const int64_t xcd = blockIdx.x & 7, rest = blockIdx.x >> 3;
    hg = rest % a.head_groups;
    split = (rest / a.head_groups) * 8 + xcd;
  } else {
    split = blockIdx.x / a.head_groups;
    hg = blockIdx.x - split * a.head_groups;
  }
  if (split >= a.splits) return;
  const int64_t b = bq / a.n_q;
  const int64_t nkm = n_keys<MODE>(a, bq);
  const int64_t nk = nkm + n_win_keys(a, bq);
  const int64_t k0 = split * a.keys_per_split;
  const int64_t k1 = min(nk, k0 + a.keys_per_split);
  const int64_t hbase = hg * HPG + wave * 16;
  // HD: every wave computes S^T (heads past n_h use head n_h-1), since every
  // wave's P block feeds all of them
  const bool active = HD || hbase < a.n_h;
  const int64_t ntile = k1 > k0 ? (k1 - k0 + 31) / 32 : 0;
  // positions behind the key codes, read once: ring slot of window key j is
  // (mbase + j) mod cap (window mode), of tail key j >= nkm (wbase + j) mod win_ring
  int64_t mbase = 0, wbase = 0;
  if constexpr (MODE == kWindow) {
    int64_t t = a.t[bq];
    t = t < 0 ? 0 : (t > a.t_max ? a.t_max : t);
    mbase = t - nkm + 1;
  }
  if (a.win != nullptr) {
    int64_t t = a.win_t[bq];
    t = t < 0 ? 0 : (t > a.win_tmax ? a.win_tmax : t);
    wbase = t - (nk - nkm) + 1 - nkm;
  }
  const bf16_raw* zrow = g_zero_row;
  asm volatile("" : "+s"(zrow));  // keep the masked-key source in SGPRs

  if constexpr (MODE == kGather) {
    for (int64_t j = tid; j < k1 - k0; j += 64 * NW) sRow[j] = int32_t(key_code<kGather>(a, bq, k0 + j, k1, nkm));
    __syncthreads();
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)DLC_LDS(sK);
  auto issue = [&](int64_t tl) {
    const uint32_t buf = lds0 + uint32_t(tl & (NST - 1)) * kTileBytes;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int row = RPW * wave + r;
      const int64_t j = k0 + tl * 32 + row;
      int64_t code;
      if constexpr (MODE == kGather) {
        code = j < k1 ? sRow[j - k0] : -1;
      } else if (j >= k1) {
        code = -1;
      } else if (j < nkm) {
        code = MODE == kWindow ? (mbase + j) % a.cap : j;
      } else {
        code = -2 - (wbase + j) % a.win_ring;
      }
      code = __builtin_amdgcn_readfirstlane(int(code));
      const bf16_raw* src = key_ptr<bf16_raw>(a, b, code);
      if (src == nullptr) src = zrow;
      dma_row(src, uint32_t(lane) * 16u, buf + uint32_t(h16_row_off(row)));
    }
  };
  auto valid_mask = [&](int64_t tl) -> uint32_t {
    const int64_t j = tl * 32 + (lane & 31);
    bool v = k0 + j < k1;
    if constexpr (MODE == kGather) v = v && sRow[j] != -1;
    return uint32_t(__ballot(v) & 0xffffffffu);
  };
  // tile 0 and Q first, waited for together; then tiles 1 and 2, so that the
  // first tile's compute starts as soon as its own rows are in (waiting for
  // three tiles of every workgroup at once put the whole first burst of the
  // call in front of it); tile i+3 is issued once every wave is past tile
  // i-1 (the barrier of step i)
  if (ntile > 0) issue(0);
  // Q^T operand: lane holds head hbase + r16, dims 32*ks + 8*g .. +7; heads
  // past n_h read head n_h-1 (their columns and outputs are never used).
  // Loaded straight into that layout, every instruction touches 64 bytes of
  // 16 rows, which the memory pipeline serves slowly; so the first QW waves
  // move their 16 rows whole (1 KB a direct-to-LDS instruction) into ring
  // buffers 1.. (free until tiles 1 and 2 are issued below), rows 1040 bytes
  // apart so that a ds_read_b128 pass over 16 rows hits 16 distinct bank
  // groups, and read the operand from there; the other waves (whose rows
  // would not fit) load it directly.
  constexpr int QROW = 1040, QW = (NST - 1) * kTileBytes / (16 * QROW) < NW ? (NST - 1) * kTileBytes / (16 * QROW) : NW;
  static_assert(QW >= 1, "Q staging");
  const bool q_lds = wave < QW;
  const uint32_t qst = lds0 + uint32_t(kTileBytes) + uint32_t(wave * 16 * QROW);
  bf16x8 qf[KS];
  if (q_lds) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t h = min(hbase + r, a.n_h - 1);
      dma_row(static_cast<const bf16_raw*>(a.q) + (bq * a.n_h + h) * CD, uint32_t(lane) * 16u, qst + uint32_t(r * QROW));
    }
  } else {
    const int64_t h = min(hbase + r16, a.n_h - 1);
    const bf16_raw* qp = static_cast<const bf16_raw*>(a.q) + (bq * a.n_h + h) * CD + g * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + ks * 32));
    // wait for Q here, so that no vector-memory wait for it lands inside the
    // tile loop (it would drain the tile loads in flight)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
  }
  wait_vm<0>();  // tile 0 and Q
  lds_barrier();  // every wave's tile-0 rows and staged Q rows
  if (q_lds) {
    const unsigned char* qs = sK + kTileBytes + wave * 16 * QROW + r16 * QROW + 16 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qs + 64 * ks);
  }
  lds_barrier();  // the staged rows are read before tiles 1 and 2 overwrite them
  if (ntile > 1) issue(1);
  if (ntile > 2) issue(2);

  f32x4 o[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;  // for head hbase + r16

  // per-lane LDS offsets: Q.K^T A operand (row r16 of each half, chunk 4*ks + g)
  const uint32_t qk_off0 = uint32_t(h16_row_off(r16) + 16 * g);
  const uint32_t qk_off1 = uint32_t(h16_row_off(16 + r16) + 16 * g);
  // P.V B operand: keys 4*g + i16/4 (+16 for the second half), dims 16*nt + 4*(i16%4)
  const uint32_t pv_off0 = uint32_t(h16_row_off(4 * g + (i16 >> 2)) + 8 * (i16 & 3));
  const uint32_t pv_off1 = uint32_t(h16_row_off(16 + 4 * g + (i16 >> 2)) + 8 * (i16 & 3));
  auto tile_ptr = [&](int64_t tl) { return sK + (tl & (NST - 1)) * kTileBytes; };
  auto kfrag = [&](const unsigned char* tile, uint32_t off, int ks) {
    return *reinterpret_cast<const bf16x8*>(tile + off + 64 * ks);
  };
  auto vfrag = [&](const unsigned char* tile, int nt) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)DLC_LDS(tile + pv_off0 + 32 * nt));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)DLC_LDS(tile + pv_off1 + 32 * nt));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // S^T of one tile alone (the first)
  f32x4 s0, s1;
  auto qk_only = [&](const unsigned char* tq) {
    s0 = f32x4{0.f, 0.f, 0.f, 0.f};
    s1 = s0;
    bf16x8 ka0 = kfrag(tq, qk_off0, 0), ka1 = kfrag(tq, qk_off1, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 kb0 = ka0, kb1 = ka1;
      if (ks + 1 < KS) {
        kb0 = kfrag(tq, qk_off0, ks + 1);
        kb1 = kfrag(tq, qk_off1, ks + 1);
      }
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1, qf[ks], s1, 0, 0, 0);
      ka0 = kb0;
      ka1 = kb1;
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // O += P . V of tile tp and, interleaved, S^T of tile tq: four MFMAs per
  // step; each operand register is refilled for the next step right after
  // the MFMA that reads it is issued
  bf16x8 pa;
  // HD: O[16 heads of block hb][dims 64*wave + 16*n] is o[4*hb + n]; the
  // tile's P blocks come from buffer pb; first the rescale that any wave's
  // softmax published for this tile
  auto hd_rescale = [&](int pb) {
    const int4 m0 = *reinterpret_cast<const int4*>(&sMove[pb][0]);
    const int4 m1 = *reinterpret_cast<const int4*>(&sMove[pb][4]);
    if ((m0.x | m0.y | m0.z | m0.w | m1.x | m1.y | m1.z | m1.w) != 0) {
#pragma unroll
      for (int hb = 0; hb < 8; ++hb) {
        const float4 al = *reinterpret_cast<const float4*>(&sAlpha[pb][16 * hb + 4 * g]);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          o[4 * hb + n][0] *= al.x;
          o[4 * hb + n][1] *= al.y;
          o[4 * hb + n][2] *= al.z;
          o[4 * hb + n][3] *= al.w;
        }
      }
    }
  };
  auto hd_pv_qk = [&](const unsigned char* tp, const unsigned char* tq, int pb) {
    hd_rescale(pb);
    s0 = f32x4{0.f, 0.f, 0.f, 0.f};
    s1 = s0;
    bf16x8 vb[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) vb[n] = vfrag(tp, 4 * wave + n);
    bf16x8 ka0 = kfrag(tq, qk_off0, 0), ka1 = kfrag(tq, qk_off1, 0);
    bf16x8 pc;
    // step pair (2hb, 2hb+1) adds head block hb's four output tiles; P block
    // hb is read two S^T MFMAs ahead of its first use (registers are too
    // tight for a second P buffer), so even steps issue both S^T MFMAs first
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int hb = ks >> 1;
      if ((ks & 1) == 0) {
        pc = sP[pb][hb][lane];
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0, qf[ks], s0, 0, 0, 0);
        if (ks + 1 < KS) ka0 = kfrag(tq, qk_off0, ks + 1);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1, qf[ks], s1, 0, 0, 0);
        if (ks + 1 < KS) ka1 = kfrag(tq, qk_off1, ks + 1);
        o[4 * hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pc, vb[0], o[4 * hb], 0, 0, 0);
        o[4 * hb + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pc, vb[1], o[4 * hb + 1], 0, 0, 0);
      } else {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0, qf[ks], s0, 0, 0, 0);
        if (ks + 1 < KS) ka0 = kfrag(tq, qk_off0, ks + 1);
        o[4 * hb + 2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pc, vb[2], o[4 * hb + 2], 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1, qf[ks], s1, 0, 0, 0);
        if (ks + 1 < KS) ka1 = kfrag(tq, qk_off1, ks + 1);
        o[4 * hb + 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pc, vb[3], o[4 * hb + 3], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto hd_pv_only = [&](const unsigned char* tp, int pb) {
    hd_rescale(pb);
    bf16x8 vb[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) vb[n] = vfrag(tp, 4 * wave + n);
    bf16x8 pc = sP[pb][0][lane];
#pragma unroll
    for (int hb = 0; hb < 8; ++hb) {
      bf16x8 pn = pc;
      if (hb + 1 < 8) pn = sP[pb][hb + 1][lane];
#pragma unroll
      for (int n = 0; n < 4; ++n)
        o[4 * hb + n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pc, vb[n], o[4 * hb + n], 0, 0, 0);
      pc = pn;
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto pv_qk = [&](const unsigned char* tp, const unsigned char* tq) {
    s0 = f32x4{0.f, 0.f, 0.f, 0.f};
    s1 = s0;
    bf16x8 ka0 = kfrag(tq, qk_off0, 0), ka1 = kfrag(tq, qk_off1, 0);
    bf16x8 va0 = vfrag(tp, 0), va1 = vfrag(tp, 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0, qf[ks], s0, 0, 0, 0);
      if (ks + 1 < KS) ka0 = kfrag(tq, qk_off0, ks + 1);
      o[2 * ks] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, va0, o[2 * ks], 0, 0, 0);
      if (ks + 1 < KS) va0 = vfrag(tp, 2 * ks + 2);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1, qf[ks], s1, 0, 0, 0);
      if (ks + 1 < KS) ka1 = kfrag(tq, qk_off1, ks + 1);
      o[2 * ks + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, va1, o[2 * ks + 1], 0, 0, 0);
      if (ks + 1 < KS) va1 = vfrag(tp, 2 * ks + 3);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto pv_only = [&](const unsigned char* tp) {
    bf16x8 va0 = vfrag(tp, 0), va1 = vfrag(tp, 1);
#pragma unroll
    for (int n2 = 0; n2 < NT; n2 += 2) {
      bf16x8 vb0 = va0, vb1 = va1;
      if (n2 + 2 < NT) {
        vb0 = vfrag(tp, n2 + 2);
        vb1 = vfrag(tp, n2 + 3);
      }
      o[n2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, va0, o[n2], 0, 0, 0);
      o[n2 + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, va1, o[n2 + 1], 0, 0, 0);
      va0 = vb0;
      va1 = vb1;
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // softmax of S^T (keys masked by vmask) into pa, rescaling O if the running
  // max grew; lane holds head r16, keys 4g+e (s0) and 16+4g+e (s1).  HD: the
  // factors, the flag and P go to LDS buffer pb instead
  auto softmax = [&](uint32_t vmask, int pb) {
    float x[8];
    const uint32_t vm = vmask >> (4 * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = ((vm >> e) & 1u) ? s0[e] * a.scale_log2 : -INFINITY;
      x[4 + e] = ((vm >> (16 + e)) & 1u) ? s1[e] * a.scale_log2 : -INFINITY;
    }
    float tmax = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, x[e]);
    tmax = rows4_max(tmax);
    // lazy running max: O is rescaled only when the max grows by more than 2^8
    const bool move = tmax > mrun + 8.f;
    const bool any_move = __any(move);
    if constexpr (HD) {
      float alpha = 1.f;
      if (any_move) {
        const float mnew = move ? tmax : mrun;
        alpha = mrun == -INFINITY ? 0.f : exp2f(mrun - mnew);
        lrun *= alpha;
        mrun = mnew;
      }
      if (g == 0) sAlpha[pb][16 * wave + r16] = alpha;
      if (lane == 0) sMove[pb][wave] = any_move ? 1 : 0;
    } else if (any_move) {
      const float mnew = move ? tmax : mrun;
      const float alpha = mrun == -INFINITY ? 0.f : exp2f(mrun - mnew);
      lrun *= alpha;
      mrun = mnew;
      // O rows are heads 4*g + e
      float al[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) al[e] = __shfl(alpha, 4 * g + e);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[nt][e] *= al[e];
    }
    const float mr = mrun == -INFINITY ? 0.f : mrun;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __builtin_amdgcn_exp2f(x[e] - mr);
      psum += p;
      pa[e] = (__bf16)p;
    }
    lrun += rows4_sum(psum);
    if constexpr (HD) sP[pb][wave][lane] = pa;
  };

  if (ntile > 0) {
    const uint32_t vmask = valid_mask(0);  // tile 0 is in LDS for every wave (the barriers above)
    if (active) {
      qk_only(tile_ptr(0));
      softmax(vmask, 0);
    }
  }
  for (int64_t it = 0; it + 1 < ntile; ++it) {
    if (it + 2 < ntile) wait_vm<RPW>(); else wait_vm<0>();
    lds_barrier();
    if (it + 3 < ntile) issue(it + 3);
    const uint32_t vmask = valid_mask(it + 1);
    if constexpr (HD) {
      hd_pv_qk(tile_ptr(it), tile_ptr(it + 1), int(it & 1));
      softmax(vmask, int((it + 1) & 1));
    } else if (active) {
      pv_qk(tile_ptr(it), tile_ptr(it + 1));
      softmax(vmask, 0);
    }
  }
  if constexpr (HD) {
    if (ntile > 0) {
      lds_barrier();  // the last tile's P blocks, from every wave
      hd_pv_only(tile_ptr(ntile - 1), int((ntile - 1) & 1));
    }
  } else if (ntile > 0 && active) {
    pv_only(tile_ptr(ntile - 1));
  }

  const int64_t slot0 = (bq * a.splits + split) * a.n_h;
  if constexpr (HD) {
    // every head's sum, from the wave that owns its softmax, to the owners
    // of the O slices; o[4*hb + n][e] is head 16*hb + 4*g + e of the
    // workgroup, dim 64*wave + 16*n + i16
    if (g == 0) sL[16 * wave + r16] = lrun;
    if (g == 0 && a.lse && hbase + r16 < a.n_h)
      a.lse[slot0 + hbase + r16] = lrun > 0.f ? (mrun + log2f(lrun)) * kLn2 : -INFINITY;
    lds_barrier();
    const int64_t h0 = hg * HPG;
    if (a.ob != nullptr) {
      // fragment order (as below): head block hb's stores j = 2*wave and
      // 2*wave+1 hold dims 16nt + i16 of nt = 2j, 2j+1
      const int64_t nh16 = (a.n_h + 15) & ~int64_t(15);
      bf16_raw* dst0 = a.ob + ((bq * a.splits + split) * nh16 + h0) * CD + 8 * lane;
#pragma unroll
      for (int hb = 0; hb < 8; ++hb) {
        if (h0 + 16 * hb >= a.n_h) break;
        const float4 l4 = *reinterpret_cast<const float4*>(&sL[16 * hb + 4 * g]);
        const float inv[4] = {l4.x > 0.f ? 1.f / l4.x : 0.f, l4.y > 0.f ? 1.f / l4.y : 0.f,
                              l4.z > 0.f ? 1.f / l4.z : 0.f, l4.w > 0.f ? 1.f / l4.w : 0.f};
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = (__bf16)(o[4 * hb + 2 * jj][e] * inv[e]);
            v[4 + e] = (__bf16)(o[4 * hb + 2 * jj + 1][e] * inv[e]);
          }
          store_partial(dst0 + int64_t(16 * hb) * CD + 512 * (2 * wave + jj), v);
        }
      }
      return;
    }
#pragma unroll
    for (int hb = 0; hb < 8; ++hb) {
      const float4 l4 = *reinterpret_cast<const float4*>(&sL[16 * hb + 4 * g]);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t h = h0 + 16 * hb + 4 * g + e;
        if (h < a.n_h) {
          const float inv = lv[e] > 0.f ? 1.f / lv[e] : 0.f;
          float* op = a.o + (slot0 + h) * CD + 64 * wave + i16;
#pragma unroll
          for (int n = 0; n < 4; ++n) op[16 * n] = o[4 * hb + n][e] * inv;
        }
      }
    }
    return;
  }
  // normalise and write: o[nt][e] is head 4*g + e, dim 16*nt + i16
  float inv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float l = __shfl(lrun, 4 * g + e);
    inv[e] = l > 0.f ? 1.f / l : 0.f;
  }
  if (active && g == 0 && a.lse && hbase + r16 < a.n_h)
    a.lse[slot0 + hbase + r16] = lrun > 0.f ? (mrun + log2f(lrun)) * kLn2 : -INFINITY;
  if (a.ob != nullptr) {
    // bf16 partials in fragment order, straight from the accumulators: the
    // wave's block of 16 heads x 512 dims is 16 stores of 16 bytes per lane,
    // store j of lane 16g + i16 holding heads 4g .. 4g+3 at dims 16nt + i16
    // of nt = 2j (elements 0..3) and 2j+1 (4..7); blocks of 16 heads follow
    // each other, n_h rounded up to 16 (combine_frag_kernel reads them)
    if (!active) return;
    const int64_t nh16 = (a.n_h + 15) & ~int64_t(15);
    bf16_raw* dst = a.ob + ((bq * a.splits + split) * nh16 + hbase) * CD + 8 * lane;
#pragma unroll
    for (int j = 0; j < NT / 2; ++j) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = (__bf16)(o[2 * j][e] * inv[e]);
        v[4 + e] = (__bf16)(o[2 * j + 1][e] * inv[e]);
      }
      store_partial(dst + 512 * j, v);
    }
    return;
  }
  if (!active) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t h = hbase + 4 * g + e;
    if (h < a.n_h) {
      float* op = a.o + (slot0 + h) * CD + i16;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) op[16 * nt] = o[nt][e] * inv[e];
    }
  }
}

// ------------------------------------------------------------------ combine

// One block per (query, head).  The split weights e^{lse_j - lse} are formed
// once in LDS; each thread then owns 4 consecutive dims (c % 4 == 0) or one
// dim and sums the splits with independent loads.  An optional extra part
// (o_in, lse_in), laid out like the final output, joins as one more split:
// the attention over the union of its keys and these (the window branch
// joined to a compressed branch).  out may be o_in: every element is read and
// written by the same thread, and lse_in is read before lse is written.
constexpr int kMaxSplits = 256;

__global__ void __launch_bounds__(128) combine_kernel(const float* op, const float* lp, int64_t splits,
                                                      int64_t n_h, int64_t c, float* out, float* lse,
                                                      const float* o_in, const float* lse_in) {
  __shared__ float wsh[kMaxSplits + 1];
  __shared__ float red[2];
  const int64_t bh = blockIdx.x;  // bq * n_h + h
  const int64_t bq = bh / n_h, h = bh - bq * n_h;
  const int tid = threadIdx.x;
  const int parts = int(splits) + (o_in ? 1 : 0);
  for (int j = tid; j < splits; j += blockDim.x) wsh[j] = lp[(bq * splits + j) * n_h + h];
  if (o_in && tid == 0) wsh[splits] = lse_in[bh];
  __syncthreads();
  if (tid < 64) {
    float M = -INFINITY;
    for (int j = tid; j < parts; j += 64) M = fmaxf(M, wsh[j]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float L = 0.f;
    for (int j = tid; j < parts; j += 64) L += (M == -INFINITY) ? 0.f : __expf(wsh[j] - M);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
    if (tid == 0) { red[0] = M; red[1] = L; }
  }
  __syncthreads();
  const float M = red[0], L = red[1];
  for (int j = tid; j < parts; j += blockDim.x) wsh[j] = (M == -INFINITY) ? 0.f : __expf(wsh[j] - M) / L;
  __syncthreads();
  const float* base = op + (bq * splits * n_h + h) * c;
  const int64_t sstride = n_h * c;
  const float w_in = o_in ? wsh[splits] : 0.f;
  if ((c & 3) == 0) {
    for (int64_t d = 4 * tid; d < c; d += 4 * blockDim.x) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
      for (int64_t j = 0; j < splits; ++j) {
        const float wj = wsh[j];
        const float4 v = *reinterpret_cast<const float4*>(base + j * sstride + d);
        acc.x = fmaf(wj, v.x, acc.x); acc.y = fmaf(wj, v.y, acc.y);
        acc.z = fmaf(wj, v.z, acc.z); acc.w = fmaf(wj, v.w, acc.w);
      }
      if (o_in) {
        const float4 v = *reinterpret_cast<const float4*>(o_in + bh * c + d);
        acc.x = fmaf(w_in, v.x, acc.x); acc.y = fmaf(w_in, v.y, acc.y);
        acc.z = fmaf(w_in, v.z, acc.z); acc.w = fmaf(w_in, v.w, acc.w);
      }
      *reinterpret_cast<float4*>(out + bh * c + d) = acc;
    }
  } else {
    for (int64_t d = tid; d < c; d += blockDim.x) {
      float acc = 0.f;
#pragma unroll 8
      for (int64_t j = 0; j < splits; ++j) acc = fmaf(wsh[j], base[j * sstride + d], acc);
      if (o_in) acc = fmaf(w_in, o_in[bh * c + d], acc);
      out[bh * c + d] = acc;
    }
  }
  if (tid == 0 && lse) lse[bh] = M == -INFINITY ? -INFINITY : M + __logf(L);
}

// The bf16 partials of attend512_kernel, in its fragment order.  A block
// covers one query, one block of 16 heads and JB of the 16 fragment stores j
// (blockIdx.y picks which), with W waves per j; blockDim.x = 64 * JB * W.
// Lane l of the waves of store j reads, for its share of the splits (every
// W-th), the 16 bytes lane l stored as its store j - heads 4g .. 4g+3 (g =
// l/16) at dims 16nt + l%16 of nt = 2j, 2j+1 - so a wave reads 1 KB of
// consecutive bytes per split; the W sums meet in LDS.  The split weights of
// the 16 heads are formed in LDS first.  The extra part (o_in, lse_in) joins
// as in combine_kernel; the host then launches JB = 16 (one block per query
// and head block), so that lse_in is read before lse is written in place.
template <int NT, int U>  // block size; partials a wave has in flight
__global__ void __launch_bounds__(NT) combine_frag_kernel(const bf16_raw* op, const float* lp, int64_t splits,
                                                          int64_t n_h, int W, float* out, float* lse,
                                                          const float* o_in, const float* lse_in) {
  constexpr int CD = 512;
  __shared__ __attribute__((aligned(16))) float wsh[(kMaxSplits + 1) * 16];  // [part][head of the block]
  __shared__ float mh[16], lh[16];
  __shared__ float4 red[8 * 2 * 64];  // wave sums [wave][2][lane] (W > 1 only with JB = 1, W <= 8)
  const int64_t nb = (n_h + 15) / 16;
  const int64_t bq = blockIdx.x / nb, hb = (int64_t(blockIdx.x) - bq * nb) * 16;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63, wid = tid >> 6, wv = wid % W;
  const int j = int(blockIdx.y) * (nthr / (64 * W)) + wid / W;
  const int parts = int(splits) + (o_in ? 1 : 0);
  const int g = lane >> 4, i16 = lane & 15;
  const int64_t sstride = nb * 16 * CD;
  const bf16_raw* base = op + (bq * splits * nb * 16 + hb) * CD + 512 * j + 8 * lane;
  // lse of every part for the block's heads (heads past n_h: -inf), four
  // heads a thread; the first round is loaded before the partials of the
  // first batch, which do not depend on the weights and stay in flight while
  // the weights are formed
  // (every load below is unconditional, from a clamped address, with the
  // result dropped when out of range: loads under branches make the
  // compiler wait for them early)
  auto lse_load = [&](int i, float* v) {
    const int p = min(i >> 2, parts - 1), e0 = 4 * (i & 3);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t h = hb + e0 + e, hc = h < n_h ? h : n_h - 1;
      const float* src = p < splits ? lp + (bq * splits + p) * n_h + hc : lse_in + bq * n_h + hc;
      const float x = *src;
      v[e] = h < n_h ? x : -INFINITY;
    }
  };
  float lv[4];
  lse_load(tid, lv);
  asm volatile("" ::: "memory");  // these loads first, so that their wait leaves the partials in flight
  uint4 u[U];
  const int64_t wstep = int64_t(W) * sstride;
  {
    const bf16_raw* pp = base + wv * sstride;
    const bf16_raw* plast = base + (splits - 1) * sstride;
#pragma unroll
    for (int i = 0; i < U; ++i, pp += wstep) u[i] = *reinterpret_cast<const uint4*>(wv + i * W < splits ? pp : plast);
  }
  if (tid < parts * 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) wsh[(tid >> 2) * 16 + 4 * (tid & 3) + e] = lv[e];
  }
  for (int i = tid + nthr; i < parts * 4; i += nthr) {
    float v[4];
    lse_load(i, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) wsh[(i >> 2) * 16 + 4 * (i & 3) + e] = v[e];
  }
  __syncthreads();
  {  // per head: max, sum and weights over the parts, nthr/16 threads a head
     // (consecutive lanes of one wave)
    const int tph = nthr >> 4, hh = tid / tph, q = tid % tph;
    float M = -INFINITY;
    for (int p = q; p < parts; p += tph) M = fmaxf(M, wsh[p * 16 + hh]);
    for (int off = 1; off < tph; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
    float L = 0.f;
    if (M != -INFINITY)
      for (int p = q; p < parts; p += tph) L += __expf(wsh[p * 16 + hh] - M);
    for (int off = 1; off < tph; off <<= 1) L += __shfl_xor(L, off);
    const float rl = M == -INFINITY ? 0.f : 1.f / L;
    for (int p = q; p < parts; p += tph) wsh[p * 16 + hh] = M == -INFINITY ? 0.f : __expf(wsh[p * 16 + hh] - M) * rl;
    if (q == 0) {
      mh[hh] = M;
      lh[hh] = L;
    }
  }
  __syncthreads();
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  auto accumulate = [&](const uint4& x, int64_t p) {
    const float4 w = *reinterpret_cast<const float4*>(&wsh[p * 16 + 4 * g]);
    acc[0] = fmaf(w.x, __uint_as_float(x.x << 16), acc[0]);
    acc[1] = fmaf(w.y, __uint_as_float(x.x & 0xffff0000u), acc[1]);
    acc[2] = fmaf(w.z, __uint_as_float(x.y << 16), acc[2]);
    acc[3] = fmaf(w.w, __uint_as_float(x.y & 0xffff0000u), acc[3]);
    acc[4] = fmaf(w.x, __uint_as_float(x.z << 16), acc[4]);
    acc[5] = fmaf(w.y, __uint_as_float(x.z & 0xffff0000u), acc[5]);
    acc[6] = fmaf(w.z, __uint_as_float(x.w << 16), acc[6]);
    acc[7] = fmaf(w.w, __uint_as_float(x.w & 0xffff0000u), acc[7]);
  };
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int64_t p = wv + int64_t(i) * W;
    if (p < splits) accumulate(u[i], p);
  }
  // further batches (more than U * W splits), U loads issued together
  for (int64_t p0 = wv + int64_t(U) * W; p0 < splits; p0 += int64_t(U) * W) {
    const bf16_raw* pp = base + p0 * sstride;
    const bf16_raw* plast = base + (splits - 1) * sstride;
#pragma unroll
    for (int i = 0; i < U; ++i, pp += wstep) u[i] = *reinterpret_cast<const uint4*>(p0 + i * W < splits ? pp : plast);
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int64_t p = p0 + int64_t(i) * W;
      if (p < splits) accumulate(u[i], p);
    }
  }
  if (W > 1) {  // the other waves of store j hand their sums to its first wave
    if (wv != 0) {
      red[(wid * 2) * 64 + lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      red[(wid * 2 + 1) * 64 + lane] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
    __syncthreads();
    if (wv != 0) return;
    for (int v = 1; v < W; ++v) {
      const float4 a0 = red[((wid + v) * 2) * 64 + lane], a1 = red[((wid + v) * 2 + 1) * 64 + lane];
      acc[0] += a0.x; acc[1] += a0.y; acc[2] += a0.z; acc[3] += a0.w;
      acc[4] += a1.x; acc[5] += a1.y; acc[6] += a1.z; acc[7] += a1.w;
    }
  }
  // element k: head hb + 4g + k%4, dim 16 (2j + k/4) + i16
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int64_t h = hb + 4 * g + (k & 3);
    if (h < n_h) {
      const int64_t at = (bq * n_h + h) * CD + 16 * (2 * j + (k >> 2)) + i16;
      float v = acc[k];
      if (o_in) v = fmaf(wsh[int(splits) * 16 + 4 * g + (k & 3)], o_in[at], v);
      out[at] = v;
    }
  }
  if (lse && j == 0 && lane < 16 && hb + lane < n_h)
    lse[bq * n_h + hb + lane] = mh[lane] == -INFINITY ? -INFINITY : mh[lane] + __logf(lh[lane]);
}

// ------------------------------------------------------------------ sink logits
//
// One logit z_h per head joins a finished attention's softmax as an extra
// key with a zero value: o' = o * e^lse / (e^lse + e^z), lse' = log(e^lse +
// e^z).  One block per (row, head); the factor is formed once, then the c
// dims are scaled in place (float4 when c % 4 == 0).
__global__ void __launch_bounds__(128) sink_kernel(float* o, float* lse, const float* z, int64_t n_h, int64_t c) {
  const int64_t rh = blockIdx.x;  // row * n_h + head
  const float l = lse[rh], zh = z[rh % n_h];
  const float m = fmaxf(l, zh);
  const float el = l == -INFINITY ? 0.f : expf(l - m), ez = expf(zh - m);
  const float f = el / (el + ez);
  float* op = o + rh * c;
  if ((c & 3) == 0) {
    for (int64_t d = threadIdx.x; d < c / 4; d += blockDim.x) {
      float4 v = reinterpret_cast<float4*>(op)[d];
      v.x *= f; v.y *= f; v.z *= f; v.w *= f;
      reinterpret_cast<float4*>(op)[d] = v;
    }
  } else {
    for (int64_t d = threadIdx.x; d < c; d += blockDim.x) op[d] *= f;
  }
  __syncthreads();
  if (threadIdx.x == 0) lse[rh] = m + logf(el + ez);
}

// ------------------------------------------------------------------ host

bool mfma_ok(int dtype, int64_t c) { return dtype == DLC_BF16 && (c == 128 || c == 256 || c == 512); }

struct Plan {
  bool mfma, bf16_parts;  // bf16_parts: the partial outputs are stored in bf16
  int64_t heads;          // heads per workgroup (MFMA paths)
  int64_t splits, kps, head_groups;
  size_t o_off, l_off, total;
};

// gather: the keys of a split are listed in LDS (kGather), which bounds a split's length
Plan plan(int dtype, int64_t BQ, int64_t n_h, int64_t c, int64_t nkeys, bool merge = false, bool gather = true) {
  Plan p{};
  p.mfma = mfma_ok(dtype, c);
  const int64_t nk1 = nkeys > 0 ? nkeys : 1;
  auto split_count = [&](int64_t per_split) {
    int64_t s = ceil_div(kTargetWorkgroups, per_split);
    const int64_t smax = ceil_div(nk1, kMinKeysPerSplit);
    s = s < smax ? s : smax;
    if (gather) {  // a split's row list fits in LDS
      const int64_t smin = ceil_div(nk1, c == 512 ? kMaxGatherKeys : 4096);
      s = s < smin ? smin : s;
    }
    return s < 1 ? 1 : (s > kMaxSplits ? kMaxSplits : s);
  };
  // c = 512: 128 heads (8 waves) per workgroup, or 64 (4 waves) when the
  // minimum split length leaves the 128-head grid at or under half the target
  // and the smaller groups add workgroups
  p.heads = p.mfma ? 128 : 1;
  p.head_groups = p.mfma ? ceil_div(n_h, p.heads) : n_h;
  int64_t s = split_count(p.mfma ? BQ * p.head_groups : BQ * n_h);
  if (p.mfma && c == 512 && n_h > 64 && 2 * BQ * p.head_groups * s <= kTargetWorkgroups) {
    const int64_t hg64 = ceil_div(n_h, 64), s64 = split_count(BQ * hg64);
    if (hg64 * s64 > p.head_groups * s) {
      p.heads = 64;
      p.head_groups = hg64;
      s = s64;
    }
  }
  p.splits = s;
  p.kps = ceil_div(nkeys > 0 ? nkeys : 1, s);
  if (p.mfma) p.kps = ceil_div(p.kps, 32) * 32;
  p.o_off = 0;
  size_t off = 0;
  p.bf16_parts = p.mfma && c == 512 && kBf16Partials;
  if (s > 1 || merge) {  // partials, combined afterwards
    // bf16 partials: blocks of 16 heads (n_h rounded up to 16)
    const int64_t nh_parts = p.bf16_parts ? (n_h + 15) / 16 * 16 : n_h;
    off = align_up(size_t(BQ) * s * nh_parts * c * (p.bf16_parts ? 2 : 4), 256);
    p.l_off = off;
    off = align_up(off + size_t(BQ) * s * n_h * 4, 256);
  } else {
    p.l_off = 0;
  }
  p.total = off;
  return p;
}

size_t ws_bound(int64_t BQ, int64_t n_h, int64_t c, int64_t nkeys, bool merge = false) {
  const Plan a = plan(DLC_BF16, BQ, n_h, c, nkeys, merge), b = plan(DLC_F32, BQ, n_h, c, nkeys, merge);
  return a.total > b.total ? a.total : b.total;
}

template <int MODE>
int run_attend(const char* name, int dtype, AttArgs a, int64_t BQ, int64_t nkeys, float* out, float* lse,
               void* ws, size_t ws_bytes, hipStream_t s, const float* o_in = nullptr,
               const float* lse_in = nullptr) {
  const bool merge = o_in != nullptr;
  const Plan p = plan(dtype, BQ, a.n_h, a.c, nkeys, merge, MODE == kGather);
  DLC_REQUIRE(p.total == 0 || (ws != nullptr && ws_bytes >= p.total), DLC_E_WORKSPACE,
              "%s: workspace of %zu bytes needed, %zu given", name, p.total, ws_bytes);
  DLC_REQUIRE(ws == nullptr || aligned(ws, 256), DLC_E_WORKSPACE, "%s: workspace must be 256-byte aligned", name);
  a.splits = p.splits;
  a.keys_per_split = p.kps;
  a.head_groups = p.head_groups;
  const bool partials = p.splits > 1 || merge;
  a.ob = nullptr;
  if (partials) {
    a.o = reinterpret_cast<float*>(static_cast<char*>(ws) + p.o_off);
    if (p.bf16_parts) a.ob = reinterpret_cast<bf16_raw*>(static_cast<char*>(ws) + p.o_off);
    a.lse = reinterpret_cast<float*>(static_cast<char*>(ws) + p.l_off);
  } else {
    a.o = out;
    a.lse = lse;
  }
  DLC_REQUIRE(BQ <= 65535 && p.splits * p.head_groups < (int64_t(1) << 31), DLC_E_UNSUPPORTED,
              "%s: grid too large", name);
  // the c = 512 kernel lists a split's gathered rows in LDS (kMaxGatherKeys)
  DLC_REQUIRE(!(MODE == kGather && p.mfma && a.c == 512) || p.kps <= kMaxGatherKeys, DLC_E_UNSUPPORTED,
              "%s: %lld gathered keys per query exceed %lld (%d splits of %d)", name, (long long)nkeys,
              (long long)kMaxSplits * kMaxGatherKeys, kMaxSplits, kMaxGatherKeys);
  StageTimer timer(MODE == kGather ? DLC_STAGE_CSA_ATTEND : MODE == kDense ? DLC_STAGE_HCA_ATTEND
                                                                             : DLC_STAGE_WINDOW_ATTEND, s);
  if (p.mfma) {
    dim3 grid{(unsigned)(p.splits * p.head_groups), (unsigned)BQ, 1u};
    if (a.c == 128) hipLaunchKernelGGL((attend_mfma_kernel<128, MODE>), grid, dim3(512), 0, s, a);
    if (a.c == 256) hipLaunchKernelGGL((attend_mfma_kernel<256, MODE>), grid, dim3(512), 0, s, a);
    if (a.c == 512) {
      // several head groups and >= 8 splits: whole chunks of 8 splits for
      // every head group (the kernel's block mapping)
      const int64_t gx = p.head_groups > 1 && p.splits >= 8 ? ceil_div(p.splits, 8) * 8 * p.head_groups
                                                             : p.splits * p.head_groups;
      const dim3 grid8{(unsigned)gx, (unsigned)BQ, 1u};
      if (p.heads == 64)
        hipLaunchKernelGGL((attend512_kernel<MODE, 4>), grid8, dim3(256), 0, s, a);
      else if (MODE == kDense && kHeadsDims && p.kps >= kHdMinKeys)
        hipLaunchKernelGGL((attend512_kernel<MODE, 8, MODE == kDense>), grid8, dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((attend512_kernel<MODE, 8>), grid8, dim3(512), 0, s, a);
    }
  } else {
    DLC_REQUIRE(a.n_h <= 65535, DLC_E_UNSUPPORTED, "%s: n_h > 65535 on the VALU path", name);
    dim3 grid{(unsigned)p.splits, (unsigned)a.n_h, (unsigned)BQ};
    if (dtype == DLC_BF16)
      hipLaunchKernelGGL((attend_valu_kernel<bf16_raw, MODE, 16>), grid, dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((attend_valu_kernel<float, MODE, 16>), grid, dim3(64), 0, s, a);
  }
  int rc = check_launch(name);
  if (rc || !partials) return rc;
  if (p.bf16_parts) {
    // merging: one block per query and head block (lse may be lse_in);
    // else four waves per fragment store, sharing the splits
    const unsigned nb = (unsigned)(BQ * ((a.n_h + 15) / 16));
    if (merge)
      hipLaunchKernelGGL((combine_frag_kernel<1024, 4>), dim3(nb, 1u, 1u), dim3(1024), 0, s, a.ob, a.lse, p.splits,
                         a.n_h, 1, out, lse, o_in, lse_in);
    else
      // each of the four waves of a store loads its share of the splits at once:
      // as many loads in flight as it has splits, up to 16 (fewer registers
      // for short split lists, so more blocks resident)
      if (p.splits <= 16)
        hipLaunchKernelGGL((combine_frag_kernel<256, 4>), dim3(nb, 16u, 1u), dim3(256), 0, s, a.ob, a.lse, p.splits,
                           a.n_h, 4, out, lse, o_in, lse_in);
      else if (p.splits <= 32)
        hipLaunchKernelGGL((combine_frag_kernel<256, 8>), dim3(nb, 16u, 1u), dim3(256), 0, s, a.ob, a.lse, p.splits,
                           a.n_h, 4, out, lse, o_in, lse_in);
      else if (kCombine8)
        hipLaunchKernelGGL((combine_frag_kernel<512, 8>), dim3(nb, 16u, 1u), dim3(512), 0, s, a.ob, a.lse, p.splits,
                           a.n_h, 8, out, lse, o_in, lse_in);
      else
        hipLaunchKernelGGL((combine_frag_kernel<256, 16>), dim3(nb, 16u, 1u), dim3(256), 0, s, a.ob, a.lse, p.splits,
                           a.n_h, 4, out, lse, o_in, lse_in);
  } else {
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(BQ * a.n_h)), dim3(128), 0, s, a.o, a.lse, p.splits, a.n_h,
                       a.c, out, lse, o_in, lse_in);
  }
  return check_launch(name);
}

int common_checks(const char* name, int dtype, int64_t B, int64_t n_q, int64_t n_h, int64_t c, const void* q,
                  const void* kv, int64_t cap, const float* out) {
  DLC_REQUIRE(dtype == DLC_F32 || dtype == DLC_BF16, DLC_E_DTYPE, "%s: unsupported dtype %d", name, dtype);
  DLC_REQUIRE(B >= 1 && n_q >= 1 && n_h >= 1 && c >= 1 && cap >= 0, DLC_E_INVAL,
              "%s: need B, n_q, n_h, c >= 1 and cap >= 0", name);
  DLC_REQUIRE(q && out && (kv || cap == 0), DLC_E_INVAL, "%s: NULL argument", name);
  DLC_REQUIRE(c <= 1024 || mfma_ok(dtype, c), DLC_E_UNSUPPORTED, "%s: c=%lld > 1024", name, (long long)c);
  if (mfma_ok(dtype, c))
    DLC_REQUIRE(aligned(q, 16) && aligned(kv, 16), DLC_E_INVAL, "%s: q and the cache must be 16-byte aligned", name);
  return DLC_OK;
}

// the joined forms: the mode's keys and the window's in one attention
int window_tail(const char* name, AttArgs& a, const void* Cwin, int64_t ring, int64_t n_win, const int64_t* t,
                int64_t t_max) {
  DLC_REQUIRE(Cwin != nullptr && t != nullptr, DLC_E_INVAL, "%s: NULL window ring or t", name);
  DLC_REQUIRE(n_win >= 1 && ring >= n_win && t_max >= 0, DLC_E_SHAPE,
              "%s: need 1 <= n_win <= ring and t_max >= 0 (n_win=%lld ring=%lld)", name, (long long)n_win,
              (long long)ring);
  DLC_REQUIRE(!mfma_ok(DLC_BF16, a.c) || aligned(Cwin, 16), DLC_E_INVAL, "%s: ring must be 16-byte aligned", name);
  a.win = Cwin; a.win_ring = ring; a.win_n = n_win; a.win_t = t; a.win_tmax = t_max;
  return DLC_OK;
}

// csa_attend with its caller-checked arguments; ws is the workspace (or the
// scratch array of csa_attend_noalloc)
int csa_attend_impl(const char* name, int dtype, int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t k,
                    const void* q, const void* Ccomp, int64_t cap, const int32_t* idx, const int32_t* count,
                    float scale, float* out, float* lse, void* ws, size_t ws_bytes, hipStream_t s) {
  AttArgs a{};
  a.q = q; a.kv = Ccomp; a.idx = idx; a.count = count;
  a.n_q = n_q; a.n_h = n_h; a.c = c; a.cap = cap; a.k = k;
  a.scale_log2 = (scale > 0.f ? scale : 1.f / std::sqrt(float(c))) * kLog2e;
  return run_attend<kGather>(name, dtype, a, B * n_q, k, out, lse, ws, ws_bytes, s);
}

int csa_attend_checks(const char* name, int dtype, int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t k,
                      const void* q, const void* Ccomp, int64_t cap, const int32_t* idx, const int32_t* count,
                      const float* out) {
  int rc = common_checks(name, dtype, B, n_q, n_h, c, q, Ccomp, cap, out);
  if (rc) return rc;
  DLC_REQUIRE(k >= 1, DLC_E_INVAL, "%s: k must be >= 1", name);
  DLC_REQUIRE(idx && count, DLC_E_INVAL, "%s: NULL idx or count", name);
  return DLC_OK;
}

}  // namespace

// ------------------------------------------------------------------ allocation-free entry point
//
// csa_attend_noalloc keeps its split partials in this file-scope device array
// instead of a caller workspace.  Every device the library runs on holds its
// own copy at its own address until the process ends.  Host code never uses
// the array's name as a device address: the address is taken once per device
// with hipGetSymbolAddress (that device current) and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the scratch array's address on the device of stream s
int scratch_for_stream(const char* name, hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipStreamGetDevice(s, &dev);
  if (e != hipSuccess) return fail(DLC_E_HIP, "%s: hipStreamGetDevice: %s", name, hipGetErrorString(e));
  DLC_REQUIRE(dev >= 0 && dev < kMaxDevices, DLC_E_UNSUPPORTED, "%s: device %d out of range", name, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(DLC_E_HIP, "%s: hipGetDevice: %s", name, hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(DLC_E_HIP, "%s: hipSetDevice: %s", name, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr)
      return fail(DLC_E_HIP, "%s: hipGetSymbolAddress: %s", name, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DLC_OK;
}
}  // namespace

}  // namespace dlc

extern "C" {

size_t csa_attend_ws(int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t k) {
  if (B < 1 || n_q < 1 || n_h < 1 || c < 1 || k < 1) return 0;
  return dlc::ws_bound(B * n_q, n_h, c, k);
}

size_t hca_attend_ws(int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t cap) {
  if (B < 1 || n_q < 1 || n_h < 1 || c < 1 || cap < 0) return 0;
  return dlc::ws_bound(B * n_q, n_h, c, cap);
}

int csa_attend(int dtype, int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t k, const void* q,
               const void* Ccomp, int64_t cap, const int32_t* idx, const int32_t* count, float scale, float* out,
               float* lse, void* ws, size_t ws_bytes, void* stream) {
  using namespace dlc;
  int rc = csa_attend_checks("csa_attend", dtype, B, n_q, n_h, c, k, q, Ccomp, cap, idx, count, out);
  if (rc) return rc;
  return csa_attend_impl("csa_attend", dtype, B, n_q, n_h, c, k, q, Ccomp, cap, idx, count, scale, out, lse, ws,
                         ws_bytes, as_stream(stream));
}

int csa_attend_noalloc(int dtype, int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t k, const void* q,
                       const void* Ccomp, int64_t cap, const int32_t* idx, const int32_t* count, float scale,
                       float* out, float* lse, void* stream) {
  using namespace dlc;
  const char* name = "csa_attend_noalloc";
  int rc = csa_attend_checks(name, dtype, B, n_q, n_h, c, k, q, Ccomp, cap, idx, count, out);
  if (rc) return rc;
  const size_t need = csa_attend_ws(B, n_q, n_h, c, k);
  DLC_REQUIRE(need <= kScratchBytes, DLC_E_UNSUPPORTED,
              "%s: this shape needs %zu bytes of scratch, more than the %zu-byte static scratch array", name, need,
              kScratchBytes);
  void* ws = nullptr;
  hipStream_t s = as_stream(stream);
  if (need > 0 && (rc = scratch_for_stream(name, s, &ws))) return rc;
  return csa_attend_impl(name, dtype, B, n_q, n_h, c, k, q, Ccomp, cap, idx, count, scale, out, lse, ws,
                         need > 0 ? kScratchBytes : 0, s);
}

int hca_attend(int dtype, int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t m_prime, const void* q,
               const void* Chca, int64_t cap, const int64_t* t, int64_t t_max, float scale, float* out, float* lse,
               void* ws, size_t ws_bytes, void* stream) {
  using namespace dlc;
  int rc = common_checks("hca_attend", dtype, B, n_q, n_h, c, q, Chca, cap, out);
  if (rc) return rc;
  DLC_REQUIRE(m_prime >= 1 && t_max >= 0, DLC_E_INVAL, "hca_attend: need m' >= 1 and t_max >= 0");
  DLC_REQUIRE(t != nullptr, DLC_E_INVAL, "hca_attend: NULL t");
  DLC_REQUIRE(t_max / m_prime <= cap, DLC_E_SHAPE, "hca_attend: floor(t_max/m')=%lld exceeds cap=%lld",
              (long long)(t_max / m_prime), (long long)cap);
  AttArgs a{};
  a.q = q; a.kv = Chca; a.t = t;
  a.n_q = n_q; a.n_h = n_h; a.c = c; a.cap = cap; a.m_prime = m_prime; a.t_max = t_max;
  a.scale_log2 = (scale > 0.f ? scale : 1.f / std::sqrt(float(c))) * kLog2e;
  return run_attend<kDense>("hca_attend", dtype, a, B * n_q, t_max / m_prime, out, lse, ws, ws_bytes,
                           as_stream(stream));
}


size_t csa_attend_window_ws(int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t k, int64_t n_win) {
  if (B < 1 || n_q < 1 || n_h < 1 || c < 1 || k < 1 || n_win < 1) return 0;
  return dlc::ws_bound(B * n_q, n_h, c, k + n_win);
}

size_t hca_attend_window_ws(int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t cap, int64_t n_win) {
  if (B < 1 || n_q < 1 || n_h < 1 || c < 1 || cap < 0 || n_win < 1) return 0;
  return dlc::ws_bound(B * n_q, n_h, c, cap + n_win);
}

int csa_attend_window(int dtype, int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t k, const void* q,
                      const void* Ccomp, int64_t cap, const int32_t* idx, const int32_t* count, const void* Cwin,
                      int64_t ring, int64_t n_win, const int64_t* t, int64_t t_max, float scale, float* out,
                      float* lse, void* ws, size_t ws_bytes, void* stream) {
  using namespace dlc;
  int rc = common_checks("csa_attend_window", dtype, B, n_q, n_h, c, q, Ccomp, cap, out);
  if (rc) return rc;
  DLC_REQUIRE(k >= 1, DLC_E_INVAL, "csa_attend_window: k must be >= 1");
  DLC_REQUIRE(idx && count, DLC_E_INVAL, "csa_attend_window: NULL idx or count");
  AttArgs a{};
  a.q = q; a.kv = Ccomp; a.idx = idx; a.count = count;
  a.n_q = n_q; a.n_h = n_h; a.c = c; a.cap = cap; a.k = k;
  a.scale_log2 = (scale > 0.f ? scale : 1.f / std::sqrt(float(c))) * kLog2e;
  if ((rc = window_tail("csa_attend_window", a, Cwin, ring, n_win, t, t_max))) return rc;
  return run_attend<kGather>("csa_attend_window", dtype, a, B * n_q, k + n_win, out, lse, ws, ws_bytes,
                             as_stream(stream));
}

int hca_attend_window(int dtype, int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t m_prime, const void* q,
                      const void* Chca, int64_t cap, const int64_t* t, int64_t t_max, const void* Cwin, int64_t ring,
                      int64_t n_win, float scale, float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  using namespace dlc;
  int rc = common_checks("hca_attend_window", dtype, B, n_q, n_h, c, q, Chca, cap, out);
  if (rc) return rc;
  DLC_REQUIRE(m_prime >= 1 && t_max >= 0, DLC_E_INVAL, "hca_attend_window: need m' >= 1 and t_max >= 0");
  DLC_REQUIRE(t != nullptr, DLC_E_INVAL, "hca_attend_window: NULL t");
  DLC_REQUIRE(t_max / m_prime <= cap, DLC_E_SHAPE, "hca_attend_window: floor(t_max/m')=%lld exceeds cap=%lld",
              (long long)(t_max / m_prime), (long long)cap);
  AttArgs a{};
  a.q = q; a.kv = Chca; a.t = t;
  a.n_q = n_q; a.n_h = n_h; a.c = c; a.cap = cap; a.m_prime = m_prime; a.t_max = t_max;
  a.scale_log2 = (scale > 0.f ? scale : 1.f / std::sqrt(float(c))) * kLog2e;
  if ((rc = window_tail("hca_attend_window", a, Cwin, ring, n_win, t, t_max))) return rc;
  return run_attend<kDense>("hca_attend_window", dtype, a, B * n_q, t_max / m_prime + n_win, out, lse, ws,
                            ws_bytes, as_stream(stream));
}

size_t window_attend_ws(int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t n_win) {
  if (B < 1 || n_q < 1 || n_h < 1 || c < 1 || n_win < 1) return 0;
  return dlc::ws_bound(B * n_q, n_h, c, n_win, true);
}

int window_attend(int dtype, int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t n_win, const void* q,
                  const void* Cwin, int64_t ring, const int64_t* t, int64_t t_max, float scale, const float* o_in,
                  const float* lse_in, float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  using namespace dlc;
  int rc = common_checks("window_attend", dtype, B, n_q, n_h, c, q, Cwin, ring, out);
  if (rc) return rc;
  DLC_REQUIRE(n_win >= 1 && t_max >= 0, DLC_E_INVAL, "window_attend: need n_win >= 1 and t_max >= 0");
  DLC_REQUIRE(ring >= n_win && Cwin != nullptr, DLC_E_SHAPE, "window_attend: ring (%lld) < n_win (%lld)",
              (long long)ring, (long long)n_win);
  DLC_REQUIRE(t != nullptr, DLC_E_INVAL, "window_attend: NULL t");
  DLC_REQUIRE((o_in == nullptr) == (lse_in == nullptr), DLC_E_INVAL,
              "window_attend: o_in and lse_in come together");
  AttArgs a{};
  a.q = q; a.kv = Cwin; a.t = t;
  a.n_q = n_q; a.n_h = n_h; a.c = c; a.cap = ring; a.n_win = n_win; a.t_max = t_max; a.m_prime = 1;
  a.scale_log2 = (scale > 0.f ? scale : 1.f / std::sqrt(float(c))) * kLog2e;
  const int64_t nkeys = t_max + 1 < n_win ? t_max + 1 : n_win;
  return run_attend<kWindow>("window_attend", dtype, a, B * n_q, nkeys, out, lse, ws, ws_bytes,
                             as_stream(stream), o_in, lse_in);
}

int attend_sink(int64_t rows, int64_t n_h, int64_t c, float* out, float* lse, const float* z, void* stream) {
  using namespace dlc;
  DLC_REQUIRE(rows >= 0 && n_h >= 1 && c >= 1, DLC_E_INVAL, "attend_sink: need rows >= 0, n_h >= 1, c >= 1");
  if (rows == 0) return DLC_OK;
  DLC_REQUIRE(out && lse && z, DLC_E_INVAL, "attend_sink: NULL argument");
  DLC_REQUIRE(aligned(out, 16), DLC_E_INVAL, "attend_sink: out must be 16-byte aligned");
  DLC_REQUIRE(rows * n_h < (int64_t(1) << 31), DLC_E_UNSUPPORTED, "attend_sink: rows*n_h too large");
  hipLaunchKernelGGL(sink_kernel, dim3((unsigned)(rows * n_h)), dim3(128), 0, as_stream(stream), out, lse, z, n_h, c);
  return check_launch("attend_sink");
}

}  // extern "C"
