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
// MFMA path (bf16, c in {128, 256, 512}): a workgroup is 8 waves and covers
// 128 heads.  All heads share each key row, so a 32-key tile is staged once in
// LDS, row-major for Q.K^T and transposed for P.V.  Wave w owns heads
// 32*(w/2) .. +31 and half w%2 of the c dimensions, and multiplies with
// v_mfma_f32_32x32x16_bf16:
//   S^T[32 keys][32 heads] = K[32 keys][half] . Q^T[half][32 heads]  (Q in registers)
//   (the two halves' partial S^T are swapped through LDS and added)
//   O[32 heads][half]     += P[32 heads][32 keys] . V[32 keys][half]
// Splitting c between two waves keeps Q (64 VGPRs) and O (128 AGPRs) of a
// wave in registers at two waves per SIMD.  The S^T accumulator already holds,
// per lane, the 16 keys of one head that the P operand needs, so P never goes
// through memory.  Tiles are double-buffered: the next tile's global loads are
// in flight while the current one is used.
// The VALU path covers fp32 and other shapes.
#include "common.hpp"

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
constexpr int kTargetWorkgroups = DLC_ATTEND_TARGET_WGS;

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

// ------------------------------------------------------------------ MFMA path, c = 512
//
// The V4-Pro shape gets a kernel that keeps every 32-key tile in LDS exactly
// once, row-major, and feeds both products from it:
//  * tiles arrive by direct global->LDS loads (global_load_lds_dwordx4: one
//    instruction moves one 1 KB key row), three stages deep with two tiles in
//    flight; no registers hold staged data;
//  * Q.K^T reads the A operand (key rows) with ds_read_b128;
//  * P.V reads the B operand with ds_read_b64_tr_b16, the gfx950 transposing
//    LDS read: in each 16-lane group, lane j receives element j%4 of the
//    8-byte chunks addressed by lanes j/4, j/4+4, j/4+8, j/4+12.  Lane i of a
//    group addresses key row base+i/4 at dims c0+4*(i%4), so lane j ends up
//    with dim c0+j of keys base..base+3 - four consecutive keys of one dim,
//    which is the packed-k layout the MFMA wants;
//  * barriers are plain s_barrier after an LDS-only wait, so the tile loads in
//    flight are never drained by a barrier; each tile is waited for with an
//    explicit vmcnt that leaves the younger tile outstanding.
// Wave w owns heads 32*(w/2) .. +31 and half w%2 of the 512 dims, as in the
// generic kernel; the two halves' partial S^T are added through LDS.

__device__ __align__(16) bf16_raw g_zero_row[512];  // masked keys load this row

__device__ __forceinline__ void wait_vmcnt(int n) {
  // s_waitcnt with only the vector-memory counter set
  if (n == 4)
    __builtin_amdgcn_s_waitcnt(0x0F74);
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);
}


__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // LDS and scalar-memory counter only
  __builtin_amdgcn_s_barrier();
}

// LDS layout of a 32-key tile (gfx950 LDS: 64 banks of 4 bytes): key row r
// starts at byte 1024*r + 16*t(r), t(4a+j) = 16a + a%4 + 4j.  Row starts then
// differ mod 256 bytes so that
//  * a ds_read_b128 of 16 consecutive rows at one 16-byte column (the Q.K^T A
//    operand, 16 lanes per pass) touches 16 distinct 4-bank groups, and
//  * a ds_read_b64_tr_b16 of 4 consecutive rows x 64 bytes (the P.V B operand,
//    32 lanes per pass) touches 4 disjoint 16-bank groups;
// both are conflict-free.  A row stays 1 KB contiguous, as one direct load
// writes it.
constexpr int kTileBytes = 34816;   // 1024*31 + 16*t(31) + 1024, rounded up to 1 KB
constexpr int kMaxGatherKeys = 2048;  // keys per split whose rows sit in LDS

__device__ __forceinline__ constexpr int tile_row_off(int r) {
  return 1024 * r + 16 * (16 * (r >> 2) + ((r >> 2) & 3) + 4 * (r & 3));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int MODE>
__global__ void __launch_bounds__(512) attend512_kernel(AttArgs a) {
  constexpr int CD = 512, HALF = 256, KSH = 16, NTH = 8;
  constexpr int NST = 3;                // tile stages, two tiles in flight
  constexpr int RPW = 4;                // key rows each wave moves per tile
  constexpr int HPG = 128;              // heads per workgroup: 4 slices of 32, each split over 2 waves
  // one array per stage: distinct objects let the compiler see that reads of
  // the current stage never alias the loads still landing in the others
  __shared__ __attribute__((aligned(1024))) unsigned char sK0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sK1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sK2[kTileBytes];
  // partial S^T of every wave: lane-major, 16 values + 4 pad per lane so that
  // four 16-byte accesses per lane are free of bank conflicts
  constexpr int XROW = 20;
  __shared__ __attribute__((aligned(16))) float sX[8 * 64 * XROW];
  __shared__ int32_t sRow[MODE == kGather ? kMaxGatherKeys : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lets addresses live in SGPRs
  const int l32 = lane & 31, g2 = lane >> 5, G = lane >> 4, i16 = lane & 15;
  const int hp = wave >> 1, dh = wave & 1;  // head slice of 32, half of c
  const int64_t bq = blockIdx.y;
  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so the
  // head groups of one key split get ids that are equal mod 8 and share that
  // XCD's L2 for the split's key rows
  const int64_t xcd = blockIdx.x & 7, rest = blockIdx.x >> 3;
  const int64_t hg = rest % a.head_groups;
  const int64_t split = (rest / a.head_groups) * 8 + xcd;
  if (split >= a.splits) return;
  const int64_t b = bq / a.n_q;
  const int64_t nkm = n_keys<MODE>(a, bq);
  const int64_t nk = nkm + n_win_keys(a, bq);
  const int64_t k0 = split * a.keys_per_split;
  const int64_t k1 = min(nk, k0 + a.keys_per_split);
  const int64_t hbase = hg * HPG + hp * 32;
  const bool active = hbase < a.n_h;
  const int64_t ntile = k1 > k0 ? (k1 - k0 + 31) / 32 : 0;

  if constexpr (MODE == kGather) {
    for (int64_t j = tid; j < k1 - k0; j += 512) sRow[j] = int32_t(key_code<kGather>(a, bq, k0 + j, k1, nkm));
    __syncthreads();  // sRow ready for the tile loads
  }
  // each wave moves rows RPW*wave .. +RPW-1 of a tile: one 1 KB DMA load per row
  auto issue = [&](unsigned char* dst, int st, int64_t tl) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int row = RPW * wave + r;
      const int64_t j = tl * 32 + row;  // key position within the split
      int64_t gr;
      if constexpr (MODE == kGather) {
        gr = (k0 + j < k1) ? sRow[j] : -1;
      } else {
        gr = key_code<MODE>(a, bq, k0 + j, k1, nkm);
      }
      gr = __builtin_amdgcn_readfirstlane(int(gr));
      const bf16_raw* src = key_ptr<bf16_raw>(a, b, gr);
      if (src == nullptr) src = g_zero_row;
      const uint32_t lds_addr = (uint32_t)(uintptr_t)DLC_LDS(dst) + uint32_t(tile_row_off(row));
      dma_row(src, uint32_t(lane) * 16u, lds_addr);
    }
  };
  // bit j: key j of tile tl is valid (masked keys were loaded as zero rows)
  auto valid_mask = [&](int64_t tl) -> uint32_t {
    const int64_t j = tl * 32 + l32;
    bool v = k0 + j < k1;
    if constexpr (MODE == kGather) v = v && sRow[j] != -1;
    return uint32_t(__ballot(v) & 0xffffffffu);
  };
  // the first two tiles and Q are in flight together
  if (ntile > 0) issue(sK0, 0, 0);
  if (ntile > 1) issue(sK1, 1, 1);
  // Q^T operand over this wave's half of c: lane holds head hbase + l32,
  // dims dh*HALF + ks*16 + g2*8 .. +7; heads past n_h read head n_h-1 (their
  // S^T columns and outputs are never used)
  bf16x8 qf[KSH];
  {
    const int64_t h = min(hbase + l32, a.n_h - 1);
    const bf16_raw* qp = static_cast<const bf16_raw*>(a.q) + (bq * a.n_h + h) * CD + dh * HALF + g2 * 8;
#pragma unroll
    for (int ks = 0; ks < KSH; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + ks * 16));
    // consume the Q loads here (this also waits for the two tiles issued
    // above), so no wait for them is left inside the tile loop
#pragma unroll
    for (int ks = 0; ks < KSH; ++ks) asm volatile("" ::"v"(qf[ks]));
  }
  f32x16 o[NTH];
#pragma unroll
  for (int nt = 0; nt < NTH; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[nt][r] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;
  // per-lane LDS byte offsets within a tile (rows laid out by tile_row_off)
  const uint32_t qk_off = uint32_t(tile_row_off(l32) + dh * 512 + 16 * g2);
  uint32_t pv_off[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      pv_off[u][h] = uint32_t(tile_row_off(16 * u + 8 * h + 4 * g2 + (i16 >> 2)) + dh * 512 + 32 * (G & 1) + 8 * (i16 & 3));

  auto tile_step = [&](const unsigned char* tile, unsigned char* next, int st, int64_t it) {
    wait_vmcnt(it + 1 < ntile ? RPW : 0);  // tile it has landed (tile it+1 may still fly)
    lds_barrier();                         // ... for every wave; stage (it+2)%3 and sX are free
    if (it + 2 < ntile) issue(next, (st + 2) % NST, it + 2);
    f32x16 sx;
#pragma unroll
    for (int r = 0; r < 16; ++r) sx[r] = 0.f;
    if (active) {
      // partial S^T = K . Q^T over this wave's half of c; the next batch of
      // fragments is in flight while the current one feeds the MFMAs
      const unsigned char* krow = tile + qk_off;
      bf16x8 ka[4], kb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) ka[u] = *reinterpret_cast<const bf16x8*>(krow + 32 * u);
#pragma unroll
      for (int k4 = 0; k4 < KSH; k4 += 4) {
        if (k4 + 4 < KSH) {
#pragma unroll
          for (int u = 0; u < 4; ++u) kb[u] = *reinterpret_cast<const bf16x8*>(krow + 32 * (k4 + 4 + u));
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int u = 0; u < 4; ++u) sx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[u], qf[k4 + u], sx, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) ka[u] = kb[u];
      }
      float4* xw = reinterpret_cast<float4*>(&sX[(wave * 64 + lane) * XROW]);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        xw[q4] = make_float4(sx[4 * q4], sx[4 * q4 + 1], sx[4 * q4 + 2], sx[4 * q4 + 3]);
    }
    const uint32_t vmask = valid_mask(it);
    lds_barrier();
    if (!active) return;
    // full S^T = both halves; lane holds head l32, keys kr(r) = 8*(r/4) + 4*g2 + r%4
    // add the partner's half, eight values at a time (bounded register use)
    {
      const float4* xr = reinterpret_cast<const float4*>(&sX[((wave ^ 1) * 64 + lane) * XROW]);
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        const float4 v0 = xr[2 * hq], v1 = xr[2 * hq + 1];
        const float ov[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * hq + e;
          sx[r] = dh == 0 ? sx[r] + ov[e] : ov[e] + sx[r];
        }
        asm volatile("" ::: "memory");
      }
    }
    float tmax = -INFINITY;
    if (vmask == 0xffffffffu) {  // a full tile (wave-uniform): no mask
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sx[r] *= a.scale_log2;
        tmax = fmaxf(tmax, sx[r]);
      }
    } else {
      const uint32_t vm = vmask >> (4 * g2);  // key 8*(r/4) + 4*g2 + r%4 -> bit 8*(r/4) + r%4
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sx[r] = ((vm >> (8 * (r >> 2) + (r & 3))) & 1u) ? sx[r] * a.scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, sx[r]);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    // lazy running max (see the generic kernel)
    const bool move = tmax > mrun + 8.f;
    if (__any(move)) {
      const float mnew = move ? tmax : mrun;
      const float alpha = mrun == -INFINITY ? 0.f : exp2f(mrun - mnew);
      lrun *= alpha;
      mrun = mnew;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float al = __shfl(alpha, 8 * (r >> 2) + 4 * g2 + (r & 3));
#pragma unroll
        for (int nt = 0; nt < NTH; ++nt) o[nt][r] *= al;
      }
    }
    // v_exp_f32 directly: masked keys give exp2(-inf) = 0; a head with nothing
    // valid yet has mrun = -inf, and exponentiates against 0 instead
    const float mr = mrun == -INFINITY ? 0.f : mrun;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sx[r] = __builtin_amdgcn_exp2f(sx[r] - mr);
      psum += sx[r];
    }
    psum += __shfl_xor(psum, 32);
    lrun += psum;
    bf16x8 pa[2];
#pragma unroll
    for (int uu = 0; uu < 2; ++uu)
#pragma unroll
      for (int e = 0; e < 8; ++e) pa[uu][e] = (__bf16)sx[8 * uu + e];
    // B operand (keys 16u + 8h + 4*g2 + 0..3 for slots 4h .. 4h+3, dim
    // dh*HALF + nt*32 + l32) from two transposing reads
    auto vfrag = [&](int nt, int u) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)DLC_LDS(tile + pv_off[u][0] + 64 * nt));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)DLC_LDS(tile + pv_off[u][1] + 64 * nt));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // fragments in batches of four (two output tiles x both key halves), the
    // next batch in flight while the current one feeds the MFMAs
    bf16x8 va[4], vb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) va[u] = vfrag(u >> 1, u & 1);
#pragma unroll
    for (int n2 = 0; n2 < NTH; n2 += 2) {
      if (n2 + 2 < NTH) {
#pragma unroll
        for (int u = 0; u < 4; ++u) vb[u] = vfrag(n2 + 2 + (u >> 1), u & 1);
      }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int u = 0; u < 4; ++u)
        o[n2 + (u >> 1)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[u & 1], va[u], o[n2 + (u >> 1)], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 4; ++u) va[u] = vb[u];
    }
  };
  for (int64_t it = 0; it < ntile; it += NST) {
    tile_step(sK0, sK2, 0, it);
    if (it + 1 < ntile) tile_step(sK1, sK0, 1, it + 1);
    if (it + 2 < ntile) tile_step(sK2, sK1, 2, it + 2);
  }

  if (!active) return;
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

// ------------------------------------------------------------------ host

bool mfma_ok(int dtype, int64_t c) { return dtype == DLC_BF16 && (c == 128 || c == 256 || c == 512); }

struct Plan {
  bool mfma;
  int64_t splits, kps, head_groups;
  size_t o_off, l_off, total;
};

Plan plan(int dtype, int64_t BQ, int64_t n_h, int64_t c, int64_t nkeys, bool merge = false) {
  Plan p{};
  p.mfma = mfma_ok(dtype, c);
  p.head_groups = p.mfma ? ceil_div(n_h, 128) : n_h;
  const int64_t per_split = p.mfma ? BQ * p.head_groups : BQ * n_h;
  int64_t s = ceil_div(kTargetWorkgroups, per_split);
  const int64_t smax = ceil_div(nkeys > 0 ? nkeys : 1, kMinKeysPerSplit);
  s = s < smax ? s : smax;
  const int64_t smin = ceil_div(nkeys > 0 ? nkeys : 1, c == 512 ? kMaxGatherKeys : 4096);  // a split's rows fit in LDS
  s = s < smin ? smin : s;
  s = s < 1 ? 1 : (s > kMaxSplits ? kMaxSplits : s);
  p.splits = s;
  p.kps = ceil_div(nkeys > 0 ? nkeys : 1, s);
  if (p.mfma) p.kps = ceil_div(p.kps, 32) * 32;
  p.o_off = 0;
  size_t off = 0;
  if (s > 1 || merge) {  // partials, combined afterwards
    off = align_up(size_t(BQ) * s * n_h * c * 4, 256);
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
  const Plan p = plan(dtype, BQ, a.n_h, a.c, nkeys, merge);
  DLC_REQUIRE(p.total == 0 || (ws != nullptr && ws_bytes >= p.total), DLC_E_WORKSPACE,
              "%s: workspace of %zu bytes needed, %zu given", name, p.total, ws_bytes);
  DLC_REQUIRE(ws == nullptr || aligned(ws, 256), DLC_E_WORKSPACE, "%s: workspace must be 256-byte aligned", name);
  a.splits = p.splits;
  a.keys_per_split = p.kps;
  a.head_groups = p.head_groups;
  const bool partials = p.splits > 1 || merge;
  if (partials) {
    a.o = reinterpret_cast<float*>(static_cast<char*>(ws) + p.o_off);
    a.lse = reinterpret_cast<float*>(static_cast<char*>(ws) + p.l_off);
  } else {
    a.o = out;
    a.lse = lse;
  }
  DLC_REQUIRE(BQ <= 65535 && p.splits * p.head_groups < (int64_t(1) << 31), DLC_E_UNSUPPORTED,
              "%s: grid too large", name);
  StageTimer timer(MODE == kGather ? DLC_STAGE_CSA_ATTEND : MODE == kDense ? DLC_STAGE_HCA_ATTEND
                                                                             : DLC_STAGE_WINDOW_ATTEND, s);
  if (p.mfma) {
    dim3 grid{(unsigned)(p.splits * p.head_groups), (unsigned)BQ, 1u};
    if (a.c == 128) hipLaunchKernelGGL((attend_mfma_kernel<128, MODE>), grid, dim3(512), 0, s, a);
    if (a.c == 256) hipLaunchKernelGGL((attend_mfma_kernel<256, MODE>), grid, dim3(512), 0, s, a);
    if (a.c == 512) hipLaunchKernelGGL((attend512_kernel<MODE>), grid, dim3(512), 0, s, a);
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
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(BQ * a.n_h)), dim3(128), 0, s, a.o, a.lse, p.splits, a.n_h,
                     a.c, out, lse, o_in, lse_in);
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
  int rc = common_checks("csa_attend", dtype, B, n_q, n_h, c, q, Ccomp, cap, out);
  if (rc) return rc;
  DLC_REQUIRE(k >= 1, DLC_E_INVAL, "csa_attend: k must be >= 1");
  DLC_REQUIRE(idx && count, DLC_E_INVAL, "csa_attend: NULL idx or count");
  AttArgs a{};
  a.q = q; a.kv = Ccomp; a.idx = idx; a.count = count;
  a.n_q = n_q; a.n_h = n_h; a.c = c; a.cap = cap; a.k = k;
  a.scale_log2 = (scale > 0.f ? scale : 1.f / std::sqrt(float(c))) * kLog2e;
  return run_attend<kGather>("csa_attend", dtype, a, B * n_q, k, out, lse, ws, ws_bytes, as_stream(stream));
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

}  // extern "C"
