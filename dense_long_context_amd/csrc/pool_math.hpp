// Softmax pooling arithmetic of the compressor ("DeepSeek-V4 Hybrid
// Attention: CSA and HCA from Scratch", §4 and §10: one softmax per column
// over the window's logits, then the weighted sum of the window's values),
// shared by csa_compress / hca_compress and the fused projection + pooling
// calls, so that both give the same bits for the same stream values.
//
// A window is consumed in chunks of kPoolChunk rows.  A chunk's partial state
// is (max, sum, acc) with its weights taken against its own max; states are
// folded left to right with merge_state, and the entry is acc / sum.  Logits
// arrive pre-scaled: (Z + bias) * log2(e), so every weight is one exp2.
#pragma once
#include "common.hpp"

namespace dlc {

#ifndef DLC_POOL_CHUNK
#define DLC_POOL_CHUNK 4
#endif
constexpr int kPoolChunk = DLC_POOL_CHUNK;
constexpr float kPoolLog2e = 1.4426950408889634f;

// Every operation below is rounded on its own (no contraction into fused
// multiply-adds beyond the explicit fmaf): contraction is the compiler's
// choice per kernel, and two kernels that contracted differently would
// disagree in the last bit.

// the scaled logit (z + bias) * log2(e)
__device__ __forceinline__ float pool_logit(float z, float bias) {
#pragma clang fp contract(off)
  return (z + bias) * kPoolLog2e;
}

// the partial state of one chunk: rows rr < nr of l (logits) and cv (values)
// for each of VEC columns
template <int VEC>
__device__ __forceinline__ void chunk_fold(const float (&l)[kPoolChunk][VEC], const float (&cv)[kPoolChunk][VEC],
                                           int nr, float* mx, float* sum, float* acc) {
#pragma clang fp contract(off)
#pragma unroll
  for (int u = 0; u < VEC; ++u) {
    float cm = -INFINITY;
#pragma unroll
    for (int rr = 0; rr < kPoolChunk; ++rr)
      if (rr < nr) cm = fmaxf(cm, l[rr][u]);
    float sm = 0.f, ac = 0.f;
    // one v_exp_f32 per logit.  A -inf logit (the page's padding) gets weight
    // exp2(-inf) = 0; a chunk whose logits are all -inf keeps max -inf and
    // weights 0 (taking its max as the reference would give -inf - -inf = NaN),
    // so it adds nothing when merged.
    const float cref = cm == -INFINITY ? 0.f : cm;
#pragma unroll
    for (int rr = 0; rr < kPoolChunk; ++rr) {
      if (rr < nr) {
        const float w = __builtin_amdgcn_exp2f(l[rr][u] - cref);
        sm += w;
        ac = fmaf(w, cv[rr][u], ac);
      }
    }
    mx[u] = cm;
    sum[u] = sm;
    acc[u] = ac;
  }
}

// state <- state (+) partial.  The same operations wherever two states meet,
// so the result depends only on the chunk order, not on which lanes held them.
template <int VEC>
__device__ __forceinline__ void merge_state(float* mS, float* sS, float* aS, const float* mP, const float* sP,
                                            const float* aP) {
#pragma clang fp contract(off)
#pragma unroll
  for (int u = 0; u < VEC; ++u) {
    const float M = fmaxf(mS[u], mP[u]);
    const float f1 = mS[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mS[u] - M);
    const float f2 = mP[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mP[u] - M);
    sS[u] = fmaf(sS[u], f1, sP[u] * f2);
    aS[u] = fmaf(aS[u], f1, aP[u] * f2);
    mS[u] = M;
  }
}

// the entry's value from its folded state
__device__ __forceinline__ float pool_value(float acc, float sum) {
#pragma clang fp contract(off)
  return acc / sum;
}

}  // namespace dlc
