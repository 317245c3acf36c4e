// Softmax + top-k of one token's E router logits, on one 64-lane wavefront.
//
// The gate's softmax runs over all E experts and the k experts with the
// largest probability are kept, their probabilities being the mixing weights
// (page "FreeToken：753B大模型塞进单卡的本地部署硬件账该怎么算", section
// "混合专家架构（MoE）的天然稀疏性").  Softmax is monotone, so the selection
// compares the fp32 logits, ties going to the lower expert index.
#pragma once
#include "common.h"

// Lane l holds logits of experts l, l+64, ..., l+64*(NV-1) (E <= 64*NV).  On
// return, lane r < k holds the rank-r expert and its weight.
// (z, e) is better than (oz, oe): larger logit, or an equal logit and a lower index.
__device__ __forceinline__ bool better(float z, int e, float oz, int oe) {
  return z > oz || (z == oz && e < oe);
}

template <int CTRL>
__device__ __forceinline__ void argmax_step(float& z, int& e) {
  const float oz = dpp_f32<CTRL>(z);
  const int oe = dpp_i32<CTRL>(e);
  if (better(oz, oe, z, e)) {
    z = oz;
    e = oe;
  }
}

// Wave-wide best (z, e), uniform result: DPP within rows, readlane across rows.
__device__ __forceinline__ void wave_argmax(float& z, int& e) {
  argmax_step<kDppXor1>(z, e);
  argmax_step<kDppXor2>(z, e);
  argmax_step<kDppHalfMirror>(z, e);
  argmax_step<kDppMirror>(z, e);
  float bz = readlane_f32(z, 0);
  int be = __builtin_amdgcn_readlane(e, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) {
    const float rz = readlane_f32(z, r);
    const int re = __builtin_amdgcn_readlane(e, r);
    if (better(rz, re, bz, be)) {
      bz = rz;
      be = re;
    }
  }
  z = bz;
  e = be;
}

// Lane l holds logits of experts l, l+64, ..., l+64*(NV-1) (E <= 64*NV, -inf
// beyond E).  On return, lane r < k holds the rank-r expert and its weight.
template <int NV>
__device__ __forceinline__ void wave_topk_regs(const float (&v)[NV], int E, int k, unsigned flags,
                                               int& my_idx, float& my_w) {
  const int lane = threadIdx.x & 63;
  float zmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV; ++i) zmax = fmaxf(zmax, v[i]);
  zmax = wave_max(zmax);
  float se = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (lane + 64 * i < E) se += expf(v[i] - zmax);
  se = wave_sum(se);
  uint32_t taken = 0;
  float selsum = 0.0f;
  my_idx = 0;
  my_w = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bz = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && better(v[i], e, bz, be)) {
        bz = v[i];
        be = e;
      }
    }
    wave_argmax(bz, be);
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    const float p = expf(bz - zmax) / se;
    selsum += p;
    if (lane == j) {
      my_idx = be;
      my_w = p;
    }
  }
  if (flags & MOE_ROUTE_RENORM) my_w /= selsum;
}

template <int NV>
__device__ __forceinline__ void wave_load_logits(const float* __restrict__ z, int E, float (&v)[NV]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? z[e] : -INFINITY;
  }
}
