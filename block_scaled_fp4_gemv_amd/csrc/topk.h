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

// Order-preserving map of an fp32 logit to uint32 (larger logit -> larger key;
// -0 and +0 map to one key).  Key 0 is below every finite logit's key.
__device__ __forceinline__ uint32_t logit_key(float z) {
  const uint32_t u = __float_as_uint(z + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Lane l holds logits of experts l, l+64, ..., l+64*(NV-1) (E <= 64*NV; values
// beyond E are ignored).  k <= 16.  `list` is 2*16 words of LDS private to this
// wave.  On return lane r < k holds the rank-r expert and its weight.
//
// Selection is a radix select on the 32-bit keys: 32 ballot/popcount rounds
// find the k-th largest key T; the experts above T plus the lowest-index ones
// equal to T form the top-k set, which is compacted into `list` and ordered
// by (logit desc, index asc) with k*k comparisons.
template <int NV>
__device__ __forceinline__ void wave_topk_radix(const float (&v)[NV], int E, int k, unsigned flags,
                                                int& my_idx, float& my_w, uint32_t* list) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  uint32_t key[NV];
  float zmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const bool ok = lane + 64 * i < E;
    key[i] = ok ? logit_key(v[i]) : 0u;
    if (ok) zmax = fmaxf(zmax, v[i]);
  }
  zmax = wave_max(zmax);
  float se = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (lane + 64 * i < E) se += __expf(v[i] - zmax);
  se = wave_sum(se);
  // k-th largest key
  uint32_t T = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) cnt += __popcll(__ballot(key[i] >= cand));
    if (cnt >= k) T = cand;
  }
  int n_gt = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) n_gt += __popcll(__ballot(key[i] > T));
  const int need = k - n_gt;  // >= 1 ties at T, taken by ascending expert index
  int ties_before = 0, sel_before = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const uint64_t tm = __ballot(key[i] == T && key[i] != 0u);
    const int tie_rank = ties_before + __popcll(tm & lt_mask);
    ties_before += __popcll(tm);
    const bool sel = key[i] > T || (key[i] == T && key[i] != 0u && tie_rank < need);
    const uint64_t sm = __ballot(sel);
    if (sel) {
      const int pos = sel_before + __popcll(sm & lt_mask);
      list[pos] = __float_as_uint(v[i]);
      list[16 + pos] = (uint32_t)(lane + 64 * i);
    }
    sel_before += __popcll(sm);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  float z = -INFINITY;
  int e = 0x7fffffff, rank = 0;
  if (lane < k) {
    z = __uint_as_float(list[lane]);
    e = (int)list[16 + lane];
    for (int s = 0; s < k; ++s) {
      const float oz = __uint_as_float(list[s]);
      const int oe = (int)list[16 + s];
      rank += better(oz, oe, z, e) ? 1 : 0;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  // scatter to rank order through the same scratch
  const float p = lane < k ? __expf(z - zmax) / se : 0.0f;
  if (lane < k) {
    list[rank] = __float_as_uint(p);
    list[16 + rank] = (uint32_t)e;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  my_idx = 0;
  my_w = 0.0f;
  if (lane < k) {
    my_w = __uint_as_float(list[lane]);
    my_idx = (int)list[16 + lane];
  }
  if (flags & MOE_ROUTE_RENORM) {
    const float tot = wave_sum(lane < k ? my_w : 0.0f);
    my_w /= tot;
  }
  __builtin_amdgcn_wave_barrier();
}

// Scratch (LDS, private to one wave) for wave_topk_regs.
struct TopkScratch {
  uint32_t cz[64];   // candidate logits (fp32 bits)
  uint32_t ce[64];   // candidate experts
  uint32_t list[32]; // radix fallback scratch
};

// Selection state of one token's top-k on one wave (uniform except bin).
template <int NV>
struct TopkSel {
  float zmax;          // max logit
  int B, m;            // threshold bin; experts in bins <= B (the candidates)
  uint64_t mask[NV];   // candidates: bit l of mask[i] is expert l + 64 i
  int bin[NV];         // per lane: bin of experts lane + 64 i (256 beyond E)
};

// Lane l holds logits of experts l, l+64, ..., l+64*(NV-1) (E <= 64*NV; values
// beyond E are ignored), 1 <= k <= min(E, 16).
//
// The logit range [zmin, zmax] is cut into 256 equal bins counted from the top,
// bin = floor((zmax - z) * 255 / (zmax - zmin)), which never decreases as z
// decreases, so the k best experts lie in the bins up to the one holding the
// k-th best; that bin B is found by an 8-step bisection over bin numbers with
// ballot counts.  Returns true when the candidates (bins <= B) are exactly k:
// they are then the top-k set, known before its order.
template <int NV>
__device__ __forceinline__ bool wave_topk_select(const float (&v)[NV], int E, int k, TopkSel<NV>& s) {
  const int lane = threadIdx.x & 63;
  float zmax = -INFINITY, zmin = INFINITY;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (lane + 64 * i < E) {
      zmax = fmaxf(zmax, v[i]);
      zmin = fminf(zmin, v[i]);
    }
  zmax = wave_max(zmax);
  zmin = wave_min(zmin);
  const float span = zmax - zmin;
  const float scale = span > 0.0f ? 255.0f / span : 0.0f;  // an infinite span gives 0: one bin
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const bool ok = lane + 64 * i < E;
    const float d = (zmax - v[i]) * scale;
    s.bin[i] = ok ? (d < 255.0f ? (int)d : 255) : 256;
  }
  s.zmax = zmax;
  // B = the largest bin number with fewer than k experts in lower bins
  int B = 0;
#pragma unroll
  for (int bit = 7; bit >= 0; --bit) {
    const int t = B + (1 << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) cnt += __popcll(__ballot(s.bin[i] < t));
    if (cnt < k) B = t;
  }
  int m = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    s.mask[i] = __ballot(s.bin[i] <= B);
    m += __popcll(s.mask[i]);
  }
  s.B = B;
  s.m = m;
  return m == k;
}

// The j-th candidate in ascending expert order (j < m; uniform).
template <int NV>
__device__ __forceinline__ int topk_candidate(const TopkSel<NV>& s, int j) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    uint64_t mk = s.mask[i];
    const int n = __popcll(mk);
    if (j < n) {
      for (; j > 0; --j) mk &= mk - 1;
      return 64 * i + __builtin_ctzll(mk);
    }
    j -= n;
  }
  return -1;
}

// Order the selection: on return lane r < k holds the rank-r expert (logit
// desc, index asc) and its softmax weight over all E experts.  The candidates
// are compacted into lanes through LDS and ranked exactly against each other;
// more than 64 candidates (many equal or clustered logits) fall back to an
// exact radix select over all keys.
template <int NV>
__device__ __forceinline__ void wave_topk_order(const float (&v)[NV], int E, int k, unsigned flags,
                                                const TopkSel<NV>& s, int& my_idx, float& my_w,
                                                TopkScratch& sc) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  const int m = s.m;
  if (m > 64) {  // degenerate: many logits in one bin
    wave_topk_radix<NV>(v, E, k, flags, my_idx, my_w, sc.list);
    return;
  }
  float se = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (lane + 64 * i < E) se += __expf(v[i] - s.zmax);
  const float inv_se = 1.0f / wave_sum(se);
  // compact the candidates into lanes 0 .. m-1 through LDS
  int pos_base = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (s.bin[i] <= s.B) {
      const int pos = pos_base + __popcll(s.mask[i] & lt_mask);
      sc.cz[pos] = __float_as_uint(v[i]);
      sc.ce[pos] = (uint32_t)(lane + 64 * i);
    }
    pos_base += __popcll(s.mask[i]);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  float z = -INFINITY;
  int e = 0x7fffffff;
  if (lane < m) {
    z = __uint_as_float(sc.cz[lane]);
    e = (int)sc.ce[lane];
  }
  int rank = 0;
  for (int s2 = 0; s2 < m; ++s2)
    rank += better(readlane_f32(z, s2), __builtin_amdgcn_readlane(e, s2), z, e) ? 1 : 0;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  if (lane < m && rank < k) {
    sc.cz[rank] = __float_as_uint(__expf(z - s.zmax) * inv_se);
    sc.ce[rank] = (uint32_t)e;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  my_idx = 0;
  my_w = 0.0f;
  if (lane < k) {
    my_w = __uint_as_float(sc.cz[lane]);
    my_idx = (int)sc.ce[lane];
  }
  if (flags & MOE_ROUTE_RENORM) {
    const float tot = wave_sum(lane < k ? my_w : 0.0f);
    my_w /= tot;
  }
  __builtin_amdgcn_wave_barrier();
}

// Softmax + top-k: selection, then order (lane r < k: rank-r expert and weight).
template <int NV>
__device__ __forceinline__ void wave_topk_regs(const float (&v)[NV], int E, int k, unsigned flags,
                                               int& my_idx, float& my_w, TopkScratch& sc) {
  TopkSel<NV> s;
  wave_topk_select<NV>(v, E, k, s);
  wave_topk_order<NV>(v, E, k, flags, s, my_idx, my_w, sc);
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
