// Per-layer VRAM expert-slot cache with least-recently-used replacement.
//
// A global LRU cache of experts in VRAM absorbs the routing overlap between
// adjacent tokens; what misses is filled into the GPU cache (page "8GB 笔记本
// 39.3 tok/s、单卡跑 753B：FreeToken 把 frontier MoE 拉回本地", section "设计核心";
// frequency-based hot/cold expert placement: page "FreeToken：753B大模型塞进单卡
// 的本地部署硬件账该怎么算", section "按带宽动态分配参数存储").
//
// One workgroup performs one step for T*k accesses, with the whole state
// staged in LDS:
//  * hits are classified against the state at the start of the step;
//  * each distinct missed expert (in order of first appearance) takes a
//    victim among slots whose expert is not requested this step: empty slots
//    by ascending index first, then occupied slots by ascending stamp;
//  * access q (pair order) advances the clock and stamps its slot, so a slot's
//    final stamp is clock0 + (last access index of its expert) + 1.
// The state is keyed: expert e of a lookup is key key_base + e, so one state
// and one slot pool can serve several layers (each layer its own key range),
// the cross-layer form of the global cache; a per-layer cache has key_base 0.
// Miss records list experts (key - key_base), as the fills index the layer's
// own host pool by expert.
#include "common.h"
#include "launch.h"
#include "topk.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxE = 1024, kMaxS = 1024;

__device__ int block_exclusive_scan(int v, int* sh, int* total) {
  // sh: kThreads/64 ints of scratch
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o);
    if (lane >= o) incl += n;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  int wbase = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int s = sh[w];
    if (w < wave) wbase += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wbase + incl - v;
}

// NV > 0: the routed experts are first selected here from `logits` (T <= 4
// tokens, one wave each: softmax + top-k, written to topk_idx / topk_w), which
// saves a dependent kernel between the router and the lookup.
constexpr int kMaxFusedPairs = (kThreads / 64) * 16;

// E: keys of the state; key_base: this lookup's first key; E_route: experts
// of the fused top-k.
template <int NV>
__global__ __launch_bounds__(kThreads) void k_lru_lookup(
    int E, int S, int32_t* __restrict__ slot_expert, int32_t* __restrict__ expert_slot,
    int64_t* __restrict__ slot_stamp, int64_t* __restrict__ clock,
    const int32_t* __restrict__ idx_in, int n, int32_t* __restrict__ pair_slot,
    int32_t* __restrict__ pair_order, int32_t* __restrict__ rec, int n_max,
    const float* __restrict__ logits, int k, unsigned flags, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int key_base, int E_route, float* __restrict__ logit_out) {
  __shared__ int s_idx[kMaxFusedPairs];
  const int32_t* idx = idx_in;
  const int tid = threadIdx.x;
  // the cache state and the clock are requested first, so that their loads
  // overlap the fused top-k
  constexpr int kPer = kMaxE / kThreads;
  static_assert(kMaxS <= kMaxE, "state registers sized by kMaxE");
  int r_eslot[kPer], r_sexp[kPer];
  long long r_stamp[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid + i * kThreads;
    r_eslot[i] = e < E ? expert_slot[e] : -1;
    r_sexp[i] = e < S ? slot_expert[e] : -1;
    r_stamp[i] = e < S ? slot_stamp[e] : 0;
  }
  const long long c0 = *clock;
  if constexpr (NV > 0) {
    __shared__ TopkScratch s_topk[kThreads / 64];
    const int wv = threadIdx.x >> 6, ln = threadIdx.x & 63, T = n / k;
    if (wv < T) {
      float v[NV];
      wave_load_logits<NV>(logits + (size_t)wv * E_route, E_route, v);
      if (logit_out)  // a copy of the logits for a later prefetch step
#pragma unroll
        for (int i = 0; i < NV; ++i)
          if (ln + 64 * i < E_route) logit_out[(size_t)wv * E_route + ln + 64 * i] = v[i];
      int e;
      float wt;
      wave_topk_regs<NV>(v, E_route, k, flags, e, wt, s_topk[wv]);
      if (ln < k) {
        s_idx[wv * k + ln] = e;
        topk_idx[wv * k + ln] = e;
        topk_w[wv * k + ln] = wt;
      }
    }
    __syncthreads();
    idx = s_idx;
  }
  __shared__ int s_first[kMaxE];   // first access index of each expert (n = none)
  __shared__ int s_last[kMaxE];    // last access index
  __shared__ int s_eslot[kMaxE];   // expert -> slot (updated in place)
  __shared__ int s_resident[kMaxE];// resident at step start
  __shared__ int s_sexp[kMaxS];    // slot -> expert
  __shared__ long long s_stamp[kMaxS];
  __shared__ int s_cand_rank[kMaxS];
  __shared__ unsigned long long s_key[kMaxS];
  __shared__ int s_victim[kMaxS];
  __shared__ int s_miss_exp[kMaxS];
  __shared__ int s_scan[kThreads / 64];
  __shared__ int s_nmiss, s_ncand;

#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid + i * kThreads;
    if (e < E) {
      s_first[e] = n;
      s_last[e] = -1;
      s_eslot[e] = r_eslot[i];
      s_resident[e] = r_eslot[i] >= 0;
    }
    if (e < S) {
      s_sexp[e] = r_sexp[i];
      s_stamp[e] = r_stamp[i];
    }
  }
  __syncthreads();
  for (int q = tid; q < n; q += blockDim.x) {
    const int e = key_base + idx[q];
    atomicMin(&s_first[e], q);
    atomicMax(&s_last[e], q);
  }
  __syncthreads();

  // rank the distinct missed experts by first appearance (scan over pairs)
  int carry = 0;
  for (int base = 0; base < n; base += blockDim.x) {
    const int q = base + tid;
    int e = -1, flag = 0;
    if (q < n) {
      e = key_base + idx[q];
      flag = (s_first[e] == q) && !s_resident[e];
    }
    int tot;
    const int r = block_exclusive_scan(flag, s_scan, &tot) + carry;
    if (flag) s_miss_exp[r < kMaxS ? r : kMaxS - 1] = e;
    carry += tot;
  }
  if (tid == 0) s_nmiss = carry;

  // candidate victims: slots whose expert is not requested this step.  Their
  // order (empty slots first, then occupied by stamp, ties by index) becomes one
  // 64-bit key per slot; a candidate's rank is the number of keys below its own.
  if (tid == 0) s_ncand = 0;
  for (int s = tid; s < S; s += blockDim.x) {
    const int e = s_sexp[s];
    const bool cand = e < 0 || s_first[e] == n;
    s_key[s] = cand ? ((unsigned long long)(e >= 0) << 62) | (unsigned long long)s_stamp[s] : ~0ull;
  }
  __syncthreads();
  for (int s = tid; s < S; s += blockDim.x) {
    const unsigned long long ks = s_key[s];
    int rank = -1;
    if (ks != ~0ull) {
      rank = 0;
      int o = 0;
      for (; o + 8 <= S; o += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const unsigned long long ko = s_key[o + u];
          rank += (ko < ks) || (ko == ks && o + u < s);
        }
      }
      for (; o < S; ++o) {
        const unsigned long long ko = s_key[o];
        rank += (ko < ks) || (ko == ks && o < s);
      }
      atomicAdd(&s_ncand, 1);
    }
    s_cand_rank[s] = rank;
  }
  __syncthreads();
  const int n_miss = s_nmiss;
  if (s_ncand < n_miss) {
    if (tid == 0) {
      rec[0] = MOE_E_CAPACITY;
      rec[1] = n_miss;
      rec[2] = 0;
      rec[3] = 0;
      rec[4] = n_max;
    }
    return;
  }
  for (int s = tid; s < S; s += blockDim.x) {
    const int r = s_cand_rank[s];
    if (r >= 0 && r < n_miss) s_victim[r] = s;
  }
  __syncthreads();
  // install the misses
  for (int r = tid; r < n_miss; r += blockDim.x) {
    const int s = s_victim[r], e = s_miss_exp[r];
    const int old = s_sexp[s];
    if (old >= 0) s_eslot[old] = -1;
    s_sexp[s] = e;
    s_eslot[e] = s;
  }
  __syncthreads();
  // stamps: last access of each requested expert
  for (int q = tid; q < n; q += blockDim.x) {
    const int e = key_base + idx[q];
    if (s_last[e] == q) s_stamp[s_eslot[e]] = c0 + q + 1;
    pair_slot[q] = s_eslot[e];
  }
  // pair order: resident-at-start pairs first, then the others, each ascending
  int nh = 0;
  {
    int c = 0;
    for (int base = 0; base < n; base += blockDim.x) {
      const int q = base + tid;
      const int f = q < n ? s_resident[key_base + idx[q]] : 0;
      int tot;
      const int r = block_exclusive_scan(f, s_scan, &tot) + c;
      if (q < n && f) pair_order[r] = q;
      c += tot;
    }
    nh = c;
    c = 0;
    for (int base = 0; base < n; base += blockDim.x) {
      const int q = base + tid;
      const int f = q < n ? !s_resident[key_base + idx[q]] : 0;
      int tot;
      const int r = block_exclusive_scan(f, s_scan, &tot) + c;
      if (q < n && f) pair_order[nh + r] = q;
      c += tot;
    }
  }
  __syncthreads();
  // write back state and the miss record
  for (int e = tid; e < E; e += blockDim.x) expert_slot[e] = s_eslot[e];
  for (int s = tid; s < S; s += blockDim.x) {
    slot_expert[s] = s_sexp[s];
    slot_stamp[s] = s_stamp[s];
  }
  for (int r = tid; r < n_miss; r += blockDim.x) {
    rec[5 + r] = s_miss_exp[r] - key_base;
    rec[5 + n_max + r] = s_victim[r];
  }
  if (tid == 0) {
    *clock = c0 + n;
    rec[0] = MOE_OK;
    rec[1] = n_miss;
    rec[2] = nh;
    rec[3] = n - n_miss;
    rec[4] = n_max;
  }
}

// ------------------------------------------------------------ one-wave step
// The same step for at most 64 accesses on at most 64 slots, on one wavefront
// and without barriers: lane q holds access q and lane s slot s, and the
// cross-lane steps are ballots and lane reads.  It writes the same state,
// pair slots, pair order and miss record as k_lru_lookup.  FUSED: the accesses
// are the top-k of one token's logits (E <= 64*NE), selected here first.

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// E_route: experts of this lookup (keys key_base .. key_base + E_route - 1;
// the fused top-k runs over them).
template <int NE, bool FUSED>
__global__ __launch_bounds__(64) void k_lru_lookup_wave(
    int E_route, int S, int32_t* __restrict__ slot_expert, int32_t* __restrict__ expert_slot,
    int64_t* __restrict__ slot_stamp, int64_t* __restrict__ clock,
    const int32_t* __restrict__ idx_in, int n, int32_t* __restrict__ pair_slot,
    int32_t* __restrict__ pair_order, int32_t* __restrict__ rec, int n_max,
    const float* __restrict__ logits, int k, unsigned flags, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int key_base, float* __restrict__ logit_out) {
  const int E = E_route;
  const int lane = threadIdx.x;
  const uint64_t lt = (1ull << lane) - 1ull;
  // the state at the step start, requested before the top-k
  int es[NE];  // expert_slot[key_base + lane + 64 i]
#pragma unroll
  for (int i = 0; i < NE; ++i) es[i] = lane + 64 * i < E ? expert_slot[key_base + lane + 64 * i] : -1;
  const int sexp0 = lane < S ? slot_expert[lane] : -1;
  const long long stamp0 = lane < S ? slot_stamp[lane] : 0;
  const long long c0 = *clock;
  // expert of access q = lane
  int e = -1;
  if constexpr (FUSED) {
    __shared__ TopkScratch s_topk;
    float v[NE];
    wave_load_logits<NE>(logits, E, v);
    if (logit_out)  // a copy of the logits for a later prefetch step
#pragma unroll
      for (int i = 0; i < NE; ++i)
        if (lane + 64 * i < E) logit_out[lane + 64 * i] = v[i];
    float wt;
    wave_topk_regs<NE>(v, E, k, flags, e, wt, s_topk);
    if (lane < k) {
      topk_idx[lane] = e;
      topk_w[lane] = wt;
    }
  } else {
    if (lane < n) e = idx_in[lane];
  }
  const bool act = lane < n;
  if (!act) e = -1;
  // the expert's slot at the step start: expert_slot[e] sits in lane e % 64, register e / 64
  int slot0 = -1;
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int v = __shfl(es[i], e & 63);
    if (act && (e >> 6) == i) slot0 = v;
  }
  // first and last access of the access's expert
  int first = lane, last = lane;
  for (int p = 0; p < n; ++p) {
    const int ep = __builtin_amdgcn_readlane(e, p);
    if (act && ep == e) {
      first = min(first, p);
      last = max(last, p);
    }
  }
  const bool resident = slot0 >= 0;
  // distinct missed experts, ranked by first access
  const uint64_t miss_first = __ballot(act && first == lane && !resident);
  const int n_miss = __popcll(miss_first);
  const int miss_rank = __popcll(miss_first & lt);
  // slots requested this step: the start slots of the resident experts accessed
  uint64_t req = 0;
  for (uint64_t m = __ballot(act && resident); m; m &= m - 1)
    req |= 1ull << __builtin_amdgcn_readlane(slot0, __builtin_ctzll(m));
  // candidate victims (lane s = slot s): slots not requested, ordered by
  // (occupied, stamp), ties by index
  const bool cand = lane < S && !((req >> lane) & 1ull);
  uint64_t key = cand ? ((uint64_t)(sexp0 >= 0) << 62) | (uint64_t)stamp0 : ~0ull;
  const int n_cand = __popcll(__ballot(cand));
  if (n_cand < n_miss) {
    if (lane == 0) {
      rec[0] = MOE_E_CAPACITY;
      rec[1] = n_miss;
      rec[2] = 0;
      rec[3] = 0;
      rec[4] = n_max;
    }
    return;
  }
  // lane r < n_miss: victim slot of the r-th missed expert (the r-th smallest key),
  // that expert and the one it evicts
  int victim = -1, new_e = -1, old_e = -1;
  uint64_t mf = miss_first;
  for (int r = 0; r < n_miss; ++r) {
    uint64_t bk = key;
    int bs = lane;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint64_t ok = shfl_xor_u64(bk, off);
      const int os = __shfl_xor(bs, off);
      if (ok < bk || (ok == bk && os < bs)) {
        bk = ok;
        bs = os;
      }
    }
    const int vs = __builtin_amdgcn_readfirstlane(bs);
    const int er = __builtin_amdgcn_readlane(e, __builtin_ctzll(mf));
    mf &= mf - 1;
    const int eo = __builtin_amdgcn_readlane(sexp0, vs);
    if (lane == vs) key = ~0ull;
    if (lane == r) {
      victim = vs;
      new_e = er;
      old_e = eo;
    }
  }
  // slot state after the install (lane s = slot s)
  int sexp = sexp0;
  long long stamp = stamp0;
  for (int r = 0; r < n_miss; ++r)
    if (lane == __builtin_amdgcn_readlane(victim, r)) sexp = key_base + __builtin_amdgcn_readlane(new_e, r);
  // the access's slot after the install: a missed expert's victim, by the
  // miss rank of its first access
  const int rr = __shfl(miss_rank, first & 63);
  const int vslot = __shfl(victim, rr & 63);
  const int slot = act && !resident ? vslot : slot0;
  // the last access of each expert stamps its slot with clock0 + index + 1
  for (uint64_t m = __ballot(act && last == lane); m; m &= m - 1) {
    const int q = __builtin_ctzll(m);
    if (lane == __builtin_amdgcn_readlane(slot, q)) stamp = c0 + q + 1;
  }
  // pair order: resident-at-start accesses first, then the others, each ascending
  const uint64_t hm = __ballot(act && resident), mm = __ballot(act && !resident);
  const int nh = __popcll(hm);
  if (act) {
    pair_slot[lane] = slot;
    pair_order[resident ? __popcll(hm & lt) : nh + __popcll(mm & lt)] = lane;
  }
  if (lane < S) {
    slot_expert[lane] = sexp;
    slot_stamp[lane] = stamp;
  }
  if (lane < n_miss) {  // slot_expert holds keys; new_e is this lookup's expert
    if (old_e >= 0) expert_slot[old_e] = -1;
    expert_slot[key_base + new_e] = victim;
    rec[5 + lane] = new_e;
    rec[5 + n_max + lane] = victim;
  }
  if (lane == 0) {
    *clock = c0 + n;
    rec[0] = MOE_OK;
    rec[1] = n_miss;
    rec[2] = nh;
    rec[3] = n - n_miss;
    rec[4] = n_max;
  }
}

__global__ void k_lru_reset(int E, int S, int32_t* slot_expert, int32_t* expert_slot,
                            int64_t* slot_stamp, int64_t* clock) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < E) expert_slot[i] = -1;
  if (i < S) {
    slot_expert[i] = -1;
    slot_stamp[i] = 0;
  }
  if (i == 0) *clock = 0;
}

}  // namespace

hipError_t launch_lru_reset(const moe_lru& l, hipStream_t s) {
  const int n = l.E > l.S ? l.E : l.S;
  hipLaunchKernelGGL(k_lru_reset, dim3((n + 255) / 256), dim3(256), 0, s, l.E, l.S, l.slot_expert,
                     l.expert_slot, l.slot_stamp, l.clock);
  return hipGetLastError();
}

hipError_t launch_lru_lookup(const moe_lru& l, const int32_t* topk_idx, int n_pairs,
                             int32_t* pair_slot, int32_t* pair_order, int32_t* miss_rec, int n_max,
                             hipStream_t s) {
  const int E_route = l.E - l.key_base;  // the experts a lookup can name
  if (l.S <= 64 && n_pairs <= 64 && E_route <= 1024) {  // one wavefront
#define W(NE)                                                                                             \
  hipLaunchKernelGGL((k_lru_lookup_wave<NE, false>), dim3(1), dim3(64), 0, s, E_route, l.S, l.slot_expert, \
                     l.expert_slot, l.slot_stamp, l.clock, topk_idx, n_pairs, pair_slot, pair_order,       \
                     miss_rec, n_max, nullptr, 0, 0u, nullptr, nullptr, l.key_base, nullptr)
    if (E_route <= 64) W(1);
    else if (E_route <= 256) W(4);
    else W(16);
#undef W
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_lru_lookup<0>, dim3(1), dim3(kThreads), 0, s, l.E, l.S, l.slot_expert,
                     l.expert_slot, l.slot_stamp, l.clock, topk_idx, n_pairs, pair_slot, pair_order,
                     miss_rec, n_max, nullptr, 0, 0u, nullptr, nullptr, l.key_base, E_route, nullptr);
  return hipGetLastError();
}

hipError_t launch_lru_lookup_topk(const moe_lru& l, const float* logits, int E_route, int T, int k, unsigned flags,
                                  int32_t* topk_idx, float* topk_w, int32_t* pair_slot, int32_t* pair_order,
                                  int32_t* miss_rec, int n_max, hipStream_t s, float* logit_out) {
  if (T > kThreads / 64 || k > 16 || E_route > 1024) return hipErrorInvalidValue;
  if (T == 1 && l.S <= 64) {  // one wavefront
#define W(NE)                                                                                             \
  hipLaunchKernelGGL((k_lru_lookup_wave<NE, true>), dim3(1), dim3(64), 0, s, E_route, l.S, l.slot_expert,  \
                     l.expert_slot, l.slot_stamp, l.clock, nullptr, k, pair_slot, pair_order, miss_rec,    \
                     n_max, logits, k, flags, topk_idx, topk_w, l.key_base, logit_out)
    if (E_route <= 64) W(1);
    else if (E_route <= 256) W(4);
    else W(16);
#undef W
    return hipGetLastError();
  }
#define L(NV)                                                                                           \
  hipLaunchKernelGGL(k_lru_lookup<NV>, dim3(1), dim3(kThreads), 0, s, l.E, l.S, l.slot_expert,          \
                     l.expert_slot, l.slot_stamp, l.clock, nullptr, T * k, pair_slot, pair_order, miss_rec, \
                     n_max, logits, k, flags, topk_idx, topk_w, l.key_base, E_route, logit_out)
  if (E_route <= 64) L(1);
  else if (E_route <= 256) L(4);
  else L(16);
#undef L
  return hipGetLastError();
}

// ---------------------------------------------------------------- device fill
// The GPU cache fill without a host round trip: the miss record is read on the
// device and each missed blob is copied from the pinned host pool (addressed
// directly over PCIe) into its victim slot with 16-byte loads and stores, four
// in flight per thread.  Blob sizes are multiples of 256 bytes.
namespace {
__global__ __launch_bounds__(256) void k_cache_fill(const int32_t* __restrict__ rec,
                                                    const uint8_t* __restrict__ host,
                                                    uint8_t* __restrict__ slots, size_t expert_bytes,
                                                    size_t stride) {
  if (rec[0] != MOE_OK) return;
  const int n_max = rec[4], n_miss = min(rec[1], n_max);
  const size_t chunks = expert_bytes / 16, step = (size_t)gridDim.x * blockDim.x;
  for (int m = 0; m < n_miss; ++m) {
    const uint4* src = reinterpret_cast<const uint4*>(host + (size_t)rec[5 + m] * stride);
    uint4* dst = reinterpret_cast<uint4*>(slots + (size_t)rec[5 + n_max + m] * stride);
    size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; c + 3 * step < chunks; c += 4 * step) {
      const uint4 a = src[c], b = src[c + step], d = src[c + 2 * step], e = src[c + 3 * step];
      dst[c] = a;
      dst[c + step] = b;
      dst[c + 2 * step] = d;
      dst[c + 3 * step] = e;
    }
    for (; c < chunks; c += step) dst[c] = src[c];
  }
}
}  // namespace

hipError_t launch_cache_fill(const int32_t* miss_rec, const uint8_t* host_pool, uint8_t* slot_pool,
                             size_t expert_bytes, size_t stride, hipStream_t s, int n_groups) {
  hipLaunchKernelGGL(k_cache_fill, dim3(n_groups), dim3(256), 0, s, miss_rec, host_pool, slot_pool, expert_bytes,
                     stride);
  return hipGetLastError();
}

// ------------------------------------------------------------- elastic resize
// One layer's slot cache rebuilt for a new slot count (the elastic GPU expert
// cache of page "8GB 笔记本 39.3 tok/s、单卡跑 753B：FreeToken 把 frontier MoE
// 拉回本地", section "设计核心": resized at a scheduler safe point without
// reloading the host-resident expert pool).  Kept: the S1 latest-stamped
// residents (occupied slots carry distinct clock values; equal stamps, which
// only a hand-written state can hold, go to the lower slot first).  A kept expert below S1 keeps its slot; the others take the lowest
// free slots below S1 in ascending order of their old slot.  Stamps and the
// clock carry over; added slots start empty.
namespace {
constexpr int kResizeThreads = 1024;

// Exclusive count of `flag` over the threads before this one, and the total.
__device__ int block_count_excl(bool flag, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t b = __ballot(flag);
  __syncthreads();  // the previous call's readers of wsum are done
  if (lane == 0) wsum[wave] = __popcll(b);
  __syncthreads();
  int before = 0, tot = 0;
  for (int w = 0; w < kResizeThreads / 64; ++w) {
    if (w < wave) before += wsum[w];
    tot += wsum[w];
  }
  *total = tot;
  return before + __popcll(b & ((1ull << lane) - 1ull));
}

// One workgroup; thread i stands for old slot i and new slot i.  Every old
// value is read before any new value is written, so the new state may occupy
// the old state's memory.  plan: [0] copy count, then (old slot, new slot)
// pairs in ascending old slot: every kept slot, or with in_place only those
// whose slot changes.
__global__ __launch_bounds__(kResizeThreads) void k_lru_resize_plan(
    int E, int S0, const int32_t* se0, const int64_t* st0, const int64_t* clk0, int S1, int32_t* se1,
    int32_t* es1, int64_t* st1, int64_t* clk1, int in_place, int32_t* __restrict__ plan) {
  __shared__ int32_t o_e[kResizeThreads], n_e[kResizeThreads], n_es[kResizeThreads], free_slot[kResizeThreads];
  __shared__ int64_t o_st[kResizeThreads], n_st[kResizeThreads];
  __shared__ int wsum[kResizeThreads / 64];
  __shared__ int64_t s_clock;
  const int i = threadIdx.x;
  const int32_t e_i = i < S0 ? se0[i] : -1;
  const int64_t st_i = i < S0 ? st0[i] : 0;
  if (i == 0) s_clock = *clk0;
  o_e[i] = e_i;
  o_st[i] = st_i;
  __syncthreads();
  // rank: occupied slots used later than this one; equal stamps (never produced
  // by the lookup, possible in a state written by hand) rank the lower slot
  // first, so at most S1 experts are kept whatever the state holds
  int rank = 0;
  if (e_i >= 0)
    for (int j = 0; j < S0; ++j) rank += (o_e[j] >= 0 && (o_st[j] > st_i || (o_st[j] == st_i && j < i))) ? 1 : 0;
  const bool kept = e_i >= 0 && rank < S1;
  const bool stay = kept && i < S1, mover = kept && i >= S1;
  const bool is_free = i < S1 && !stay;  // new slot i, not held by a staying expert
  int n_free, n_mov, n_copy;
  const int fi = block_count_excl(is_free, wsum, &n_free);
  if (is_free) free_slot[fi] = i;
  const int mi = block_count_excl(mover, wsum, &n_mov);
  n_e[i] = -1;
  n_st[i] = 0;
  n_es[i] = -1;
  __syncthreads();
  const int dst = stay ? i : mover ? free_slot[mi] : -1;
  if (dst >= 0) {
    n_e[dst] = e_i;
    n_st[dst] = st_i;
    n_es[e_i] = dst;
  }
  const bool copy = in_place ? mover : kept;
  const int ci = block_count_excl(copy, wsum, &n_copy);  // its barriers also publish n_e / n_st / n_es
  if (copy) {
    plan[1 + 2 * ci] = i;
    plan[2 + 2 * ci] = dst;
  }
  if (i == 0) plan[0] = n_copy;
  if (i < S1) {
    se1[i] = n_e[i];
    st1[i] = n_st[i];
  }
  if (i < E) es1[i] = n_es[i];
  if (i == 0) *clk1 = s_clock;
}

// Blob copies of a plan: blockIdx.y picks the copy, the x blocks split the blob.
__global__ __launch_bounds__(256) void k_lru_resize_copy(const int32_t* __restrict__ plan,
                                                         const uint8_t* from, uint8_t* to,
                                                         size_t expert_bytes, size_t stride) {
  const int m = blockIdx.y;
  if (m >= plan[0]) return;
  const uint4* src = reinterpret_cast<const uint4*>(from + (size_t)plan[1 + 2 * m] * stride);
  uint4* dst = reinterpret_cast<uint4*>(to + (size_t)plan[2 + 2 * m] * stride);
  const size_t chunks = expert_bytes / 16, step = (size_t)gridDim.x * blockDim.x;
  for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks; c += step) dst[c] = src[c];
}
}  // namespace

hipError_t launch_lru_resize(const moe_lru& from, const uint8_t* from_pool, const moe_lru& to, uint8_t* to_pool,
                             size_t expert_bytes, size_t stride, int32_t* plan, hipStream_t s) {
  const int in_place = from_pool == to_pool ? 1 : 0;
  hipLaunchKernelGGL(k_lru_resize_plan, dim3(1), dim3(kResizeThreads), 0, s, from.E, from.S, from.slot_expert,
                     from.slot_stamp, from.clock, to.S, to.slot_expert, to.expert_slot, to.slot_stamp, to.clock,
                     in_place, plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_lru_resize_copy, dim3(16, to.S), dim3(256), 0, s, plan, from_pool, to_pool, expert_bytes,
                     stride);
  return hipGetLastError();
}
