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
//  * hits are judged against the state at the start of the step;
//  * each distinct missed expert (in order of first appearance) takes a
//    victim among slots whose expert is not requested this step: empty slots
//    by ascending index first, then occupied slots by ascending stamp;
//  * access q (pair order) advances the clock and stamps its slot, so a slot's
//    final stamp is clock0 + (last access index of its expert) + 1.
#include "common.h"
#include "launch.h"

namespace {

constexpr int kThreads = 1024;
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

__global__ __launch_bounds__(kThreads) void k_lru_lookup(
    int E, int S, int32_t* __restrict__ slot_expert, int32_t* __restrict__ expert_slot,
    int64_t* __restrict__ slot_stamp, int64_t* __restrict__ clock,
    const int32_t* __restrict__ idx, int n, int32_t* __restrict__ pair_slot,
    int32_t* __restrict__ pair_order, int32_t* __restrict__ rec, int n_max) {
  __shared__ int s_first[kMaxE];   // first access index of each expert (n = none)
  __shared__ int s_last[kMaxE];    // last access index
  __shared__ int s_eslot[kMaxE];   // expert -> slot (updated in place)
  __shared__ int s_resident[kMaxE];// resident at step start
  __shared__ int s_sexp[kMaxS];    // slot -> expert
  __shared__ long long s_stamp[kMaxS];
  __shared__ int s_cand_rank[kMaxS];
  __shared__ int s_victim[kMaxS];
  __shared__ int s_miss_exp[kMaxS];
  __shared__ int s_scan[kThreads / 64];
  __shared__ int s_nmiss, s_ncand;
  const int tid = threadIdx.x;

  for (int e = tid; e < E; e += blockDim.x) {
    s_first[e] = n;
    s_last[e] = -1;
    const int sl = expert_slot[e];
    s_eslot[e] = sl;
    s_resident[e] = sl >= 0;
  }
  for (int s = tid; s < S; s += blockDim.x) {
    s_sexp[s] = slot_expert[s];
    s_stamp[s] = slot_stamp[s];
  }
  __syncthreads();
  for (int q = tid; q < n; q += blockDim.x) {
    const int e = idx[q];
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
      e = idx[q];
      flag = (s_first[e] == q) && !s_resident[e];
    }
    int tot;
    const int r = block_exclusive_scan(flag, s_scan, &tot) + carry;
    if (flag) s_miss_exp[r < kMaxS ? r : kMaxS - 1] = e;
    carry += tot;
  }
  if (tid == 0) s_nmiss = carry;

  // candidate victims: slots whose expert is not requested this step
  for (int s = tid; s < S; s += blockDim.x) {
    const int e = s_sexp[s];
    const bool cand = e < 0 || s_first[e] == n;
    int rank = -1;
    if (cand) {
      rank = 0;
      const int ke = e < 0 ? 0 : 1;
      const long long ks = s_stamp[s];
      for (int o = 0; o < S; ++o) {
        const int eo = s_sexp[o];
        if (!(eo < 0 || s_first[eo] == n)) continue;
        const int koe = eo < 0 ? 0 : 1;
        const long long kos = s_stamp[o];
        if (koe < ke || (koe == ke && (kos < ks || (kos == ks && o < s)))) ++rank;
      }
    }
    s_cand_rank[s] = rank;
  }
  __syncthreads();
  int ncand_local = 0;
  for (int s = tid; s < S; s += blockDim.x) ncand_local += s_cand_rank[s] >= 0;
  {
    int tot;
    block_exclusive_scan(ncand_local, s_scan, &tot);
    if (tid == 0) s_ncand = tot;
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
  const long long c0 = *clock;
  // stamps: last access of each requested expert
  for (int q = tid; q < n; q += blockDim.x) {
    const int e = idx[q];
    if (s_last[e] == q) s_stamp[s_eslot[e]] = c0 + q + 1;
    pair_slot[q] = s_eslot[e];
  }
  // pair order: resident-at-start pairs first, then the others, each ascending
  int nh = 0;
  {
    int c = 0;
    for (int base = 0; base < n; base += blockDim.x) {
      const int q = base + tid;
      const int f = q < n ? s_resident[idx[q]] : 0;
      int tot;
      const int r = block_exclusive_scan(f, s_scan, &tot) + c;
      if (q < n && f) pair_order[r] = q;
      c += tot;
    }
    nh = c;
    c = 0;
    for (int base = 0; base < n; base += blockDim.x) {
      const int q = base + tid;
      const int f = q < n ? !s_resident[idx[q]] : 0;
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
    rec[5 + r] = s_miss_exp[r];
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
  hipLaunchKernelGGL(k_lru_lookup, dim3(1), dim3(kThreads), 0, s, l.E, l.S, l.slot_expert,
                     l.expert_slot, l.slot_stamp, l.clock, topk_idx, n_pairs, pair_slot, pair_order,
                     miss_rec, n_max);
  return hipGetLastError();
}
