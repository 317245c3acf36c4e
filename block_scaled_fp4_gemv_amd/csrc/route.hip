// Router, softmax, top-k and the token-by-expert permutation.
//
// The gate is a linear layer followed by a softmax over all experts; the top-K
// experts by probability are kept with their probabilities as mixing weights
// (page "FreeToken：753B大模型塞进单卡的本地部署硬件账该怎么算", section
// "混合专家架构（MoE）的天然稀疏性").  Selection compares fp32 logits (softmax
// is monotone) with ties going to the lower expert index.
//
// Logits of every expert are produced by the same instruction sequence (same
// summation order), so experts with identical router rows tie exactly.
#include "common.h"
#include "launch.h"
#include "topk.h"

namespace {

constexpr int kMaxE = 1024;

// ------------------------------------------------------- small-T router (decode)
// One wave per expert row: every lane issues all of its loads of R and x first
// (H/256 float4 of R per lane), then runs one fp32 FMA chain per token and a
// butterfly reduction.  Every expert uses the same sequence, so experts with
// identical router rows produce identical logits.
constexpr int kGemvMaxT = 4;
constexpr int kRouterSplitK = 4;  // large-T router GEMM: K split 4 ways, partials summed by k_topk
// Pairs per expert for the permutation are counted by the top-k kernel in
// kCountCopies copies ([copy][E], copy = top-k workgroup mod kCountCopies), so
// that few increments meet at one address; the permutation adds the copies.
constexpr int kCountCopies = 64;
static_assert(kCountCopies == 64, "the router GEMV zeroes one copy per lane of its 64-lane workgroup");

template <int NT, int NC>
__global__ __launch_bounds__(64) void k_router_logits(const uint16_t* __restrict__ x,
                                                      const float* __restrict__ R, int H, int E,
                                                      float* __restrict__ logits, int32_t* __restrict__ counts) {
  const int lane = threadIdx.x, e = blockIdx.x;
  if (counts) counts[lane * E + e] = 0;  // this expert's count copies (one per lane), for the top-k kernel
  const float4* r4 = reinterpret_cast<const float4*>(R + (size_t)e * H);
  float4 r[NC];
  uint2 xv[NT][NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) r[c] = r4[lane + 64 * c];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int c = 0; c < NC; ++c) xv[t][c] = reinterpret_cast<const uint2*>(x + (size_t)t * H)[lane + 64 * c];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      acc = fmaf(bf16_to_f32(xv[t][c].x & 0xffff), r[c].x, acc);
      acc = fmaf(bf16_to_f32(xv[t][c].x >> 16), r[c].y, acc);
      acc = fmaf(bf16_to_f32(xv[t][c].y & 0xffff), r[c].z, acc);
      acc = fmaf(bf16_to_f32(xv[t][c].y >> 16), r[c].w, acc);
    }
    const float s = wave_sum(acc);
    if (lane == 0) logits[(size_t)t * E + e] = s;
  }
}

template <int NT>
hipError_t router_logits_nt(const uint16_t* x, const float* R, int H, int E, float* logits, int32_t* counts,
                            hipStream_t s) {
#define L(NC) \
  case NC * 256: \
    hipLaunchKernelGGL((k_router_logits<NT, NC>), dim3(E), dim3(64), 0, s, x, R, H, E, logits, counts); break;
  switch (H) {
    L(1) L(2) L(4) L(8) L(16) L(24) L(32)
    default: return hipErrorInvalidValue;
  }
#undef L
  return hipGetLastError();
}

// ---------------------------------------------------------- large-T router GEMM
// logits[T][E] = x[T][H] . R[E][H]^T on bf16 MFMA with fp32 accuracy: an fp32
// router weight splits exactly into three bf16 terms (hi + mid + lo covers the
// 24-bit significand for every |w| in [2^-100, 3.3e38] and zero), x is already
// bf16, so each product is exact in fp32 and the three MFMA chains accumulate
// in fp32.  64x64 tile per workgroup (4 waves of 32x32), K staged through LDS
// 64 at a time with the next step's global loads issued before the current
// step's MFMAs.  The planes are written by a small kernel on every call, or
// once per weight set by moe_router_prepare.
typedef __bf16 rbf16x8_t __attribute__((ext_vector_type(8)));
typedef float rfloatx16_t __attribute__((ext_vector_type(16)));
constexpr int RBM = 64, RBN = 64, RBK = 64, RLD = RBK + 8, RTHREADS = 256;

__global__ __launch_bounds__(256) void k_router_split(const float* __restrict__ R, size_t n,
                                                      uint16_t* __restrict__ planes) {
  const size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  const float4 v = *reinterpret_cast<const float4*>(R + i);
  const float f[4] = {v.x, v.y, v.z, v.w};
  uint16_t hh[4], mm[4], ll[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    hh[q] = f32_to_bf16_rne(f[q]);
    const float r1 = f[q] - bf16_to_f32(hh[q]);
    mm[q] = f32_to_bf16_rne(r1);
    ll[q] = f32_to_bf16_rne(r1 - bf16_to_f32(mm[q]));
  }
  *reinterpret_cast<uint2*>(planes + i) = make_uint2(hh[0] | ((uint32_t)hh[1] << 16), hh[2] | ((uint32_t)hh[3] << 16));
  *reinterpret_cast<uint2*>(planes + n + i) = make_uint2(mm[0] | ((uint32_t)mm[1] << 16), mm[2] | ((uint32_t)mm[3] << 16));
  *reinterpret_cast<uint2*>(planes + 2 * n + i) = make_uint2(ll[0] | ((uint32_t)ll[1] << 16), ll[2] | ((uint32_t)ll[3] << 16));
}

__global__ __launch_bounds__(RTHREADS) void k_router_gemm(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ planes, int T, int H,
                                                           int E, float* __restrict__ logits,
                                                           int32_t* __restrict__ counts) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[RBM * RLD];
  __shared__ __attribute__((aligned(16))) uint16_t rs[3][RBN * RLD];
  if (counts) {  // zero the permutation's count copies for the top-k kernel, a slice per workgroup
    const int nb = gridDim.x * gridDim.y * gridDim.z;
    const int b = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int n = kCountCopies * E, per = (n + nb - 1) / nb;
    for (int j = b * per + (int)threadIdx.x; j < min(n, (b + 1) * per); j += RTHREADS) counts[j] = 0;
  }
  // Workgroups go to the 8 XCDs round-robin by linear index.  Tile (bx, by, bz)
  // is taken from the XCD-contiguous order instead: XCD c runs the c-th eighth
  // of the tiles in x-fastest order, so the column tiles of one (row tile, K
  // slice) run one after another on one XCD and fetch their x rows into its L2
  // once (in grid order they sat on different XCDs and each read x from HBM).
  int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  {
    const int n = gridDim.x * gridDim.y * gridDim.z;
    if (n % 8 == 0) {
      const int b = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
      const int l = (b & 7) * (n >> 3) + (b >> 3);
      bx = l % gridDim.x;
      by = (l / gridDim.x) % gridDim.y;
      bz = l / (gridDim.x * gridDim.y);
    }
  }
  // split K: workgroup z sums k in [z*H/Z, (z+1)*H/Z) into partial z of logits
  const int kz = H / gridDim.z, k0 = bz * kz;
  logits += (size_t)bz * T * E;
  const int tm = by * RBM, tn = bx * RBN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5;
  // staging: thread -> row tid/4, 16 columns at (tid%4)*16 of each of x and the 3 planes
  const int sr = tid >> 2, sc = (tid & 3) * 16;
  const bool xrow_ok = tm + sr < T, rrow_ok = tn + sr < E;
  const size_t plane = (size_t)E * H;
  const uint16_t* xp = x + (size_t)(xrow_ok ? tm + sr : 0) * H + sc;
  const uint16_t* rp = planes + (size_t)(rrow_ok ? tn + sr : 0) * H + sc;
  uint4 xa[2], ra[3][2];
  auto gload = [&](int kb) {
#pragma unroll
    for (int j = 0; j < 2; ++j) xa[j] = xrow_ok ? reinterpret_cast<const uint4*>(xp + kb)[j] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        ra[p][j] = rrow_ok ? reinterpret_cast<const uint4*>(rp + p * plane + kb)[j] : make_uint4(0, 0, 0, 0);
  };
  rfloatx16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  gload(k0);
  for (int kb = k0; kb < k0 + kz; kb += RBK) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      *reinterpret_cast<uint4*>(xs + sr * RLD + sc + 8 * j) = xa[j];
#pragma unroll
      for (int p = 0; p < 3; ++p) *reinterpret_cast<uint4*>(rs[p] + sr * RLD + sc + 8 * j) = ra[p][j];
    }
    __syncthreads();
    if (kb + RBK < k0 + kz) gload(kb + RBK);
#pragma unroll
    for (int i = 0; i < RBK / 16; ++i) {
      const rbf16x8_t a = *reinterpret_cast<const rbf16x8_t*>(xs + (32 * wm + (lane & 31)) * RLD + 16 * i + 8 * h);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const rbf16x8_t b = *reinterpret_cast<const rbf16x8_t*>(rs[p] + (32 * wn + (lane & 31)) * RLD + 16 * i + 8 * h);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
      }
    }
  }
  const int e = tn + 32 * wn + (lane & 31);
  if (e < E) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int t = tm + 32 * wm + 8 * (v >> 2) + 4 * h + (v & 3);
      if (t < T) logits[(size_t)t * E + e] = acc[v];
    }
  }
}

// logits holds nsplit partial sums [nsplit][T][E]; they are added in order.
// With counts != NULL (kCountCopies copies of [E], zeroed by the router
// kernel) every selected pair adds 1 to its expert's count in copy
// blockIdx.x % kCountCopies (integer atomics: the sums do not depend on order).
template <int NV>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              unsigned flags, int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_w, int nsplit, int32_t* __restrict__ counts) {
  __shared__ TopkScratch scr[4];
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= T) return;
  float v[NV];
  wave_load_logits<NV>(logits + (size_t)t * E, E, v);
  for (int z = 1; z < nsplit; ++z) {
    float p[NV];
    wave_load_logits<NV>(logits + ((size_t)z * T + t) * E, E, p);
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] += p[i];
  }
  int idx;
  float w;
  wave_topk_regs<NV>(v, E, k, flags, idx, w, scr[threadIdx.x >> 6]);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = idx;
    topk_w[(size_t)t * k + lane] = w;
    if (counts) atomicAdd(&counts[(blockIdx.x % kCountCopies) * E + idx], 1);
  }
}

hipError_t topk_impl(const float* logits, int T, int E, int k, unsigned flags, int32_t* idx,
                     float* w, int nsplit, int32_t* counts, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  if (E <= 64)
    hipLaunchKernelGGL(k_topk<1>, grid, dim3(256), 0, s, logits, T, E, k, flags, idx, w, nsplit, counts);
  else if (E <= 256)
    hipLaunchKernelGGL(k_topk<4>, grid, dim3(256), 0, s, logits, T, E, k, flags, idx, w, nsplit, counts);
  else
    hipLaunchKernelGGL(k_topk<16>, grid, dim3(256), 0, s, logits, T, E, k, flags, idx, w, nsplit, counts);
  return hipGetLastError();
}

// ------------------------------------------------------------ permutation
// Stable counting sort of the pairs by expert in one kernel: workgroup e
// reads the pairs per expert (counted by the top-k kernel), takes its
// expert's offset from their exclusive scan, then writes the pairs of expert e
// in ascending pair order.  Wave w owns the w-th sixteenth of the pairs
// and walks it 64 pairs at a time (one coalesced load per lane); a ballot
// ranks the matches inside a 64-pair chunk and the waves' match counts, scanned
// once, order the sixteenths.  With tile_rows > 0 it also writes the grouped
// path's tile list (one entry per tile_rows pairs of each expert, in expert
// order).
constexpr int kPermThreads = 1024, kPermWaves = kPermThreads / 64, kPermUnroll = 16;

// Exclusive scan over the workgroup's threads' values; *total = the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o);
    if (lane >= o) incl += n;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kPermWaves; ++w) {
    base += w < wave ? wsum[w] : 0;
    tot += wsum[w];
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// ONE: every wave's share fits one batch of kPermUnroll chunks (n <=
// kPermWaves * 64 * kPermUnroll); its pair experts stay in registers between
// the passes.
template <bool ONE>
__global__ __launch_bounds__(kPermThreads) void k_perm_experts(const int32_t* __restrict__ idx,
                                                              const int32_t* __restrict__ counts, int n, int E,
                                                              int32_t* __restrict__ pair_perm,
                                                              int32_t* __restrict__ expert_off, int tile_rows,
                                                              int32_t* __restrict__ tile_e,
                                                              int32_t* __restrict__ tile_m0,
                                                              int32_t* __restrict__ n_tiles) {
  __shared__ int hist[kMaxE];
  __shared__ int wsum[kPermWaves];
  __shared__ int s_wcnt[kPermWaves];
  __shared__ int s_off, s_tbase;
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int j = tid; j < E; j += kPermThreads) {
    int c = 0;
    for (int r = 0; r < kCountCopies; ++r) c += counts[r * E + j];
    hist[j] = c;
  }
  // this wave's share [b0, b1), in chunks of 64 pairs: this wave's matches of e
  const int qn = (n + kPermWaves - 1) / kPermWaves, b0 = min(n, wave * qn), b1 = min(n, b0 + qn);
  int wcnt = 0;
  int v[kPermUnroll];
  for (int c = b0; c < b1; c += 64 * kPermUnroll) {
#pragma unroll
    for (int u = 0; u < kPermUnroll; ++u) {
      const int q = c + 64 * u + lane;
      v[u] = q < b1 ? idx[q] : -1;
    }
#pragma unroll
    for (int u = 0; u < kPermUnroll; ++u) wcnt += __popcll(__ballot(v[u] == e));
    if (ONE) break;
  }
  if (lane == 0) s_wcnt[wave] = wcnt;
  __syncthreads();
  // offsets of expert e (pairs and tiles): sums over the experts before it, the
  // experts split into contiguous runs of ceil(E / kPermThreads) per thread
  const int epr = (E + kPermThreads - 1) / kPermThreads, j0 = tid * epr, j1 = min(E, j0 + epr);
  int cnt = 0, tl = 0;
  for (int j = j0; j < j1; ++j) {
    cnt += hist[j];
    if (tile_rows > 0) tl += (hist[j] + tile_rows - 1) / tile_rows;
  }
  int total, tiles_total;
  const int cnt_before = block_excl_scan(cnt, wsum, &total);
  const int tl_before = block_excl_scan(tl, wsum, &tiles_total);
  if (e >= j0 && e < j1) {  // the thread whose run holds e adds the experts of its run before e
    int o = cnt_before, tb = tl_before;
    for (int j = j0; j < e; ++j) {
      o += hist[j];
      if (tile_rows > 0) tb += (hist[j] + tile_rows - 1) / tile_rows;
    }
    s_off = o;
    s_tbase = tb;
  }
  __syncthreads();
  const int off = s_off, ce = hist[e];
  int w = off;
  for (int i = 0; i < wave; ++i) w += s_wcnt[i];
  for (int c = b0; c < b1; c += 64 * kPermUnroll) {
    if (!ONE) {
#pragma unroll
      for (int u = 0; u < kPermUnroll; ++u) {
        const int q = c + 64 * u + lane;
        v[u] = q < b1 ? idx[q] : -1;
      }
    }
#pragma unroll
    for (int u = 0; u < kPermUnroll; ++u) {
      const uint64_t m = __ballot(v[u] == e);
      if (v[u] == e) pair_perm[w + __popcll(m & lt)] = c + 64 * u + lane;
      w += __popcll(m);
    }
    if (ONE) break;
  }
  if (tid == 0) {
    expert_off[e] = off;
    if (e == E - 1) expert_off[E] = off + ce;
    if (tile_rows > 0 && e == 0) *n_tiles = tiles_total;
  }
  if (tile_rows > 0) {
    const int nt = (ce + tile_rows - 1) / tile_rows, tb = s_tbase;
    for (int j = tid; j < nt; j += kPermThreads) {
      tile_e[tb + j] = e;
      tile_m0[tb + j] = j * tile_rows;
    }
  }
}

__global__ void k_fill_zero(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, const float* R, int T, int H, int E, float* logits,
                                hipStream_t s, int32_t* counts) {
  if (T <= kGemvMaxT) {
    switch (T) {
      case 1: return router_logits_nt<1>(x, R, H, E, logits, counts, s);
      case 2: return router_logits_nt<2>(x, R, H, E, logits, counts, s);
      case 3: return router_logits_nt<3>(x, R, H, E, logits, counts, s);
      default: return router_logits_nt<4>(x, R, H, E, logits, counts, s);
    }
  }
  return hipErrorInvalidValue;  // large T needs the split planes (launch_router_gemm)
}

hipError_t launch_router_split(const float* R, int E, int H, uint16_t* planes, hipStream_t s) {
  const size_t n = (size_t)E * H;
  hipLaunchKernelGGL(k_router_split, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s, R, n, planes);
  return hipGetLastError();
}

hipError_t launch_router_gemm(const uint16_t* x, const float* R, int T, int H, int E, float* logits,
                              uint16_t* planes, hipStream_t s, const uint16_t* planes_ready, int32_t* counts) {
  if (!planes_ready) {
    hipError_t e = launch_router_split(R, E, H, planes, s);
    if (e != hipSuccess) return e;
  }
  dim3 grid((E + RBN - 1) / RBN, (T + RBM - 1) / RBM, kRouterSplitK);
  hipLaunchKernelGGL(k_router_gemm, grid, dim3(RTHREADS), 0, s, x, planes_ready ? planes_ready : planes, T, H, E,
                     logits, counts);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, unsigned flags, int32_t* idx,
                       float* w, hipStream_t s, int nsplit, int32_t* counts) {
  return topk_impl(logits, T, E, k, flags, idx, w, nsplit, counts, s);
}

static size_t logits_bytes(int T, int E) {
  return align256((size_t)T * E * 4 * (T > kGemvMaxT ? kRouterSplitK : 1));
}

size_t route_ws_bytes(int T, int H, int E, int k) {
  (void)k;
  const size_t planes = T > kGemvMaxT ? align256((size_t)3 * E * H * 2) : 0;
  return logits_bytes(T, E) + align256((size_t)kCountCopies * E * 4) + planes;
}

void route_ws_carve(RouteArgs& a, void* ws) {
  uint8_t* p = static_cast<uint8_t*>(ws);
  a.logits = reinterpret_cast<float*>(p);
  p += logits_bytes(a.T, a.E);
  a.counts = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)kCountCopies * a.E * 4);
  a.planes = a.T > kGemvMaxT ? reinterpret_cast<uint16_t*>(p) : nullptr;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) {
    if (a.expert_off)
      hipLaunchKernelGGL(k_fill_zero, dim3((a.E + 1 + 255) / 256), dim3(256), 0, s, a.expert_off, a.E + 1);
    return hipGetLastError();
  }
  // the per-expert pair counts of the permutation: zeroed by the router
  // kernel, counted by the top-k kernel
  int32_t* counts = a.pair_perm ? a.counts : nullptr;
  hipError_t e = a.T <= kGemvMaxT
                     ? launch_router_logits(a.x, a.router, a.T, a.H, a.E, a.logits, s, counts)
                     : launch_router_gemm(a.x, a.router, a.T, a.H, a.E, a.logits, a.planes, s, a.planes_ready, counts);
  if (e != hipSuccess) return e;
  e = launch_topk(a.logits, a.T, a.E, a.k, a.flags, a.topk_idx, a.topk_w, s,
                  a.T <= kGemvMaxT ? 1 : kRouterSplitK, counts);
  if (e != hipSuccess || !a.pair_perm) return e;
  const int n = a.T * a.k;
  int32_t* te = a.tile_rows > 0 ? a.tiles : nullptr;
  if (n <= kPermWaves * 64 * kPermUnroll)
    hipLaunchKernelGGL(k_perm_experts<true>, dim3(a.E), dim3(kPermThreads), 0, s, a.topk_idx, counts, n, a.E, a.pair_perm,
                       a.expert_off, a.tile_rows, te, te ? te + a.max_tiles : nullptr,
                       te ? te + 2 * a.max_tiles : nullptr);
  else
    hipLaunchKernelGGL(k_perm_experts<false>, dim3(a.E), dim3(kPermThreads), 0, s, a.topk_idx, counts, n, a.E, a.pair_perm,
                       a.expert_off, a.tile_rows, te, te ? te + a.max_tiles : nullptr,
                       te ? te + 2 * a.max_tiles : nullptr);
  return hipGetLastError();
}
