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

constexpr int kPermChunk = 256;  // pairs per permutation block
constexpr int kMaxE = 1024;

// ------------------------------------------------------- small-T router (decode)
// One wave per expert row: every lane issues all of its loads of R and x first
// (H/256 float4 of R per lane), then runs one fp32 FMA chain per token and a
// butterfly reduction.  Every expert uses the same sequence, so experts with
// identical router rows produce identical logits.
constexpr int kGemvMaxT = 4;
constexpr int kRouterSplitK = 4;  // large-T router GEMM: K split 4 ways, partials summed by k_topk

template <int NT, int NC>
__global__ __launch_bounds__(64) void k_router_logits(const uint16_t* __restrict__ x,
                                                      const float* __restrict__ R, int H, int E,
                                                      float* __restrict__ logits) {
  const int lane = threadIdx.x, e = blockIdx.x;
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
hipError_t router_logits_nt(const uint16_t* x, const float* R, int H, int E, float* logits, hipStream_t s) {
#define L(NC) \
  case NC * 256: hipLaunchKernelGGL((k_router_logits<NT, NC>), dim3(E), dim3(64), 0, s, x, R, H, E, logits); break;
  switch (H) {
    L(1) L(2) L(4) L(8) L(16) L(24) L(32)
    default: return hipErrorInvalidValue;
  }
#undef L
  return hipGetLastError();
}

// ---------------------------------------------------------- large-T router GEMM
// logits[T][E] = x[T][H] . R[E][H]^T on bf16 MFMA with fp32 accuracy: every fp32
// router weight splits exactly into three bf16 terms (hi + mid + lo covers the
// 24-bit significand; a small kernel writes the three planes once per call), x
// is already bf16, so each product is exact in fp32 and the three MFMA chains
// accumulate in fp32.  64x64 tile per workgroup (4 waves of 32x32), K staged
// through LDS 64 at a time with the next step's global loads issued before the
// current step's MFMAs.
typedef __bf16 rbf16x8_t __attribute__((ext_vector_type(8)));
typedef float rfloatx16_t __attribute__((ext_vector_type(16)));
constexpr int RBM = 64, RBN = 64, RBK = 64, RLD = RBK + 8;

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

__global__ __launch_bounds__(256) void k_router_gemm(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ planes, int T, int H,
                                                     int E, float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[RBM * RLD];
  __shared__ __attribute__((aligned(16))) uint16_t rs[3][RBN * RLD];
  // split K: workgroup z sums k in [z*H/Z, (z+1)*H/Z) into partial z of logits
  const int kz = H / gridDim.z, k0 = blockIdx.z * kz;
  logits += (size_t)blockIdx.z * T * E;
  const int tm = blockIdx.y * RBM, tn = blockIdx.x * RBN;
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
template <int NV>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              unsigned flags, int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_w, int nsplit) {
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
  }
}

hipError_t topk_impl(const float* logits, int T, int E, int k, unsigned flags, int32_t* idx,
                     float* w, int nsplit, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  if (E <= 64) hipLaunchKernelGGL(k_topk<1>, grid, dim3(256), 0, s, logits, T, E, k, flags, idx, w, nsplit);
  else if (E <= 256) hipLaunchKernelGGL(k_topk<4>, grid, dim3(256), 0, s, logits, T, E, k, flags, idx, w, nsplit);
  else hipLaunchKernelGGL(k_topk<16>, grid, dim3(256), 0, s, logits, T, E, k, flags, idx, w, nsplit);
  return hipGetLastError();
}

// ------------------------------------------------------------ permutation
// Stable counting sort of the pairs by expert, in three kernels (no device-wide
// fences): per-chunk expert counts, one block turning them into expert_off and
// per-chunk base offsets, then a scatter that ranks each pair among the earlier
// pairs of its chunk with the same expert.
__global__ __launch_bounds__(256) void k_perm_count(const int32_t* __restrict__ idx, int n, int E,
                                                    int32_t* __restrict__ chunk_cnt) {
  __shared__ int cnt[kMaxE];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int q = blockIdx.x * kPermChunk + threadIdx.x;
  if (q < n) atomicAdd(&cnt[idx[q]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) chunk_cnt[(size_t)blockIdx.x * E + e] = cnt[e];
}

// One workgroup: expert e's column of chunk counts is split over tpe = 1024/E
// threads (contiguous chunk ranges, up to 16 counts kept in registers), the
// per-thread sums are combined in LDS, an exclusive scan over the expert totals
// gives expert_off, and each thread rewrites its counts as running offsets.
__global__ __launch_bounds__(1024) void k_perm_scan(int nchunk, int E, int32_t* __restrict__ chunk_cnt,
                                                    int32_t* __restrict__ expert_off) {
  __shared__ int s_part[1024];
  __shared__ int s_tot[kMaxE];
  __shared__ int s_off[kMaxE];
  __shared__ int wsum[16];
  const int tid = threadIdx.x, tpe = blockDim.x / E;
  const int e = tid / tpe, sub = tid % tpe;
  const bool valid = e < E;
  const int per = (nchunk + tpe - 1) / tpe, c0 = sub * per, c1 = min(nchunk, c0 + per);
  int v[16];
  int sum = 0;
  if (valid) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = c0 + i < c1 ? chunk_cnt[(size_t)(c0 + i) * E + e] : 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += v[i];
    for (int c = c0 + 16; c < c1; ++c) sum += chunk_cnt[(size_t)c * E + e];
  }
  s_part[tid] = sum;
  __syncthreads();
  int before = 0;  // this thread's offset inside its expert
  if (valid) {
    for (int j = 0; j < sub; ++j) before += s_part[e * tpe + j];
    if (sub == tpe - 1) s_tot[e] = before + sum;
  }
  __syncthreads();
  // exclusive scan of the expert totals (experts on threads 0..E-1)
  const int lane = tid & 63, wave = tid >> 6;
  const int t = tid < E ? s_tot[tid] : 0;
  int incl = t;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o);
    if (lane >= o) incl += n;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  if (tid < E) {
    s_off[tid] = base + incl - t;
    expert_off[tid] = base + incl - t;
    if (tid == E - 1) expert_off[E] = base + incl;
  }
  __syncthreads();
  if (valid) {
    int run = s_off[e] + before;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (c0 + i < c1) {
        chunk_cnt[(size_t)(c0 + i) * E + e] = run;
        run += v[i];
      }
    for (int c = c0 + 16; c < c1; ++c) {
      const size_t i = (size_t)c * E + e;
      const int x = chunk_cnt[i];
      chunk_cnt[i] = run;
      run += x;
    }
  }
}

__global__ __launch_bounds__(256) void k_perm_scatter(const int32_t* __restrict__ idx, int n, int E,
                                                      const int32_t* __restrict__ chunk_base,
                                                      int32_t* __restrict__ pair_perm) {
  __shared__ int wcnt[4][kMaxE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * E; i += blockDim.x) wcnt[i / E][i % E] = 0;
  __syncthreads();
  const int q = blockIdx.x * kPermChunk + threadIdx.x;
  const bool valid = q < n;
  const int e = valid ? idx[q] : 0;
  uint64_t same = __ballot(valid);
  for (int b = 0; (1 << b) < E; ++b) {
    const uint64_t m = __ballot(valid && ((e >> b) & 1));
    same &= ((e >> b) & 1) ? m : ~m;
  }
  const int rank = __popcll(same & ((1ull << lane) - 1ull));
  if (valid && rank == 0) wcnt[wave][e] = __popcll(same);
  __syncthreads();
  if (valid) {
    int base = chunk_base[(size_t)blockIdx.x * E + e] + rank;
    for (int w = 0; w < wave; ++w) base += wcnt[w][e];
    pair_perm[base] = q;
  }
}

__global__ void k_fill_zero(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, const float* R, int T, int H, int E, float* logits,
                                hipStream_t s) {
  if (T <= kGemvMaxT) {
    switch (T) {
      case 1: return router_logits_nt<1>(x, R, H, E, logits, s);
      case 2: return router_logits_nt<2>(x, R, H, E, logits, s);
      case 3: return router_logits_nt<3>(x, R, H, E, logits, s);
      default: return router_logits_nt<4>(x, R, H, E, logits, s);
    }
  }
  return hipErrorInvalidValue;  // large T needs the split planes (launch_router_gemm)
}

hipError_t launch_router_gemm(const uint16_t* x, const float* R, int T, int H, int E, float* logits,
                              uint16_t* planes, hipStream_t s) {
  const size_t n = (size_t)E * H;
  hipLaunchKernelGGL(k_router_split, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s, R, n, planes);
  dim3 grid((E + RBN - 1) / RBN, (T + RBM - 1) / RBM, kRouterSplitK);
  hipLaunchKernelGGL(k_router_gemm, grid, dim3(256), 0, s, x, planes, T, H, E, logits);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, unsigned flags, int32_t* idx,
                       float* w, hipStream_t s, int nsplit) {
  return topk_impl(logits, T, E, k, flags, idx, w, nsplit, s);
}

static size_t logits_bytes(int T, int E) {
  return align256((size_t)T * E * 4 * (T > kGemvMaxT ? kRouterSplitK : 1));
}

size_t route_ws_bytes(int T, int H, int E, int k) {
  const size_t n = (size_t)T * k;
  const size_t nchunk = (n + kPermChunk - 1) / kPermChunk;
  const size_t planes = T > kGemvMaxT ? align256((size_t)3 * E * H * 2) : 0;
  return logits_bytes(T, E) + align256(nchunk * E * 4 + 4) + planes;
}

void route_ws_carve(RouteArgs& a, void* ws) {
  uint8_t* p = static_cast<uint8_t*>(ws);
  a.logits = reinterpret_cast<float*>(p);
  p += logits_bytes(a.T, a.E);
  a.chunk_cnt = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)((a.T * a.k + kPermChunk - 1) / kPermChunk) * a.E * 4 + 4);
  a.planes = a.T > kGemvMaxT ? reinterpret_cast<uint16_t*>(p) : nullptr;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) {
    if (a.expert_off)
      hipLaunchKernelGGL(k_fill_zero, dim3((a.E + 1 + 255) / 256), dim3(256), 0, s, a.expert_off, a.E + 1);
    return hipGetLastError();
  }
  hipError_t e = a.T <= kGemvMaxT ? launch_router_logits(a.x, a.router, a.T, a.H, a.E, a.logits, s)
                                  : launch_router_gemm(a.x, a.router, a.T, a.H, a.E, a.logits, a.planes, s);
  if (e != hipSuccess) return e;
  e = launch_topk(a.logits, a.T, a.E, a.k, a.flags, a.topk_idx, a.topk_w, s,
                  a.T <= kGemvMaxT ? 1 : kRouterSplitK);
  if (e != hipSuccess || !a.pair_perm) return e;
  const int n = a.T * a.k;
  const int nchunk = (n + kPermChunk - 1) / kPermChunk;
  hipLaunchKernelGGL(k_perm_count, dim3(nchunk), dim3(kPermChunk), 0, s, a.topk_idx, n, a.E,
                     a.chunk_cnt);
  hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, s, nchunk, a.E, a.chunk_cnt, a.expert_off);
  hipLaunchKernelGGL(k_perm_scatter, dim3(nchunk), dim3(kPermChunk), 0, s, a.topk_idx, n, a.E,
                     a.chunk_cnt, a.pair_perm);
  return hipGetLastError();
}
