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
// logits[T][E] = x[T][H] . R[E][H]^T in fp32; 64x64 tile per block, 4x4 per thread,
// K staged through LDS 32 at a time; each output is one sequential fp32 FMA chain.
constexpr int RBM = 64, RBN = 64, RBK = 32;

__global__ __launch_bounds__(256) void k_router_gemm(const uint16_t* __restrict__ x,
                                                     const float* __restrict__ R, int T, int H, int E,
                                                     float* __restrict__ logits) {
  __shared__ float xs[RBK][RBM + 4];
  __shared__ float rs[RBK][RBN + 4];
  const int tm = blockIdx.y * RBM, tn = blockIdx.x * RBN;
  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < H; k0 += RBK) {
    // x tile: 64 rows x 32 k bf16 -> 8 elements per thread
    {
      const int r = tid / 4, c = (tid % 4) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (tm + r < T) v = *reinterpret_cast<const uint4*>(x + (size_t)(tm + r) * H + k0 + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xs[c + 2 * i][r] = bf16_to_f32(w[i] & 0xffff);
        xs[c + 2 * i + 1][r] = bf16_to_f32(w[i] >> 16);
      }
    }
    // R tile: 64 rows x 32 k fp32 -> 8 per thread
    {
      const int r = tid / 4, c = (tid % 4) * 8;
      float4 a = make_float4(0, 0, 0, 0), b = a;
      if (tn + r < E) {
        const float4* p = reinterpret_cast<const float4*>(R + (size_t)(tn + r) * H + k0 + c);
        a = p[0];
        b = p[1];
      }
      rs[c + 0][r] = a.x; rs[c + 1][r] = a.y; rs[c + 2][r] = a.z; rs[c + 3][r] = a.w;
      rs[c + 4][r] = b.x; rs[c + 5][r] = b.y; rs[c + 6][r] = b.z; rs[c + 7][r] = b.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < RBK; ++kk) {
      float xa[4], rb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = xs[kk][ty * 4 + i];
#pragma unroll
      for (int i = 0; i < 4; ++i) rb[i] = rs[kk][tx * 4 + i];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xa[i], rb[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = tm + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tn + tx * 4 + j;
      if (e < E) logits[(size_t)t * E + e] = acc[i][j];
    }
  }
}

template <int NV>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              unsigned flags, int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_w) {
  __shared__ uint32_t lists[4][32];
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= T) return;
  float v[NV];
  wave_load_logits<NV>(logits + (size_t)t * E, E, v);
  int idx;
  float w;
  wave_topk_regs<NV>(v, E, k, flags, idx, w, lists[threadIdx.x >> 6]);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = idx;
    topk_w[(size_t)t * k + lane] = w;
  }
}

hipError_t topk_impl(const float* logits, int T, int E, int k, unsigned flags, int32_t* idx,
                     float* w, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  if (E <= 64) hipLaunchKernelGGL(k_topk<1>, grid, dim3(256), 0, s, logits, T, E, k, flags, idx, w);
  else if (E <= 256) hipLaunchKernelGGL(k_topk<4>, grid, dim3(256), 0, s, logits, T, E, k, flags, idx, w);
  else hipLaunchKernelGGL(k_topk<16>, grid, dim3(256), 0, s, logits, T, E, k, flags, idx, w);
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

__global__ __launch_bounds__(1024) void k_perm_scan(int nchunk, int E, int32_t* __restrict__ chunk_cnt,
                                                    int32_t* __restrict__ expert_off) {
  __shared__ int tot[kMaxE];
  __shared__ int wsum[16];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  int s = 0;
  if (e < E)
    for (int c = 0; c < nchunk; ++c) s += chunk_cnt[(size_t)c * E + e];
  // exclusive scan of the per-expert totals over the block
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  const int excl = base + incl - s;
  if (e < E) {
    expert_off[e] = excl;
    tot[e] = excl;
    int run = excl;
    for (int c = 0; c < nchunk; ++c) {
      const size_t i = (size_t)c * E + e;
      const int v = chunk_cnt[i];
      chunk_cnt[i] = run;
      run += v;
    }
    if (e == E - 1) expert_off[E] = run;
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
  dim3 grid((E + RBN - 1) / RBN, (T + RBM - 1) / RBM);
  hipLaunchKernelGGL(k_router_gemm, grid, dim3(256), 0, s, x, R, T, H, E, logits);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, unsigned flags, int32_t* idx,
                       float* w, hipStream_t s) {
  return topk_impl(logits, T, E, k, flags, idx, w, s);
}

size_t route_ws_bytes(int T, int E, int k) {
  const size_t n = (size_t)T * k;
  const size_t nchunk = (n + kPermChunk - 1) / kPermChunk;
  return align256((size_t)T * E * 4) + align256(nchunk * E * 4 + 4);
}

void route_ws_carve(RouteArgs& a, void* ws) {
  uint8_t* p = static_cast<uint8_t*>(ws);
  a.logits = reinterpret_cast<float*>(p);
  p += align256((size_t)a.T * a.E * 4);
  a.chunk_cnt = reinterpret_cast<int32_t*>(p);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) {
    if (a.expert_off)
      hipLaunchKernelGGL(k_fill_zero, dim3((a.E + 1 + 255) / 256), dim3(256), 0, s, a.expert_off, a.E + 1);
    return hipGetLastError();
  }
  hipError_t e = launch_router_logits(a.x, a.router, a.T, a.H, a.E, a.logits, s);
  if (e != hipSuccess) return e;
  e = launch_topk(a.logits, a.T, a.E, a.k, a.flags, a.topk_idx, a.topk_w, s);
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
