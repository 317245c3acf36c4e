// Batch-1 (decode-shaped) expert FFN: weight-streaming GEMV on block-scaled
// weights, dequantized in registers.
//
// Expert FFN h = bf16(silu(G x) * (U x)), y = D h  (each expert an independent
// FFN: page "FreeToken：753B大模型塞进单卡的本地部署硬件账该怎么算", section
// "混合专家架构（MoE）的天然稀疏性"; dequantization at compute time: page
// "8GB显存跑35B MoE模型：FreeToken引擎本地部署实战", §2.1).
//
// Mapping onto a 64-lane wavefront: a matrix row of K elements is C 16-byte
// chunks (C = K/32 for FP4, K/16 for FP8).  A wave owns RB consecutive rows
// (RB*C chunks) and lane l loads chunks l, l+64, ... of that run: one fully
// coalesced 1 KiB dwordx4 load per "slot".  Because C divides 64 or 64 divides
// C, each lane always meets the same chunk columns, so its slice of the input
// vector stays in registers for every row.  Partial dot products use the gfx950
// FP4/FP8 -> bf16 conversions and v_dot2_f32_bf16 (fp32 accumulate), and rows
// are finished with cross-lane reductions.
#include "common.h"
#include "launch.h"
#include "topk.h"

namespace {

template <int FMT, int C, int RB>
struct Gemv {
  static constexpr bool kFP8 = FMT == MOE_FMT_FP8_E4M3;
  static constexpr int NS = RB * C / 64;            // 16-byte slots per lane
  static constexpr int XS = C >= 64 ? C / 64 : 1;   // x slices per lane
  static constexpr int XW = kFP8 ? 8 : 16;          // bf16 pairs per x slice
  static constexpr int EPC = kFP8 ? 16 : 32;        // elements per chunk
  static constexpr int RPS = C >= 64 ? 1 : 64 / C;  // rows per slot
  static constexpr int NOUT = C >= 64 ? RB : NS;    // per-lane results
  static_assert(NS >= 1 && (RB * C) % 64 == 0, "bad row block");
  static_assert(C % 64 == 0 || 64 % C == 0, "bad chunk count");

  uint4 code[NS];
  uint32_t sc[NS];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ codes,
                                       const uint8_t* __restrict__ scales, int row0, int lane) {
    const size_t g0 = (size_t)row0 * C + lane;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const size_t g = g0 + 64 * s;
      code[s] = reinterpret_cast<const uint4*>(codes)[g];
      if constexpr (FMT == MOE_FMT_NVFP4)
        sc[s] = reinterpret_cast<const uint16_t*>(scales)[g];
      else if constexpr (FMT == MOE_FMT_MXFP4)
        sc[s] = scales[g];
      else
        sc[s] = reinterpret_cast<const uint32_t*>(scales)[g >> 3];
    }
  }

  static __device__ __forceinline__ void load_x(const uint16_t* __restrict__ xrow, int lane,
                                                uint32_t (&xs)[XS][XW]) {
#pragma unroll
    for (int i = 0; i < XS; ++i) {
      const int col = C >= 64 ? 64 * i + lane : lane % C;
      const uint4* p = reinterpret_cast<const uint4*>(xrow + (size_t)col * EPC);
#pragma unroll
      for (int j = 0; j < XW / 4; ++j) {
        uint4 v = p[j];
        xs[i][4 * j + 0] = v.x;
        xs[i][4 * j + 1] = v.y;
        xs[i][4 * j + 2] = v.z;
        xs[i][4 * j + 3] = v.w;
      }
    }
  }

  __device__ __forceinline__ void compute(const uint32_t (&xs)[XS][XW], float (&out)[NOUT]) const {
    float p[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int xi = C >= 64 ? s % XS : 0;
      if constexpr (FMT == MOE_FMT_NVFP4) {
        const float slo = e4m3_byte0_to_f32(sc[s]), shi = e4m3_byte0_to_f32(sc[s] >> 8);
        p[s] = chunk_dot_nvfp4(code[s], slo, shi, xs[xi]);
      } else if constexpr (FMT == MOE_FMT_MXFP4) {
        p[s] = chunk_dot_mxfp4(code[s], e8m0_to_f32(sc[s]), xs[xi], 0.0f);
      } else {
        p[s] = __uint_as_float(sc[s]) * chunk_dot_fp8(code[s], xs[xi], 0.0f);
      }
    }
    if constexpr (C >= 64) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < XS; ++i) a += p[r * XS + i];
        out[r] = wave_sum(a);
      }
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) out[s] = group_sum<C>(p[s]);
    }
  }

  // Row (relative to row0) of result i in this lane, and whether this lane writes it.
  static __device__ __forceinline__ int row_of(int i, int lane) {
    return C >= 64 ? i : i * RPS + lane / C;
  }
  static __device__ __forceinline__ bool owner(int i, int lane) {
    return C >= 64 ? lane == (i & 63) : (lane % C) == 0;
  }
};

// Rows per wave for a matrix of C chunks per row: about four 16-byte slots per lane.
constexpr int rows_per_wave(int C) { return C >= 256 ? 1 : 256 / C; }
// Down + combine: at most 8 rows per workgroup so that a 2048-row layer spreads
// over >= 256 workgroups (one wave per routed pair in each).
constexpr int rows_per_wave_down(int C) {
  return (64 / C > (rows_per_wave(C) < 8 ? rows_per_wave(C) : 8)) ? 64 / C
                                                                    : (rows_per_wave(C) < 8 ? rows_per_wave(C) : 8);
}

template <int FMT, int C, int RB, int WPB>
__global__ __launch_bounds__(WPB * 64) void k_gateup_gemv(
    const uint8_t* __restrict__ pool, size_t stride, BlobLayout L, int H, int F,
    const uint16_t* __restrict__ x, int k, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ pair_slot, const int32_t* __restrict__ pair_subset,
    uint16_t* __restrict__ hbuf) {
  using G = Gemv<FMT, C, RB>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = pair_subset ? pair_subset[blockIdx.y] : (int)blockIdx.y;
  const int slot = pair_slot ? pair_slot[q] : topk_idx[q];
  const uint8_t* blob = pool + (size_t)slot * stride;
  const int row0 = (blockIdx.x * WPB + wave) * RB;
  G g, u;
  g.load(blob + L.cg, blob + L.sg, row0, lane);
  u.load(blob + L.cu, blob + L.su, row0, lane);
  uint32_t xs[G::XS][G::XW];
  G::load_x(x + (size_t)(q / k) * H, lane, xs);
  float og[G::NOUT], ou[G::NOUT];
  g.compute(xs, og);
  u.compute(xs, ou);
  float tg = 1.0f, tu = 1.0f;
  if constexpr (FMT == MOE_FMT_NVFP4) {
    const float* tau = reinterpret_cast<const float*>(blob + L.tau);
    tg = tau[0];
    tu = tau[1];
  }
#pragma unroll
  for (int i = 0; i < G::NOUT; ++i) {
    if (G::owner(i, lane)) {
      const float gv = og[i] * tg, uv = ou[i] * tu;
      hbuf[(size_t)q * F + row0 + G::row_of(i, lane)] = f32_to_bf16_rne(silu_f32(gv) * uv);
    }
  }
}

// Gate/up for a decode layer that starts from the router logits: wave 0 of
// every workgroup runs the softmax + top-k of its token (identical in every
// workgroup), which saves a dependent kernel between routing and the experts.
// The token's first pair, column-block 0, writes topk_idx / topk_w.
template <int FMT, int C, int RB, int WPB, int NV>
__global__ __launch_bounds__(WPB * 64) void k_gateup_gemv_topk(
    const uint8_t* __restrict__ pool, size_t stride, BlobLayout L, int H, int F, int E, int k,
    unsigned flags, const uint16_t* __restrict__ x, const float* __restrict__ logits,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, uint16_t* __restrict__ hbuf) {
  using G = Gemv<FMT, C, RB>;
  __shared__ int s_expert;
  __shared__ TopkScratch s_topk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = blockIdx.y, t = q / k, j = q % k;
  uint32_t xs[G::XS][G::XW];
  G::load_x(x + (size_t)t * H, lane, xs);
  if (wave == 0) {
    float v[NV];
    wave_load_logits<NV>(logits + (size_t)t * E, E, v);
    int idx;
    float w;
    wave_topk_regs<NV>(v, E, k, flags, idx, w, s_topk);
    if (lane == j) s_expert = idx;
    if (blockIdx.x == 0 && j == 0 && lane < k) {
      topk_idx[(size_t)t * k + lane] = idx;
      topk_w[(size_t)t * k + lane] = w;
    }
  }
  __syncthreads();
  const uint8_t* blob = pool + (size_t)s_expert * stride;
  const int row0 = (blockIdx.x * WPB + wave) * RB;
  G g, u;
  g.load(blob + L.cg, blob + L.sg, row0, lane);
  u.load(blob + L.cu, blob + L.su, row0, lane);
  float og[G::NOUT], ou[G::NOUT];
  g.compute(xs, og);
  u.compute(xs, ou);
  float tg = 1.0f, tu = 1.0f;
  if constexpr (FMT == MOE_FMT_NVFP4) {
    const float* tau = reinterpret_cast<const float*>(blob + L.tau);
    tg = tau[0];
    tu = tau[1];
  }
#pragma unroll
  for (int i = 0; i < G::NOUT; ++i) {
    if (G::owner(i, lane)) {
      const float gv = og[i] * tg, uv = ou[i] * tu;
      hbuf[(size_t)q * F + row0 + G::row_of(i, lane)] = f32_to_bf16_rne(silu_f32(gv) * uv);
    }
  }
}

template <int FMT, int C, int RB, int WPB>
__global__ __launch_bounds__(WPB * 64) void k_down_gemv(
    const uint8_t* __restrict__ pool, size_t stride, BlobLayout L, int H, int F, int k,
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ pair_slot,
    const int32_t* __restrict__ pair_subset, const uint16_t* __restrict__ hbuf,
    float* __restrict__ y) {
  using G = Gemv<FMT, C, RB>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = pair_subset ? pair_subset[blockIdx.y] : (int)blockIdx.y;
  const int slot = pair_slot ? pair_slot[q] : topk_idx[q];
  const uint8_t* blob = pool + (size_t)slot * stride;
  const int row0 = (blockIdx.x * WPB + wave) * RB;
  G d;
  d.load(blob + L.cd, blob + L.sd, row0, lane);
  uint32_t xs[G::XS][G::XW];
  G::load_x(hbuf + (size_t)q * F, lane, xs);
  float o[G::NOUT];
  d.compute(xs, o);
  float td = 1.0f;
  if constexpr (FMT == MOE_FMT_NVFP4) td = reinterpret_cast<const float*>(blob + L.tau)[2];
#pragma unroll
  for (int i = 0; i < G::NOUT; ++i)
    if (G::owner(i, lane)) y[(size_t)q * H + row0 + G::row_of(i, lane)] = o[i] * td;
}

// Down GEMV for all k pairs of one token with the gate-weighted combine fused:
// wave j computes y[t*k+j] on RB rows, then out[t] = bf16(sum_j w_j * y_j).
template <int FMT, int C, int RB>
__global__ __launch_bounds__(1024) void k_down_combine_gemv(
    const uint8_t* __restrict__ pool, size_t stride, BlobLayout L, int H, int F, int k,
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ pair_slot,
    const uint16_t* __restrict__ hbuf, const float* __restrict__ topk_w, float* __restrict__ y,
    uint16_t* __restrict__ out) {
  using G = Gemv<FMT, C, RB>;
  __shared__ float ys[16][RB];
  const int lane = threadIdx.x & 63, j = threadIdx.x >> 6;
  const int t = blockIdx.y, q = t * k + j;
  const int slot = pair_slot ? pair_slot[q] : topk_idx[q];
  const uint8_t* blob = pool + (size_t)slot * stride;
  const int row0 = blockIdx.x * RB;
  G d;
  d.load(blob + L.cd, blob + L.sd, row0, lane);
  uint32_t xs[G::XS][G::XW];
  G::load_x(hbuf + (size_t)q * F, lane, xs);
  float o[G::NOUT];
  d.compute(xs, o);
  float td = 1.0f;
  if constexpr (FMT == MOE_FMT_NVFP4) td = reinterpret_cast<const float*>(blob + L.tau)[2];
#pragma unroll
  for (int i = 0; i < G::NOUT; ++i) {
    if (G::owner(i, lane)) {
      const int r = G::row_of(i, lane);
      const float v = o[i] * td;
      ys[j][r] = v;
      if (y) y[(size_t)q * H + row0 + r] = v;
    }
  }
  __syncthreads();
  if (threadIdx.x < RB) {
    const float* w = topk_w + (size_t)t * k;
    float acc = 0.0f;
    for (int jj = 0; jj < k; ++jj) acc = fmaf(w[jj], ys[jj][threadIdx.x], acc);
    out[(size_t)t * H + row0 + threadIdx.x] = f32_to_bf16_rne(acc);
  }
}



template <int FMT, int C>
hipError_t launch_gateup_c(const FfnArgs& a, hipStream_t s) {
  constexpr int RB = rows_per_wave(C), WPB = 4;
  if (a.F % (RB * WPB)) return hipErrorInvalidValue;
  dim3 grid(a.F / (RB * WPB), a.n_pairs);
  hipLaunchKernelGGL((k_gateup_gemv<FMT, C, RB, WPB>), grid, dim3(WPB * 64), 0, s, a.pool, a.stride,
                     a.L, a.H, a.F, a.x, a.k, a.topk_idx, a.pair_slot, a.pair_subset, a.hbuf);
  return hipGetLastError();
}

template <int FMT, int C>
hipError_t launch_down_c(const FfnArgs& a, hipStream_t s) {
  constexpr int RB = rows_per_wave(C);
  constexpr int RBC = rows_per_wave_down(C);
  if (a.out) {
    if (a.H % RBC || a.k > 16) return hipErrorInvalidValue;
    dim3 grid(a.H / RBC, a.T);
    hipLaunchKernelGGL((k_down_combine_gemv<FMT, C, RBC>), grid, dim3(64 * a.k), 0, s, a.pool,
                       a.stride, a.L, a.H, a.F, a.k, a.topk_idx, a.pair_slot, a.hbuf, a.topk_w,
                       a.y, a.out);
  } else {
    constexpr int WPB = 4;
    if (a.H % (RB * WPB)) return hipErrorInvalidValue;
    dim3 grid(a.H / (RB * WPB), a.n_pairs);
    hipLaunchKernelGGL((k_down_gemv<FMT, C, RB, WPB>), grid, dim3(WPB * 64), 0, s, a.pool, a.stride,
                       a.L, a.H, a.F, a.k, a.topk_idx, a.pair_slot, a.pair_subset, a.hbuf, a.y);
  }
  return hipGetLastError();
}

template <int FMT, int C>
hipError_t launch_gateup_topk_c(const FfnArgs& a, const float* logits, unsigned flags, int32_t* idx,
                                float* w, hipStream_t s) {
  constexpr int RB = rows_per_wave(C), WPB = 4;
  if (a.F % (RB * WPB)) return hipErrorInvalidValue;
  dim3 grid(a.F / (RB * WPB), a.T * a.k);
  if (a.E <= 256)
    hipLaunchKernelGGL((k_gateup_gemv_topk<FMT, C, RB, WPB, 4>), grid, dim3(WPB * 64), 0, s, a.pool,
                       a.stride, a.L, a.H, a.F, a.E, a.k, flags, a.x, logits, idx, w, a.hbuf);
  else
    hipLaunchKernelGGL((k_gateup_gemv_topk<FMT, C, RB, WPB, 16>), grid, dim3(WPB * 64), 0, s, a.pool,
                       a.stride, a.L, a.H, a.F, a.E, a.k, flags, a.x, logits, idx, w, a.hbuf);
  return hipGetLastError();
}

// Chunks per row for the supported K values: FP4 K/32, FP8 K/16.
#define MOE_FOR_FP4_C(X) X(8) X(16) X(32) X(64) X(128) X(192) X(256)
#define MOE_FOR_FP8_C(X) X(16) X(32) X(64) X(128) X(256) X(384) X(512)

template <int FMT>
hipError_t gateup_fmt(const FfnArgs& a, int C, hipStream_t s) {
#define CASE(c) \
  case c: return launch_gateup_c<FMT, c>(a, s);
  if constexpr (FMT == MOE_FMT_FP8_E4M3) {
    switch (C) { MOE_FOR_FP8_C(CASE) }
  } else {
    switch (C) { MOE_FOR_FP4_C(CASE) }
  }
#undef CASE
  return hipErrorInvalidValue;
}

template <int FMT>
hipError_t gateup_topk_fmt(const FfnArgs& a, int C, const float* logits, unsigned flags, int32_t* idx,
                           float* w, hipStream_t s) {
#define CASE(c) \
  case c: return launch_gateup_topk_c<FMT, c>(a, logits, flags, idx, w, s);
  if constexpr (FMT == MOE_FMT_FP8_E4M3) {
    switch (C) { MOE_FOR_FP8_C(CASE) }
  } else {
    switch (C) { MOE_FOR_FP4_C(CASE) }
  }
#undef CASE
  return hipErrorInvalidValue;
}

template <int FMT>
hipError_t down_fmt(const FfnArgs& a, int C, hipStream_t s) {
#define CASE(c) \
  case c: return launch_down_c<FMT, c>(a, s);
  if constexpr (FMT == MOE_FMT_FP8_E4M3) {
    switch (C) { MOE_FOR_FP8_C(CASE) }
  } else {
    switch (C) { MOE_FOR_FP4_C(CASE) }
  }
#undef CASE
  return hipErrorInvalidValue;
}

int chunks_per_row(int fmt, int K) { return fmt == MOE_FMT_FP8_E4M3 ? K / 16 : K / 32; }

}  // namespace

hipError_t launch_ffn_gemv(const FfnArgs& a, hipStream_t s) {
  if (a.n_pairs == 0) return hipSuccess;
  const int Cg = chunks_per_row(a.fmt, a.H), Cd = chunks_per_row(a.fmt, a.F);
  hipError_t e;
  switch (a.fmt) {
    case MOE_FMT_NVFP4: e = gateup_fmt<MOE_FMT_NVFP4>(a, Cg, s); break;
    case MOE_FMT_MXFP4: e = gateup_fmt<MOE_FMT_MXFP4>(a, Cg, s); break;
    default: e = gateup_fmt<MOE_FMT_FP8_E4M3>(a, Cg, s); break;
  }
  if (e != hipSuccess) return e;
  switch (a.fmt) {
    case MOE_FMT_NVFP4: return down_fmt<MOE_FMT_NVFP4>(a, Cd, s);
    case MOE_FMT_MXFP4: return down_fmt<MOE_FMT_MXFP4>(a, Cd, s);
    default: return down_fmt<MOE_FMT_FP8_E4M3>(a, Cd, s);
  }
}

hipError_t launch_decode_layer(const FfnArgs& a0, const float* logits, unsigned route_flags,
                               int32_t* topk_idx, float* topk_w, hipStream_t s) {
  if (a0.T == 0) return hipSuccess;
  const int Cg = chunks_per_row(a0.fmt, a0.H), Cd = chunks_per_row(a0.fmt, a0.F);
  hipError_t e;
  switch (a0.fmt) {
    case MOE_FMT_NVFP4: e = gateup_topk_fmt<MOE_FMT_NVFP4>(a0, Cg, logits, route_flags, topk_idx, topk_w, s); break;
    case MOE_FMT_MXFP4: e = gateup_topk_fmt<MOE_FMT_MXFP4>(a0, Cg, logits, route_flags, topk_idx, topk_w, s); break;
    default: e = gateup_topk_fmt<MOE_FMT_FP8_E4M3>(a0, Cg, logits, route_flags, topk_idx, topk_w, s); break;
  }
  if (e != hipSuccess) return e;
  FfnArgs a = a0;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.pair_slot = nullptr;
  a.pair_subset = nullptr;
  a.n_pairs = a.T * a.k;
  switch (a.fmt) {
    case MOE_FMT_NVFP4: return down_fmt<MOE_FMT_NVFP4>(a, Cd, s);
    case MOE_FMT_MXFP4: return down_fmt<MOE_FMT_MXFP4>(a, Cd, s);
    default: return down_fmt<MOE_FMT_FP8_E4M3>(a, Cd, s);
  }
}
