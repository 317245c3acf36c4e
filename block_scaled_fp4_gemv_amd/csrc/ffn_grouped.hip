// Expert-grouped expert FFN for many tokens (prefill shape) on bf16 MFMA.
//
// Each expert is an independent FFN evaluated on the tokens routed to it (page
// "FreeToken：753B大模型塞进单卡的本地部署硬件账该怎么算", section
// "混合专家架构（MoE）的天然稀疏性"); its low-precision weights are dequantized
// at compute time (page "8GB显存跑35B MoE模型：FreeToken引擎本地部署实战", §2.1),
// here in registers, straight into MFMA operands.
//
// Pairs arrive sorted by expert (pair_perm / expert_off).  A device-built tile
// list holds one (expert, first row) entry per 64 rows of each expert.  A
// workgroup (4 waves) owns one tile x 128 output columns per matrix: wave w
// takes columns [32w, 32w+32) for all 64 rows (two 32x32 MFMA subtiles), so each
// dequantized weight fragment feeds two MFMAs.
//
// K runs in steps of 128.  Lane (n = l%32, h = l/32) loads the contiguous 64
// weight elements [64h, 64h+64) of row n for the step (FP4: 32 bytes, FP8: 64
// bytes) and MFMA i (0..7) takes elements 64h + 8i .. +7 from every lane; the
// activation operand is read from LDS with the same k order, so the products
// pair up exactly as in the plain k order.
//   MXFP4: e2m1 -> bf16 with the E8M0 scale folded into the conversion (exact).
//   NVFP4: e2m1 -> fp32, times the E4M3 block scale (exact in bf16: <= 6
//          significant bits), high halves packed to bf16; tau in the epilogue.
//   FP8  : e4m3 -> bf16 exactly; the fp32 scale of the 128-element block is
//          applied to each step's partial sums.
// Gate/up writes h = bf16(silu(g) * u) in expert-sorted row order; down
// writes y (fp32) to the rows of the original pairs.
#include "common.h"
#include "launch.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 64, BNW = 32, NWAVE = 4, BN = BNW * NWAVE, BK = 128;
constexpr int LDA = BK + 8;  // bf16 elements per LDS row (16-byte pad)

__global__ __launch_bounds__(1024) void k_build_tiles(const int32_t* __restrict__ expert_off, int E,
                                                      int32_t* __restrict__ tile_e,
                                                      int32_t* __restrict__ tile_m0,
                                                      int32_t* __restrict__ n_tiles) {
  __shared__ int wsum[16];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  const int ne = e < E ? expert_off[e + 1] - expert_off[e] : 0;
  const int c = (ne + BM - 1) / BM;
  int incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) base += wsum[w];
    tot += wsum[w];
  }
  base += incl - c;
  for (int j = 0; j < c; ++j) {
    tile_e[base + j] = e;
    tile_m0[base + j] = j * BM;
  }
  if (e == 0) *n_tiles = tot;
}

template <int FMT>
struct WFrag {
  static constexpr bool kFP8 = FMT == MOE_FMT_FP8_E4M3;
  static constexpr int NQ = kFP8 ? 4 : 2;  // 16-byte code loads per lane per step
  uint4 c[NQ];
  uint32_t s;  // NVFP4: 4 scale bytes; MXFP4: 2 bytes; FP8: fp32 bits

  __device__ __forceinline__ void load(const uint8_t* __restrict__ codes,
                                       const uint8_t* __restrict__ scales, int K, int n, int h,
                                       int kb) {
    const size_t rowb = kFP8 ? (size_t)n * K : (size_t)n * (K / 2);
    const int off = kFP8 ? kb + 64 * h : (kb + 64 * h) / 2;
    const uint4* p = reinterpret_cast<const uint4*>(codes + rowb + off);
#pragma unroll
    for (int i = 0; i < NQ; ++i) c[i] = p[i];
    if constexpr (FMT == MOE_FMT_NVFP4)
      s = *reinterpret_cast<const uint32_t*>(scales + (size_t)n * (K / 16) + (kb + 64 * h) / 16);
    else if constexpr (FMT == MOE_FMT_MXFP4)
      s = *reinterpret_cast<const uint16_t*>(scales + (size_t)n * (K / 32) + (kb + 64 * h) / 32);
    else
      s = reinterpret_cast<const uint32_t*>(scales)[(size_t)n * (K / 128) + kb / 128];
  }

  __device__ __forceinline__ uint32_t word(int w) const {  // 4-byte word w of the lane's codes
    const uint4& q = c[w >> 2];
    switch (w & 3) {
      case 0: return q.x;
      case 1: return q.y;
      case 2: return q.z;
      default: return q.w;
    }
  }

  // bf16 operand (8 elements) for MFMA i.
  __device__ __forceinline__ bf16x8_t operand(int i) const {
    uint32_t o[4];
    if constexpr (FMT == MOE_FMT_MXFP4) {
      const float sc = e8m0_to_f32((s >> (8 * (i >> 2))) & 0xff);
      const uint32_t w = word(i);
      o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
      o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
      o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
      o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
    } else if constexpr (FMT == MOE_FMT_NVFP4) {
      const float sc = __builtin_amdgcn_cvt_f32_fp8((int)(s >> (8 * (i >> 1))), 0);
      const uint32_t w = word(i);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float2 f;
        if (b == 0) f = __builtin_bit_cast(float2, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0));
        else if (b == 1) f = __builtin_bit_cast(float2, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1));
        else if (b == 2) f = __builtin_bit_cast(float2, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2));
        else f = __builtin_bit_cast(float2, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3));
        const uint32_t lo = __float_as_uint(f.x * sc), hi = __float_as_uint(f.y * sc);
        o[b] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);  // exact: low halves are zero
      }
    } else {
      const uint32_t w0 = word(2 * i), w1 = word(2 * i + 1);
      o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
      o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
      o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
      o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
    }
    return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
  }

  __device__ __forceinline__ float step_scale() const {  // FP8 block scale
    return __uint_as_float(s);
  }
};

// A fragment for MFMA i: row m of the LDS tile, elements 64h + 8i .. +7.
__device__ __forceinline__ bf16x8_t a_operand(const uint16_t* As, int row, int h, int i) {
  return *reinterpret_cast<const bf16x8_t*>(As + row * LDA + 64 * h + 8 * i);
}

// NMAT = 2: gate/up with SwiGLU into hout (expert-sorted rows, width N).
// NMAT = 1: down into y rows of the original pairs.
template <int FMT, int NMAT>
__global__ __launch_bounds__(256) void k_grouped(
    const uint8_t* __restrict__ pool, size_t stride, BlobLayout L, int K, int N, int k_top,
    const uint16_t* __restrict__ a_src, int a_by_token, const int32_t* __restrict__ pair_perm,
    const int32_t* __restrict__ expert_off, const int32_t* __restrict__ tile_e,
    const int32_t* __restrict__ tile_m0, const int32_t* __restrict__ n_tiles, int n_col_tiles,
    uint16_t* __restrict__ hout, float* __restrict__ yout) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDA];
  // Workgroups are handed to the 8 XCDs round-robin by index; within each run of
  // 8 * n_col_tiles indices, the column tiles of one row tile share an XCD (and
  // its L2 copy of the gathered activation rows).
  const int grp = blockIdx.x / (8 * n_col_tiles), r8 = blockIdx.x % (8 * n_col_tiles);
  const int tile = grp * 8 + (r8 & 7), ct = r8 >> 3;
  if (tile >= *n_tiles) return;
  const int e = tile_e[tile], m0 = tile_m0[tile];
  const int row_base = expert_off[e] + m0;
  const int rows = min(BM, expert_off[e + 1] - row_base);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_lane = ct * BN + BNW * wave + (lane & 31), h = lane >> 5;
  const uint8_t* blob = pool + (size_t)e * stride;
  const uint8_t* codes0 = blob + (NMAT == 2 ? L.cg : L.cd);
  const uint8_t* scales0 = blob + (NMAT == 2 ? L.sg : L.sd);

  // A rows handled by this thread for LDS staging: row r = tid / 4, 32 columns each
  const int ar = tid >> 2, ac = (tid & 3) * 32;
  const uint16_t* arow = nullptr;
  if (ar < rows) {
    const int p = row_base + ar;
    arow = a_by_token ? a_src + (size_t)(pair_perm[p] / k_top) * K : a_src + (size_t)p * K;
  }

  floatx16_t acc[NMAT][2];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[m][s][v] = 0.0f;

  // software pipeline: the next step's weights and activations are loaded into
  // registers while the current step runs its MFMAs
  WFrag<FMT> wf[NMAT];
  uint4 av[4];
  auto gload = [&](int kb) {
    wf[0].load(codes0, scales0, K, n_lane, h, kb);
    if constexpr (NMAT == 2) wf[1].load(blob + L.cu, blob + L.su, K, n_lane, h, kb);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      av[j] = arow ? reinterpret_cast<const uint4*>(arow + kb + ac)[j] : make_uint4(0, 0, 0, 0);
  };
  gload(0);
  for (int kb = 0; kb < K; kb += BK) {
    __syncthreads();  // previous step's LDS reads are done
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(As + ar * LDA + ac + 8 * j) = av[j];
    __syncthreads();
    WFrag<FMT> cur[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) cur[m] = wf[m];
    if (kb + BK < K) gload(kb + BK);
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      floatx16_t part[2];
      const bool fp8 = FMT == MOE_FMT_FP8_E4M3;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int v = 0; v < 16; ++v) part[s][v] = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8_t b = cur[m].operand(i);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8_t a = a_operand(As, 32 * s + (lane & 31), h, i);
          if (fp8)
            part[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, part[s], 0, 0, 0);
          else
            acc[m][s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m][s], 0, 0, 0);
        }
      }
      if (fp8) {
        const float sg = cur[m].step_scale();
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[m][s][v] = fmaf(sg, part[s][v], acc[m][s][v]);
      }
    }
  }

  // epilogue: lane holds column n_lane, rows 32s + 8(v/4) + 4h + v%4
  const float* tau = reinterpret_cast<const float*>(blob + L.tau);
  if constexpr (NMAT == 2) {
    const float tg = FMT == MOE_FMT_NVFP4 ? tau[0] : 1.0f, tu = FMT == MOE_FMT_NVFP4 ? tau[1] : 1.0f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * s + 8 * (v >> 2) + 4 * h + (v & 3);
        if (r < rows) {
          const float g = acc[0][s][v] * tg, u = acc[1][s][v] * tu;
          hout[(size_t)(row_base + r) * N + n_lane] = f32_to_bf16_rne(silu_f32(g) * u);
        }
      }
  } else {
    const float td = FMT == MOE_FMT_NVFP4 ? tau[2] : 1.0f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * s + 8 * (v >> 2) + 4 * h + (v & 3);
        if (r < rows) yout[(size_t)pair_perm[row_base + r] * N + n_lane] = acc[0][s][v] * td;
      }
  }
}

template <int FMT>
hipError_t grouped_fmt(const FfnArgs& a, int32_t* tiles, hipStream_t s) {
  const int n_pairs = a.T * a.k;
  const int max_tiles = ((n_pairs + BM - 1) / BM + a.E + 7) / 8 * 8;
  int32_t *tile_e = tiles, *tile_m0 = tiles + max_tiles, *n_tiles = tiles + 2 * max_tiles;
  hipLaunchKernelGGL(k_build_tiles, dim3(1), dim3(1024), 0, s, a.expert_off, a.E, tile_e, tile_m0,
                     n_tiles);
  if (a.F % BN || a.H % BN || a.H % BK || a.F % BK) return hipErrorInvalidValue;
  // gate/up: A = x rows by token, K = H, N = F, h rows in expert order (hbuf)
  const int nct_gu = a.F / BN;
  hipLaunchKernelGGL((k_grouped<FMT, 2>), dim3(max_tiles * nct_gu), dim3(256), 0, s, a.pool,
                     a.stride, a.L, a.H, a.F, a.k, a.x, 1, a.pair_perm, a.expert_off, tile_e, tile_m0,
                     n_tiles, nct_gu, a.hbuf, nullptr);
  // down: A = h rows in expert order, K = F, N = H, y rows of the pairs
  float* y = a.y ? a.y : a.ybuf;
  const int nct_d = a.H / BN;
  hipLaunchKernelGGL((k_grouped<FMT, 1>), dim3(max_tiles * nct_d), dim3(256), 0, s, a.pool, a.stride,
                     a.L, a.F, a.H, a.k, a.hbuf, 0, a.pair_perm, a.expert_off, tile_e, tile_m0,
                     n_tiles, nct_d, nullptr, y);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.out) return e;
  return launch_combine(y, a.topk_w, a.T, a.H, a.k, a.out, s);
}

}  // namespace

size_t grouped_tiles_bytes(int T, int k, int E) {
  const int max_tiles = ((T * k + BM - 1) / BM + E + 7) / 8 * 8;
  return align256((size_t)(2 * max_tiles + 1) * 4);
}

hipError_t launch_ffn_grouped(const FfnArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  switch (a.fmt) {
    case MOE_FMT_NVFP4: return grouped_fmt<MOE_FMT_NVFP4>(a, a.tiles, s);
    case MOE_FMT_MXFP4: return grouped_fmt<MOE_FMT_MXFP4>(a, a.tiles, s);
    default: return grouped_fmt<MOE_FMT_FP8_E4M3>(a, a.tiles, s);
  }
}
