// Expert-grouped expert FFN for many tokens (prefill shape) on bf16 MFMA.
//
// Each expert is an independent FFN evaluated on the tokens routed to it (page
// "FreeToken：753B大模型塞进单卡的本地部署硬件账该怎么算", section
// "混合专家架构（MoE）的天然稀疏性"); its low-precision weights are dequantized
// at compute time (page "8GB显存跑35B MoE模型：FreeToken引擎本地部署实战", §2.1),
// here in registers, straight into MFMA operands.
//
// Pairs arrive sorted by expert (pair_perm / expert_off).  A device-built tile
// list holds one (expert, first row) entry per 128 rows of each expert (64 for
// FP8, whose per-step partial sums need more registers, and for native MXFP4,
// whose FP8 operand sets do).  A workgroup of NW
// waves (8 when the output width allows, else 4) owns one tile x NW*32 output columns
// per matrix for gate/up (NW*64 for down): wave w takes the weight fragments
// of its 32 (64) columns and all rows of the tile (up to eight 16-row
// subtiles for gate/up, six for down, v_mfma_f32_16x16x32_bf16), so each
// dequantized weight operand feeds one MFMA per subtile and an expert's gate
// and up weights are fetched and dequantized once per column tile whenever it
// has at most 128 rows (FP8, native MXFP4: 64).  The subtile count is a template parameter
// chosen per tile, so the inner loop has no branches.
//
// K runs in steps of 128 (one weight fragment).  The pre-shuffled blob gives
// lane l its 32 consecutive k of the fragment with one 16-byte load; MFMA i
// (0..3) takes elements 8i..8i+7 of them, and the activation operand is read
// from LDS with the same k order, so products pair up as in the plain k order.
//   MXFP4: e2m1 -> bf16 with the E8M0 scale folded into the conversion (exact).
//   NVFP4: e2m1 -> fp32, times the E4M3 block scale (exact in bf16: <= 6
//          significant bits), high halves packed to bf16; tau in the epilogue.
//   FP8  : e4m3 -> bf16 exactly; the fp32 scale of the 128-element block is
//          applied to each step's partial sums.
// Activation tiles (rows x 128 k bf16) are double-buffered in LDS with the
// 16-byte chunks of row r stored at chunk ^ (r & 15), which keeps both the
// staging writes and the MFMA operand reads free of bank conflicts; the next
// step's activations and the step after next's weights are in flight while a
// step computes, with one barrier per step.
// Gate/up writes h = bf16(silu(g) * u) in expert-sorted row order; down
// writes y (fp32) to the rows of the original pairs.
//
// MXFP4 also runs natively on the gfx950 scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4): the weight operand is the FP4 codes and
// E8M0 block scales exactly as the blob stores them (lane l's 16 bytes and
// scale byte of a fragment are the operand layout of that instruction), and
// the bf16 activations enter as two FP8 E4M3 terms, hi = e4m3(a / 2^e) with
// 2^e mapping the 32-element block's largest |a| into [128, 256), and lo the
// same for the remainder a - hi * 2^e, each with its E8M0 block scale.  For a
// bf16 value the two terms are exact unless it lies some 2^14 below its
// block's largest (then its lowest bits fall below lo's subnormal step).  The
// x rows are split once by a small kernel, h rows by the gate/up epilogue; a
// 128-k step is two MFMAs per 16x16 tile and no weight is converted.  On that
// instruction lane l of the 8-bit operand holds k 16(l/16)..+15 and
// 64+16(l/16)..+15 of row l%16, while the 4-bit operand holds k 32(l/16)..+31,
// and lane group b supplies the scale of k-block b for both.
#include "common.h"
#include "launch.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// Internal format tag: MXFP4 blobs run on the scaled MFMA (see above).
constexpr int kMxNat = 4;
template <int FMT>
constexpr bool kNat = FMT == kMxNat;
constexpr int kNatScaleRow = 8;  // LDS bytes of scales per activation row per step: (hi, lo) x 4 blocks

constexpr int BK = kFragK;   // k per step
// 16-column weight groups per wave: each activation operand read from LDS
// feeds NMAT * CG MFMAs; down (one matrix) takes four groups so that LDS reads
// stay at half the MFMA rate, gate/up two (its two matrices double the reuse).
template <int NMAT>
constexpr int kCG = NMAT == 2 ? 2 : 4;
// output columns per matrix per column tile of a workgroup of NW waves
template <int NMAT, int NW>
constexpr int kBN = NW * kCG<NMAT> * kFragRows;
constexpr int ROWB = BK * 2;                 // LDS bytes per activation row per step

// 16-row subtiles per tile of the list (gate/up runs a whole tile; down runs
// tiles of more than 6 subtiles as two halves, its accumulators being twice
// as wide)
template <int FMT>
constexpr int kSubMax = FMT == MOE_FMT_FP8_E4M3 || FMT == kMxNat ? 4 : 8;
template <int FMT>
constexpr int kTileRows = kFragRows * kSubMax<FMT>;

__global__ __launch_bounds__(1024) void k_build_tiles(const int32_t* __restrict__ expert_off, int E,
                                                      int rb, int32_t* __restrict__ tile_e,
                                                      int32_t* __restrict__ tile_m0,
                                                      int32_t* __restrict__ n_tiles) {
  __shared__ int wsum[16];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  const int ne = e < E ? expert_off[e + 1] - expert_off[e] : 0;
  const int c = (ne + rb - 1) / rb;
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
    tile_m0[base + j] = j * rb;
  }
  if (e == 0) *n_tiles = tot;
}

// One weight fragment (16 columns x 128 k) as held by a lane: 32 consecutive k.
template <int FMT>
struct BFrag {
  static constexpr bool kFP8 = FMT == MOE_FMT_FP8_E4M3;
  u32x4_t c[kFP8 ? 2 : 1];
  uint32_t s;  // NVFP4: 2 scale bytes; MXFP4: 1 byte; FP8: fp32 bits

  __device__ __forceinline__ void load(const uint8_t* __restrict__ codes,
                                       const uint8_t* __restrict__ scales, size_t f, int lane) {
    if constexpr (kFP8) {
      c[0] = reinterpret_cast<const u32x4_t*>(codes + f * 2048)[lane];
      c[1] = reinterpret_cast<const u32x4_t*>(codes + f * 2048 + 1024)[lane];
      s = reinterpret_cast<const uint32_t*>(scales + f * 64)[lane & 15];
    } else {
      c[0] = reinterpret_cast<const u32x4_t*>(codes + f * 1024)[lane];
      if constexpr (FMT == MOE_FMT_NVFP4)
        s = reinterpret_cast<const uint16_t*>(scales + f * 128)[lane];
      else
        s = scales[f * 64 + lane];
    }
  }

  __device__ __forceinline__ static uint32_t word(const u32x4_t& q, int w) { return q[w]; }

  // bf16 operand for MFMA i: elements 8i .. 8i+7 of the lane's 32.
  __device__ __forceinline__ bf16x8_t operand(int i) const {
    uint32_t o[4];
    if constexpr (FMT == MOE_FMT_MXFP4) {
      const float sc = e8m0_to_f32(s & 0xff);
      const uint32_t w = word(c[0], i);
      o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
      o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
      o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
      o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
    } else if constexpr (FMT == MOE_FMT_NVFP4) {
      const float sc = __builtin_amdgcn_cvt_f32_fp8((int)(s >> (8 * (i >> 1))), 0);
      const uint32_t w = word(c[0], i);
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
      const u32x4_t& q = c[i >> 1];
      const uint32_t w0 = word(q, 2 * (i & 1)), w1 = word(q, 2 * (i & 1) + 1);
      o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
      o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
      o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
      o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
    }
    return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
  }

  __device__ __forceinline__ float step_scale() const { return __uint_as_float(s); }  // FP8
};

constexpr int kPatchLd = 68, kPatchFloats = 16 * kPatchLd;  // down epilogue patch per wave (16 x 64 fp32, padded)
constexpr int kHPatchLd = 40, kHPatchHalfs = 16 * kHPatchLd;  // gate/up epilogue patch per wave (16 x 32 bf16, padded)

struct TileArgs {
  uint8_t* epi;               // LDS: down epilogue patches
  const int32_t* rows_perm;   // LDS: pair_perm of the tile's rows (down)
  const uint8_t* blob;
  BlobLayout L;
  int K, N, k_top, a_by_token, ct, npass, row_base, rows;
  const uint16_t* a_src;
  const int32_t* pair_perm;
  uint16_t* hout;
  float* yout;
  // native MXFP4: activation rows as FP8 terms (lo plane a_plane bytes after
  // the hi plane) and their scales; gate/up writes h the same way
  const uint8_t* a_q;
  size_t a_plane;
  const uint8_t* a_s;
  uint8_t* hq;
  uint8_t* hs;
  size_t h_plane;
  uint8_t* sbuf;  // LDS: the staged scales, [2][rows][kNatScaleRow]
};

// ------------------------------------------------ FP8 two-term split (native MXFP4)

// E8M0 exponent e (clamped to [-127, 120]) with m / 2^e in [128, 256) for a
// normal m > 0; 0 for m = 0.
__device__ __forceinline__ int block_exp(float m) {
  if (m == 0.0f) return 0;
  const int e = (int)((__float_as_uint(m) >> 23) & 0xffu) - 127 - 7;
  return e < -127 ? -127 : (e > 120 ? 120 : e);
}
__device__ __forceinline__ float exp2_neg(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }  // 2^-e

__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  return fmaxf(v, dpp_f32<kDppXor2>(v));
}

// Eight values (one quarter of a 32-element block; the block's other quarters
// are held by the other lanes of this lane's aligned quad, all of which must
// be active) -> their hi and lo FP8 codes and the block's scales (byte 0: hi
// E8M0, byte 1: lo E8M0).
__device__ __forceinline__ uint32_t split_quad8(const float (&f)[8], uint2& hi, uint2& lo) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  const int eh = block_exp(quad_max(m));
  const float sh = exp2_neg(eh), uh = exp2_neg(-eh);
  uint32_t ch[2];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * w] * sh, f[4 * w + 1] * sh, 0, false);
    c = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * w + 2] * sh, f[4 * w + 3] * sh, c, true);
    ch[w] = (uint32_t)c;
  }
  float r[8], rm = 0.0f;
#pragma unroll
  for (int w = 0; w < 2; ++w) {  // remainders, exact in fp32
    r[4 * w + 0] = f[4 * w + 0] - __builtin_amdgcn_cvt_f32_fp8((int)ch[w], 0) * uh;
    r[4 * w + 1] = f[4 * w + 1] - __builtin_amdgcn_cvt_f32_fp8((int)ch[w], 1) * uh;
    r[4 * w + 2] = f[4 * w + 2] - __builtin_amdgcn_cvt_f32_fp8((int)ch[w], 2) * uh;
    r[4 * w + 3] = f[4 * w + 3] - __builtin_amdgcn_cvt_f32_fp8((int)ch[w], 3) * uh;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) rm = fmaxf(rm, fabsf(r[i]));
  const int el = block_exp(quad_max(rm));
  const float sl = exp2_neg(el);
  uint32_t cl[2];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * w] * sl, r[4 * w + 1] * sl, 0, false);
    c = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * w + 2] * sl, r[4 * w + 3] * sl, c, true);
    cl[w] = (uint32_t)c;
  }
  hi = make_uint2(ch[0], ch[1]);
  lo = make_uint2(cl[0], cl[1]);
  return (uint32_t)(eh + 127) | ((uint32_t)(el + 127) << 8);
}

__device__ __forceinline__ void unpack_bf16x8(uint4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Rows of bf16 [n_rows][K] -> FP8 terms q (hi plane, then lo plane `plane`
// bytes later, both [n_rows][K]) and scales s [n_rows][K/32][2]; one thread per
// 8 elements (n8 = n_rows * K / 8, a multiple of 4).
__global__ __launch_bounds__(256) void k_split_rows(const uint16_t* __restrict__ x, size_t n8, size_t plane,
                                                    uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;  // whole quads only (n8 % 4 == 0, blocks of 256)
  float f[8];
  unpack_bf16x8(reinterpret_cast<const uint4*>(x)[i], f);
  uint2 hi, lo;
  const uint32_t sc = split_quad8(f, hi, lo);
  reinterpret_cast<uint2*>(q)[i] = hi;
  reinterpret_cast<uint2*>(q + plane)[i] = lo;
  if ((i & 3) == 0) reinterpret_cast<uint16_t*>(s)[i >> 2] = (uint16_t)sc;
}

// Activation staging by the 64*NW threads: thread -> rows tid/16 + 4*NW*j
// (j < NP), 16-byte chunk tid%16, NP passes covering the tile's 16*NS rows.
// Row r's chunk c sits at slot c ^ (r & 15): sixteen lanes writing one row, or
// reading one chunk of sixteen consecutive rows, touch sixteen distinct slots.
template <int NS, int NW>
constexpr int kStagePasses = (4 * NS + NW - 1) / NW;

template <int NP>
__device__ __forceinline__ void a_load(u32x4_t (&av)[NP], const uint16_t* const (&arow)[NP], int s, int sc) {
#pragma unroll
  for (int j = 0; j < NP; ++j) av[j] = reinterpret_cast<const u32x4_t*>(arow[j] + s * BK)[sc];
}

template <int NP, int NW>
__device__ __forceinline__ void a_store(const u32x4_t (&av)[NP], uint8_t* __restrict__ buf, int sr, int sc) {
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int r = sr + 4 * NW * j;
    *reinterpret_cast<u32x4_t*>(buf + r * ROWB + ((sc ^ (r & 15)) << 4)) = av[j];
  }
}

template <int FMT, int NMAT>
__device__ __forceinline__ void b_load(BFrag<FMT> (&dst)[NMAT][kCG<NMAT>], const uint8_t* const (&codes)[NMAT],
                                       const uint8_t* const (&scales)[NMAT], int g0, int S, int s, int lane) {
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int cg = 0; cg < kCG<NMAT>; ++cg) dst[m][cg].load(codes[m], scales[m], (size_t)(g0 + cg) * S + s, lane);
}

// One step: MFMAs of every subtile against the step's weight fragments.
// FP4: i outer, each dequantized operand feeds the NS subtiles at once.
// FP8: per column group the step's operands are converted first, then subtile
// by subtile a four-MFMA partial sum is scaled by the fragment's fp32 block
// scale.
template <int FMT, int NMAT, int NS>
__device__ __forceinline__ void tile_step(floatx4_t (&acc)[NMAT][kCG<NMAT>][NS], const uint8_t* __restrict__ buf,
                                          const BFrag<FMT> (&wf)[NMAT][kCG<NMAT>], int lane,
                                          const uint8_t* __restrict__ sbuf = nullptr) {
  const int am = lane & 15, aq = lane >> 4;
  if constexpr (kNat<FMT>) {
    // per 16-row subtile: the hi and lo terms of rows 16r + lane%16 (k chunks
    // aq and 4 + aq of each 128-byte term row), two scaled MFMAs per weight
    // fragment; the FP4 codes and E8M0 scale go in exactly as loaded
    i32x8_t bo[NMAT][kCG<NMAT>];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int cg = 0; cg < kCG<NMAT>; ++cg) {
        const u32x4_t& c = wf[m][cg].c[0];
        bo[m][cg] = i32x8_t{(int)c[0], (int)c[1], (int)c[2], (int)c[3], 0, 0, 0, 0};
      }
    // the hi terms of every subtile, then the lo terms; the operand of subtile
    // r + 1 is read from LDS while subtile r's MFMAs run, and the reads of later
    // subtiles are not hoisted.  The LDS bases pass through an empty asm so that
    // the per-subtile addresses (base + constant) are formed inside the step
    // rather than hoisted out of the k loop into registers of their own.
    int lz = 0;
    asm volatile("" : "+v"(lz));
    const uint8_t* bufl = buf + lz;
    const uint8_t* sbufl = sbuf + lz;
    const auto read_a = [&](int r, int term, i32x8_t& av8, int& sc) {
      const int row = kFragRows * r + am, sw = row & 15;
      const uint8_t* rp = bufl + row * ROWB;
      const u32x4_t c0 = *reinterpret_cast<const u32x4_t*>(rp + (((8 * term + aq) ^ sw) << 4));
      const u32x4_t c1 = *reinterpret_cast<const u32x4_t*>(rp + (((8 * term + 4 + aq) ^ sw) << 4));
      av8 = i32x8_t{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
      // lane group aq supplies the scale of k-block aq of its row
      sc = (int)sbufl[row * kNatScaleRow + 2 * aq + term];
    };
#pragma unroll
    for (int term = 0; term < 2; ++term) {
      i32x8_t cur, nxt;
      int s_cur, s_nxt;
      read_a(0, term, cur, s_cur);
#pragma unroll
      for (int r = 0; r < NS; ++r) {
        if (r + 1 < NS) read_a(r + 1, term, nxt, s_nxt);
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int cg = 0; cg < kCG<NMAT>; ++cg)
            acc[m][cg][r] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                cur, bo[m][cg], acc[m][cg][r], 0, 4, 0, s_cur, 0, (int)(wf[m][cg].s & 0xffu));
        // an empty asm with a memory clobber keeps the compiler's IR passes from
        // hoisting later reads; the scheduling barrier does so for the machine scheduler
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if (r + 1 < NS) {
          cur = nxt;
          s_cur = s_nxt;
        }
      }
    }
    // the step's MFMAs stay in the step: without this the compiler sinks them
    // below the next barrier, beside the next step's LDS reads, and the operands
    // of both steps spill
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int cg = 0; cg < kCG<NMAT>; ++cg)
#pragma unroll
        for (int r = 0; r < NS; ++r) asm volatile("" : "+v"(acc[m][cg][r]));
  } else if constexpr (FMT != MOE_FMT_FP8_E4M3) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x8_t b[NMAT][kCG<NMAT>];
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int cg = 0; cg < kCG<NMAT>; ++cg) b[m][cg] = wf[m][cg].operand(i);
      // row 16r + lane%16, chunk 4(lane/16) + i, swizzled by row & 15
      const int slot = ((4 * aq + i) ^ am) << 4;
#pragma unroll
      for (int r = 0; r < NS; ++r) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(buf + (kFragRows * r + am) * ROWB + slot);
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int cg = 0; cg < kCG<NMAT>; ++cg)
            acc[m][cg][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[m][cg], acc[m][cg][r], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int cg = 0; cg < kCG<NMAT>; ++cg) {
      bf16x8_t b[4][NMAT];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) b[i][m] = wf[m][cg].operand(i);
#pragma unroll
      for (int r = 0; r < NS; ++r) {
        floatx4_t part[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) part[m] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int slot = ((4 * aq + i) ^ am) << 4;
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(buf + (kFragRows * r + am) * ROWB + slot);
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
            part[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[i][m], part[m], 0, 0, 0);
        }
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          const float sg = wf[m][cg].step_scale();
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[m][cg][r][v] = fmaf(sg, part[m][v], acc[m][cg][r][v]);
        }
      }
    }
  }
}

// Results of one column tile: lane holds column 16*g + lane%16 of each of its
// groups, rows 16r + 4(lane/16) + v of the tile.
// tau: the expert's NVFP4 tensor scales (gate, up, down), read when the tile starts.
template <int FMT, int NMAT, int NS>
__device__ __forceinline__ void tile_epilogue(const TileArgs& t, const floatx4_t (&acc)[NMAT][kCG<NMAT>][NS], int g0,
                                              const float (&tau)[3], int lane) {
  const int am = lane & 15, aq = lane >> 4;
  if constexpr (NMAT == 2) {
    // h = bf16(silu(g) * u): each 16-row subtile (this wave's 32 columns) goes
    // through the wave's LDS patch so that a store covers 16 B per lane and the
    // 64 contiguous bytes of a row per 4 lanes
    const float tg = FMT == MOE_FMT_NVFP4 ? tau[0] : 1.0f, tu = FMT == MOE_FMT_NVFP4 ? tau[1] : 1.0f;
    uint16_t* patch = reinterpret_cast<uint16_t*>(t.epi) + (threadIdx.x >> 6) * kHPatchHalfs;
    const int col0 = g0 * kFragRows;
#pragma unroll
    for (int r = 0; r < NS; ++r) {
#pragma unroll
      for (int cg = 0; cg < kCG<NMAT>; ++cg)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gv = acc[0][cg][r][v] * tg, uv = acc[1][cg][r][v] * tu;
          patch[(4 * aq + v) * kHPatchLd + 16 * cg + am] = f32_to_bf16_rne(silu_f32(gv) * uv);
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int rl = lane >> 2, c8 = 8 * (lane & 3), row = kFragRows * r + rl;
      const uint4 val = *reinterpret_cast<const uint4*>(patch + rl * kHPatchLd + c8);
      if constexpr (kNat<FMT>) {
        // the row's 32 columns are one scale block, held by this lane's quad
        float f[8];
        unpack_bf16x8(val, f);
        uint2 qh, ql;
        const uint32_t sc = split_quad8(f, qh, ql);
        if (row < t.rows) {
          const size_t pr = (size_t)(t.row_base + row);
          *reinterpret_cast<uint2*>(t.hq + pr * t.N + col0 + c8) = qh;
          *reinterpret_cast<uint2*>(t.hq + t.h_plane + pr * t.N + col0 + c8) = ql;
          if ((lane & 3) == 0) reinterpret_cast<uint16_t*>(t.hs)[pr * (t.N / 32) + col0 / 32] = (uint16_t)sc;
        }
      } else {
        if (row < t.rows) *reinterpret_cast<uint4*>(t.hout + (size_t)(t.row_base + row) * t.N + col0 + c8) = val;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  if constexpr (NMAT == 1) {
    // y rows of the pairs: each 16-row subtile goes through this wave's LDS
    // patch (16 rows x 64 columns) so that a store covers 16 B per lane and
    // 256 contiguous bytes of a row per 16 lanes
    const float td = FMT == MOE_FMT_NVFP4 ? tau[2] : 1.0f;
    float* patch = reinterpret_cast<float*>(t.epi) + (threadIdx.x >> 6) * kPatchFloats;
    const int col0 = g0 * kFragRows;
#pragma unroll
    for (int r = 0; r < NS; ++r) {
#pragma unroll
      for (int cg = 0; cg < kCG<NMAT>; ++cg)
#pragma unroll
        for (int v = 0; v < 4; ++v) patch[(4 * aq + v) * kPatchLd + 16 * cg + am] = acc[0][cg][r][v] * td;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rl = 4 * j + (lane >> 4), row = kFragRows * r + rl, c4 = 4 * (lane & 15);
        const float4 val = *reinterpret_cast<const float4*>(patch + rl * kPatchLd + c4);
        if (row < t.rows)
          *reinterpret_cast<float4*>(t.yout + (size_t)t.rows_perm[row] * t.N + col0 + c4) = val;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

template <int NMAT, int NS>
__device__ __forceinline__ void zero_acc(floatx4_t (&acc)[NMAT][kCG<NMAT>][NS]) {
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int cg = 0; cg < kCG<NMAT>; ++cg)
#pragma unroll
      for (int r = 0; r < NS; ++r) acc[m][cg][r] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
}

// One tile with NS 16-row subtiles (rows <= 16*NS), NW waves.
template <int FMT, int NMAT, int NS, int NW>
__device__ __forceinline__ void grouped_tile(const TileArgs& t, uint8_t* __restrict__ As) {
  constexpr int NP = kStagePasses<NS, NW>;
  constexpr int RB = kTileRows<FMT>;       // LDS rows per buffer
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = t.K / BK;

  // weight fragments of this wave: column groups 2*(4ct + wave) + cg
  const uint8_t* codes[NMAT];
  const uint8_t* scales[NMAT];
  codes[0] = t.blob + (NMAT == 2 ? t.L.cg : t.L.cd);
  scales[0] = t.blob + (NMAT == 2 ? t.L.sg : t.L.sd);
  if constexpr (NMAT == 2) {
    codes[NMAT - 1] = t.blob + t.L.cu;
    scales[NMAT - 1] = t.blob + t.L.su;
  }
  // NVFP4 tensor scales, requested now so that the epilogue does not wait for them
  float tau[3] = {1.0f, 1.0f, 1.0f};
  if constexpr (FMT == MOE_FMT_NVFP4) {
    const float* tp = reinterpret_cast<const float*>(t.blob + t.L.tau);
    tau[0] = tp[0];
    tau[1] = tp[1];
    tau[2] = tp[2];
  }

  // activation staging rows (rows past the end repeat the last row; they land
  // in buffer rows no subtile reads).  A row index is a token (gate/up) or an
  // expert-sorted pair (down).
  const int sr = tid >> 4, sc = tid & 15;
  const auto src_row = [&](int r) -> size_t {
    const int p = t.row_base + min(r, t.rows - 1);
    return t.a_by_token ? (size_t)(t.pair_perm[p] / t.k_top) : (size_t)p;
  };
  const uint16_t* arow[NP];
  const uint8_t* qrow[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const size_t ar = src_row(sr + 4 * NW * j);
    if constexpr (kNat<FMT>)  // 16-byte chunk sc: hi chunk sc (< 8) or lo chunk sc - 8
      qrow[j] = t.a_q + ar * t.K + (sc >= 8 ? t.a_plane : 0) + (size_t)(sc & 7) * 16;
    else
      arow[j] = t.a_src + ar * t.K;
  }
  // native: the block scales of staged row tid (threads below the tile's rows)
  const bool s_stage = kNat<FMT> && tid < kFragRows * NS;
  const uint8_t* srow = kNat<FMT> ? t.a_s + src_row(tid) * (size_t)(t.K / 32) * 2 : nullptr;
  uint2 sv = make_uint2(0u, 0u);
  u32x4_t av[NP];
  const auto load_act = [&](int s) {
    if constexpr (kNat<FMT>) {
#pragma unroll
      for (int j = 0; j < NP; ++j) av[j] = *reinterpret_cast<const u32x4_t*>(qrow[j] + (size_t)s * BK);
      if (s_stage) sv = *reinterpret_cast<const uint2*>(srow + (size_t)s * kNatScaleRow);
    } else {
      a_load<NP>(av, arow, s, sc);
    }
  };
  const auto store_act = [&](uint8_t* buf, uint8_t* sb) {
    a_store<NP, NW>(av, buf, sr, sc);
    if constexpr (kNat<FMT>)
      if (s_stage) *reinterpret_cast<uint2*>(sb + tid * kNatScaleRow) = sv;
  };
  uint8_t* sbuf0 = t.sbuf;
  uint8_t* sbuf1 = kNat<FMT> ? t.sbuf + kTileRows<FMT> * kNatScaleRow : nullptr;
  BFrag<FMT> wb0[NMAT][kCG<NMAT>], wb1[NMAT][kCG<NMAT>];
  floatx4_t acc[NMAT][kCG<NMAT>][NS];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int cg = 0; cg < kCG<NMAT>; ++cg)
#pragma unroll
      for (int r = 0; r < NS; ++r) acc[m][cg][r] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // The workgroup sweeps npass column tiles (t.ct ...; npass = 1 for gate/up) of its row tile as one
  // pipeline of U = npass * S steps; step u is k-step u % S of column tile
  // t.ct + u / S.  Step u uses LDS buffer u&1 and weight registers wb(u&1);
  // writing buffer u&1 is safe after the previous step's barrier, since its
  // last reader was step u-2.  The activation tile does not depend on the
  // column tile, so it is staged again (from L2) on each pass.
  const int U = t.npass * S;
  const int gw = wave * kCG<NMAT>;  // this wave's first group inside a column tile
  // Prefetches past the last step re-load the last step's data (cached, never
  // used): every load is unconditional, so the compiler's wait counts stay
  // exact and a wait for the activations never waits for a newer weight load.
  const auto grp_of = [&](int v) { return (t.ct + min(v, U - 1) / S) * (kBN<NMAT, NW> / kFragRows) + gw; };
  const auto k_of = [&](int v) { return min(v, U - 1) % S; };
  uint8_t* buf0 = As;
  uint8_t* buf1 = As + RB * ROWB;
  load_act(0);
  b_load<FMT, NMAT>(wb0, codes, scales, grp_of(0), S, 0, lane);
  b_load<FMT, NMAT>(wb1, codes, scales, grp_of(1), S, k_of(1), lane);
  // Down writes a column tile's results after its last k-step (an odd step:
  // sweeps need S even), before the next weight prefetch is issued, so that
  // later waits for activation loads never wait for those weights.  The
  // scheduling barriers keep each prefetch after the step that frees its
  // registers.
  int u = 0;
  for (; u + 1 < U; u += 2) {
    store_act(buf0, sbuf0);
    load_act(k_of(u + 1));
    __syncthreads();
    tile_step<FMT, NMAT, NS>(acc, buf0, wb0, lane, sbuf0);
    __builtin_amdgcn_sched_barrier(0);
    b_load<FMT, NMAT>(wb0, codes, scales, grp_of(u + 2), S, k_of(u + 2), lane);
    store_act(buf1, sbuf1);
    load_act(k_of(u + 2));
    __syncthreads();
    tile_step<FMT, NMAT, NS>(acc, buf1, wb1, lane, sbuf1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NMAT == 1) {
      if ((u + 1) % S == S - 1) {
        tile_epilogue<FMT, NMAT, NS>(t, acc, grp_of(u + 1), tau, lane);
        zero_acc<NMAT, NS>(acc);
      }
    }
    b_load<FMT, NMAT>(wb1, codes, scales, grp_of(u + 3), S, k_of(u + 3), lane);
  }
  if (u < U) {  // odd step count: the last step (a pass end)
    store_act(buf0, sbuf0);
    __syncthreads();
    tile_step<FMT, NMAT, NS>(acc, buf0, wb0, lane, sbuf0);
    if constexpr (NMAT == 1) tile_epilogue<FMT, NMAT, NS>(t, acc, grp_of(u), tau, lane);
  }
  if constexpr (NMAT == 2) tile_epilogue<FMT, NMAT, NS>(t, acc, t.ct * (kBN<NMAT, NW> / kFragRows) + gw, tau, lane);
}

// NMAT = 2: gate/up with SwiGLU into hout (expert-sorted rows, width N).
// NMAT = 1: down into y rows of the original pairs.
// Native MXFP4 (FMT = kMxNat): a_q / a_plane / a_s replace a_src, and gate/up
// writes h's FP8 terms (hq, lo plane h_plane bytes on) and scales (hs) instead of hout.
template <int FMT, int NMAT, int NW>
__global__ __launch_bounds__(64 * NW, NW == 4 && FMT != MOE_FMT_FP8_E4M3 && !kNat<FMT> ? 2 : 1) void k_grouped(
    const uint8_t* __restrict__ pool, size_t stride, BlobLayout L, int K, int N, int k_top,
    const uint16_t* __restrict__ a_src, int a_by_token, const int32_t* __restrict__ pair_perm,
    const int32_t* __restrict__ expert_off, const int32_t* __restrict__ tile_e,
    const int32_t* __restrict__ tile_m0, const int32_t* __restrict__ n_tiles, int tile_rows, int n_sweeps,
    int npass, uint16_t* __restrict__ hout, float* __restrict__ yout, const uint8_t* __restrict__ a_q, size_t a_plane,
    const uint8_t* __restrict__ a_s, uint8_t* __restrict__ hq, uint8_t* __restrict__ hs, size_t h_plane) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2 * kTileRows<FMT> * ROWB +
                                                   (NMAT == 1 ? NW * kPatchFloats * 4 : NW * kHPatchHalfs * 2) +
                                                   (kNat<FMT> ? 2 * kTileRows<FMT> * kNatScaleRow : 0)];
  __shared__ int s_rows[NMAT == 1 ? kTileRows<FMT> : 1];
  // A workgroup takes one row tile and a sweep of npass consecutive column
  // tiles.  Workgroups are handed to the 8 XCDs round-robin by index (the grid,
  // max_tiles * n_sweeps, is a multiple of 8); XCD c takes the c-th eighth of
  // the tile list, in order, every tile with all its sweeps.  The sweeps of a
  // row tile then share that XCD's L2 copy of the gathered activation rows, and
  // the row tiles of one expert (consecutive in the list) its copy of the
  // expert's weights.
  const int nt = *n_tiles, per = (nt + 7) >> 3;
  const int j = blockIdx.x >> 3, tl = j / n_sweeps;
  const int tile = (blockIdx.x & 7) * per + tl;
  if (tl >= per || tile >= nt) return;
  TileArgs t;
  const int e = tile_e[tile];
  t.row_base = expert_off[e] + tile_m0[tile];
  // (bounded by the format's tile rows, so that the compiler drops the subtile
  // counts a format never reaches)
  t.rows = min(min(tile_rows, kTileRows<FMT>), expert_off[e + 1] - t.row_base);
  t.epi = As + 2 * kTileRows<FMT> * ROWB;
  t.rows_perm = s_rows;
  if constexpr (NMAT == 1)  // read before the first epilogue, after the pipeline's first barrier
    for (int i = threadIdx.x; i < t.rows; i += blockDim.x) s_rows[i] = pair_perm[t.row_base + i];
  t.blob = pool + (size_t)e * stride;
  t.L = L;
  t.K = K;
  t.N = N;
  t.k_top = k_top;
  t.a_by_token = a_by_token;
  t.ct = (j % n_sweeps) * npass;
  t.npass = npass;
  t.a_src = a_src;
  t.pair_perm = pair_perm;
  t.hout = hout;
  t.yout = yout;
  t.a_q = a_q;
  t.a_plane = a_plane;
  t.a_s = a_s;
  t.hq = hq;
  t.hs = hs;
  t.h_plane = h_plane;
  t.sbuf = t.epi + (NMAT == 1 ? NW * kPatchFloats * 4 : NW * kHPatchHalfs * 2);
  const int ns = (t.rows + kFragRows - 1) / kFragRows;
  if (NMAT == 1 && ns > 6) {
    // down: the first 64 rows, then the rest, each with the tile's sweep
    TileArgs t2 = t;
    t.rows = 4 * kFragRows;
    grouped_tile<FMT, NMAT, 4, NW>(t, As);
    t2.row_base += 4 * kFragRows;
    t2.rows -= 4 * kFragRows;
    t2.rows_perm += 4 * kFragRows;
    __syncthreads();  // the first half's last LDS reads are done before the second stages
    switch (ns - 4) {
      case 3: grouped_tile<FMT, NMAT, 3, NW>(t2, As); break;
      default: grouped_tile<FMT, NMAT, 4, NW>(t2, As); break;
    }
    return;
  }
  switch (ns) {
    case 1: grouped_tile<FMT, NMAT, 1, NW>(t, As); break;
    case 2: grouped_tile<FMT, NMAT, 2, NW>(t, As); break;
    case 3: grouped_tile<FMT, NMAT, 3, NW>(t, As); break;
    case 4: grouped_tile<FMT, NMAT, 4, NW>(t, As); break;
    default:
      if constexpr (kSubMax<FMT> >= 6) {
        switch (ns) {
          case 5: grouped_tile<FMT, NMAT, 5, NW>(t, As); break;
          case 6: grouped_tile<FMT, NMAT, 6, NW>(t, As); break;
          default:
            if constexpr (NMAT == 2) {
              if (ns == 7) grouped_tile<FMT, NMAT, 7, NW>(t, As);
              else grouped_tile<FMT, NMAT, 8, NW>(t, As);
            }
            break;
        }
      }
      break;
  }
}

// Column tiles per workgroup: enough for about 16 k-steps in one pipeline,
// a power of two that divides the column tile count.
int sweep_len(int n_col_tiles, int S) {
  int n = 1;
  if (S % 2) return n;  // a pass must end on an odd step
  while (n * 2 * S <= 16 && n_col_tiles % (n * 2) == 0) n *= 2;
  return n;
}

// Entries of a tile list of rb-row tiles: a multiple of 8 (k_grouped maps
// tiles to XCDs by eighths).
int max_tiles_rows(int n_pairs, int E, int rb) { return ((n_pairs + rb - 1) / rb + E + 7) / 8 * 8; }
template <int FMT>
int max_tiles_for(int n_pairs, int E) {
  return max_tiles_rows(n_pairs, E, kTileRows<FMT>);
}

// Row tiles of the FP4 down kernel when experts average more than this many
// rows: its accumulators hold at most six 16-row subtiles without spilling, so
// a 128-row tile runs as two passes (64 rows + the rest), each streaming the
// expert's down weights and dequantizing them for few rows.  A list of 96-row
// tiles (built after the gate/up kernel, over the same buffer) needs one pass
// per tile: 16384 tokens of the 35B-class layer take 1501 instead of 2120
// passes, the 753B-class layer at 4096 tokens 511 instead of 635.
constexpr int kDownRows = 96;

// One grouped kernel: NMAT = 2 gate/up (A = x rows by token, K = H, N = F,
// h rows in expert order), NMAT = 1 down (A = h rows in expert order, K = F,
// N = H, y rows of the pairs).  FP4 formats: eight waves (twice the columns
// per staged activation tile, so half the activation reads) when N allows;
// else four.
template <int FMT, int NMAT>
void launch_grouped_k(const FfnArgs& a, int max_tiles, const int32_t* tile_e, const int32_t* tile_m0,
                      const int32_t* n_tiles, int tile_rows, float* y, hipStream_t s) {
  const int K = NMAT == 2 ? a.H : a.F, N = NMAT == 2 ? a.F : a.H;
  const uint16_t* a_src = NMAT == 2 ? a.x : a.hbuf;
  // native MXFP4: x's FP8 terms (gate/up) or h's (down; they replace the bf16 h rows in hbuf)
  const size_t n_pairs = (size_t)a.T * a.k;
  uint8_t* hq = reinterpret_cast<uint8_t*>(a.hbuf);
  const uint8_t* a_q = NMAT == 2 ? a.xq : hq;
  const size_t a_plane = NMAT == 2 ? (size_t)a.T * a.H : n_pairs * a.F;
  const uint8_t* a_s = NMAT == 2 ? a.xs : a.hs;
#define GK(NW)                                                                                                \
  {                                                                                                           \
    const int nct = N / kBN<NMAT, NW>;                                                                        \
    const int np = NMAT == 2 ? 1 : sweep_len(nct, K / BK); /* gate/up keeps its epilogue out of the loop */   \
    hipLaunchKernelGGL((k_grouped<FMT, NMAT, NW>), dim3(max_tiles * (nct / np)), dim3(64 * NW), 0, s, a.pool, \
                       a.stride, a.L, K, N, a.k, a_src, NMAT == 2 ? 1 : 0, a.pair_perm, a.expert_off, tile_e,  \
                       tile_m0, n_tiles, tile_rows, nct / np, np, NMAT == 2 ? a.hbuf : nullptr,                \
                       NMAT == 2 ? nullptr : y,                                                               \
                       a_q, a_plane, a_s, hq, a.hs, n_pairs * a.F);                                           \
  }
  // gate/up widths are multiples of 256 (8-wave tiles); down takes 4 waves for hidden 256.
  // Native MXFP4 runs 8-wave workgroups on 64-row tiles: with 128-row tiles its
  // scaled-MFMA operands and accumulators spill at two waves per SIMD.
  if constexpr (NMAT == 2) GK(8) else if (N % kBN<NMAT, 8> == 0) GK(8) else GK(4)
#undef GK
}

template <int FMT>
hipError_t grouped_fmt(const FfnArgs& a, int32_t* tiles, hipStream_t s) {
  const int n_pairs = a.T * a.k;
  const bool nat = FMT == MOE_FMT_MXFP4 && a.mx_native;
  const int max_tiles = nat ? max_tiles_for<kMxNat>(n_pairs, a.E) : max_tiles_for<FMT>(n_pairs, a.E);
  int32_t *tile_e = tiles, *tile_m0 = tiles + max_tiles, *n_tiles = tiles + 2 * max_tiles;
  if (a.F % kBN<2, 8> || a.H % kBN<1, 4> || a.H % BK || a.F % BK) return hipErrorInvalidValue;
  if (!a.tiles_ready)  // else the permutation kernel wrote the list (grouped_tile_rows / grouped_max_tiles)
    hipLaunchKernelGGL(k_build_tiles, dim3(1), dim3(1024), 0, s, a.expert_off, a.E,
                       nat ? kTileRows<kMxNat> : kTileRows<FMT>, tile_e, tile_m0, n_tiles);
  float* y = a.y ? a.y : a.ybuf;
  if (nat) {
    // x rows into their FP8 terms once, then both grouped kernels on the scaled MFMA
    const size_t n8 = (size_t)a.T * a.H / 8;
    hipLaunchKernelGGL(k_split_rows, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, a.x, n8,
                       (size_t)a.T * a.H, a.xq, a.xs);
    launch_grouped_k<kMxNat, 2>(a, max_tiles, tile_e, tile_m0, n_tiles, kTileRows<kMxNat>, y, s);
    launch_grouped_k<kMxNat, 1>(a, max_tiles, tile_e, tile_m0, n_tiles, kTileRows<kMxNat>, y, s);
  } else {
    launch_grouped_k<FMT, 2>(a, max_tiles, tile_e, tile_m0, n_tiles, kTileRows<FMT>, y, s);
    if (kTileRows<FMT> > kDownRows && n_pairs > kDownRows * a.E) {
      // the down kernel's own list of 96-row tiles, written over the gate/up
      // kernel's list once that kernel is done (same stream); the buffer holds
      // the longest list (64-row tiles)
      const int mt = max_tiles_rows(n_pairs, a.E, kDownRows);
      hipLaunchKernelGGL(k_build_tiles, dim3(1), dim3(1024), 0, s, a.expert_off, a.E, kDownRows, tiles,
                         tiles + mt, tiles + 2 * mt);
      launch_grouped_k<FMT, 1>(a, mt, tiles, tiles + mt, tiles + 2 * mt, kDownRows, y, s);
    } else {
      launch_grouped_k<FMT, 1>(a, max_tiles, tile_e, tile_m0, n_tiles, kTileRows<FMT>, y, s);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.out) return e;
  return launch_combine(y, a.topk_w, a.T, a.H, a.k, a.out, s);
}

}  // namespace

size_t grouped_tiles_bytes(int T, int k, int E) {
  // the FP4 formats use 128-row tiles and FP8 64-row tiles: size for the longer list
  const int max_tiles = max_tiles_for<MOE_FMT_FP8_E4M3>(T * k, E);
  return align256((size_t)(2 * max_tiles + 1) * 4);
}

int grouped_tile_rows(int fmt, int mx_native) {
  if (fmt == MOE_FMT_MXFP4 && mx_native) return kTileRows<kMxNat>;
  return fmt == MOE_FMT_FP8_E4M3 ? kTileRows<MOE_FMT_FP8_E4M3> : kTileRows<MOE_FMT_NVFP4>;
}

int grouped_max_tiles(int fmt, int mx_native, int n_pairs, int E) {
  if (fmt == MOE_FMT_MXFP4 && mx_native) return max_tiles_for<kMxNat>(n_pairs, E);
  return fmt == MOE_FMT_FP8_E4M3 ? max_tiles_for<MOE_FMT_FP8_E4M3>(n_pairs, E)
                                 : max_tiles_for<MOE_FMT_NVFP4>(n_pairs, E);
}

hipError_t launch_ffn_grouped(const FfnArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  switch (a.fmt) {
    case MOE_FMT_NVFP4: return grouped_fmt<MOE_FMT_NVFP4>(a, a.tiles, s);
    case MOE_FMT_MXFP4: return grouped_fmt<MOE_FMT_MXFP4>(a, a.tiles, s);
    default: return grouped_fmt<MOE_FMT_FP8_E4M3>(a, a.tiles, s);
  }
}
