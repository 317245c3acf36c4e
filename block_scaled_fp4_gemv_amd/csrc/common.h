// Shared device helpers and blob geometry for the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_fp4.h"

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- blob geometry
// One expert blob: gate/up/down codes, then their scales, then tau[3]; every
// section begins on a 256-byte boundary.  A matrix [N][K] (blocks along K) is
// stored as fragments of 16 rows x 128 k, N/16 row groups by S = K/128 steps,
// fragment f = g*S + s.  Lane l (0..63) of a wavefront owns row 16g + l%16 and
// the 32 consecutive elements 128s + 32(l/16) .. +31 of fragment f: the k set
// lane l supplies to four consecutive v_mfma_f32_16x16x32_bf16 operands, and a
// 32-element dot product for a GEMV lane.  Inside a fragment:
//   FP4 codes    64 x 16 B: lane l at byte 16l (canonical byte order inside)
//   FP8 codes    2 pieces x 64 x 16 B: elements 16p..16p+15 of lane l at 1024p + 16l
//   NVFP4 scales 64 x 2 B: the lane's two 16-element blocks, lower k first
//   MXFP4 scales 64 x 1 B: the lane's 32-element block
//   FP8 scales   16 x fp32: row r's scale for the step at float r
// so each wavefront-wide 16-byte load of a fragment reads 1 KiB contiguously.
constexpr int kFragRows = 16, kFragK = 128;
__host__ __device__ constexpr size_t frag_code_bytes(int fmt) { return fmt == MOE_FMT_FP8_E4M3 ? 2048 : 1024; }
__host__ __device__ constexpr size_t frag_scale_bytes(int fmt) {
  return fmt == MOE_FMT_NVFP4 ? 128 : 64;
}

struct BlobLayout {
  size_t cg, cu, cd, sg, su, sd, tau, total;
};

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static inline size_t code_bytes(int fmt, size_t N, size_t K) {
  return fmt == MOE_FMT_FP8_E4M3 ? N * K : N * K / 2;
}
static inline size_t scale_bytes(int fmt, size_t N, size_t K) {
  switch (fmt) {
    case MOE_FMT_NVFP4: return N * (K / 16);
    case MOE_FMT_MXFP4: return N * (K / 32);
    default: return N * (K / 128) * 4;
  }
}

static inline BlobLayout blob_layout(int fmt, int H, int F) {
  BlobLayout b;
  size_t cgu = align256(code_bytes(fmt, F, H)), cd = align256(code_bytes(fmt, H, F));
  size_t sgu = align256(scale_bytes(fmt, F, H)), sd = align256(scale_bytes(fmt, H, F));
  b.cg = 0;
  b.cu = b.cg + cgu;
  b.cd = b.cu + cgu;
  b.sg = b.cd + cd;
  b.su = b.sg + sgu;
  b.sd = b.su + sgu;
  b.tau = b.sd + sd;
  b.total = b.tau + 256;
  return b;
}

// ---------------------------------------------------------------- scalar helpers
__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E8M0 scale byte -> fp32 2^(s-127) (s = 0 gives the fp32 denormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);
}

// E4M3 (OCP FN) byte 0 of v -> fp32, hardware conversion.
__device__ __forceinline__ float e4m3_byte0_to_f32(uint32_t v) {
  return __builtin_amdgcn_cvt_f32_fp8((int)v, 0);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

// acc + a.lo*b.lo + a.hi*b.hi  (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2_bf16(bf16x2_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, as_bf16x2(b), acc, false);
}

// ---------------------------------------------------------------- cross-lane
// DPP moves within 16-lane rows (no LDS round trip): quad_perm(1,0,3,2) = xor 1,
// quad_perm(2,3,0,1) = xor 2, row_half_mirror pairs the two quads of each
// 8-lane half, row_mirror pairs the two halves of a row.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Every lane of each aligned group of W (<= 16) lanes gets the group's sum.
template <int W>
__device__ __forceinline__ float group_sum_dpp(float v) {
  if constexpr (W >= 2) v += dpp_f32<kDppXor1>(v);
  if constexpr (W >= 4) v += dpp_f32<kDppXor2>(v);
  if constexpr (W >= 8) v += dpp_f32<kDppHalfMirror>(v);
  if constexpr (W >= 16) v += dpp_f32<kDppMirror>(v);
  return v;
}

// Sum over the 64-lane wavefront (uniform result).
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum_dpp<16>(v);
  return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)), fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

__device__ __forceinline__ float wave_min(float v) {
  v = fminf(v, dpp_f32<kDppXor1>(v));
  v = fminf(v, dpp_f32<kDppXor2>(v));
  v = fminf(v, dpp_f32<kDppHalfMirror>(v));
  v = fminf(v, dpp_f32<kDppMirror>(v));
  return fminf(fminf(readlane_f32(v, 0), readlane_f32(v, 16)), fminf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

// Sum over aligned groups of W lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (W <= 16) {
    return group_sum_dpp<W>(v);
  } else {
    v = group_sum_dpp<16>(v);
    v += __shfl_xor(v, 16);
    if constexpr (W == 64) v += __shfl_xor(v, 32);
    return v;
  }
}

// silu(g) = g / (1 + e^-g), with the hardware reciprocal (about 1 ulp) in
// place of a full-precision division
__device__ __forceinline__ float silu_f32(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// ---------------------------------------------------------------- chunk dot products
// One 16-byte code chunk against the matching x slice (bf16 pairs in registers).

// The gfx950 scaled conversions (v_cvt_scalef32_pk_*) apply only the exponent
// of their fp32 scale operand, i.e. a power-of-two scale.

// MXFP4: 32 elements with one E8M0 scale, folded into the e2m1 -> bf16
// conversion (e2m1 * 2^e is exact in bf16).
__device__ __forceinline__ float chunk_dot_mxfp4(uint4 c, float s_pow2, const uint32_t* xs, float acc) {
  const uint32_t d[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], s_pow2, 0), xs[4 * i + 0], acc);
    acc = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], s_pow2, 1), xs[4 * i + 1], acc);
    acc = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], s_pow2, 2), xs[4 * i + 2], acc);
    acc = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], s_pow2, 3), xs[4 * i + 3], acc);
  }
  return acc;
}

// NVFP4: 32 elements = two 16-element blocks; each block's dot product with the
// unscaled (exact) e2m1 values is multiplied by its E4M3 scale s_lo / s_hi.
__device__ __forceinline__ float chunk_dot_nvfp4(uint4 c, float s_lo, float s_hi, const uint32_t* xs) {
  const uint32_t d[4] = {c.x, c.y, c.z, c.w};
  float a[2] = {0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float& acc = a[i >> 1];
    acc = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 0), xs[4 * i + 0], acc);
    acc = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 1), xs[4 * i + 1], acc);
    acc = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 2), xs[4 * i + 2], acc);
    acc = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 3), xs[4 * i + 3], acc);
  }
  return a[0] * s_lo + a[1] * s_hi;
}

// FP8 E4M3: 16 elements, exact in bf16; the block scale is applied by the caller.
__device__ __forceinline__ float chunk_dot_fp8(uint4 c, const uint32_t* xs, float acc) {
  const uint32_t d[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[i], 1.0f, false), xs[2 * i + 0], acc);
    acc = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[i], 1.0f, true), xs[2 * i + 1], acc);
  }
  return acc;
}
