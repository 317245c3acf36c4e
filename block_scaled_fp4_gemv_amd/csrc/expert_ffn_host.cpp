// Host (CPU) expert FFN on packed blobs in host memory: the CPU side of the
// decode scheduler's split of a step's cache misses between a GPU cache fill
// and CPU compute, chosen from the two bandwidths (page "8GB 笔记本 39.3 tok/s、
// 单卡跑 753B：FreeToken 把 frontier MoE 拉回本地", section "设计核心", the
// bandwidth-adaptive execution principle).
//
// For one routed pair: h = bf16(silu(G x) * (U x)), y = D h, with the weights
// of the expert's blob decoded in place (the fragment layout the GPU kernels
// read: matrix [N][K] as fragments of 16 rows x 128 k, lane l of a fragment
// holding row l%16 and elements 32(l/16) .. +31 of the fragment's 128), fp32
// accumulation.  Plain C++ compiled by the host compiler with OpenMP: rows of a
// batch of pairs are shared among the threads.
#include <immintrin.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include "moe_fp4.h"

namespace {

// Blob sections (the same geometry as the device code; every section starts
// on a 256-byte boundary).
struct Sections {
  size_t cg, cu, cd, sg, su, sd, tau;
};

size_t a256(size_t v) { return (v + 255) & ~(size_t)255; }

Sections sections(int fmt, size_t H, size_t F) {
  const bool f8 = fmt == MOE_FMT_FP8_E4M3;
  const size_t cgu = a256(f8 ? F * H : F * H / 2), cd = a256(f8 ? H * F : H * F / 2);
  auto sb = [&](size_t N, size_t K) {
    return fmt == MOE_FMT_NVFP4 ? N * (K / 16) : fmt == MOE_FMT_MXFP4 ? N * (K / 32) : N * (K / 128) * 4;
  };
  const size_t sgu = a256(sb(F, H)), sd = a256(sb(H, F));
  Sections s;
  s.cg = 0;
  s.cu = s.cg + cgu;
  s.cd = s.cu + cgu;
  s.sg = s.cd + cd;
  s.su = s.sg + sgu;
  s.sd = s.su + sgu;
  s.tau = s.sd + sd;
  return s;
}

float bf16f(uint16_t v) {
  uint32_t u = (uint32_t)v << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint16_t f2bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E4M3 (OCP "FN") and E2M1 values
float e4m3_value(uint32_t b) {
  const int e = (b >> 3) & 15, m = b & 7;
  const float v = e ? ldexpf(1.0f + m / 8.0f, e - 7) : ldexpf(m / 8.0f, -6);
  return (b & 0x80) ? -v : v;
}
// byte -> value tables: E4M3, and half of each E8M0 power of two (the FP4
// table of fp4x32_dot2 decodes twice the E2M1 values)
struct Tables {
  float e4m3[256], e4m3_half[256], e8m0_half[256];
  Tables() {
    for (int b = 0; b < 256; ++b) {
      e4m3[b] = e4m3_value(b);
      e4m3_half[b] = 0.5f * e4m3[b];
      e8m0_half[b] = 0.5f * ldexpf(1.0f, b - 127);  // b = 0: 2^-127, a subnormal, as the format defines
    }
  }
};
const Tables kTab;
float e4m3f(uint32_t b) { return kTab.e4m3[b & 0xff]; }
const float kE2M1[16] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f,
                         -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f};

// 32 FP4 codes (16 bytes, element 2i in the low nibble of byte i) against 32
// floats with AVX2: the two 16-element halves' dot products as 8-wide partial
// sums, each carrying a factor 2 (the codes decode through a table of twice the
// E2M1 values, which are small integers).
inline void fp4x32_dot2(const uint8_t* c16, const float* x, __m256& half0, __m256& half1) {
  const __m128i raw = _mm_loadu_si128(reinterpret_cast<const __m128i*>(c16));
  const __m128i m4 = _mm_set1_epi8(0x0F);
  const __m128i lo = _mm_and_si128(raw, m4), hi = _mm_and_si128(_mm_srli_epi16(raw, 4), m4);
  const __m128i lut = _mm_setr_epi8(0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12);
  const __m128i v0 = _mm_shuffle_epi8(lut, _mm_unpacklo_epi8(lo, hi));  // elements 0..15
  const __m128i v1 = _mm_shuffle_epi8(lut, _mm_unpackhi_epi8(lo, hi));  // elements 16..31
  const __m256 f0 = _mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(v0));
  const __m256 f1 = _mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(_mm_srli_si128(v0, 8)));
  const __m256 f2 = _mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(v1));
  const __m256 f3 = _mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(_mm_srli_si128(v1, 8)));
  half0 = _mm256_fmadd_ps(f1, _mm256_loadu_ps(x + 8), _mm256_mul_ps(f0, _mm256_loadu_ps(x)));
  half1 = _mm256_fmadd_ps(f3, _mm256_loadu_ps(x + 24), _mm256_mul_ps(f2, _mm256_loadu_ps(x + 16)));
}

inline float hsum8(__m256 v) {
  __m128 s = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
  s = _mm_add_ps(s, _mm_movehl_ps(s, s));
  s = _mm_add_ss(s, _mm_shuffle_ps(s, s, 1));
  return _mm_cvtss_f32(s);
}

// Row n of an FP4 matrix [N][K] against xf[K], vectorized.
float row_dot_fp4(int fmt, const uint8_t* codes, const uint8_t* scales, int K, int n, const float* xf) {
  const int S = K / 128, g = n / 16, r = n % 16;
  __m256 acc = _mm256_setzero_ps();
  for (int s = 0; s < S; ++s) {
    const size_t f = (size_t)g * S + s;
    for (int q = 0; q < 4; ++q) {
      const int l = 16 * q + r;
      __m256 h0, h1;
      fp4x32_dot2(codes + f * 1024 + (size_t)l * 16, xf + 128 * s + 32 * q, h0, h1);
      if (fmt == MOE_FMT_NVFP4) {
        const uint8_t* sc = scales + f * 128 + (size_t)l * 2;
        acc = _mm256_fmadd_ps(h0, _mm256_set1_ps(kTab.e4m3_half[sc[0]]), acc);
        acc = _mm256_fmadd_ps(h1, _mm256_set1_ps(kTab.e4m3_half[sc[1]]), acc);
      } else {
        acc = _mm256_fmadd_ps(_mm256_add_ps(h0, h1), _mm256_set1_ps(kTab.e8m0_half[scales[f * 64 + l]]), acc);
      }
    }
  }
  return hsum8(acc);
}

// Row n of matrix [N][K] (codes at `codes`, scales at `scales`) against xf[K].
float row_dot(int fmt, const uint8_t* codes, const uint8_t* scales, int K, int n, const float* xf) {
  if (fmt != MOE_FMT_FP8_E4M3) return row_dot_fp4(fmt, codes, scales, K, n, xf);
  const int S = K / 128, g = n / 16, r = n % 16;
  float acc = 0.0f;
  for (int s = 0; s < S; ++s) {
    const size_t f = (size_t)g * S + s;
    for (int q = 0; q < 4; ++q) {
      const int l = 16 * q + r;
      const float* xs = xf + 128 * s + 32 * q;
      if (fmt == MOE_FMT_FP8_E4M3) {
        float a = 0.0f;
        for (int p = 0; p < 2; ++p) {
          const uint8_t* c = codes + f * 2048 + (size_t)p * 1024 + (size_t)l * 16;
          for (int i = 0; i < 16; ++i) a += e4m3f(c[i]) * xs[16 * p + i];
        }
        float sg;
        memcpy(&sg, scales + f * 64 + (size_t)r * 4, 4);
        acc += a * sg;
      } else {
        const uint8_t* c = codes + f * 1024 + (size_t)l * 16;
        float blk[2] = {0.0f, 0.0f};
        for (int i = 0; i < 16; ++i) {
          blk[i >> 3] += kE2M1[c[i] & 15] * xs[2 * i] + kE2M1[c[i] >> 4] * xs[2 * i + 1];
        }
        if (fmt == MOE_FMT_NVFP4) {
          const uint8_t* sc = scales + f * 128 + (size_t)l * 2;
          acc += blk[0] * e4m3f(sc[0]) + blk[1] * e4m3f(sc[1]);
        } else {
          const uint32_t e = scales[f * 64 + l];
          acc += (blk[0] + blk[1]) * (e ? ldexpf(1.0f, (int)e - 127) : ldexpf(1.0f, -127));
        }
      }
    }
  }
  return acc;
}

}  // namespace

extern "C" int moe_host_expert_ffn(int fmt, int H, int F, int n, const void* const* blobs, const uint16_t* const* xs,
                                   float* const* ys, float* scratch, int n_threads) {
  if (fmt != MOE_FMT_NVFP4 && fmt != MOE_FMT_MXFP4 && fmt != MOE_FMT_FP8_E4M3) return MOE_E_FORMAT;
  if (n < 0 || H < 128 || F < 128 || H % 128 || F % 128 || H > 8192 || F > 8192) return MOE_E_ARG;
  if (n == 0) return MOE_OK;
  if (!blobs || !xs || !ys || !scratch) return MOE_E_ARG;
  for (int i = 0; i < n; ++i)
    if (!blobs[i] || !xs[i] || !ys[i]) return MOE_E_ARG;
  const Sections L = sections(fmt, H, F);
  // scratch: n * H floats of x, then n * F floats of h (rounded to bf16 values)
  float* xf = scratch;
  float* hf = scratch + (size_t)n * H;
  const int nt = n_threads > 0 ? n_threads : 1;
#pragma omp parallel num_threads(nt)
  {
#pragma omp for schedule(static)
    for (int p = 0; p < n; ++p)
      for (int i = 0; i < H; ++i) xf[(size_t)p * H + i] = bf16f(xs[p][i]);
    // gate/up rows of every pair, then the SwiGLU with h rounded to bf16
#pragma omp for schedule(static)
    for (long i = 0; i < (long)n * F; ++i) {
      const int p = (int)(i / F), row = (int)(i % F);
      const uint8_t* b = static_cast<const uint8_t*>(blobs[p]);
      float tg = 1.0f, tu = 1.0f;
      if (fmt == MOE_FMT_NVFP4) {
        memcpy(&tg, b + L.tau, 4);
        memcpy(&tu, b + L.tau + 4, 4);
      }
      const float gv = row_dot(fmt, b + L.cg, b + L.sg, H, row, xf + (size_t)p * H) * tg;
      const float uv = row_dot(fmt, b + L.cu, b + L.su, H, row, xf + (size_t)p * H) * tu;
      hf[i] = bf16f(f2bf16_rne(gv / (1.0f + expf(-gv)) * uv));
    }
    // down rows
#pragma omp for schedule(static)
    for (long i = 0; i < (long)n * H; ++i) {
      const int p = (int)(i / H), row = (int)(i % H);
      const uint8_t* b = static_cast<const uint8_t*>(blobs[p]);
      float td = 1.0f;
      if (fmt == MOE_FMT_NVFP4) memcpy(&td, b + L.tau + 8, 4);
      ys[p][row] = row_dot(fmt, b + L.cd, b + L.sd, F, row, hf + (size_t)p * F) * td;
    }
  }
  return MOE_OK;
}
