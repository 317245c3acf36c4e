/* Seeded synthetic inputs for the routed MoE layer: normal draws, bf16
 * activations, and the quantization of fp32 expert weights into canonical
 * NVFP4 / MXFP4 / FP8 bytes.
 *
 * This module produces inputs only.  It holds none of the layer's arithmetic
 * (no router product, softmax, selection, dequantized product, SwiGLU or
 * combine); both the GPU path and the CPU checker read the bytes it writes.
 *
 * Random numbers: Philox4x32-10, the counter-based generator of Salmon,
 * Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
 * (SC'11).  A stream is a 64-bit key derived from (seed, config, kind, layer,
 * expert, matrix, attempt) with the SplitMix64 finaliser; element i of a
 * stream takes word i%4 of the Philox block at counter i/4.  Normals come from
 * the Box-Muller transform of consecutive word pairs.
 *
 * Quantizers (test-data generation; the decoders live elsewhere):
 *   NVFP4: tau = amax(W)/(6*448); s = e4m3_rne(amax_blk16/(6*tau));
 *          c = e2m1_rne_sat(w/(s*tau)); a zero scale gives zero codes.
 *   MXFP4: X = 2^(floor(log2 amax_blk32) - 2), exponent clamped to
 *          [-127, 127] (OCP MX v1.0); c = e2m1_rne_sat(w/X); zero block ->
 *          scale byte 127, codes 0.
 *   FP8  : sigma = fp32(amax_blk128/448) (1 for a zero block);
 *          c = e4m3_rne_sat(w/sigma).
 * Built with -ffp-contract=off so that every machine writes the same bytes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define FMT_NVFP4 1
#define FMT_MXFP4 2
#define FMT_FP8 3

/* ---------------------------------------------------------------- Philox */

static inline void mulhilo32(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; ++r) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo32(0xD2511F53u, c0, &hi0, &lo0);
    mulhilo32(0xCD9E8D57u, c2, &hi1, &lo1);
    uint32_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline uint64_t splitmix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t synth_stream(uint64_t seed, uint32_t cfg, uint32_t kind, uint32_t layer,
                      uint32_t expert, uint32_t matrix, uint32_t attempt) {
  uint64_t h = splitmix64(seed);
  h = splitmix64(h ^ cfg);
  h = splitmix64(h ^ kind);
  h = splitmix64(h ^ layer);
  h = splitmix64(h ^ expert);
  h = splitmix64(h ^ matrix);
  h = splitmix64(h ^ attempt);
  return h;
}

/* Four standard normals from Philox block `blk` of `stream`. */
static inline void normal4(uint64_t stream, uint64_t blk, double z[4]) {
  uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u};
  uint32_t key[2] = {(uint32_t)stream, (uint32_t)(stream >> 32)};
  uint32_t w[4];
  synth_philox4x32_10(ctr, key, w);
  for (int p = 0; p < 2; ++p) {
    double u1 = ((double)w[2 * p] + 1.0) * 0x1p-32;  /* (0, 1] */
    double u2 = (double)w[2 * p + 1] * 0x1p-32;       /* [0, 1) */
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925286766559 * u2;
    z[2 * p] = r * cos(t);
    z[2 * p + 1] = r * sin(t);
  }
}

/* out[i] = float(mean + std * N_{first+i}) */
void synth_normal(uint64_t stream, uint64_t first, size_t n, double mean, double std, float* out) {
#pragma omp parallel for schedule(static) if (n > (1u << 16))
  for (int64_t b = (int64_t)(first / 4); b < (int64_t)((first + n + 3) / 4); ++b) {
    double z[4];
    normal4(stream, (uint64_t)b, z);
    for (int q = 0; q < 4; ++q) {
      uint64_t i = (uint64_t)b * 4 + (uint64_t)q;
      if (i >= first && i < first + n) out[i - first] = (float)(mean + std * z[q]);
    }
  }
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

void synth_f32_to_bf16(const float* in, size_t n, uint16_t* out) {
  for (size_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

static inline float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

void synth_normal_bf16(uint64_t stream, uint64_t first, size_t n, double mean, double std,
                       uint16_t* out) {
  float* tmp = (float*)malloc(n * sizeof(float));
  synth_normal(stream, first, n, mean, std, tmp);
  synth_f32_to_bf16(tmp, n, out);
  free(tmp);
}

/* h_new = bf16(rho * h_prev + c * eps), rho*h and c*eps formed in fp64, one
 * rounding to fp32 of the sum, then bf16 RNE (the AR(1) decode-state recipe). */
void synth_ar1_bf16(const uint16_t* h_prev, const float* eps, size_t n, double rho, double c,
                    uint16_t* out) {
  for (size_t i = 0; i < n; ++i) {
    double v = rho * (double)bf16_to_f32(h_prev[i]) + c * (double)eps[i];
    out[i] = f32_to_bf16_rne((float)v);
  }
}

/* ------------------------------------------------------------ quantizers */

static uint8_t e2m1_rne_sat(double v) {
  double a = fabs(v);
  uint8_t m;
  if (a <= 0.25) m = 0;
  else if (a < 0.75) m = 1;
  else if (a <= 1.25) m = 2;
  else if (a < 1.75) m = 3;
  else if (a <= 2.5) m = 4;
  else if (a < 3.5) m = 5;
  else if (a <= 5.0) m = 6;
  else m = 7;
  return (uint8_t)((v < 0 && m) ? (8 | m) : m);
}

static uint8_t e4m3_rne_sat(double v) {
  uint8_t s = v < 0 ? 0x80 : 0;
  double a = fabs(v);
  if (a != a) return 0x7F;
  if (a >= 448.0) return (uint8_t)(s | 0x7E);
  if (a < 0x1p-6) {                  /* subnormal: multiples of 2^-9 */
    double q = nearbyint(a * 512.0); /* ties to even; q == 8 is code 0x08 = 2^-6 */
    return (uint8_t)(s | (uint8_t)q);
  }
  int e;
  double m = frexp(a, &e);           /* a = m * 2^e, m in [0.5, 1) */
  int E = e - 1;
  double q = nearbyint((2.0 * m - 1.0) * 8.0);
  if (q == 8.0) { q = 0.0; E += 1; }
  int code = ((E + 7) << 3) | (int)q;
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)(s | code);
}

static double e4m3_decode_nonneg(uint8_t c) {
  int e = (c >> 3) & 15, m = c & 7;
  if (e == 0) return m * 0x1p-9;
  return (1.0 + m / 8.0) * ldexp(1.0, e - 7);
}

uint8_t synth_e2m1_encode(double v) { return e2m1_rne_sat(v); }
uint8_t synth_e4m3_encode(double v) { return e4m3_rne_sat(v); }

static double amax_of(const float* w, size_t n) {
  double a = 0.0;
  for (size_t i = 0; i < n; ++i) {
    double t = fabs((double)w[i]);
    if (t > a) a = t;
  }
  return a;
}

/* w: fp32 [N, K] row-major.  Outputs in canonical layout.  Returns 0 / -1. */
int synth_quantize(int fmt, const float* w, int N, int K, uint8_t* codes, void* scales, float* tau) {
  if (fmt == FMT_NVFP4) {
    if (K % 16) return -1;
    double at = amax_of(w, (size_t)N * K);
    float t = at > 0.0 ? (float)(at / (6.0 * 448.0)) : 1.0f;
    *tau = t;
    uint8_t* sc = (uint8_t*)scales;
    for (int n = 0; n < N; ++n) {
      const float* row = w + (size_t)n * K;
      for (int b = 0; b < K / 16; ++b) {
        double ab = amax_of(row + b * 16, 16);
        uint8_t scode = e4m3_rne_sat(ab / (6.0 * (double)t));
        sc[(size_t)n * (K / 16) + b] = scode;
        double denom = e4m3_decode_nonneg(scode) * (double)t;
        for (int i = 0; i < 16; i += 2) {
          uint8_t lo = denom > 0 ? e2m1_rne_sat(row[b * 16 + i] / denom) : 0;
          uint8_t hi = denom > 0 ? e2m1_rne_sat(row[b * 16 + i + 1] / denom) : 0;
          codes[(size_t)n * (K / 2) + (b * 16 + i) / 2] = (uint8_t)(lo | (hi << 4));
        }
      }
    }
    return 0;
  }
  if (fmt == FMT_MXFP4) {
    if (K % 32) return -1;
    if (tau) *tau = 1.0f;
    uint8_t* sc = (uint8_t*)scales;
    for (int n = 0; n < N; ++n) {
      const float* row = w + (size_t)n * K;
      for (int b = 0; b < K / 32; ++b) {
        double ab = amax_of(row + b * 32, 32);
        int xexp;
        if (ab > 0) {
          int e;
          frexp(ab, &e);             /* ab = m*2^e, m in [0.5,1): floor(log2 ab) = e-1 */
          xexp = (e - 1) - 2;
          if (xexp < -127) xexp = -127;
          if (xexp > 127) xexp = 127;
        } else {
          xexp = 0;
        }
        sc[(size_t)n * (K / 32) + b] = (uint8_t)(xexp + 127);
        double X = ldexp(1.0, xexp);
        for (int i = 0; i < 32; i += 2) {
          uint8_t lo = ab > 0 ? e2m1_rne_sat(row[b * 32 + i] / X) : 0;
          uint8_t hi = ab > 0 ? e2m1_rne_sat(row[b * 32 + i + 1] / X) : 0;
          codes[(size_t)n * (K / 2) + (b * 32 + i) / 2] = (uint8_t)(lo | (hi << 4));
        }
      }
    }
    return 0;
  }
  if (fmt == FMT_FP8) {
    if (K % 128) return -1;
    if (tau) *tau = 1.0f;
    float* sc = (float*)scales;
    for (int n = 0; n < N; ++n) {
      const float* row = w + (size_t)n * K;
      for (int b = 0; b < K / 128; ++b) {
        double ab = amax_of(row + b * 128, 128);
        float sg = ab > 0 ? (float)(ab / 448.0) : 1.0f;
        sc[(size_t)n * (K / 128) + b] = sg;
        for (int i = 0; i < 128; ++i)
          codes[(size_t)n * K + b * 128 + i] = e4m3_rne_sat((double)row[b * 128 + i] / (double)sg);
      }
    }
    return 0;
  }
  return -1;
}

/* bytes of canonical codes / scales of one [N, K] matrix */
static size_t code_bytes(int fmt, int N, int K) {
  return fmt == FMT_FP8 ? (size_t)N * K : (size_t)N * K / 2;
}
static size_t scale_bytes(int fmt, int N, int K) {
  if (fmt == FMT_NVFP4) return (size_t)N * (K / 16);
  if (fmt == FMT_MXFP4) return (size_t)N * (K / 32);
  return (size_t)N * (K / 128) * 4;
}

/* Generate and quantize `n_exp` experts (e0 .. e0+n_exp-1) of one layer.
 * G, U are [F, H] and D is [H, F]; each is N(0, std^2) fp32 drawn from
 * stream(seed, cfg, kind=3, layer, expert, matrix, 0), matrix 0/1/2 = G/U/D.
 * Outputs are contiguous per matrix kind with the expert as the leading
 * index: codes_g [n_exp][F][..], scales_g [n_exp][F][..], tau [n_exp][3]. */
int synth_experts(int fmt, uint64_t seed, uint32_t cfg, uint32_t layer, uint32_t e0, int n_exp,
                  int H, int F, double std, uint8_t* codes_g, uint8_t* codes_u, uint8_t* codes_d,
                  uint8_t* scales_g, uint8_t* scales_u, uint8_t* scales_d, float* tau) {
  int bad = 0;
  size_t cb_gu = code_bytes(fmt, F, H), cb_d = code_bytes(fmt, H, F);
  size_t sb_gu = scale_bytes(fmt, F, H), sb_d = scale_bytes(fmt, H, F);
#pragma omp parallel
  {
    float* tmp = (float*)malloc((size_t)H * F * sizeof(float));
#pragma omp for schedule(dynamic, 1)
    for (int task = 0; task < n_exp * 3; ++task) {
      int ei = task / 3, m = task % 3;
      uint64_t st = synth_stream(seed, cfg, 3u, layer, e0 + (uint32_t)ei, (uint32_t)m, 0u);
      size_t n = (size_t)H * F;
      for (size_t b = 0; b < n / 4; ++b) {
        double z[4];
        normal4(st, b, z);
        for (int q = 0; q < 4; ++q) tmp[b * 4 + q] = (float)(std * z[q]);
      }
      int r;
      if (m == 0)
        r = synth_quantize(fmt, tmp, F, H, codes_g + ei * cb_gu, scales_g + ei * sb_gu, tau + ei * 3 + 0);
      else if (m == 1)
        r = synth_quantize(fmt, tmp, F, H, codes_u + ei * cb_gu, scales_u + ei * sb_gu, tau + ei * 3 + 1);
      else
        r = synth_quantize(fmt, tmp, H, F, codes_d + ei * cb_d, scales_d + ei * sb_d, tau + ei * 3 + 2);
      if (r) {
#pragma omp atomic write
        bad = 1;
      }
    }
    free(tmp);
  }
  return bad ? -1 : 0;
}

void synth_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int synth_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
