// Gate-weighted combine: out[t] = bf16(sum_j w[t][j] * y[t*k+j]), an fp32 FMA
// chain in j order (the weighted sum of the top-K expert outputs: page
// "FreeToken：753B大模型塞进单卡的本地部署硬件账该怎么算", section
// "混合专家架构（MoE）的天然稀疏性").
#include "common.h"
#include "launch.h"

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One float4 of y, read once: a non-temporal load (y is streamed through once,
// so it is not kept in the caches; 16384 tokens: 4% faster layer).
__device__ __forceinline__ float4 y_load(const float* __restrict__ y, size_t row, int H, int n4) {
  const f32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(y + row * H) + n4);
  return make_float4(q.x, q.y, q.z, q.w);
}

// K known at compile time: every thread requests its K rows' float4 before the
// first FMA (with a run-time trip count each load waited for the one before).
template <int K>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y,
                                                 const float* __restrict__ w, int H,
                                                 uint16_t* __restrict__ out, const int32_t* __restrict__ rec) {
  if (rec && rec[0] != MOE_OK) return;  // the pairs did not run (cache capacity error)
  const int t = blockIdx.y;
  const int n4 = blockIdx.x * blockDim.x + threadIdx.x;
  if (n4 * 4 >= H) return;
  float4 v[K];
  float wj[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    v[j] = y_load(y, (size_t)t * K + j, H, n4);
    wj[j] = w[(size_t)t * K + j];
  }
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    a0 = fmaf(wj[j], v[j].x, a0);
    a1 = fmaf(wj[j], v[j].y, a1);
    a2 = fmaf(wj[j], v[j].z, a2);
    a3 = fmaf(wj[j], v[j].w, a3);
  }
  uint2 o;
  o.x = (uint32_t)f32_to_bf16_rne(a0) | ((uint32_t)f32_to_bf16_rne(a1) << 16);
  o.y = (uint32_t)f32_to_bf16_rne(a2) | ((uint32_t)f32_to_bf16_rne(a3) << 16);
  reinterpret_cast<uint2*>(out + (size_t)t * H)[n4] = o;
}

// Any k (above 16): one row at a time.
__global__ __launch_bounds__(256) void k_combine_any(const float* __restrict__ y,
                                                     const float* __restrict__ w, int H, int k,
                                                     uint16_t* __restrict__ out, const int32_t* __restrict__ rec) {
  if (rec && rec[0] != MOE_OK) return;
  const int t = blockIdx.y;
  const int n4 = blockIdx.x * blockDim.x + threadIdx.x;
  if (n4 * 4 >= H) return;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const float4 v = y_load(y, (size_t)t * k + j, H, n4);
    a0 = fmaf(wj, v.x, a0);
    a1 = fmaf(wj, v.y, a1);
    a2 = fmaf(wj, v.z, a2);
    a3 = fmaf(wj, v.w, a3);
  }
  uint2 o;
  o.x = (uint32_t)f32_to_bf16_rne(a0) | ((uint32_t)f32_to_bf16_rne(a1) << 16);
  o.y = (uint32_t)f32_to_bf16_rne(a2) | ((uint32_t)f32_to_bf16_rne(a3) << 16);
  reinterpret_cast<uint2*>(out + (size_t)t * H)[n4] = o;
}

hipError_t combine_k(const float* y, const float* w, int T, int H, int k, uint16_t* out, const int32_t* rec,
                     hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((H / 4 + 255) / 256, T);
#define C(K) \
  case K: hipLaunchKernelGGL(k_combine<K>, grid, dim3(256), 0, s, y, w, H, out, rec); break;
  switch (k) {
    C(1) C(2) C(3) C(4) C(5) C(6) C(7) C(8) C(9) C(10) C(11) C(12) C(13) C(14) C(15) C(16)
    default: hipLaunchKernelGGL(k_combine_any, grid, dim3(256), 0, s, y, w, H, k, out, rec); break;
  }
#undef C
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const float* y, const float* w, int T, int H, int k, uint16_t* out,
                          hipStream_t s) {
  return combine_k(y, w, T, H, k, out, nullptr, s);
}

hipError_t launch_combine_rec(const float* y, const float* w, int T, int H, int k, uint16_t* out,
                              const int32_t* rec, hipStream_t s) {
  return combine_k(y, w, T, H, k, out, rec, s);
}
