// Gate-weighted combine: out[t] = bf16(sum_j w[t][j] * y[t*k+j]), an fp32 FMA
// chain in j order (the weighted sum of the top-K expert outputs: page
// "FreeToken：753B大模型塞进单卡的本地部署硬件账该怎么算", section
// "混合专家架构（MoE）的天然稀疏性").
#include "common.h"
#include "launch.h"

namespace {

__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y,
                                                 const float* __restrict__ w, int H, int k,
                                                 uint16_t* __restrict__ out, const int32_t* __restrict__ rec) {
  if (rec && rec[0] != MOE_OK) return;  // the pairs did not run (cache capacity error)
  const int t = blockIdx.y;
  const int n4 = blockIdx.x * blockDim.x + threadIdx.x;
  if (n4 * 4 >= H) return;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const float4 v = reinterpret_cast<const float4*>(y + ((size_t)t * k + j) * H)[n4];
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

}  // namespace

hipError_t launch_combine(const float* y, const float* w, int T, int H, int k, uint16_t* out,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((H / 4 + 255) / 256, T);
  hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, s, y, w, H, k, out, nullptr);
  return hipGetLastError();
}

hipError_t launch_combine_rec(const float* y, const float* w, int T, int H, int k, uint16_t* out,
                              const int32_t* rec, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((H / 4 + 255) / 256, T);
  hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, s, y, w, H, k, out, rec);
  return hipGetLastError();
}
