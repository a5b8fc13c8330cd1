// One-time weight preprocessing kernels (the Swin talk "大規模なビジュアル モデル…",
// section 3: work that needs doing only once is done ahead of inference and reused).
#include "device.h"
#include "launch.h"

namespace tel {

template <typename T>
__global__ __launch_bounds__(256) void widen_kernel(const T* __restrict__ src, float* __restrict__ dst,
                                                    int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) dst[i] = to_f32(src[i]);
}

hipError_t launch_widen_f32(int dtype, const void* src, float* dst, int n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int grid = min((n + 255) / 256, 1024);
  switch (dtype) {
    case DT_F16: widen_kernel<f16><<<grid, 256, 0, stream>>>((const f16*)src, dst, n); break;
    case DT_BF16: widen_kernel<bf16><<<grid, 256, 0, stream>>>((const bf16*)src, dst, n); break;
    case DT_F32: widen_kernel<float><<<grid, 256, 0, stream>>>((const float*)src, dst, n); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

constexpr int STORE_F32_MAX = 16;
struct F32xN { float v[STORE_F32_MAX]; };

__global__ void store_f32_kernel(float* __restrict__ dst, F32xN vals, int n) {
  if (threadIdx.x < n) dst[threadIdx.x] = vals.v[threadIdx.x];
}

// Small host-known constants into device memory through kernel arguments (no host buffer
// has to outlive the call).
hipError_t launch_store_f32(float* dst, const float* vals, int n, hipStream_t stream) {
  if (n <= 0 || n > STORE_F32_MAX) return hipErrorInvalidValue;
  F32xN a{};
  for (int i = 0; i < n; ++i) a.v[i] = vals[i];
  store_f32_kernel<<<1, 64, 0, stream>>>(dst, a, n);
  return hipGetLastError();
}

}  // namespace tel
