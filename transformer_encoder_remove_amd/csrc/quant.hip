// INT8 quantisation kernels (the Swin talk "大規模なビジュアル モデル…", section 3, INT8
// paragraph: inputs and weights are quantised to INT8 before the INT8 GEMM, whose INT32
// result is dequantised). Symmetric codes in [-127, 127], round half to even.
//  * weights, once at preprocessing, per output channel: s[n] = max_k |W[n][k]| / 127
//    (1 for an all-zero row), code = clamp(rne(W[n][k] / s[n])), float32 arithmetic;
//    the per-column dequantisation scale dq[n] = act_scale * s[n] is stored beside them;
//  * activations, per tensor with a static scale: code = clamp(rne(float(x) * inv)).
#include "device.h"
#include "launch.h"

namespace tel {

constexpr int QW_THREADS = 256;

// One workgroup per weight row.
template <typename T>
__global__ __launch_bounds__(QW_THREADS) void quantize_weight_kernel(const T* __restrict__ w,
                                                                     int8_t* __restrict__ q,
                                                                     float* __restrict__ s_w,
                                                                     float* __restrict__ dq,
                                                                     float act_scale, int K) {
  __shared__ float wave_max[QW_THREADS / 64];
  const int n = blockIdx.x, tid = threadIdx.x;
  const T* row = w + (size_t)n * K;
  float m = 0.f;
  for (int k = tid; k < K; k += QW_THREADS) m = fmaxf(m, fabsf(to_f32(row[k])));
  m = group_max<64>(m);
  if ((tid & 63) == 0) wave_max[tid >> 6] = m;
  __syncthreads();
  float amax = wave_max[0];
#pragma unroll
  for (int i = 1; i < QW_THREADS / 64; ++i) amax = fmaxf(amax, wave_max[i]);
  const float s = amax > 0.f ? amax / 127.f : 1.f;   // correctly rounded float32 division
  for (int k = tid; k < K; k += QW_THREADS) {
    const float r = __builtin_rintf(to_f32(row[k]) / s);
    q[(size_t)n * K + k] = (int8_t)fminf(fmaxf(r, -127.f), 127.f);
  }
  if (tid == 0) {
    s_w[n] = s;
    if (dq) dq[n] = act_scale * s;
  }
}

hipError_t launch_quantize_weight(int dtype, const void* w, int8_t* q, float* s_w, float* dq,
                                  float act_scale, int N, int K, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  switch (dtype) {
    case DT_F16:
      quantize_weight_kernel<f16><<<N, QW_THREADS, 0, stream>>>((const f16*)w, q, s_w, dq, act_scale, K);
      break;
    case DT_BF16:
      quantize_weight_kernel<bf16><<<N, QW_THREADS, 0, stream>>>((const bf16*)w, q, s_w, dq, act_scale, K);
      break;
    case DT_F32:
      quantize_weight_kernel<float><<<N, QW_THREADS, 0, stream>>>((const float*)w, q, s_w, dq, act_scale, K);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Activations: 8 elements per thread per step (one 16-byte load for 16-bit types),
// grid-stride; the tail (n % 8) is handled element by element.
template <typename T>
__global__ __launch_bounds__(256) void quantize_act_kernel(const T* __restrict__ x,
                                                           int8_t* __restrict__ q, size_t n,
                                                           const float* __restrict__ inv_dev,
                                                           float inv_host,
                                                           const float* __restrict__ amax_stat,
                                                           float* __restrict__ amax_out,
                                                           float* __restrict__ zero,
                                                           int n_zero) {
  // zero: statistics later kernels raise, cleared here to save a launch (never the one this
  // kernel reads)
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_zero * AMAX_SLOTS; i += 256)
      zero[(size_t)(i / AMAX_SLOTS) * AMAX_STAT_FLOATS + (i % AMAX_SLOTS) * AMAX_STRIDE] = 0.f;
  // dynamic scale: 1 / s = 127 / max-abs of the tensor (1 for an all-zero tensor); every
  // wavefront folds the statistic's copies itself (256 threads: four whole wavefronts)
  float inv = inv_dev ? *inv_dev : inv_host;
  if (amax_stat) {
    const float a = amax_fold(amax_stat);
    if (blockIdx.x == 0 && threadIdx.x == 0) *amax_out = a;
    inv = a > 0.f ? 127.f / a : 1.f;
  }
  const size_t nv = n / 8;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nv; i += (size_t)gridDim.x * 256) {
    int8_t c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float r = __builtin_rintf(to_f32(x[i * 8 + e]) * inv);
      c[e] = (int8_t)fminf(fmaxf(r, -127.f), 127.f);
    }
    uint2 packed;
    __builtin_memcpy(&packed, c, 8);
    *reinterpret_cast<uint2*>(q + i * 8) = packed;
  }
  if (blockIdx.x == 0) {
    for (size_t i = nv * 8 + threadIdx.x; i < n; i += 256) {
      const float r = __builtin_rintf(to_f32(x[i]) * inv);
      q[i] = (int8_t)fminf(fmaxf(r, -127.f), 127.f);
    }
  }
}

hipError_t launch_quantize_act(int dtype, const void* x, int8_t* q, size_t n, const float* inv_dev,
                               float inv_host, hipStream_t stream, const float* amax_stat,
                               float* amax_out, float* zero, int n_zero) {
  if (n == 0) return hipSuccess;
  if (n_zero < 0 || n_zero > 8 || (n_zero && !zero) || (amax_stat && !amax_out))
    return hipErrorInvalidValue;
  size_t blocks = (n / 8 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  switch (dtype) {
    case DT_F16:
      quantize_act_kernel<f16><<<blocks, 256, 0, stream>>>((const f16*)x, q, n, inv_dev, inv_host,
                                                           amax_stat, amax_out, zero, n_zero);
      break;
    case DT_BF16:
      quantize_act_kernel<bf16><<<blocks, 256, 0, stream>>>((const bf16*)x, q, n, inv_dev, inv_host,
                                                            amax_stat, amax_out, zero, n_zero);
      break;
    case DT_F32:
      quantize_act_kernel<float><<<blocks, 256, 0, stream>>>((const float*)x, q, n, inv_dev,
                                                             inv_host, amax_stat, amax_out, zero,
                                                             n_zero);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Calibration statistic: *out = max(*out, max_i |x[i]|). Non-negative floats order like
// their bit patterns, so an unsigned atomic max is exact and order-independent. The
// workgroup reduces through LDS first: one atomic per workgroup, not per wavefront (atomics
// on one address serialise).
// Each thread reads 16 bytes per step (8 16-bit or 4 float32 values); workgroup 0 takes the
// tail of n that does not fill a vector.
template <typename T>
__global__ __launch_bounds__(256) void absmax_kernel(const T* __restrict__ x, size_t n,
                                                     float* __restrict__ out, bool stat) {
  constexpr int VEC = 16 / sizeof(T);
  __shared__ float wave_max[4];
  float m = 0.f;
  const size_t nv = n / VEC;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nv; i += (size_t)gridDim.x * 256) {
    T v[VEC];
    const u32x4 raw = *reinterpret_cast<const u32x4*>(x + i * VEC);
    __builtin_memcpy(v, &raw, 16);
#pragma unroll
    for (int e = 0; e < VEC; ++e) m = fmaxf(m, fabsf(to_f32(v[e])));
  }
  if (blockIdx.x == 0)
    for (size_t i = nv * VEC + threadIdx.x; i < n; i += 256) m = fmaxf(m, fabsf(to_f32(x[i])));
  m = group_max<64>(m);
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
    if (stat) amax_raise(out, m);
    else atomicMax(reinterpret_cast<unsigned int*>(out), __float_as_uint(m));
  }
}

hipError_t launch_absmax(int dtype, const void* x, size_t n, float* out, hipStream_t stream,
                         bool stat) {
  if (n == 0) return hipSuccess;
  if ((uintptr_t)x & 15u) return hipErrorInvalidValue;   // 16-byte vector loads
  // one workgroup per compute unit at most: atomics to the one address serialise (a few
  // ns each), so fewer, longer workgroups finish sooner than one per 4 KiB of input
  size_t blocks = (n * dtype_size(dtype) / 16 + 255) / 256;
  if (blocks > 256) blocks = 256;
  if (blocks == 0) blocks = 1;
  switch (dtype) {
    case DT_F16: absmax_kernel<f16><<<blocks, 256, 0, stream>>>((const f16*)x, n, out, stat); break;
    case DT_BF16: absmax_kernel<bf16><<<blocks, 256, 0, stream>>>((const bf16*)x, n, out, stat); break;
    case DT_F32: absmax_kernel<float><<<blocks, 256, 0, stream>>>((const float*)x, n, out, stat); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Every copy of n max-abs statistics set to 0 (a kernel, not a memset: graph capture).
__global__ __launch_bounds__(256) void clear_amax_kernel(float* __restrict__ stats, int n) {
  for (int i = threadIdx.x; i < n * AMAX_SLOTS; i += 256)
    stats[(size_t)(i / AMAX_SLOTS) * AMAX_STAT_FLOATS + (i % AMAX_SLOTS) * AMAX_STRIDE] = 0.f;
}

hipError_t launch_clear_amax(float* stats, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  clear_amax_kernel<<<1, 256, 0, stream>>>(stats, n);
  return hipGetLastError();
}

}  // namespace tel
