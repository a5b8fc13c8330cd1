// 2:4 structured sparsity of the projection weights (TensorRT 8 overview, "通過稀疏支持和
// Transformer優化增強AI推理", the paragraphs on sparsity of the Ampere architecture: weak
// connections are pruned, about half of the weights, and the matrix hardware skips them).
// Magnitude pruning along the input dimension: in every group of four consecutive weights of
// an output row the two of largest |w| are kept (ties to the lower k) and stored compressed
// in the operand form of the sparse MFMA: kept values [N][K/2] in increasing k, and one
// 16-bit index word per 16 k whose bits 4g..4g+3 hold group g's two positions (first in the
// low two bits). Done once, when a layer's weights are prepared.
#include "device.h"
#include "launch.h"

namespace tel {

// One thread per 16 consecutive weights of a row (one index word).
template <typename T>
__global__ __launch_bounds__(256) void prune_2of4_kernel(const T* __restrict__ w,
                                                         T* __restrict__ values,
                                                         uint16_t* __restrict__ index,
                                                         long long words) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= words) return;
  const Vec16<T> lo = *reinterpret_cast<const Vec16<T>*>(w + t * 16);
  const Vec16<T> hi = *reinterpret_cast<const Vec16<T>*>(w + t * 16 + 8);
  T x[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = lo.v[i];
    x[8 + i] = hi.v[i];
  }
  Vec16<T> out;
  uint32_t word = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float m[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) m[q] = fabsf(to_f32(x[4 * g + q]));
    // first: the largest magnitude, lowest position among equals
    int p0 = 0;
#pragma unroll
    for (int q = 1; q < 4; ++q) if (m[q] > m[p0]) p0 = q;
    // second: the largest of the other three, lowest position among equals
    int p1 = p0 == 0 ? 1 : 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) if (q != p0 && m[q] > m[p1]) p1 = q;
    const int a = p0 < p1 ? p0 : p1, b = p0 < p1 ? p1 : p0;
    out.v[2 * g] = x[4 * g + a];
    out.v[2 * g + 1] = x[4 * g + b];
    word |= (uint32_t)(a | (b << 2)) << (4 * g);
  }
  *reinterpret_cast<Vec16<T>*>(values + t * 8) = out;
  index[t] = (uint16_t)word;
}

hipError_t launch_prune_2of4(int dtype, const void* w, void* values, uint16_t* index, int N,
                             int K, hipStream_t stream) {
  if (N <= 0 || K <= 0 || K % 16) return hipErrorInvalidValue;
  const long long words = (long long)N * (K / 16);
  const unsigned grid = (unsigned)((words + 255) / 256);
  switch (dtype) {
    case DT_F16:
      prune_2of4_kernel<f16><<<grid, 256, 0, stream>>>((const f16*)w, (f16*)values, index, words);
      break;
    case DT_BF16:
      prune_2of4_kernel<bf16><<<grid, 256, 0, stream>>>((const bf16*)w, (bf16*)values, index,
                                                          words);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tel
