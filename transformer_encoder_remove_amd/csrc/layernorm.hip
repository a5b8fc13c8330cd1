// LayerNorm over the hidden dimension, one row per group of G lanes.
//
// The row is read once into a register array whose size is a template parameter and
// whose indices are compile-time after unrolling (the register-array technique of the
// Swin talk "大規模なビジュアル モデル…", section 3), so the two statistics passes
// (mean, then the variance of the centred values) re-read registers, not memory.
// Element assignment is strided so that the G lanes of a row read G consecutive
// 16-byte vectors per load (coalesced), and reductions are G-lane butterflies.
#include "device.h"
#include "launch.h"

namespace tel {

constexpr int LN_THREADS = 256;

template <typename T, int G, int NV>
__global__ __launch_bounds__(LN_THREADS) void layernorm_kernel(const T* __restrict__ x,
                                                               T* __restrict__ y,
                                                               const float* __restrict__ gamma,
                                                               const float* __restrict__ beta,
                                                               int rows, float eps) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int H = G * NV * VEC;
  const int row = blockIdx.x * (LN_THREADS / G) + threadIdx.x / G;
  const int sub = threadIdx.x % G;
  if (row >= rows) return;   // whole G-lane groups leave together
  const T* xr = x + (size_t)row * H;
  float v[NV][VEC];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const Vec16<T> t = *reinterpret_cast<const Vec16<T>*>(xr + (k * G + sub) * VEC);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      v[k][e] = to_f32(t.v[e]);
      s += v[k][e];
    }
  }
  const float mean = group_sum<G>(s) * (1.f / H);
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      v[k][e] -= mean;
      q += v[k][e] * v[k][e];
    }
  const float rstd = rsqrtf(group_sum<G>(q) * (1.f / H) + eps);
  T* yr = y + (size_t)row * H;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int c0 = (k * G + sub) * VEC;
    Vec16<T> o;
#pragma unroll
    for (int e = 0; e < VEC; e += 4) {
      const float4 g = *reinterpret_cast<const float4*>(gamma + c0 + e);
      const float4 b = *reinterpret_cast<const float4*>(beta + c0 + e);
      o.v[e + 0] = from_f32<T>(v[k][e + 0] * rstd * g.x + b.x);
      o.v[e + 1] = from_f32<T>(v[k][e + 1] * rstd * g.y + b.y);
      o.v[e + 2] = from_f32<T>(v[k][e + 2] * rstd * g.z + b.z);
      o.v[e + 3] = from_f32<T>(v[k][e + 3] * rstd * g.w + b.w);
    }
    *reinterpret_cast<Vec16<T>*>(yr + c0) = o;
  }
}

// Lanes per row G and vectors per lane NV with G * NV * (16 / sizeof(T)) == width.
static bool pick_ln(int dtype, int width, int* g, int* nv) {
  const int vec = 16 / dtype_size(dtype);
  if (width <= 0 || width % vec) return false;
  const int nvec = width / vec;
  for (int G = 64; G >= 1; G >>= 1) {
    if (nvec % G) continue;
    const int n = nvec / G;
    if (n == 1 || n == 2 || n == 3 || n == 4 || n == 6 || n == 8) {
      *g = G;
      *nv = n;
      return true;
    }
  }
  return false;
}

bool layernorm_supported(int dtype, int width) {
  int g, nv;
  if (dtype != DT_F16 && dtype != DT_BF16 && dtype != DT_F32) return false;
  return pick_ln(dtype, width, &g, &nv);
}

template <typename T, int G, int NV>
static void run_ln(const void* x, void* y, const float* g, const float* b, int rows, float eps,
                   hipStream_t stream) {
  constexpr int RPB = LN_THREADS / G;
  layernorm_kernel<T, G, NV><<<(rows + RPB - 1) / RPB, LN_THREADS, 0, stream>>>(
      (const T*)x, (T*)y, g, b, rows, eps);
}

template <typename T, int G>
static bool run_ln_nv(int nv, const void* x, void* y, const float* g, const float* b, int rows,
                      float eps, hipStream_t s) {
  switch (nv) {
    case 1: run_ln<T, G, 1>(x, y, g, b, rows, eps, s); return true;
    case 2: run_ln<T, G, 2>(x, y, g, b, rows, eps, s); return true;
    case 3: run_ln<T, G, 3>(x, y, g, b, rows, eps, s); return true;
    case 4: run_ln<T, G, 4>(x, y, g, b, rows, eps, s); return true;
    case 6: run_ln<T, G, 6>(x, y, g, b, rows, eps, s); return true;
    case 8: run_ln<T, G, 8>(x, y, g, b, rows, eps, s); return true;
  }
  return false;
}

template <typename T>
static bool run_ln_g(int G, int nv, const void* x, void* y, const float* g, const float* b,
                     int rows, float eps, hipStream_t s) {
  switch (G) {
    case 1: return run_ln_nv<T, 1>(nv, x, y, g, b, rows, eps, s);
    case 2: return run_ln_nv<T, 2>(nv, x, y, g, b, rows, eps, s);
    case 4: return run_ln_nv<T, 4>(nv, x, y, g, b, rows, eps, s);
    case 8: return run_ln_nv<T, 8>(nv, x, y, g, b, rows, eps, s);
    case 16: return run_ln_nv<T, 16>(nv, x, y, g, b, rows, eps, s);
    case 32: return run_ln_nv<T, 32>(nv, x, y, g, b, rows, eps, s);
    case 64: return run_ln_nv<T, 64>(nv, x, y, g, b, rows, eps, s);
  }
  return false;
}

hipError_t launch_layernorm(int dtype, const void* x, void* y, const float* gamma,
                            const float* beta, int rows, int width, float eps,
                            hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  int G, nv;
  if (!pick_ln(dtype, width, &G, &nv)) return hipErrorInvalidValue;
  bool ok = false;
  switch (dtype) {
    case DT_F16: ok = run_ln_g<f16>(G, nv, x, y, gamma, beta, rows, eps, stream); break;
    case DT_BF16: ok = run_ln_g<bf16>(G, nv, x, y, gamma, beta, rows, eps, stream); break;
    case DT_F32: ok = run_ln_g<float>(G, nv, x, y, gamma, beta, rows, eps, stream); break;
  }
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tel
