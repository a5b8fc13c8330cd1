// LayerNorm over the hidden dimension, one row per group of G lanes.
//
// The row is read once into a register array whose size is a template parameter and
// whose indices are compile-time after unrolling (the register-array technique of the
// Swin talk "大規模なビジュアル モデル…", section 3), so the two statistics passes
// (mean, then the variance of the centred values) re-read registers, not memory.
// Each lane owns NV groups of 8 consecutive elements (one 16-byte load for 16-bit
// types, two for float32); group k of lane s starts at element (k * G + s) * 8, so the
// G lanes of a row read G consecutive groups per load (coalesced). Reductions are
// G-lane butterflies. The input may be float32 (a bf16 layer's pre-LN sums) and the
// result may also be written a second time in float32 (its residual stream).
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace tel {

constexpr int LN_THREADS = 256;

template <typename T> __device__ __forceinline__ void load8(const T* p, float* v) {
  if constexpr (sizeof(T) == 4) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const Vec16<T> t = *reinterpret_cast<const Vec16<T>*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = to_f32(t.v[e]);
  }
}

template <typename T> __device__ __forceinline__ void store8(T* p, const float* v) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    Vec16<T> t;
#pragma unroll
    for (int e = 0; e < 8; ++e) t.v[e] = from_f32<T>(v[e]);
    *reinterpret_cast<Vec16<T>*>(p) = t;
  }
}

// Q8: also write the int8 codes of the output for an int8 GEMM that consumes it, taken
// from the stored (TO-rounded) value: code = clamp(rne(float(y) * inv), -127, 127).
// GATHER: output row r reads input row geom.src_row(r) (the shifted-window partition:
// LayerNorm, cyclic shift and window partition in one pass).
// AMAX: also raise the max-abs statistic amax by max |y| over the stored (TO-rounded)
// outputs, the statistic of a dynamically scaled int8 GEMM that reads y: reduced over the
// workgroup through LDS, then one atomic max per workgroup on one of the statistic's copies
// (amax_raise). Rows past the end
// then compute on the last row instead of leaving, so that every lane reaches the barrier.
template <typename TI, typename TO, bool COPY, int G, int NV, bool Q8 = false, bool GATHER = false,
          bool AMAX = false>
__global__ __launch_bounds__(LN_THREADS) void layernorm_kernel(const TI* __restrict__ x,
                                                               TO* __restrict__ y,
                                                               float* __restrict__ y32,
                                                               const float* __restrict__ gamma,
                                                               const float* __restrict__ beta,
                                                               int rows, float eps,
                                                               int8_t* __restrict__ yq = nullptr,
                                                               const float* __restrict__ qinv = nullptr,
                                                               SwinGeom geom = SwinGeom{},
                                                               float* __restrict__ amax = nullptr) {
  constexpr int H = G * NV * 8;
  int row = blockIdx.x * (LN_THREADS / G) + threadIdx.x / G;
  const int sub = threadIdx.x % G;
  const bool live = row < rows;
  if constexpr (AMAX) {
    row = live ? row : rows - 1;
  } else {
    if (!live) return;   // whole G-lane groups leave together
  }
  float ymax = 0.f;
  const TI* xr = x + (size_t)(GATHER ? geom.src_row(row) : row) * H;
  float v[NV][8];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    load8(xr + (k * G + sub) * 8, v[k]);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += v[k][e];
  }
  const float mean = group_sum<G>(s) * (1.f / H);
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[k][e] -= mean;
      q += v[k][e] * v[k][e];
    }
  const float rstd = rsqrtf(group_sum<G>(q) * (1.f / H) + eps);
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int c0 = (k * G + sub) * 8;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; e += 4) {
      const float4 g = *reinterpret_cast<const float4*>(gamma + c0 + e);
      const float4 b = *reinterpret_cast<const float4*>(beta + c0 + e);
      o[e + 0] = v[k][e + 0] * rstd * g.x + b.x;
      o[e + 1] = v[k][e + 1] * rstd * g.y + b.y;
      o[e + 2] = v[k][e + 2] * rstd * g.z + b.z;
      o[e + 3] = v[k][e + 3] * rstd * g.w + b.w;
    }
    if constexpr (AMAX) {
      if (live) store8(y + (size_t)row * H + c0, o);
#pragma unroll
      for (int e = 0; e < 8; ++e) ymax = fmaxf(ymax, fabsf(to_f32(from_f32<TO>(o[e]))));
    } else {
      store8(y + (size_t)row * H + c0, o);
    }
    if constexpr (COPY) store8(y32 + (size_t)row * H + c0, o);
    if constexpr (Q8) {
      const float inv = *qinv;
      int8_t c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float r = __builtin_rintf(to_f32(from_f32<TO>(o[e])) * inv);
        c[e] = (int8_t)fminf(fmaxf(r, -127.f), 127.f);
      }
      uint2 packed;
      __builtin_memcpy(&packed, c, 8);
      *reinterpret_cast<uint2*>(yq + (size_t)row * H + c0) = packed;
    }
  }
  if constexpr (AMAX) {
    __shared__ float wave_max[LN_THREADS / 64];
    ymax = group_max<64>(live ? ymax : 0.f);
    if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = ymax;
    __syncthreads();
    if (threadIdx.x == 0) {
      float m = wave_max[0];
#pragma unroll
      for (int w = 1; w < LN_THREADS / 64; ++w) m = fmaxf(m, wave_max[w]);
      amax_raise(amax, m);
    }
  }
}

// LayerNorm of a sum that a split GEMM left unfinished: the row is assembled from the
// k-split partial sums (float32, fp16 (part16) added in float32, or int32 dequantised by
// dq[n]), the bias and the residual,
// then normalised as above. This is where the output projection's and FFN2's bias +
// residual + LayerNorm epilogue ([SW] section 3, the fused add-bias-residual-LayerNorm)
// happens once the GEMM's k-splits are summed.
constexpr int LNR_MAX_SPLITS = 8;

struct LnRedParams {
  const void* part; int nsplit; const float* dq; const float* bias; const void* resid;
  void* y; float* y32; int8_t* yq; const float* qinv;
  const float* gamma; const float* beta; int rows; float eps; int round_pre; int part16;
  const void* ahead; size_t ahead_bytes; int main_blocks;   // workgroups past main_blocks
};                                                           // only read ahead

template <typename TR, typename TO, int G, int NV>
__global__ __launch_bounds__(LN_THREADS) void layernorm_reduce_kernel(LnRedParams p) {
  constexpr int H = G * NV * 8;
  constexpr bool TO_HALF = std::is_same<TO, f16>::value;
  if ((int)blockIdx.x >= p.main_blocks) {   // no barrier below: these may leave at once
    read_ahead(p.ahead, p.ahead_bytes, blockIdx.x - p.main_blocks, gridDim.x - p.main_blocks);
    return;
  }
  const int row = blockIdx.x * (LN_THREADS / G) + threadIdx.x / G;
  const int sub = threadIdx.x % G;
  if (row >= p.rows) return;
  const size_t split_stride = (size_t)p.rows * H;
  const TR* rr = (const TR*)p.resid + (size_t)row * H;
  float v[NV][8];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int c0 = (k * G + sub) * 8;
    const size_t off = (size_t)row * H + c0;
    float a[8];
    if (p.dq) {   // int32 partial sums: the integer sum is exact, then dequantise
      int32_t acc[8];
      {
        const int4 x0 = *reinterpret_cast<const int4*>((const int32_t*)p.part + off);
        const int4 x1 = *reinterpret_cast<const int4*>((const int32_t*)p.part + off + 4);
        acc[0] = x0.x; acc[1] = x0.y; acc[2] = x0.z; acc[3] = x0.w;
        acc[4] = x1.x; acc[5] = x1.y; acc[6] = x1.z; acc[7] = x1.w;
      }
#pragma unroll
      for (int sp = 1; sp < LNR_MAX_SPLITS; ++sp) {   // unrolled: the loads overlap
        if (sp >= p.nsplit) break;
        const int32_t* q = (const int32_t*)p.part + sp * split_stride + off;
        const int4 x0 = *reinterpret_cast<const int4*>(q);
        const int4 x1 = *reinterpret_cast<const int4*>(q + 4);
        acc[0] += x0.x; acc[1] += x0.y; acc[2] += x0.z; acc[3] += x0.w;
        acc[4] += x1.x; acc[5] += x1.y; acc[6] += x1.z; acc[7] += x1.w;
      }
      float dq[8], b[8];
      load8(p.dq + c0, dq);
      load8(p.bias + c0, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = (float)acc[e] * dq[e] + b[e];
    } else if (TO_HALF && p.part16) {   // fp16 partial sums, added in float32
      load8((const f16*)p.part + off, a);
#pragma unroll
      for (int sp = 1; sp < LNR_MAX_SPLITS; ++sp) {
        if (sp >= p.nsplit) break;
        float t[8];
        load8((const f16*)p.part + sp * split_stride + off, t);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] += t[e];
      }
      float b[8];
      load8(p.bias + c0, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] += b[e];
    } else {
      load8((const float*)p.part + off, a);
#pragma unroll
      for (int sp = 1; sp < LNR_MAX_SPLITS; ++sp) {   // unrolled: the loads overlap
        if (sp >= p.nsplit) break;
        float t[8];
        load8((const float*)p.part + sp * split_stride + off, t);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] += t[e];
      }
      float b[8];
      load8(p.bias + c0, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] += b[e];
    }
    float r[8];
    load8(rr + c0, r);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] += r[e];
      if (p.round_pre) a[e] = to_f32(from_f32<TO>(a[e]));
      v[k][e] = a[e];
      s += a[e];
    }
  }
  const float mean = group_sum<G>(s) * (1.f / H);
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[k][e] -= mean;
      q += v[k][e] * v[k][e];
    }
  const float rstd = rsqrtf(group_sum<G>(q) * (1.f / H) + p.eps);
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int c0 = (k * G + sub) * 8;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; e += 4) {
      const float4 g = *reinterpret_cast<const float4*>(p.gamma + c0 + e);
      const float4 b = *reinterpret_cast<const float4*>(p.beta + c0 + e);
      o[e + 0] = v[k][e + 0] * rstd * g.x + b.x;
      o[e + 1] = v[k][e + 1] * rstd * g.y + b.y;
      o[e + 2] = v[k][e + 2] * rstd * g.z + b.z;
      o[e + 3] = v[k][e + 3] * rstd * g.w + b.w;
    }
    store8((TO*)p.y + (size_t)row * H + c0, o);
    if (p.y32) store8(p.y32 + (size_t)row * H + c0, o);
    if (p.yq) {
      const float inv = *p.qinv;
      int8_t c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float r = __builtin_rintf(to_f32(from_f32<TO>(o[e])) * inv);
        c[e] = (int8_t)fminf(fmaxf(r, -127.f), 127.f);
      }
      uint2 packed;
      __builtin_memcpy(&packed, c, 8);
      *reinterpret_cast<uint2*>(p.yq + (size_t)row * H + c0) = packed;
    }
  }
}

// Lanes per row G and groups per lane NV with G * NV * 8 == width.
static bool pick_ln(int width, int* g, int* nv) {
  if (width <= 0 || width % 8) return false;
  const int groups = width / 8;
  for (int G = 64; G >= 1; G >>= 1) {
    if (groups % G) continue;
    const int n = groups / G;
    if (n >= 1 && n <= 4) {
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
  return pick_ln(width, &g, &nv);
}

struct LnArgs {
  const void* x;
  void* y;
  float* y32;
  const float* g;
  const float* b;
  int rows;
  float eps;
  int8_t* yq = nullptr;
  const float* qinv = nullptr;
  const SwinGeom* geom = nullptr;
  float* amax = nullptr;
};

template <typename TI, typename TO, bool COPY, int G, int NV>
static void run_ln(const LnArgs& a, hipStream_t s) {
  constexpr int RPB = LN_THREADS / G;
  if (a.geom) {
    if constexpr (std::is_same<TI, TO>::value && !COPY) {
      layernorm_kernel<TI, TO, COPY, G, NV, false, true>
          <<<(a.rows + RPB - 1) / RPB, LN_THREADS, 0, s>>>((const TI*)a.x, (TO*)a.y, a.y32, a.g, a.b,
                                                          a.rows, a.eps, nullptr, nullptr, *a.geom);
    }
    return;
  }
  if (a.amax) {
    if constexpr (std::is_same<TI, f16>::value && std::is_same<TO, f16>::value && !COPY) {
      layernorm_kernel<TI, TO, COPY, G, NV, false, false, true>
          <<<(a.rows + RPB - 1) / RPB, LN_THREADS, 0, s>>>((const TI*)a.x, (TO*)a.y, a.y32, a.g,
                                                          a.b, a.rows, a.eps, nullptr, nullptr,
                                                          SwinGeom{}, a.amax);
    }
    return;
  }
  if (a.yq) {
    if constexpr (std::is_same<TI, f16>::value && std::is_same<TO, f16>::value && !COPY) {
      layernorm_kernel<TI, TO, COPY, G, NV, true><<<(a.rows + RPB - 1) / RPB, LN_THREADS, 0, s>>>(
          (const TI*)a.x, (TO*)a.y, a.y32, a.g, a.b, a.rows, a.eps, a.yq, a.qinv);
    }
    return;
  }
  layernorm_kernel<TI, TO, COPY, G, NV><<<(a.rows + RPB - 1) / RPB, LN_THREADS, 0, s>>>(
      (const TI*)a.x, (TO*)a.y, a.y32, a.g, a.b, a.rows, a.eps);
}

template <typename TI, typename TO, bool COPY, int G>
static bool run_ln_nv(int nv, const LnArgs& a, hipStream_t s) {
  switch (nv) {
    case 1: run_ln<TI, TO, COPY, G, 1>(a, s); return true;
    case 2: run_ln<TI, TO, COPY, G, 2>(a, s); return true;
    case 3: run_ln<TI, TO, COPY, G, 3>(a, s); return true;
    case 4: run_ln<TI, TO, COPY, G, 4>(a, s); return true;
  }
  return false;
}

template <typename TI, typename TO, bool COPY>
static bool run_ln_g(int G, int nv, const LnArgs& a, hipStream_t s) {
  switch (G) {
    case 1: return run_ln_nv<TI, TO, COPY, 1>(nv, a, s);
    case 2: return run_ln_nv<TI, TO, COPY, 2>(nv, a, s);
    case 4: return run_ln_nv<TI, TO, COPY, 4>(nv, a, s);
    case 8: return run_ln_nv<TI, TO, COPY, 8>(nv, a, s);
    case 16: return run_ln_nv<TI, TO, COPY, 16>(nv, a, s);
    case 32: return run_ln_nv<TI, TO, COPY, 32>(nv, a, s);
    case 64: return run_ln_nv<TI, TO, COPY, 64>(nv, a, s);
  }
  return false;
}

hipError_t launch_layernorm(int dtype_in, int dtype_out, const void* x, void* y, float* y32,
                            const float* gamma, const float* beta, int rows, int width, float eps,
                            hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  int G, nv;
  if (!pick_ln(width, &G, &nv)) return hipErrorInvalidValue;
  const LnArgs a{x, y, y32, gamma, beta, rows, eps};
  bool ok = false;
  if (dtype_in == dtype_out && !y32) {
    switch (dtype_in) {
      case DT_F16: ok = run_ln_g<f16, f16, false>(G, nv, a, stream); break;
      case DT_BF16: ok = run_ln_g<bf16, bf16, false>(G, nv, a, stream); break;
      case DT_F32: ok = run_ln_g<float, float, false>(G, nv, a, stream); break;
    }
  } else if (dtype_in == DT_F32 && dtype_out == DT_BF16) {
    ok = y32 ? run_ln_g<float, bf16, true>(G, nv, a, stream)
             : run_ln_g<float, bf16, false>(G, nv, a, stream);
  }
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_layernorm_gather(int dtype, const void* x, void* y, const float* gamma,
                                   const float* beta, int rows, int width, float eps,
                                   const SwinGeom& geom, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  int G, nv;
  if (!pick_ln(width, &G, &nv)) return hipErrorInvalidValue;
  LnArgs a{x, y, nullptr, gamma, beta, rows, eps};
  a.geom = &geom;
  bool ok = false;
  switch (dtype) {
    case DT_F16: ok = run_ln_g<f16, f16, false>(G, nv, a, stream); break;
    case DT_BF16: ok = run_ln_g<bf16, bf16, false>(G, nv, a, stream); break;
    case DT_F32: ok = run_ln_g<float, float, false>(G, nv, a, stream); break;
  }
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_layernorm_amax(const void* x, void* y, float* amax, const float* gamma,
                                 const float* beta, int rows, int width, float eps,
                                 hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  int G, nv;
  if (!pick_ln(width, &G, &nv) || !amax) return hipErrorInvalidValue;
  LnArgs a{x, y, nullptr, gamma, beta, rows, eps};
  a.amax = amax;
  if (!run_ln_g<f16, f16, false>(G, nv, a, stream)) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_layernorm_q8(const void* x, void* y, int8_t* yq, const float* qinv,
                               const float* gamma, const float* beta, int rows, int width,
                               float eps, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  int G, nv;
  if (!pick_ln(width, &G, &nv)) return hipErrorInvalidValue;
  LnArgs a{x, y, nullptr, gamma, beta, rows, eps};
  a.yq = yq;
  a.qinv = qinv;
  if (!run_ln_g<f16, f16, false>(G, nv, a, stream)) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tel

namespace tel {

// Read-ahead workgroups beside the reduce's own: 16,384 threads, each with its 16-byte
// copies all in flight (a sweep at a 128-token BERT-large stack found 8,192 and 32,768 or
// more threads slower: more compete with the reduce's own loads, fewer cannot cover the
// memory latency).
constexpr int LNR_AHEAD_BLOCKS = 64;

template <typename TR, typename TO, int G>
static bool run_lnr_nv(int nv, const LnRedParams& p, hipStream_t s) {
  const int blocks = p.main_blocks + (p.ahead_bytes ? LNR_AHEAD_BLOCKS : 0);
  switch (nv) {
    case 1: layernorm_reduce_kernel<TR, TO, G, 1><<<blocks, LN_THREADS, 0, s>>>(p); return true;
    case 2: layernorm_reduce_kernel<TR, TO, G, 2><<<blocks, LN_THREADS, 0, s>>>(p); return true;
    case 3: layernorm_reduce_kernel<TR, TO, G, 3><<<blocks, LN_THREADS, 0, s>>>(p); return true;
    case 4: layernorm_reduce_kernel<TR, TO, G, 4><<<blocks, LN_THREADS, 0, s>>>(p); return true;
  }
  return false;
}

template <typename TR, typename TO>
static bool run_lnr(int G, int nv, const LnRedParams& p, hipStream_t s) {
  switch (G) {
    case 1: return run_lnr_nv<TR, TO, 1>(nv, p, s);
    case 2: return run_lnr_nv<TR, TO, 2>(nv, p, s);
    case 4: return run_lnr_nv<TR, TO, 4>(nv, p, s);
    case 8: return run_lnr_nv<TR, TO, 8>(nv, p, s);
    case 16: return run_lnr_nv<TR, TO, 16>(nv, p, s);
    case 32: return run_lnr_nv<TR, TO, 32>(nv, p, s);
    case 64: return run_lnr_nv<TR, TO, 64>(nv, p, s);
  }
  return false;
}

hipError_t launch_layernorm_reduce(const LnReduceArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  int G, nv;
  if (!pick_ln(a.width, &G, &nv) || a.nsplit < 1 || a.nsplit > LNR_MAX_SPLITS)
    return hipErrorInvalidValue;
  if (a.part16 && (a.out_dt != DT_F16 || a.dq)) return hipErrorInvalidValue;
  if (a.prefetch_bytes >= 16 && (!a.prefetch || (uintptr_t)a.prefetch % 16))
    return hipErrorInvalidValue;
  const int main_blocks = (a.rows + LN_THREADS / G - 1) / (LN_THREADS / G);
  const LnRedParams p{a.part, a.nsplit, a.dq, a.bias, a.resid, a.y, a.y32, a.yq, a.qinv,
                      a.gamma, a.beta, a.rows, a.eps, a.round_pre, a.part16, a.prefetch,
                      a.prefetch_bytes >= 16 ? a.prefetch_bytes : 0, main_blocks};
  bool ok = false;
  if (a.resid_dt == DT_F16 && a.out_dt == DT_F16) ok = run_lnr<f16, f16>(G, nv, p, stream);
  else if (a.resid_dt == DT_BF16 && a.out_dt == DT_BF16) ok = run_lnr<bf16, bf16>(G, nv, p, stream);
  else if (a.resid_dt == DT_F32 && a.out_dt == DT_BF16) ok = run_lnr<float, bf16>(G, nv, p, stream);
  else if (a.resid_dt == DT_F32 && a.out_dt == DT_F32) ok = run_lnr<float, float>(G, nv, p, stream);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tel
