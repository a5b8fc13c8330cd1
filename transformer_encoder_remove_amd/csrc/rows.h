// Token-row operands of the row-wise MFMA kernels (the skinny GEMMs of the shifted-window
// block and its fused halves): a wavefront holds 16 token rows as MFMA B fragments (lane l:
// row l % 16, 8 consecutive k per 32-deep step at k offset 8 (l / 16)), loads them in one
// of three row orders and applies a LayerNorm to them in registers.
#pragma once

#include "device.h"

namespace tel {

// Input-row modes of the skinny kernel: rows as stored, the shifted-window partition
// (row r reads image row geom.src_row(r)), or patch merging (row r is the concatenation of
// the four image rows geom.merge_src(r, k), each K / 4 wide).
enum RowMode { ROWS_PLAIN = 0, ROWS_WINDOW = 1, ROWS_MERGE = 2 };

template <typename T, int KS, int MODE>
__device__ __forceinline__ void rows_load(typename Mfma<T>::frag (&buf)[KS], const T* A, int M,
                                          int row0, int lr, int lg, const SwinGeom& geom) {
  constexpr int K = KS * 32;
  int row = min(row0 + lr, M - 1);
  if constexpr (MODE == ROWS_MERGE) {
    constexpr int C = K / 4, TP = KS / 4;           // 32-wide k chunks per part
    static_assert(KS % 4 == 0, "a k chunk must not straddle two parts");
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const T* src = A + (size_t)geom.merge_src(row, k) * C + lg * 8;
#pragma unroll
      for (int t = 0; t < TP; ++t)
        buf[k * TP + t] = *reinterpret_cast<const typename Mfma<T>::frag*>(src + t * 32);
    }
    return;
  } else {
    if constexpr (MODE == ROWS_WINDOW) row = geom.src_row(row);
    const T* src = A + (size_t)row * K + lg * 8;
#pragma unroll
    for (int t = 0; t < KS; ++t) buf[t] = *reinterpret_cast<const typename Mfma<T>::frag*>(src + t * 32);
  }
}

// LayerNorm of the rows held in fragments: the 4 lanes lg = 0..3 of a row hold its K values
// (8 per k-step each), so the two-pass statistics are the lane's own sums plus butterflies
// over xor 16 and xor 32; the normalised values replace the fragments (rounded to T, as a
// stored LayerNorm output would be). g, b: the lane's gamma/beta for its K/4 positions.
// Wide rows (K > 96): the same two-pass statistics without a float copy of the values (each
// value is converted again where it is needed: the same float operations, bit-identical
// results, 8 * KS fewer registers), gamma / beta read from LDS as float4 vectors.
template <typename T, int KS>
__device__ __forceinline__ void rows_layernorm_wide(typename Mfma<T>::frag (&buf)[KS],
                                                    const float* sG, const float* sB, int lg,
                                                    float eps) {
  constexpr int K = KS * 32;
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < KS; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) s += to_f32(buf[t][e]);
  s += __shfl_xor(s, 16, 64);
  s += __shfl_xor(s, 32, 64);
  const float mean = s * (1.f / K);
  float q = 0.f;
#pragma unroll
  for (int t = 0; t < KS; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c = to_f32(buf[t][e]) - mean;
      q += c * c;
    }
  q += __shfl_xor(q, 16, 64);
  q += __shfl_xor(q, 32, 64);
  const float rstd = rsqrtf(q * (1.f / K) + eps);
#pragma unroll
  for (int t = 0; t < KS; ++t)
#pragma unroll
    for (int h = 0; h < 2; ++h) {   // four values at a time: 8 live gamma / beta floats
      const float4 g4 = *reinterpret_cast<const float4*>(sG + t * 32 + lg * 8 + 4 * h);
      const float4 b4 = *reinterpret_cast<const float4*>(sB + t * 32 + lg * 8 + 4 * h);
      const float g[4] = {g4.x, g4.y, g4.z, g4.w};
      const float b[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        buf[t][4 * h + e] = from_f32<T>((to_f32(buf[t][4 * h + e]) - mean) * rstd * g[e] + b[e]);
    }
}

// gb(t, e, &g, &b) gives the lane's gamma and beta of its value e of k-step t.
template <typename T, int KS, typename GB>
__device__ __forceinline__ void rows_layernorm(typename Mfma<T>::frag (&buf)[KS], const GB& gb,
                                               float eps) {
  constexpr int K = KS * 32;
  float v[KS][8];
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < KS; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[t][e] = to_f32(buf[t][e]);
      s += v[t][e];
    }
  s += __shfl_xor(s, 16, 64);
  s += __shfl_xor(s, 32, 64);
  const float mean = s * (1.f / K);
  float q = 0.f;
#pragma unroll
  for (int t = 0; t < KS; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[t][e] -= mean;
      q += v[t][e] * v[t][e];
    }
  q += __shfl_xor(q, 16, 64);
  q += __shfl_xor(q, 32, 64);
  const float rstd = rsqrtf(q * (1.f / K) + eps);
#pragma unroll
  for (int t = 0; t < KS; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float g, b;
      gb(t, e, g, b);
      buf[t][e] = from_f32<T>(v[t][e] * rstd * g + b);
    }
}


}  // namespace tel
