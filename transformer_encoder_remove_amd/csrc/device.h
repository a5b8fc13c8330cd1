// Device-side helpers shared by the library's HIP kernels (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tel {

typedef _Float16 f16;
typedef __bf16 bf16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// 16 bytes of elements, the unit of every vector global load/store here.
template <typename T> struct alignas(16) Vec16 {
  static constexpr int N = 16 / sizeof(T);
  T v[N];
};
// 4 elements (8 bytes for 16-bit types, 16 for fp32): the epilogue store unit.
template <typename T> struct alignas(4 * sizeof(T)) Vec4 { T v[4]; };

// ------------------------------------------------------------------ MFMA 16x16 shapes
// One wavefront computes D[16][16] += A[16][K] * B[K][16]. Lane l holds KPL consecutive
// k of A row (l % 16) and of B column (l % 16), at k offset KPL * (l / 16) (the same
// mapping for both operands, which is all a dot product needs); it receives
// D[4 * (l / 16) + i][l % 16] for i = 0..3.
template <typename T> struct Mfma;

template <> struct Mfma<f16> {
  static constexpr int KPL = 8;                 // 16x16x32
  typedef f16x8 frag;
  typedef f32x4 acc;
  __device__ __forceinline__ static acc mma(frag a, frag b, acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<bf16> {
  static constexpr int KPL = 8;                 // 16x16x32
  typedef bf16x8 frag;
  typedef f32x4 acc;
  __device__ __forceinline__ static acc mma(frag a, frag b, acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  static constexpr int KPL = 1;                 // 16x16x4
  typedef float frag;
  typedef f32x4 acc;
  __device__ __forceinline__ static acc mma(frag a, frag b, acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<int8_t> {
  static constexpr int KPL = 16;                // 16x16x64, int32 accumulation
  typedef i32x4 frag;
  typedef i32x4 acc;
  __device__ __forceinline__ static acc mma(frag a, frag b, acc c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  }
};

// ------------------------------------------------------------------ sparse MFMA 16x16x64
// D[16][16] += A[16][64] * B[64][16] with A 2:4-sparse along k (two non-zeros in every
// group of four), gfx950 v_smfmac_f32_16x16x64_{f16,bf16}. Lane l (row l % 16, lane group
// a = l / 16) holds the 8 kept values of A row l % 16 at dense k [16a, 16a + 16), two per
// group of four in increasing k, and in bits 4g .. 4g+3 of its index word the positions
// (0..3) of the two values of group g (first in the low two bits). B: lane l holds column
// l % 16 at k [8a, 8a + 8) in elements 0..7 and k [32 + 8a, 32 + 8a + 8) in elements 8..15.
// D as for the dense shapes. (Layout established by probing the instruction.)
template <typename T> struct Smfma;
template <> struct Smfma<f16> {
  typedef f16x8 afrag;
  typedef f16x16 bfrag;
  typedef f32x4 acc;
  __device__ __forceinline__ static acc mma(afrag a, bfrag b, acc c, int idx) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, b, c, idx, 0, 0);
  }
};
template <> struct Smfma<bf16> {
  typedef bf16x8 afrag;
  typedef bf16x16 bfrag;
  typedef f32x4 acc;
  __device__ __forceinline__ static acc mma(afrag a, bfrag b, acc c, int idx) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a, b, c, idx, 0, 0);
  }
};

// ------------------------------------------------------------------ wavefront reductions
template <int G> __device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
template <int G> __device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Max-abs statistics of the dynamically scaled int8 layer. Many workgroups raise one such
// statistic at the end of a short kernel, nearly at once, and device atomics on one address
// serialise (a few ns each: ~3 us for the ~360 workgroups of a LayerNorm). So a statistic
// is kept in AMAX_SLOTS copies 128 bytes apart, workgroup w raises copy w % AMAX_SLOTS, and
// its reader folds the copies (amax_fold). Non-negative floats order like their bit
// patterns, so the unsigned atomic max is exact and independent of arrival order.
constexpr int AMAX_SLOTS = 64, AMAX_STRIDE = 32;              // copies, floats apart
constexpr size_t AMAX_STAT_FLOATS = (size_t)AMAX_SLOTS * AMAX_STRIDE;

__device__ __forceinline__ void amax_raise(float* stat, float m) {
  const unsigned int wg = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  atomicMax(reinterpret_cast<unsigned int*>(stat + (wg % AMAX_SLOTS) * AMAX_STRIDE),
            __float_as_uint(m));
}

// The statistic's value, in every lane of the calling wavefront (all 64 lanes must call).
__device__ __forceinline__ float amax_fold(const float* stat) {
  return group_max<64>(stat[(threadIdx.x & 63) * AMAX_STRIDE]);
}

// A workgroup of nw wavefronts raises a statistic with one global atomic: each wavefront
// folds its maximum into lds[0] with an LDS atomic max, then increments the counter lds[1];
// the wavefront that brings the counter to nw (its increment is ordered after every other
// wavefront's maximum) raises the statistic. There is no barrier, so wavefronts that have
// already left (a GEMM's producers) are not waited for. lds[0] and lds[1] must hold 0
// before any wavefront gets here, and each of the nw wavefronts calls this once.
__device__ __forceinline__ void wg_atomic_max(float m, float* stat, unsigned int* lds, int nw) {
  m = group_max<64>(m);
  if ((threadIdx.x & 63) == 0) {
    __hip_atomic_fetch_max(&lds[0], __float_as_uint(m), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    const unsigned int n = __hip_atomic_fetch_add(&lds[1], 1u, __ATOMIC_ACQ_REL,
                                                  __HIP_MEMORY_SCOPE_WORKGROUP);
    if (n == (unsigned int)nw - 1) {
      const unsigned int v = __hip_atomic_load(&lds[0], __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_WORKGROUP);
      amax_raise(stat, __uint_as_float(v));
    }
  }
}

// ------------------------------------------------------------------ shifted windows
// Token order maps of the shifted-window block. Image order: row b * Hs * Ws + y * Ws + x.
// Window order: windows row-major inside each image, images outermost, tokens row-major
// inside a window (p = py * M + px). The block computes on the cyclically shifted image
// (roll by -s on both axes), so window-order row r holds image row src(r) with
// y = (wy * M + py + s) mod Hs, x = (wx * M + px + s) mod Ws. The same map serves the
// gather before attention and the scatter (window reverse + roll by +s) after it.
struct SwinGeom {
  int Hs, Ws, M, s;   // image height/width, window size, shift
  int nWx, nW, N;     // windows per image row, windows per image, tokens per window

  __device__ __forceinline__ int src_row(int r) const {
    const int per_img = nW * N;
    const int b = r / per_img, rem = r - b * per_img;
    const int w = rem / N, p = rem - w * N;
    const int wy = w / nWx, wx = w - wy * nWx;
    const int py = p / M, px = p - py * M;
    int y = wy * M + py + s, x = wx * M + px + s;
    if (y >= Hs) y -= Hs;
    if (x >= Ws) x -= Ws;
    return b * Hs * Ws + y * Ws + x;
  }
  // Patch merging (the downsampling between stages): merged token r of the (Hs/2) x (Ws/2)
  // grid, part k = 0..3, reads image row (2i + (k & 1), 2j + (k >> 1)) of the Hs x Ws
  // image, i.e. the parts in (row, column) offset order (0,0), (1,0), (0,1), (1,1).
  __device__ __forceinline__ int merge_src(int r, int k) const {
    const int Wo = Ws >> 1, per_img = (Hs >> 1) * Wo;
    const int b = r / per_img, rem = r - b * per_img;
    const int i = rem / Wo, j = rem - i * Wo;
    return b * Hs * Ws + (2 * i + (k & 1)) * Ws + 2 * j + (k >> 1);
  }
  // Shift-mask region of window-order token p of window w (image-local window index):
  // per axis, [0, L-M) -> 0, [L-M, L-s) -> 1, [L-s, L) -> 2 in the shifted frame; no mask
  // (one region) when s == 0.
  __device__ __forceinline__ int region(int w, int p) const {
    if (s == 0) return 0;
    const int wy = w / nWx, wx = w - wy * nWx;
    const int py = p / M, px = p - py * M;
    const int Y = wy * M + py, X = wx * M + px;
    const int ry = Y < Hs - M ? 0 : (Y < Hs - s ? 1 : 2);
    const int rx = X < Ws - M ? 0 : (X < Ws - s ? 1 : 2);
    return 3 * ry + rx;
  }
};

// Wait until at most N of this wavefront's vector memory operations are outstanding.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup `wg` of `nwg` reads its share of [p, p + bytes) (16-byte aligned; a tail under
// 16 bytes is skipped) once and discards it: a later kernel then finds those bytes cached
// instead of in HBM. The reads are direct global -> LDS copies into one 1 KiB scratch slot
// that every wavefront overwrites (a copy into LDS is never dropped as unused, unlike a load
// into registers whose value nothing reads); all of them have landed before the return.
__device__ inline void read_ahead(const void* p, size_t bytes, int wg, int nwg) {
  __shared__ __attribute__((aligned(1024))) char slot[1024];
  const char* q = (const char*)p;
  const size_t n16 = bytes / 16;
  const size_t stride = (size_t)nwg * blockDim.x;
  for (size_t i = (size_t)wg * blockDim.x + threadIdx.x; i < n16; i += stride)
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(q + i * 16),
                                     (void __attribute__((address_space(3)))*)slot, 16, 0, 0);
  wait_vmcnt<0>();
}

// GELU with the exact (erf) form, 0.5 z (1 + erf(z / sqrt 2)). erf comes from the rational
// approximation of Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.26 (after
// Hastings): erf(x) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2), t = 1 / (1 + p x),
// x >= 0, absolute error at most 1.5e-7; odd symmetry for x < 0. Substituting it gives, for
// either sign of z, GELU(z) = max(z, 0) - |z| t Q(t) exp(-z^2 / 2) with x = |z| / sqrt 2 and
// Q = (a1 + t (a2 + ...)) / 2: one reciprocal, one exp2, four FMAs for Q and five other
// operations (no 1 - erf cancellation for negative z), below half an ulp of the 16-bit
// outputs it feeds (float32 max error 3.3e-7 against the exact function on [-12, 12]).
__device__ __forceinline__ float gelu_erf(float z) {
  const float a = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752f, a, 1.0f));
  const float q = fmaf(fmaf(fmaf(fmaf(0.5f * 1.061405429f, t, 0.5f * -1.453152027f), t,
                                 0.5f * 1.421413741f), t, 0.5f * -0.284496736f), t,
                       0.5f * 0.254829592f);
  const float e = __builtin_amdgcn_exp2f((z * z) * (-0.5f * 1.4426950408889634f));
  return fmaf(-(a * t) * q, e, fmaxf(z, 0.0f));
}

}  // namespace tel
