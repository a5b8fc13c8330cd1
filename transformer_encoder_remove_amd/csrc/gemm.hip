// Projection GEMMs of the encoder layer on gfx950 MFMA, with fused epilogues.
//
// C[m][n] = epilogue(sum_k A[m][k] * W[n][k]) for activations A [M][K] (M = packed tokens)
// and weights W [N][K] (nn.Linear layout). Both operands are K-contiguous, which is the
// operand layout MFMA wants, so no transpose is needed anywhere.
//
// Epilogues are the fusions of the Swin talk ("大規模なビジュアル モデル…", section 3:
// GEMM + bias, GEMM + bias + activation, QKV GEMM + bias written in the layout the
// attention kernel reads) and of the Kuaishou article (Fig. 6). Where the post-op is
// LayerNorm the bias and residual are added here and the LayerNorm runs in its own
// kernel, as that talk advises for complex post-ops.
//
// Kernel design (CDNA4, 64-wide wavefronts):
//  * workgroup tile BM tokens x BN weight rows, BK-deep k slices staged through LDS,
//    double-buffered: the next slice is fetched into registers (16-byte global loads,
//    8 consecutive threads cover a 128-byte row segment) while MFMAs consume the
//    current one; one barrier per slice;
//  * LDS rows padded by 16 bytes so that both the 16-byte stores and the fragment
//    reads (16 rows x 16 bytes per quarter-wave) hit distinct banks;
//  * WM x WN wavefronts, each owning a (BM/WM) x (BN/WN) sub-tile of 16x16 MFMA blocks;
//  * the weight tile is the MFMA A operand and the activation tile the B operand, so a
//    lane receives 4 consecutive output columns n of one token row m: the epilogue reads
//    4 biases with one 16-byte load and stores 4 outputs with one 8-byte store;
//  * ragged M and N: rows past the end are clamped on load (their results are never
//    stored); K % (16 bytes) == 0 is required, slices past K are zero-filled.
#include <type_traits>

#include <algorithm>
#include <cmath>

#include "device.h"
#include "launch.h"
#include "rows.h"

namespace tel {

// Epilogue operands. The residual and the output of EPI_BIAS_RESID may be float32
// (TR, TO) so that a bf16 layer can keep its pre-LayerNorm sums and residual stream in
// float32. With int8 operands the int32 accumulator is dequantised by a per-column scale
// (dq[n] = activation scale x weight scale); an int8 output (TO = int8_t) is quantised
// again for the next int8 GEMM: the value is first rounded to fp16, the storage type it
// would otherwise have, then q = clamp(rne(v * qinv), -127, 127).
template <typename T, typename TR, typename TO> struct EpiArgs {
  const float* bias;
  const TR* resid;
  TO* C;
  int M, N, heads;
  const float* dq;     // int8 operands: per-column dequantisation scale [N]
  const float* qinv;   // int8 output: device scalar, 1 / activation scale of the consumer
  SwinGeom geom;       // EPI_SWIN_SCATTER: window order -> image order
  const float* dyn_amax = nullptr;   // int8 operands, dynamic scale: dq = s_w, s_a from max-abs
  float* out_amax = nullptr;         // EPI_BIAS_GELU_AMAX: max-abs statistic of the stored
                                     // outputs (AMAX_SLOTS copies, amax_raise)
};

constexpr bool epi_gelu(int epi) { return epi == EPI_BIAS_GELU || epi == EPI_BIAS_GELU_AMAX; }

// Activation scale of a dynamically scaled int8 GEMM: max-abs / 127 (1 for an all-zero input).
__device__ __forceinline__ float dyn_act_scale(const float* amax) {
  const float a = *amax;
  return a > 0.f ? a / 127.f : 1.f;
}

__device__ __forceinline__ int8_t quantize_code(float v, float inv) {
  const float r = __builtin_rintf((float)(f16)v * inv);
  return (int8_t)fminf(fmaxf(r, -127.f), 127.f);
}

// Returns the max-abs of the stored outputs for EPI_BIAS_GELU_AMAX, 0 otherwise.
template <int EPI, typename T, typename TR, typename TO, typename ACC>
__device__ __forceinline__ float epilogue_store(const EpiArgs<T, TR, TO>& e, int m, int n,
                                                ACC acc) {
  if constexpr (EPI == EPI_PARTIAL && sizeof(TO) == 2) {
    // partial sums rounded to the 16-bit output type
    Vec4<TO> out;
#pragma unroll
    for (int i = 0; i < 4; ++i) out.v[i] = from_f32<TO>(acc[i]);
    *reinterpret_cast<Vec4<TO>*>(e.C + (size_t)m * e.N + n) = out;
    return 0.f;
  } else if constexpr (EPI == EPI_RAW_I32 || EPI == EPI_PARTIAL) {
    // the raw 32-bit accumulators (int32 for int8 operands), no epilogue arithmetic
    *reinterpret_cast<ACC*>(reinterpret_cast<int32_t*>(e.C) + (size_t)m * e.N + n) = acc;
    return 0.f;
  } else {
    const float4 b = EPI == EPI_PLAIN ? make_float4(0.f, 0.f, 0.f, 0.f)
                                      : *reinterpret_cast<const float4*>(e.bias + n);
    float v[4];
    if constexpr (std::is_same<T, int8_t>::value) {
      float4 d = *reinterpret_cast<const float4*>(e.dq + n);
      if (e.dyn_amax) {   // per-column dequantisation scale s_a * s_w[n], formed here
        const float sa = dyn_act_scale(e.dyn_amax);
        d = make_float4(sa * d.x, sa * d.y, sa * d.z, sa * d.w);
      }
      v[0] = (float)acc[0] * d.x + b.x;
      v[1] = (float)acc[1] * d.y + b.y;
      v[2] = (float)acc[2] * d.z + b.z;
      v[3] = (float)acc[3] * d.w + b.w;
    } else {
      v[0] = acc[0] + b.x;
      v[1] = acc[1] + b.y;
      v[2] = acc[2] + b.z;
      v[3] = acc[3] + b.w;
    }
    Vec4<TO> out;
    size_t idx;
    if constexpr (epi_gelu(EPI)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = gelu_erf(v[i]);
    }
    if constexpr (EPI == EPI_BIAS_RESID || EPI == EPI_SWIN_SCATTER) {
      // the scatter epilogue reads the residual at the image-order row it writes
      const size_t row = EPI == EPI_SWIN_SCATTER ? (size_t)e.geom.src_row(m) : (size_t)m;
      const Vec4<TR> r = *reinterpret_cast<const Vec4<TR>*>(e.resid + row * e.N + n);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += to_f32(r.v[i]);
    }
    if constexpr (EPI == EPI_QKV_SPLIT) {
      // [3][heads][M][d]: the attention kernel reads each head's Q, K and V as
      // contiguous [tokens][d] blocks.
      const int H = e.N / 3, d = H / e.heads;
      const int which = n / H, rem = n - which * H, hh = rem / d, c = rem - hh * d;
      idx = (((size_t)which * e.heads + hh) * e.M + m) * d + c;
    } else if constexpr (EPI == EPI_SWIN_SCATTER) {
      idx = (size_t)e.geom.src_row(m) * e.N + n;
    } else {
      idx = (size_t)m * e.N + n;
    }
    if constexpr (std::is_same<TO, int8_t>::value) {
      // head-split int8 output (int8 attention): Q, K and V each at its own scale
      const float inv = EPI == EPI_QKV_SPLIT ? e.qinv[n / (e.N / 3)] : *e.qinv;
#pragma unroll
      for (int i = 0; i < 4; ++i) out.v[i] = quantize_code(v[i], inv);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) out.v[i] = from_f32<TO>(v[i]);
    }
    *reinterpret_cast<Vec4<TO>*>(e.C + idx) = out;
    float am = 0.f;
    if constexpr (EPI == EPI_BIAS_GELU_AMAX) {
#pragma unroll
      for (int i = 0; i < 4; ++i) am = fmaxf(am, fabsf(to_f32(out.v[i])));
    }
    return am;
  }
}

// The same epilogue on 8 consecutive columns n..n+7 of row m (n % 8 == 0), with the
// column constants (bias bb, int8 dequantisation dd) and the residual r already in
// registers: one 16-byte store for 16-bit outputs, 8 bytes for int8 codes, 2 x 16 bytes for
// float32 and int32.
template <typename T8> struct alignas(sizeof(T8) * 8) Vec8 { T8 v[8]; };

template <int EPI, typename T, typename TR, typename TO>
__device__ __forceinline__ float epilogue_apply8(const EpiArgs<T, TR, TO>& e, int m, int n,
                                                 const float* acc, const float* bb,
                                                 const float* dd, const Vec8<TR>& r) {
  if constexpr (EPI == EPI_PARTIAL && sizeof(TO) == 2) {
    Vec8<TO> o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o.v[i] = from_f32<TO>(acc[i]);
    *reinterpret_cast<Vec8<TO>*>(e.C + (size_t)m * e.N + n) = o;
    return 0.f;
  } else if constexpr (EPI == EPI_RAW_I32 || EPI == EPI_PARTIAL) {
    Vec8<int32_t> o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o.v[i] = __float_as_int(acc[i]);   // staged as raw bits
    *reinterpret_cast<Vec8<int32_t>*>(reinterpret_cast<int32_t*>(e.C) + (size_t)m * e.N + n) = o;
    return 0.f;
  } else {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (std::is_same<T, int8_t>::value) v[i] = (float)__float_as_int(acc[i]) * dd[i] + bb[i];
      else v[i] = acc[i] + bb[i];
    }
    if constexpr (epi_gelu(EPI)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = gelu_erf(v[i]);
    }
    size_t row = (size_t)m;
    if constexpr (EPI == EPI_SWIN_SCATTER) row = (size_t)e.geom.src_row(m);
    if constexpr (EPI == EPI_BIAS_RESID || EPI == EPI_SWIN_SCATTER) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += to_f32(r.v[i]);
    }
    size_t idx;
    if constexpr (EPI == EPI_QKV_SPLIT) {
      const int H = e.N / 3, d = H / e.heads;
      const int which = n / H, rem = n - which * H, hh = rem / d, c = rem - hh * d;
      idx = (((size_t)which * e.heads + hh) * e.M + m) * d + c;
    } else {
      idx = row * e.N + n;
    }
    Vec8<TO> out;
    if constexpr (std::is_same<TO, int8_t>::value) {
      const float inv = EPI == EPI_QKV_SPLIT ? e.qinv[n / (e.N / 3)] : *e.qinv;
#pragma unroll
      for (int i = 0; i < 8; ++i) out.v[i] = quantize_code(v[i], inv);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) out.v[i] = from_f32<TO>(v[i]);
    }
    // non-temporal: the output is read by the next kernel, on other XCDs; leaving it
    // dirty in this XCD's L2 only lengthens the write-back at the end of the kernel
    if constexpr (sizeof(Vec8<TO>) == 16) {
      u32x4 bits;
      __builtin_memcpy(&bits, &out, 16);
      __builtin_nontemporal_store(bits, reinterpret_cast<u32x4*>(e.C + idx));
    } else if constexpr (sizeof(Vec8<TO>) == 8) {
      u32x2 bits;
      __builtin_memcpy(&bits, &out, 8);
      __builtin_nontemporal_store(bits, reinterpret_cast<u32x2*>(e.C + idx));
    } else {
      *reinterpret_cast<Vec8<TO>*>(e.C + idx) = out;
    }
    float am = 0.f;
    if constexpr (EPI == EPI_BIAS_GELU_AMAX) {
#pragma unroll
      for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(to_f32(out.v[i])));
    }
    return am;
  }
}

template <typename T, int BM, int BN, int BK, int WM, int WN, int EPI, typename TR, typename TO>
__global__ __launch_bounds__(WM* WN * 64) void gemm_nt_kernel(const T* __restrict__ A,
                                                              const T* __restrict__ W, int K,
                                                              EpiArgs<T, TR, TO> e) {
  using MF = Mfma<T>;
  typedef typename MF::frag frag;
  constexpr int NT = WM * WN * 64;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int LDK = BK + VEC;
  constexpr int KPL = MF::KPL, KMF = 4 * KPL;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int VPR = BK / VEC;
  constexpr int LA = BM * VPR / NT, LW = BN * VPR / NT;
  static_assert(BM * VPR % NT == 0 && BN * VPR % NT == 0, "tile/thread mismatch");
  static_assert(TM % 16 == 0 && TN % 16 == 0 && BK % KMF == 0, "bad tile");

  __shared__ __attribute__((aligned(16))) T sA[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) T sW[2][BN * LDK];
  __shared__ unsigned int amax_lds[2];   // EPI_BIAS_GELU_AMAX: workgroup max-abs, counter
  if constexpr (EPI == EPI_BIAS_GELU_AMAX) {
    if (threadIdx.x == 0) amax_lds[0] = amax_lds[1] = 0u;   // before the first barrier
  }

  const int M = e.M, N = e.N;
  const int tiles_m = (M + BM - 1) / BM;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int lr = lane & 15, lg = lane >> 4;

  // Per-thread global load coordinates, fixed across k slices: thread t loads the
  // 16-byte vector (t % VPR) of rows t / VPR + i * RSTEP of each tile.
  constexpr int RSTEP = NT / VPR;
  static_assert(NT % VPR == 0, "threads per row");
  const int row0 = tid / VPR, kv = (tid % VPR) * VEC;
  const T* gA = A + kv;
  const T* gW = W + kv;
  size_t offA[LA], offW[LW];
#pragma unroll
  for (int i = 0; i < LA; ++i) offA[i] = (size_t)min(m0 + row0 + i * RSTEP, M - 1) * K;
#pragma unroll
  for (int i = 0; i < LW; ++i) offW[i] = (size_t)min(n0 + row0 + i * RSTEP, N - 1) * K;
  const int lds_st = row0 * LDK + kv;

  u32x4 ga[LA], gw[LW];   // 16 raw bytes per vector; native vectors stay in VGPRs
#define TEL_GEMM_FETCH(k0)                                                                  \
  do {                                                                                      \
    const bool kin = (k0) + kv < K;                                                         \
    _Pragma("unroll") for (int i = 0; i < LA; ++i) ga[i] =                                  \
        kin ? *reinterpret_cast<const u32x4*>(gA + offA[i] + (k0)) : u32x4{0u, 0u, 0u, 0u}; \
    _Pragma("unroll") for (int i = 0; i < LW; ++i) gw[i] =                                  \
        kin ? *reinterpret_cast<const u32x4*>(gW + offW[i] + (k0)) : u32x4{0u, 0u, 0u, 0u}; \
  } while (0)
#define TEL_GEMM_STASH(buf)                                                                 \
  do {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < LA; ++i)                                          \
        *reinterpret_cast<u32x4*>(&sA[buf][lds_st + i * RSTEP * LDK]) = ga[i];              \
    _Pragma("unroll") for (int i = 0; i < LW; ++i)                                          \
        *reinterpret_cast<u32x4*>(&sW[buf][lds_st + i * RSTEP * LDK]) = gw[i];              \
  } while (0)

  typename MF::acc acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = typename MF::acc{};

  const int nk = (K + BK - 1) / BK;
  TEL_GEMM_FETCH(0);
  TEL_GEMM_STASH(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) TEL_GEMM_FETCH((kt + 1) * BK);
    const T* tA = sA[buf] + (wm * TM + lr) * LDK + lg * KPL;
    const T* tW = sW[buf] + (wn * TN + lr) * LDK + lg * KPL;
#pragma unroll
    for (int kk = 0; kk < BK; kk += KMF) {
      frag fa[FN], fb[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i) fa[i] = *reinterpret_cast<const frag*>(tW + i * 16 * LDK + kk);
#pragma unroll
      for (int j = 0; j < FM; ++j) fb[j] = *reinterpret_cast<const frag*>(tA + j * 16 * LDK + kk);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = MF::mma(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < nk) TEL_GEMM_STASH(buf ^ 1);
    __syncthreads();
  }

  float am = 0.f;
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int n = n0 + wn * TN + i * 16 + lg * 4;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = m0 + wm * TM + j * 16 + lr;
      if (m < M && n < N) am = fmaxf(am, epilogue_store<EPI, T, TR, TO>(e, m, n, acc[i][j]));
    }
  }
  if constexpr (EPI == EPI_BIAS_GELU_AMAX) wg_atomic_max(am, e.out_amax, amax_lds, WM * WN);
#undef TEL_GEMM_FETCH
#undef TEL_GEMM_STASH
}

// ------------------------------------------------------------------ pipelined variant
// Same contract as gemm_nt_kernel, for K % (128 bytes) == 0. Warp-specialised:
//  * WM x WN compute wavefronts read MFMA fragments from LDS and run the MFMAs;
//  * DENSE_PRODUCERS producer wavefronts copy k-slices from global memory straight into LDS with the
//    gfx950 direct path (global_load_lds_dwordx4: lane i's 16 bytes land at LDS base +
//    16 * i, no VGPR staging), keeping S - 1 slices in flight in an S-stage LDS ring.
// One barrier per slice: a producer passes barrier kt once slice kt has landed (its own
// vmcnt), a compute wave reaches it once its reads of slice kt - 1 are done; after it the
// producers refill the stage of slice kt - 1. Keeping the copies out of the compute
// wavefronts matters for the schedule: with copies in the same instruction stream the
// compiler's wait-count analysis waits for every outstanding LDS read before each MFMA
// block, serialising LDS reads and MFMAs. Compute wavefronts double-buffer fragments in
// registers: the next k-step's reads (also across a slice boundary) are issued before
// the current k-step's MFMAs. Several producers: one wavefront can have at most 63 copies
// outstanding, and the loops are bound by how fast each compute unit streams its operands,
// which more copies in flight raise.
//
// LDS rows are 128 bytes (8 chunks of 16 bytes) with no padding; bank conflicts are avoided
// by an XOR swizzle: chunk c of row r is stored in slot c ^ (r % 8). A copy instruction
// fills a block of 8 rows (1 KiB); lane i fills slot i % 8 of row i / 8, so it fetches chunk
// (i % 8) ^ (i / 8) of that row: 8 lanes still cover each 128-byte row segment.
//
// Workgroup -> tile order is XCD-aware: the dispatcher hands consecutive workgroup ids to
// the 8 XCDs in turn, so ids are regrouped so that each XCD walks a contiguous run of
// tiles (M-fastest), i.e. the tiles that share weight columns share that XCD's L2.

// Producer wavefronts per workgroup: four in the dense kernel (measured against two at
// BERT-base shapes, bit-identical results: FFN2's 64x128 tile 21.3 -> 18.4 us, QKV 15.7 ->
// 14.8, O 8.4 -> 7.7, FFN1 19.4 -> 18.8), two in the 2:4-sparse kernel, whose stages are
// split between exactly two (a 59-block stage as 30 + 29).
constexpr int PIPE_PRODUCERS = 2;
constexpr int DENSE_PRODUCERS = 4;

__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

__device__ __forceinline__ int xcd_tile(int bid, int ntiles) {
  constexpr int NX = 8;
  const int per = ntiles / NX, extra = ntiles % NX;   // the first `extra` XCDs get one more
  const int x = bid % NX, i = bid / NX;
  if (i >= per + (x < extra ? 1 : 0)) return bid;     // unreachable when grid == ntiles
  return x * per + min(x, extra) + i;
}

// The largest divisor of n that is at most 8 (epilogue passes grouped for their loads).
constexpr int group_passes(int n) {
  for (int g = 8; g > 1; --g)
    if (n % g == 0) return g;
  return 1;
}

// Epilogue of the pipelined kernels, for one compute wavefront's TM x TN accumulators
// (lane: 4 consecutive columns n of one row m per 16x16 block, the MFMA output layout).
template <int EPI, typename T, typename TR, typename TO, int TM, int TN, typename ACC, int FN,
          int FM>
__device__ __forceinline__ void pipe_epilogue(const ACC (&acc)[FN][FM], char* smem,
                                              const EpiArgs<T, TR, TO>& e, int m0, int n0,
                                              int wm, int wn, int wave, int lane,
                                              unsigned int* amax_lds = nullptr, int nw = 0) {
  const int M = e.M, N = e.N;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int LDC = TN + 4;                       // floats per staged epilogue row
  // Epilogue through LDS. Every copy has landed and every real fragment read is done
  // (the producers drained before the last barrier), so the ring is free: each wavefront
  // parks its TM x TN accumulators there (row m, 4 consecutive n per lane), then reads
  // them back as 8 consecutive columns per lane so that 8 lanes cover one 128-byte row
  // segment of the output, and applies the epilogue per 8-column chunk.
  float* stg = reinterpret_cast<float*>(smem) + wave * TM * LDC;
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      float4 v;
      if constexpr (std::is_same<T, int8_t>::value) {
        v = make_float4(__int_as_float(acc[i][j][0]), __int_as_float(acc[i][j][1]),
                        __int_as_float(acc[i][j][2]), __int_as_float(acc[i][j][3]));
      } else {
        v = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
      *reinterpret_cast<float4*>(stg + (j * 16 + lr) * LDC + i * 16 + lg * 4) = v;
    }
  // Lane -> (row rr of every pass, 8-column chunk c8): the chunk is fixed per lane, so
  // the column constants are loaded once; RP rows per pass, lanes past RP * CPR idle.
  constexpr int CPR = TN / 8;
  constexpr int RP = 64 / CPR;
  constexpr int NPASS = (TM + RP - 1) / RP;
  constexpr int GP = group_passes(NPASS);     // passes whose residuals are loaded together
  static_assert(TN % 8 == 0 && CPR <= 64 && NPASS % GP == 0, "epilogue chunking");
  const int c8 = lane % CPR, rr = lane / CPR;
  const int n = n0 + wn * TN + c8 * 8;
  const bool lane_on = rr < RP && n < N;
  const bool full8 = n + 8 <= N && (EPI != EPI_QKV_SPLIT || ((N / 3) / e.heads) % 8 == 0);
  constexpr bool IS_I8 = std::is_same<T, int8_t>::value;
  constexpr bool HAS_R = EPI == EPI_BIAS_RESID || EPI == EPI_SWIN_SCATTER;
  float bb[8], dd[8];
  float am = 0.f;   // EPI_BIAS_GELU_AMAX: this lane's max-abs of its stored outputs
#pragma unroll
  for (int i = 0; i < 8; ++i) bb[i] = dd[i] = 0.f;
  if constexpr (EPI != EPI_RAW_I32 && EPI != EPI_PARTIAL) {
    if (lane_on && full8) {
      const float4 b0 = *reinterpret_cast<const float4*>(e.bias + n);
      const float4 b1 = *reinterpret_cast<const float4*>(e.bias + n + 4);
      bb[0] = b0.x; bb[1] = b0.y; bb[2] = b0.z; bb[3] = b0.w;
      bb[4] = b1.x; bb[5] = b1.y; bb[6] = b1.z; bb[7] = b1.w;
      if constexpr (IS_I8) {
        const float4 d0 = *reinterpret_cast<const float4*>(e.dq + n);
        const float4 d1 = *reinterpret_cast<const float4*>(e.dq + n + 4);
        dd[0] = d0.x; dd[1] = d0.y; dd[2] = d0.z; dd[3] = d0.w;
        dd[4] = d1.x; dd[5] = d1.y; dd[6] = d1.z; dd[7] = d1.w;
        if (e.dyn_amax) {   // dynamic activation scale: s_a * s_w[n]
          const float sa = dyn_act_scale(e.dyn_amax);
#pragma unroll
          for (int i = 0; i < 8; ++i) dd[i] = sa * dd[i];
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < NPASS / GP; ++g) {
    // residual rows of GP passes first (loads issued back to back), then the stores
    Vec8<TR> rv[GP];
    if constexpr (HAS_R) {
#pragma unroll
      for (int q = 0; q < GP; ++q) {
        const int r = rr + RP * (g * GP + q), m = m0 + wm * TM + r;
        if (lane_on && full8 && r < TM && m < M) {
          size_t row = (size_t)m;
          if constexpr (EPI == EPI_SWIN_SCATTER) row = (size_t)e.geom.src_row(m);
          rv[q] = *reinterpret_cast<const Vec8<TR>*>(e.resid + row * N + n);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < GP; ++q) {
      const int r = rr + RP * (g * GP + q), m = m0 + wm * TM + r;
      if (!lane_on || r >= TM || m >= M) continue;
      float v[8];
      const float4 a0 = *reinterpret_cast<const float4*>(stg + r * LDC + c8 * 8);
      const float4 a1 = *reinterpret_cast<const float4*>(stg + r * LDC + c8 * 8 + 4);
      v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
      v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
      if (full8) {
        am = fmaxf(am, epilogue_apply8<EPI, T, TR, TO>(e, m, n, v, bb, dd, rv[q]));
      } else {   // ragged N (N % 8 == 4) or head_dim % 8 == 4: two 4-column stores
        ACC lo, hi;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (IS_I8) {
            lo[i] = __float_as_int(v[i]);
            hi[i] = __float_as_int(v[4 + i]);
          } else {
            lo[i] = v[i];
            hi[i] = v[4 + i];
          }
        }
        am = fmaxf(am, epilogue_store<EPI, T, TR, TO>(e, m, n, lo));
        if (n + 4 < N) am = fmaxf(am, epilogue_store<EPI, T, TR, TO>(e, m, n + 4, hi));
      }
    }
  }
  if constexpr (EPI == EPI_BIAS_GELU_AMAX) wg_atomic_max(am, e.out_amax, amax_lds, nw);
}

template <typename T, int BM, int BN, int WM, int WN, int S, int EPI, typename TR, typename TO>
__global__ __launch_bounds__((WM * WN + DENSE_PRODUCERS) * 64) void gemm_nt_pipe_kernel(
    const T* __restrict__ A, const T* __restrict__ W, int K, int splits, int gn,
    EpiArgs<T, TR, TO> e) {
  using MF = Mfma<T>;
  typedef typename MF::frag frag;
  constexpr int NW = WM * WN;                       // compute wavefronts
  constexpr int VEC = 16 / sizeof(T);
  constexpr int BK = 8 * VEC;                       // 128-byte rows
  constexpr int KPL = MF::KPL, KMF = 4 * KPL;
  constexpr int KS = BK / KMF;                      // k-steps per slice (even)
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int NB = (BM + BN) / 8;                 // 1 KiB blocks per slice
  constexpr int LJ = NB / DENSE_PRODUCERS;           // copies per producer per slice
  constexpr int STAGE = (BM + BN) * 128;
  constexpr int INFLIGHT = LJ * (S - 2) < 63 ? LJ * (S - 2) : 63;
  static_assert(NB % DENSE_PRODUCERS == 0 && BM % 8 == 0 && BN % 8 == 0, "copy split");
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile");
  static_assert(KS % 2 == 0, "k-steps per slice must be even");
  static_assert(S >= 2, "stages");

  constexpr int LDC = TN + 4;                       // floats per staged epilogue row
  constexpr int STAGED = TM * LDC * 4 * NW;         // epilogue staging bytes
  __shared__ __attribute__((aligned(1024))) char smem[S * STAGE > STAGED ? S * STAGE : STAGED];
  __shared__ unsigned int amax_lds[2];   // EPI_BIAS_GELU_AMAX: workgroup max-abs, counter
  if constexpr (EPI == EPI_BIAS_GELU_AMAX) {
    // compute wavefront 0 clears them; every wavefront passes the first barrier after this
    if (threadIdx.x == 0) {
      amax_lds[0] = amax_lds[1] = 0u;
      wait_lgkmcnt0();
    }
  }

  const int M = e.M, N = e.N;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  // blockIdx -> (output tile, k-split). Each XCD (own L2) takes a contiguous run of the
  // tile order, and the order walks groups of gn tile columns row by row, so one XCD's
  // tiles form a compact block of rows x columns that share their A rows and W columns
  // in its L2. The k-splits of a tile are neighbours in the run.
  const int ts = xcd_tile(blockIdx.x, gridDim.x);
  const int tile = ts / splits, split = ts - tile * splits;
  const int g = tile / (tiles_m * gn), r = tile - g * (tiles_m * gn);
  const int gw = min(gn, tiles_n - g * gn);
  const int tm = r / gw, tn = g * gn + (r - (r / gw) * gw);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nk = K / BK / splits;                   // k-slices of this split
  A += (size_t)split * nk * BK;
  W += (size_t)split * nk * BK;
  if constexpr (EPI == EPI_PARTIAL) e.C += (size_t)split * M * N;

  if (wave >= NW) {
    // ---------------- producer: block b = p + DENSE_PRODUCERS * j of every slice
    const int p = wave - NW;
    const T* src[LJ];
    const int chunk = (lane & 7) ^ (lane >> 3);
#pragma unroll
    for (int j = 0; j < LJ; ++j) {
      const int b = p + DENSE_PRODUCERS * j;
      if (b < BM / 8) {
        src[j] = A + (size_t)min(m0 + b * 8 + (lane >> 3), M - 1) * K + chunk * VEC;
      } else {
        src[j] = W + (size_t)min(n0 + (b - BM / 8) * 8 + (lane >> 3), N - 1) * K + chunk * VEC;
      }
    }
    // copy k-slice `data` into the stage of slice number `slot`
    auto issue = [&](int slot, int data) {
      char* dst = smem + (slot % S) * STAGE + p * 1024;
      const size_t koff = (size_t)data * BK;
#pragma unroll
      for (int j = 0; j < LJ; ++j)
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(src[j] + koff),
            (void __attribute__((address_space(3)))*)(dst + j * DENSE_PRODUCERS * 1024), 16, 0, 0);
    };
#pragma unroll
    for (int s = 0; s < S - 1; ++s) issue(s, min(s, nk - 1));
    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt<INFLIGHT>();                   // slice kt has landed
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue(kt + S - 1, min(kt + S - 1, nk - 1));   // into the stage of slice kt - 1
    }
    wait_vmcnt<0>();   // every copy has landed before the LDS is reused for the epilogue
    __builtin_amdgcn_s_barrier();   // matches the compute wavefronts' final barrier
    return;
  }

  // ---------------- compute wavefronts
  const int wm = wave % WM, wn = wave / WM;
  const int lr = lane & 15, lg = lane >> 4;
  const int xr = lr & 7;
  const int rowA = (wm * TM + lr) * 128, rowW = BM * 128 + (wn * TN + lr) * 128;
  frag fa[2][FN], fb[2][FM];
#define TEL_PIPE_FRAGS(buf, slice, kk)                                                      \
  do {                                                                                      \
    const char* st_ = smem + ((slice) % S) * STAGE;                                         \
    const int k_ = (kk) * KMF + lg * KPL;                                                   \
    const int off_ = (((k_ / VEC) ^ xr) * 16) + (k_ % VEC) * (int)sizeof(T);                \
    _Pragma("unroll") for (int i = 0; i < FN; ++i) fa[buf][i] =                            \
        *reinterpret_cast<const frag*>(st_ + rowW + i * 16 * 128 + off_);                   \
    _Pragma("unroll") for (int j = 0; j < FM; ++j) fb[buf][j] =                            \
        *reinterpret_cast<const frag*>(st_ + rowA + j * 16 * 128 + off_);                   \
  } while (0)

  typename MF::acc acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = typename MF::acc{};

  // Materialise the epilogue's kernel arguments before the loop: a scalar load still in
  // flight there would make the compiler wait for every LDS read before each MFMA block.
  asm volatile("" ::"s"(e.bias), "s"(e.resid), "s"(e.C), "s"(e.N), "s"(e.M), "s"(e.heads),
               "s"(e.dq), "s"(e.qinv), "s"(e.dyn_amax));
  if constexpr (EPI == EPI_BIAS_GELU_AMAX) asm volatile("" ::"s"(e.out_amax));
  if constexpr (EPI == EPI_SWIN_SCATTER)
    asm volatile("" ::"s"(e.geom.Hs), "s"(e.geom.Ws), "s"(e.geom.M), "s"(e.geom.s),
                 "s"(e.geom.nWx), "s"(e.geom.nW), "s"(e.geom.N));
  __builtin_amdgcn_s_barrier();                     // slice 0 has landed
  asm volatile("" ::: "memory");
  TEL_PIPE_FRAGS(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < KS) {
        TEL_PIPE_FRAGS(cur ^ 1, kt, kk + 1);
      } else {
        // Branch-free on purpose (a conditional here makes the compiler wait for every
        // outstanding LDS read before the MFMAs below). After the last slice this is one
        // extra barrier, matched by the producers, and a read nobody uses.
        wait_lgkmcnt0();                            // reads of slice kt are done
        __builtin_amdgcn_s_barrier();               // slice kt + 1 has landed
        asm volatile("" ::: "memory");
        TEL_PIPE_FRAGS(cur ^ 1, min(kt + 1, nk - 1), 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = MF::mma(fa[cur][i], fb[cur][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#undef TEL_PIPE_FRAGS

  pipe_epilogue<EPI, T, TR, TO, TM, TN>(acc, smem, e, m0, n0, wm, wn, wave, lane, amax_lds, NW);
}

// ------------------------------------------------------------------ 2:4 sparse weights
// C = epilogue(A W^T) with W pruned 2:4 along k and stored compressed: Wv [N][K/2] (the two
// kept weights of every group of four, increasing k) and Wi [N][K/16] (one 16-bit word per
// 16 k; group g's two positions in bits 4g..4g+3), which is the operand form of the sparse
// MFMA (Smfma). The weight tile is the sparse A operand, so the epilogue is the dense
// kernel's. Same pipeline as gemm_nt_pipe_kernel, with 128 dense k per slice: a stage holds
// the activation rows (256 bytes: two 128-byte halves, chunk c of row r in slot c ^ (r % 8)
// like the dense rows), the compressed weight rows (128 bytes, same swizzle) and the index
// rows (16 bytes), each part a whole number of 1 KiB copy blocks; one sparse MFMA covers
// 64 dense k, two per slice. Half the weight bytes cross HBM and LDS, and each MFMA does
// the work of two dense ones.
template <typename T, int BM, int BN, int WM, int WN, int S, int EPI, typename TR, typename TO>
__global__ __launch_bounds__((WM * WN + PIPE_PRODUCERS) * 64) void gemm_sp_pipe_kernel(
    const T* __restrict__ A, const T* __restrict__ Wv, const uint16_t* __restrict__ Wi, int K,
    int gn, EpiArgs<T, TR, TO> e) {
  using SM = Smfma<T>;
  typedef typename SM::afrag afrag;
  typedef typename SM::bfrag bfrag;
  constexpr int NW = WM * WN;
  constexpr int BK = 128;                           // dense k per slice
  constexpr int NB_A = BM / 4, NB_W = BN / 8, NB_I = BN / 64;   // 1 KiB copy blocks
  constexpr int NB = NB_A + NB_W + NB_I;
  // copies per producer per slice: producer 0 takes the odd block out when NB is odd
  constexpr int LJ0 = (NB + 1) / PIPE_PRODUCERS, LJ1 = NB / PIPE_PRODUCERS;
  constexpr int STAGE = NB * 1024;
  constexpr int W_OFF = NB_A * 1024, I_OFF = (NB_A + NB_W) * 1024;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  static_assert(BN % 64 == 0 && BM % 8 == 0 && PIPE_PRODUCERS == 2, "copy split");
  static_assert(TM % 16 == 0 && TN % 16 == 0 && S >= 2, "wave tile, stages");
  constexpr int LDC = TN + 4;
  constexpr int STAGED = TM * LDC * 4 * NW;
  __shared__ __attribute__((aligned(1024))) char smem[S * STAGE > STAGED ? S * STAGE : STAGED];

  const int M = e.M, N = e.N;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int g = tile / (tiles_m * gn), r = tile - g * (tiles_m * gn);
  const int gw = min(gn, tiles_n - g * gn);
  const int tm = r / gw, tn = g * gn + (r - (r / gw) * gw);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nk = K / BK;

  if (wave >= NW) {
    // ---------------- producer: block b = p + PIPE_PRODUCERS * j of every slice; lane i of
    // a block fills bytes 16 i .. 16 i + 15 of it
    const int p = wave - NW;
    auto produce = [&](auto lj_c) {
    constexpr int LJ = decltype(lj_c)::value;
    constexpr int INFLIGHT = LJ * (S - 2) < 63 ? LJ * (S - 2) : 63;
    const char* src[LJ];
    int step[LJ];                                   // bytes of the block's rows per slice
    const int sub = lane >> 3, slot = lane & 7;
#pragma unroll
    for (int j = 0; j < LJ; ++j) {
      const int b = p + PIPE_PRODUCERS * j;
      if (b < NB_A) {                               // activation: half rows 8b .. 8b + 7
        const int hr = 8 * b + sub, row = hr >> 1, half = hr & 1;
        const int chunk = slot ^ (row & 7);
        src[j] = reinterpret_cast<const char*>(A + (size_t)min(m0 + row, M - 1) * K +
                                               half * 64 + chunk * 8);
        step[j] = BK * 2;
      } else if (b < NB_A + NB_W) {                 // compressed weights: rows 8 b' ..
        const int row = 8 * (b - NB_A) + sub, chunk = slot ^ (row & 7);
        src[j] = reinterpret_cast<const char*>(Wv + (size_t)min(n0 + row, N - 1) * (K / 2) +
                                               chunk * 8);
        step[j] = BK;
      } else {                                      // index words: rows 64 b'' + lane
        const int row = 64 * (b - NB_A - NB_W) + lane;
        src[j] = reinterpret_cast<const char*>(Wi + (size_t)min(n0 + row, N - 1) * (K / 16));
        step[j] = BK / 8;
      }
    }
    auto issue = [&](int slot_no, int data) {
      char* dst = smem + (slot_no % S) * STAGE + p * 1024;
#pragma unroll
      for (int j = 0; j < LJ; ++j)
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(src[j] + (size_t)data * step[j]),
            (void __attribute__((address_space(3)))*)(dst + j * PIPE_PRODUCERS * 1024), 16, 0, 0);
    };
#pragma unroll
    for (int s = 0; s < S - 1; ++s) issue(s, min(s, nk - 1));
    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt<INFLIGHT>();                   // slice kt has landed
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue(kt + S - 1, min(kt + S - 1, nk - 1));   // into the stage of slice kt - 1
    }
    wait_vmcnt<0>();
    };
    if (p == 0) produce(std::integral_constant<int, LJ0>{});
    else produce(std::integral_constant<int, LJ1>{});
    __builtin_amdgcn_s_barrier();   // matches the compute wavefronts' final barrier
    return;
  }

  // ---------------- compute wavefronts
  const int wm = wave % WM, wn = wave / WM;
  const int lr = lane & 15, lg = lane >> 4;
  const int xr = lr & 7;
  const int rowA = (wm * TM + lr) * 256;
  const int rowW = W_OFF + (wn * TN + lr) * 128, rowI = I_OFF + (wn * TN + lr) * 16;
  typename SM::acc acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = typename SM::acc{};
  asm volatile("" ::"s"(e.bias), "s"(e.resid), "s"(e.C), "s"(e.N), "s"(e.M), "s"(e.heads));

  if constexpr (FN >= 8) {
    // Wide wave tile (TN >= 128 weight rows): too many registers to double-buffer both
    // operands, so the activation fragments (8 registers each) go through a two-slot ring
    // one column block ahead, while the weight fragments of the next k-step are loaded two
    // per column block during the current one. The slice barrier sits in the last column
    // block of the second k-step, after the last read of the old slice.
    afrag wa[2][FN];
    int wi[2][FN];
    bfrag br[2];
#define TEL_SPW_W(buf, slice, kk, i)                                                        \
  do {                                                                                      \
    const char* st_ = smem + ((slice) % S) * STAGE;                                         \
    wa[buf][i] = *reinterpret_cast<const afrag*>(st_ + rowW + (i) * 16 * 128 +              \
                                                 ((((kk) * 4 + lg) ^ xr) * 16));            \
    wi[buf][i] = *reinterpret_cast<const uint16_t*>(st_ + rowI + (i) * 16 * 16 +            \
                                                    ((kk) * 4 + lg) * 2);                   \
  } while (0)
#define TEL_SPW_B(r, slice, kk, j)                                                          \
  do {                                                                                      \
    const char* a_ = smem + ((slice) % S) * STAGE + rowA + (j) * 16 * 256 + (kk) * 128;     \
    const afrag lo_ = *reinterpret_cast<const afrag*>(a_ + ((lg ^ xr) * 16));               \
    const afrag hi_ = *reinterpret_cast<const afrag*>(a_ + (((lg + 4) ^ xr) * 16));         \
    br[r] = __builtin_shufflevector(lo_, hi_, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13,  \
                                    14, 15);                                                \
  } while (0)
    __builtin_amdgcn_s_barrier();                   // slice 0 has landed
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < FN; ++i) TEL_SPW_W(0, 0, 0, i);
    TEL_SPW_B(0, 0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
      for (int j = 0; j < FM; ++j) {               // k-step 0 of slice kt
        if (j + 1 < FM) TEL_SPW_B((j + 1) & 1, kt, 0, j + 1);
        else TEL_SPW_B(FM & 1, kt, 1, 0);
#pragma unroll
        for (int i = j * FN / FM; i < (j + 1) * FN / FM; ++i) TEL_SPW_W(1, kt, 1, i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < FN; ++i) acc[i][j] = SM::mma(wa[0][i], br[j & 1], acc[i][j], wi[0][i]);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < FM; ++j) {               // k-step 1 of slice kt
        const int r = (FM + j) & 1;                 // ring slot holding column block j
        if (j + 1 < FM) {
          TEL_SPW_B(r ^ 1, kt, 1, j + 1);
        } else {
          wait_lgkmcnt0();                          // reads of slice kt are done
          __builtin_amdgcn_s_barrier();             // slice kt + 1 has landed
          asm volatile("" ::: "memory");
          const int nx = min(kt + 1, nk - 1);
          TEL_SPW_B(r ^ 1, nx, 0, 0);
#pragma unroll
          for (int i = 0; i < FN; ++i) TEL_SPW_W(0, nx, 0, i);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < FN; ++i) acc[i][j] = SM::mma(wa[1][i], br[r], acc[i][j], wi[1][i]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#undef TEL_SPW_W
#undef TEL_SPW_B
    pipe_epilogue<EPI, T, TR, TO, TM, TN>(acc, smem, e, m0, n0, wm, wn, wave, lane);
    return;
  }

  afrag fa[2][FN];
  int fi[2][FN];
  bfrag fb[2][FM];
#define TEL_SP_FRAGS(buf, slice, kk)                                                        \
  do {                                                                                      \
    const char* st_ = smem + ((slice) % S) * STAGE;                                         \
    const int wc_ = ((((kk) * 4 + lg) ^ xr) * 16);                                          \
    _Pragma("unroll") for (int i = 0; i < FN; ++i) {                                        \
      fa[buf][i] = *reinterpret_cast<const afrag*>(st_ + rowW + i * 16 * 128 + wc_);        \
      fi[buf][i] = *reinterpret_cast<const uint16_t*>(st_ + rowI + i * 16 * 16 +            \
                                                      ((kk) * 4 + lg) * 2);                 \
    }                                                                                       \
    _Pragma("unroll") for (int j = 0; j < FM; ++j) {                                        \
      const char* a_ = st_ + rowA + j * 16 * 256 + (kk) * 128;                              \
      const afrag lo_ = *reinterpret_cast<const afrag*>(a_ + ((lg ^ xr) * 16));             \
      const afrag hi_ = *reinterpret_cast<const afrag*>(a_ + (((lg + 4) ^ xr) * 16));       \
      fb[buf][j] = __builtin_shufflevector(lo_, hi_, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11,  \
                                           12, 13, 14, 15);                                 \
    }                                                                                       \
  } while (0)

  __builtin_amdgcn_s_barrier();                     // slice 0 has landed
  asm volatile("" ::: "memory");
  TEL_SP_FRAGS(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int cur = kk & 1;
      if (kk == 0) {
        TEL_SP_FRAGS(1, kt, 1);
      } else {
        wait_lgkmcnt0();                            // reads of slice kt are done
        __builtin_amdgcn_s_barrier();               // slice kt + 1 has landed
        asm volatile("" ::: "memory");
        TEL_SP_FRAGS(0, min(kt + 1, nk - 1), 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = SM::mma(fa[cur][i], fb[cur][j], acc[i][j], fi[cur][i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#undef TEL_SP_FRAGS
  pipe_epilogue<EPI, T, TR, TO, TM, TN>(acc, smem, e, m0, n0, wm, wn, wave, lane);
}

// ------------------------------------------------------------------ skinny GEMMs
// Narrow, HBM-bound GEMMs of the shifted-window block (channels 96: QKV 96 -> 288, proj
// 96 -> 96, fc1 96 -> 384, fc2 384 -> 96, over ~2e5 tokens). A tile narrower than N
// would re-read the token matrix once per tile column; here each workgroup keeps the
// whole weight matrix (N x K <= 384 x 96 or 96 x 384) in LDS and owns full output rows, so
// every token row is read exactly once. At channels 192 (stage 2: QKV 192 -> 576, proj
// 192 -> 192, fc1 192 -> 768) a workgroup holds a 192-column slice of the weights (75 KiB),
// and the slices run side by side, each reading the token rows once. Persistent: a workgroup walks row blocks of 64
// tokens (16 per wavefront) with a stride of the grid, holding the token fragments of its
// next two blocks in registers while it computes the current one. The weight tile is the
// MFMA A operand, so each lane ends with 4 consecutive columns of one token and the
// 4-column epilogue above (bias, GELU, QKV split, window scatter, residual) applies as is.

// Output fragments in groups of G and k in chunks of KC steps (6 and 3; 4 and 1 for the
// 8-wavefront patch-merging workgroup), with scheduling barriers between them: the live
// weight fragments stay at G x KC instead of the whole weight slice, which keeps two or three
// wavefronts per SIMD resident.
template <typename T, int NF, int KS, int EPI, typename TR, typename TO, int KC = 3, int G = 6>
__device__ __forceinline__ void rows_block(const typename Mfma<T>::frag (&a)[KS], const T* sW,
                                           const EpiArgs<T, TR, TO>& e, int row0, int lr,
                                           int lg, int n0) {
  using MF = Mfma<T>;
  constexpr int LDW = KS * 32 + 8;
  static_assert(NF % G == 0 && KS % KC == 0, "fragment groups");
  const int m = row0 + lr;
#pragma unroll
  for (int g = 0; g < NF / G; ++g) {
    typename MF::acc acc[G];
#pragma unroll
    for (int i = 0; i < G; ++i) acc[i] = typename MF::acc{};
#pragma unroll
    for (int t0 = 0; t0 < KS; t0 += KC) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = t0; t < t0 + KC; ++t)
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const typename MF::frag w = *reinterpret_cast<const typename MF::frag*>(
              sW + ((g * G + i) * 16 + lr) * LDW + t * 32 + lg * 8);
          acc[i] = MF::mma(w, a[t], acc[i]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (m < e.M) {
#pragma unroll
      for (int i = 0; i < G; ++i)
        epilogue_store<EPI, T, TR, TO>(e, m, n0 + (g * G + i) * 16 + lg * 4, acc[i]);
    }
  }
}

// LayerNorm parameters of the A operand: up to K = 96 the lane keeps its gamma / beta in
// registers; wider rows (patch merging, K = 384) would need 2 * K / 4 registers, so they
// are staged in LDS beside the weights and read per value (lanes of one lg read the same
// address: a broadcast).
template <int KS> constexpr bool ln_in_lds() { return KS > 3; }

template <typename T, int NF, int KS, bool LNA>
constexpr int rows_lds_bytes() {
  return NF * 16 * (KS * 32 + 8) * (int)sizeof(T) + (LNA && ln_in_lds<KS>() ? 2 * KS * 32 * 4 : 0);
}

// NTH threads: 256 (4 wavefronts, 64 rows per step), or 512 for the fp16 patch-merging shape,
// whose workgroup has a compute unit's LDS to itself and needs more rows in flight.
template <typename T, int NF, int KS, int EPI, typename TR, typename TO, bool LNA, int MODE,
          int NTH = 256>
__global__ __launch_bounds__(NTH, KS == 6 ? 2 : 1) void gemm_rows_kernel(const T* __restrict__ A,
                                                        const T* __restrict__ W,
                                                        EpiArgs<T, TR, TO> e,
                                                        const float* __restrict__ ln_g,
                                                        const float* __restrict__ ln_b,
                                                        float ln_eps) {
  using MF = Mfma<T>;
  static_assert(MF::KPL == 8, "16-bit operands");
  constexpr int N = NF * 16, K = KS * 32, LDW = K + 8;
  constexpr bool GB_LDS = LNA && ln_in_lds<KS>();
  __shared__ __attribute__((aligned(16))) char smem_rows[rows_lds_bytes<T, NF, KS, LNA>()];
  T* sW = reinterpret_cast<T*>(smem_rows);
  float* sG = reinterpret_cast<float*>(smem_rows + N * LDW * sizeof(T));
  float* sB = sG + K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int RWG = NTH / 64 * 16;   // rows per workgroup step
  // column slice blockIdx.y: weight rows [n0, n0 + N) of an e.N-wide output
  const int n0 = blockIdx.y * N;
  W += (size_t)n0 * K;
  for (int idx = tid; idx < N * (K / 8); idx += NTH) {
    const int r = idx / (K / 8), c = idx - r * (K / 8);
    *reinterpret_cast<u32x4*>(sW + r * LDW + c * 8) =
        *reinterpret_cast<const u32x4*>(W + (size_t)r * K + c * 8);
  }
  if constexpr (GB_LDS) {
    for (int k = tid; k < K; k += NTH) {
      sG[k] = ln_g[k];
      sB[k] = ln_b[k];
    }
  }
  __syncthreads();
  const int M = e.M, stride = gridDim.x * RWG;
  // the lane's gamma / beta of the A-operand LayerNorm: k = t * 32 + lg * 8 + j
  constexpr int KR = LNA && !GB_LDS ? KS : 1;
  float lg_g[KR][8], lg_b[KR][8];
  if constexpr (LNA && !GB_LDS) {
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int j = 0; j < 8; j += 4) {
        const float4 gv = *reinterpret_cast<const float4*>(ln_g + t * 32 + lg * 8 + j);
        const float4 bv = *reinterpret_cast<const float4*>(ln_b + t * 32 + lg * 8 + j);
        lg_g[t][j] = gv.x; lg_g[t][j + 1] = gv.y; lg_g[t][j + 2] = gv.z; lg_g[t][j + 3] = gv.w;
        lg_b[t][j] = bv.x; lg_b[t][j + 1] = bv.y; lg_b[t][j + 2] = bv.z; lg_b[t][j + 3] = bv.w;
      }
  }
  auto gb = [&](int t, int j, float& g, float& b) {
    if constexpr (GB_LDS) {
      g = sG[t * 32 + lg * 8 + j];
      b = sB[t * 32 + lg * 8 + j];
    } else {
      g = lg_g[t][j];
      b = lg_b[t][j];
    }
  };
  auto layernorm = [&](typename MF::frag (&buf)[KS]) {
    if constexpr (GB_LDS) rows_layernorm_wide<T, KS>(buf, sG, sB, lg, ln_eps);
    else rows_layernorm<T, KS>(buf, gb, ln_eps);
  };
  int rb = blockIdx.x * RWG + wave * 16;   // this wavefront's 16 rows of the block
  if constexpr (NTH == 512) {
    // 8 wavefronts per compute unit: one row block in registers per wavefront, the other
    // wavefronts' work covers the load latency
    typename MF::frag a0[KS];
    for (; rb < M; rb += stride) {
      rows_load<T, KS, MODE>(a0, A, M, rb, lr, lg, e.geom);
      if constexpr (LNA) layernorm(a0);
      rows_block<T, NF, KS, EPI, TR, TO, 1, 4>(a0, sW, e, rb, lr, lg, 0);   // never sliced
    }
    return;
  }
  // K 192 holds 12 token fragments in registers: output groups of 4 keep the QKV split's
  // epilogue within two wavefronts per SIMD
  constexpr int GR = KS == 6 ? 4 : 6;
  typename MF::frag a0[KS], a1[KS];
  if (rb < M) rows_load<T, KS, MODE>(a0, A, M, rb, lr, lg, e.geom);
  if (rb + stride < M) rows_load<T, KS, MODE>(a1, A, M, rb + stride, lr, lg, e.geom);
  for (; rb < M; rb += 2 * stride) {
    if constexpr (LNA) layernorm(a0);
    rows_block<T, NF, KS, EPI, TR, TO, 3, GR>(a0, sW, e, rb, lr, lg, n0);
    if (rb + 2 * stride < M) rows_load<T, KS, MODE>(a0, A, M, rb + 2 * stride, lr, lg, e.geom);
    if (rb + stride >= M) break;
    if constexpr (LNA) layernorm(a1);
    rows_block<T, NF, KS, EPI, TR, TO, 3, GR>(a1, sW, e, rb + stride, lr, lg, n0);
    if (rb + 3 * stride < M) rows_load<T, KS, MODE>(a1, A, M, rb + 3 * stride, lr, lg, e.geom);
  }
}

template <typename T, int NF, int KS>
static hipError_t launch_rows_nk(const GemmArgs& a, hipStream_t stream) {
  // persistent: two workgroups per CU when one takes <= 80 KiB of LDS, else one; the
  // one-per-CU shape (patch merging) runs 8 wavefronts per workgroup in fp16 (bf16's
  // conversions need a few more registers than 8 wavefronts leave: 4 wavefronts there)
  // An output wider than the NF * 16 columns whose weights one workgroup holds runs as
  // column slices (grid y), each reading every token row once: N / (NF * 16) reads of the
  // token matrix instead of one, still far below a tiled kernel's.
  const int per_cu = rows_lds_bytes<T, NF, KS, true>() <= 80 * 1024 ? 2 : 1;
  constexpr int NTH = (NF == 12 && KS == 12 && std::is_same<T, f16>::value) ? 512 : 256;
  const int rows_wg = NTH / 64 * 16;
  const int blocks = (a.M + rows_wg - 1) / rows_wg;
  if (a.N % (NF * 16)) return hipErrorInvalidValue;
  const int slices = a.N / (NF * 16);
  const dim3 grid(std::max(1, std::min(blocks, 256 * per_cu / slices)), slices);
#define TEL_ROWS_LN(EPI, LNA, MODE)                                                          \
  do {                                                                                       \
    EpiArgs<T, T, T> e{a.bias, (const T*)a.resid, (T*)a.C, a.M, a.N, a.heads, a.dq, a.qinv, \
                       a.geom};                                                              \
    gemm_rows_kernel<T, NF, KS, EPI, T, T, LNA, MODE, NTH><<<grid, NTH, 0, stream>>>(       \
        (const T*)a.A, (const T*)a.W, e, a.ln_g, a.ln_b, a.ln_eps);                         \
  } while (0)
#define TEL_ROWS(EPI) TEL_ROWS_LN(EPI, false, ROWS_PLAIN)
  if constexpr (NF == 12 && KS == 12) {   // patch merging only: gather of four rows, LN, no bias
    if (!a.ln_g || !a.ln_b || !a.ln_merge || a.epi != EPI_PLAIN) return hipErrorInvalidValue;
    TEL_ROWS_LN(EPI_PLAIN, true, ROWS_MERGE);
    return hipGetLastError();
  } else {
  if (a.ln_g) {   // A-operand LayerNorm: the shifted-window block's LN1 (+ partition) and LN2
    if (!a.ln_b) return hipErrorInvalidValue;
    if (a.ln_merge) return hipErrorInvalidValue;
    if (a.epi == EPI_QKV_SPLIT && a.ln_gather) TEL_ROWS_LN(EPI_QKV_SPLIT, true, ROWS_WINDOW);
    else if (a.epi == EPI_QKV_SPLIT) TEL_ROWS_LN(EPI_QKV_SPLIT, true, ROWS_PLAIN);
    else if (a.epi == EPI_BIAS_GELU && !a.ln_gather) TEL_ROWS_LN(EPI_BIAS_GELU, true, ROWS_PLAIN);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  switch (a.epi) {
    case EPI_BIAS: TEL_ROWS(EPI_BIAS); break;
    case EPI_BIAS_GELU: TEL_ROWS(EPI_BIAS_GELU); break;
    case EPI_BIAS_RESID: TEL_ROWS(EPI_BIAS_RESID); break;
    case EPI_QKV_SPLIT: TEL_ROWS(EPI_QKV_SPLIT); break;
    case EPI_SWIN_SCATTER: TEL_ROWS(EPI_SWIN_SCATTER); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
  }
#undef TEL_ROWS
#undef TEL_ROWS_LN
}

bool gemm_rows_supported(int dtype, int N, int K) {
  if (dtype != DT_F16 && dtype != DT_BF16) return false;
  return (N == 288 && K == 96) || (N == 96 && K == 96) || (N == 384 && K == 96) ||
         (N == 96 && K == 384) || (K == 192 && (N == 192 || N == 576 || N == 768));
}

bool patch_merging_supported(int dtype, int channels) {
  return (dtype == DT_F16 || dtype == DT_BF16) && channels == 96;
}

// The (N, K) shapes the skinny kernel is built for; false: use the tiled kernels.
template <typename T>
static bool launch_rows(const GemmArgs& a, hipStream_t stream, hipError_t* err) {
  if (a.resid_f32 || a.out_f32) return false;
  if (a.N == 288 && a.K == 96) *err = launch_rows_nk<T, 18, 3>(a, stream);
  else if (a.N == 96 && a.K == 96) *err = launch_rows_nk<T, 6, 3>(a, stream);
  else if (a.N == 384 && a.K == 96) *err = launch_rows_nk<T, 24, 3>(a, stream);
  else if (a.N == 96 && a.K == 384) *err = launch_rows_nk<T, 6, 12>(a, stream);
  // channels 192 (Swin stage 2): QKV 576, proj 192 and fc1 768 columns as 192-column slices
  else if (a.K == 192 && (a.N == 192 || a.N == 576 || a.N == 768) && !a.ln_merge)
    *err = launch_rows_nk<T, 12, 6>(a, stream);
  else if (a.N == 192 && a.K == 384 && a.ln_merge) *err = launch_rows_nk<T, 12, 12>(a, stream);
  else return false;
  return true;
}

// ------------------------------------------------------------------ dispatch
// Tile configurations. The register-staged kernel (gemm_nt_kernel) serves K that is not a
// multiple of 128 bytes; every other shape uses the pipelined kernel with one of these
// tiles (the GEMM-configuration tuning of the Kuaishou article, Fig. 11).
struct PipeCfg { int bm, bn, wm, wn, s; };
constexpr PipeCfg PIPE_CFGS[] = {
    {128, 256, 2, 4, 3},   // 0: 8 waves, wave tile 64x64, 144 KiB LDS
    {128, 192, 2, 4, 3},   // 1: 8 waves, wave tile 64x48, 120 KiB
    {128, 128, 2, 2, 4},   // 2: 4 waves, wave tile 64x64, 128 KiB
    {64, 128, 2, 4, 4},    // 3: 8 waves, wave tile 32x32, 96 KiB
    {64, 64, 2, 2, 4},     // 4: 4 waves, wave tile 32x32, 64 KiB
    {128, 256, 2, 2, 3},   // 5: 4 waves, wave tile 64x128, 144 KiB
    {256, 128, 2, 2, 3},   // 6: 4 waves, wave tile 128x64, 144 KiB
    {128, 128, 2, 2, 2},   // 7: 4 waves, wave tile 64x64, 64 KiB (two workgroups per CU)
    {64, 128, 2, 2, 4},    // 8: 4 waves, wave tile 32x64, 96 KiB
    {192, 192, 2, 4, 3},   // 9: 8 waves, wave tile 96x48, 144 KiB
    {96, 128, 2, 4, 4},    // 10: 8 waves, wave tile 48x32, 112 KiB
    {32, 64, 2, 2, 4},     // 11: 4 waves, wave tile 16x32, 48 KiB
};
constexpr int N_PIPE_CFGS = sizeof(PIPE_CFGS) / sizeof(PIPE_CFGS[0]);

// Tiles of the 2:4-sparse kernel (stage = BM/4 + BN/8 + BN/64 KiB of copy blocks).
constexpr PipeCfg SP_CFGS[] = {
    {64, 128, 2, 4, 4},    // 0: 8 waves, wave tile 32x32, 136 KiB
    {128, 128, 2, 2, 3},   // 1: 4 waves, wave tile 64x64, 150 KiB
    {64, 256, 2, 4, 2},    // 2: 8 waves, wave tile 32x64, 104 KiB
    {128, 256, 2, 2, 2},   // 3: 4 waves, wave tile 64x128 (activation ring), 136 KiB
    {128, 192, 2, 2, 2},   // 4: 4 waves, wave tile 64x96, 118 KiB (59 blocks: 30 + 29)
};
constexpr int N_SP_CFGS = sizeof(SP_CFGS) / sizeof(SP_CFGS[0]);

template <typename T, int BM, int BN, int WM, int WN, int EPI, typename TR, typename TO>
static void launch_one(const GemmArgs& a, hipStream_t stream) {
  constexpr int BK = 128 / sizeof(T);   // 128-byte k slices
  EpiArgs<T, TR, TO> e{a.bias, (const TR*)a.resid, (TO*)a.C, a.M, a.N, a.heads, a.dq, a.qinv, a.geom};
  e.dyn_amax = a.dyn_amax;
  e.out_amax = a.out_amax;
  const int grid = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  gemm_nt_kernel<T, BM, BN, BK, WM, WN, EPI, TR, TO><<<grid, WM * WN * 64, 0, stream>>>(
      (const T*)a.A, (const T*)a.W, a.K, e);
}

// Width (in tile columns) of the column groups of the tile order: one XCD's run of
// about tiles / 8 consecutive tiles then covers rows x cols = ceil(per / gn) x gn tiles,
// and streams (rows * BM + cols * BN) k-long operand rows through its L2; take the width
// that minimises that, a width that does not divide the column count paying for its
// ragged last group (ties: the wider group). When the run is longer than the 32 tiles an
// XCD's compute units hold at once (several rounds), what the L2 can reuse is the window of
// tiles resident together, so the width minimises that window's operand rows instead: at
// BERT-large's 13,537 tokens FFN1 (1,696 tiles) took 160 -> 150 us and QKV 108 -> 103 us.
static int xcd_group_width(int tiles_m, int tiles_n, int bm, int bn) {
  constexpr long XCD_CUS = 32;
  const long per = std::min<long>(((long)tiles_m * tiles_n + 7) / 8, XCD_CUS);
  int best = tiles_n;
  long best_cost = -1;
  for (int gn = 1; gn <= tiles_n; ++gn) {
    const long rows = std::min<long>((per + gn - 1) / gn, tiles_m);
    const long cols = std::min<long>(gn, per);
    const long cost = rows * bm + cols * bn + (tiles_n % gn ? bn / 2 : 0);
    if (best_cost < 0 || cost <= best_cost) {
      best_cost = cost;
      best = gn;
    }
  }
  return best;
}

template <typename T, int C, int EPI, typename TR, typename TO>
static void launch_pipe(const GemmArgs& a, hipStream_t stream) {
  constexpr PipeCfg c = PIPE_CFGS[C];
  EpiArgs<T, TR, TO> e{a.bias, (const TR*)a.resid, (TO*)a.C, a.M, a.N, a.heads, a.dq, a.qinv, a.geom};
  e.dyn_amax = a.dyn_amax;
  e.out_amax = a.out_amax;
  const int tm = (a.M + c.bm - 1) / c.bm, tn = (a.N + c.bn - 1) / c.bn;
  const int grid = tm * tn * a.splits;
  gemm_nt_pipe_kernel<T, c.bm, c.bn, c.wm, c.wn, c.s, EPI, TR, TO>
      <<<grid, (c.wm * c.wn + DENSE_PRODUCERS) * 64, 0, stream>>>(
          (const T*)a.A, (const T*)a.W, a.K, a.splits, xcd_group_width(tm, tn, c.bm, c.bn), e);
}

template <typename T, int C, int EPI, typename TR, typename TO>
static void launch_sp(const GemmArgs& a, hipStream_t stream) {
  constexpr PipeCfg c = SP_CFGS[C];
  EpiArgs<T, TR, TO> e{a.bias, (const TR*)a.resid, (TO*)a.C, a.M, a.N, a.heads, a.dq, a.qinv, a.geom};
  const int tm = (a.M + c.bm - 1) / c.bm, tn = (a.N + c.bn - 1) / c.bn;
  gemm_sp_pipe_kernel<T, c.bm, c.bn, c.wm, c.wn, c.s, EPI, TR, TO>
      <<<tm * tn, (c.wm * c.wn + PIPE_PRODUCERS) * 64, 0, stream>>>(
          (const T*)a.A, (const T*)a.W, a.w_idx, a.K, xcd_group_width(tm, tn, c.bm, c.bn), e);
}

template <typename T, int EPI, typename TR, typename TO>
static void launch_sp_cfg(int cfg, const GemmArgs& a, hipStream_t stream) {
  switch (cfg) {
    case 0: launch_sp<T, 0, EPI, TR, TO>(a, stream); break;
    case 1: launch_sp<T, 1, EPI, TR, TO>(a, stream); break;
    case 2: launch_sp<T, 2, EPI, TR, TO>(a, stream); break;
    case 3: launch_sp<T, 3, EPI, TR, TO>(a, stream); break;
    default: launch_sp<T, 4, EPI, TR, TO>(a, stream); break;
  }
}

template <typename T>
static hipError_t run_epi_sp(int cfg, const GemmArgs& a, hipStream_t stream) {
  switch (a.epi) {
    case EPI_BIAS: launch_sp_cfg<T, EPI_BIAS, T, T>(cfg, a, stream); break;
    case EPI_BIAS_GELU: launch_sp_cfg<T, EPI_BIAS_GELU, T, T>(cfg, a, stream); break;
    case EPI_QKV_SPLIT: launch_sp_cfg<T, EPI_QKV_SPLIT, T, T>(cfg, a, stream); break;
    case EPI_BIAS_RESID:
      if constexpr (std::is_same<T, bf16>::value) {
        if (a.resid_f32 && a.out_f32) {
          launch_sp_cfg<T, EPI_BIAS_RESID, float, float>(cfg, a, stream);
          break;
        }
        if (a.out_f32 && !a.resid_f32) {
          launch_sp_cfg<T, EPI_BIAS_RESID, T, float>(cfg, a, stream);
          break;
        }
      }
      if (a.resid_f32 || a.out_f32) return hipErrorInvalidValue;
      launch_sp_cfg<T, EPI_BIAS_RESID, T, T>(cfg, a, stream);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// cfg < 0: register-staged 64x64 kernel; otherwise PIPE_CFGS[cfg].
template <typename T, int EPI, typename TR, typename TO>
static void launch_cfg(int cfg, const GemmArgs& a, hipStream_t stream) {
  switch (cfg) {
    case 0: launch_pipe<T, 0, EPI, TR, TO>(a, stream); break;
    case 1: launch_pipe<T, 1, EPI, TR, TO>(a, stream); break;
    case 2: launch_pipe<T, 2, EPI, TR, TO>(a, stream); break;
    case 3: launch_pipe<T, 3, EPI, TR, TO>(a, stream); break;
    case 4: launch_pipe<T, 4, EPI, TR, TO>(a, stream); break;
    case 5: launch_pipe<T, 5, EPI, TR, TO>(a, stream); break;
    case 6: launch_pipe<T, 6, EPI, TR, TO>(a, stream); break;
    case 7: launch_pipe<T, 7, EPI, TR, TO>(a, stream); break;
    case 8: launch_pipe<T, 8, EPI, TR, TO>(a, stream); break;
    case 9: launch_pipe<T, 9, EPI, TR, TO>(a, stream); break;
    case 10: launch_pipe<T, 10, EPI, TR, TO>(a, stream); break;
    case 11: launch_pipe<T, 11, EPI, TR, TO>(a, stream); break;
    default: launch_one<T, 64, 64, 2, 2, EPI, TR, TO>(a, stream); break;
  }
}

template <typename T>
static hipError_t run_epi(int cfg, const GemmArgs& a, hipStream_t stream) {
  switch (a.epi) {
    case EPI_BIAS: launch_cfg<T, EPI_BIAS, T, T>(cfg, a, stream); break;
    case EPI_BIAS_GELU: launch_cfg<T, EPI_BIAS_GELU, T, T>(cfg, a, stream); break;
    case EPI_QKV_SPLIT: launch_cfg<T, EPI_QKV_SPLIT, T, T>(cfg, a, stream); break;
    case EPI_SWIN_SCATTER: launch_cfg<T, EPI_SWIN_SCATTER, T, T>(cfg, a, stream); break;
    case EPI_PARTIAL:
      if constexpr (std::is_same<T, f16>::value) {
        if (a.part16) {
          launch_cfg<T, EPI_PARTIAL, T, T>(cfg, a, stream);
          break;
        }
      }
      if (a.part16) return hipErrorInvalidValue;
      launch_cfg<T, EPI_PARTIAL, T, float>(cfg, a, stream);
      break;
    case EPI_BIAS_RESID:
      if constexpr (std::is_same<T, bf16>::value) {
        if (a.resid_f32 && a.out_f32) {
          launch_cfg<T, EPI_BIAS_RESID, float, float>(cfg, a, stream);
          break;
        }
        if (a.out_f32 && !a.resid_f32) {
          launch_cfg<T, EPI_BIAS_RESID, T, float>(cfg, a, stream);
          break;
        }
      }
      if (a.resid_f32 || a.out_f32) return hipErrorInvalidValue;
      launch_cfg<T, EPI_BIAS_RESID, T, T>(cfg, a, stream);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// int8 operands: the epilogue output type follows the epilogue (fp16 activations,
// int8 codes for the GELU output that feeds the next int8 GEMM, raw int32).
static hipError_t run_epi_i8(int cfg, const GemmArgs& a, hipStream_t stream) {
  typedef int8_t T;
  switch (a.epi) {
    case EPI_QKV_SPLIT:   // int8 codes of Q, K, V (int8 attention), or fp16 values
      if (a.out_i8) launch_cfg<T, EPI_QKV_SPLIT, f16, int8_t>(cfg, a, stream);
      else launch_cfg<T, EPI_QKV_SPLIT, f16, f16>(cfg, a, stream);
      break;
    case EPI_BIAS_RESID: launch_cfg<T, EPI_BIAS_RESID, f16, f16>(cfg, a, stream); break;
    case EPI_BIAS: launch_cfg<T, EPI_BIAS, f16, f16>(cfg, a, stream); break;
    case EPI_BIAS_GELU:
      if (a.out_i8) launch_cfg<T, EPI_BIAS_GELU, f16, int8_t>(cfg, a, stream);
      else launch_cfg<T, EPI_BIAS_GELU, f16, f16>(cfg, a, stream);
      break;
    case EPI_BIAS_GELU_AMAX:
      if (!a.out_amax || a.out_i8) return hipErrorInvalidValue;
      launch_cfg<T, EPI_BIAS_GELU_AMAX, f16, f16>(cfg, a, stream);
      break;
    case EPI_RAW_I32: launch_cfg<T, EPI_RAW_I32, f16, int32_t>(cfg, a, stream); break;
    case EPI_PARTIAL: launch_cfg<T, EPI_PARTIAL, f16, int32_t>(cfg, a, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Tile choice by a small cost model. All workgroups of these tiles fit one per compute
// unit, so a launch runs in rounds of 256 tiles, and each round costs the tile's MFMA loop
// plus a fixed ~3.5 us (first slice in flight, epilogue, stores). The loop rate per compute
// unit is the one measured for the 128x256 tile (3.19e6 MACs/us for 16-bit operands, 1.9x
// that for int8 codes), scaled by each smaller tile's measured efficiency. A grid just
// past a multiple of 256 pays a whole extra round (wave quantisation), which the model
// sees and the plain "enough tiles" rule did not. Shapes whose K is not a multiple of 128
// bytes use the register-staged kernel.
static int pick_cfg(const GemmArgs& a, int elem_bytes) {
  if (((long long)a.K * elem_bytes) % 128) return -1;
  // (tile, loop efficiency relative to the 128x256 tile); 192x192 and 96x128 fill one
  // round of 256 tiles at token counts where 128x256 or 64x128 would spill into a second;
  // 32x64 puts twice the compute units of 64x64 on a 128-token batch (BERT-large at 128
  // tokens, back to back: QKV 6.2 -> 5.4 us, FFN1 6.2 -> 5.3, unsplit FFN2 13.5 -> 10.6)
  struct Cand { int cfg; double eff; };
  constexpr Cand CANDS[] = {{0, 1.0}, {1, 0.9}, {2, 0.65}, {3, 0.62}, {4, 0.5}, {9, 0.95},
                            {10, 0.55}, {11, 0.35}};
  constexpr double FIXED_US = 3.5, CUS = 256;
  const double rate = elem_bytes == 1 ? 6.06e6 : elem_bytes == 2 ? 3.19e6 : 0.2e6;
  int best = 0;
  double best_us = -1;
  for (const Cand& c : CANDS) {
    const PipeCfg& p = PIPE_CFGS[c.cfg];
    const double tiles = (double)((a.M + p.bm - 1) / p.bm) * ((a.N + p.bn - 1) / p.bn);
    const double rounds = std::ceil(tiles / CUS);
    const double us = rounds * ((double)p.bm * p.bn * a.K / (rate * c.eff) + FIXED_US);
    if (best_us < 0 || us < best_us) {
      best_us = us;
      best = c.cfg;
    }
  }
  return best;
}

// Partial-sum GEMMs: a shape whose tile grid leaves most compute units idle (few tokens,
// e.g. one 128-token sequence) is split over k. The tile is the one the unsplit kernel
// would take; the split count is the smallest power of two that reaches about 100
// workgroups, then doubled while the grid fits one round of 256, as long as every split
// keeps at least 8 k-slices (fewer make the prologue and the partial-sum traffic
// dominate). Returns 1 when splitting does not pay.
constexpr int SPLIT_MIN_TILES = 100, SPLIT_MIN_SLICES = 8, SPLIT_MAX = 8;

//
// fp16 partial sums (part16, half the bytes of float32) are available to callers of
// tel_gemm_partial; the plan itself no longer picks them. A rule that split BERT-base's FFN2
// (2557 x 768, K 3072, one round of 64 x 128 tiles) into two k-splits of 128 x 128 tiles
// with fp16 partials won back to back, but after the GEMM gained its four producer
// wavefronts the unsplit tile + LayerNorm was 0.9 % faster per 12-layer step end to end
// (three alternating runs on one box: 1.037 against 1.046 ms).

static int tiles_of(int cfg, int M, int N) {
  const PipeCfg& p = PIPE_CFGS[cfg];
  return ((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
}

int gemm_partial_plan(int dtype, int M, int N, int K, int* cfg, int* part16) {
  const int es = dtype_size(dtype);
  *part16 = 0;
  GemmArgs a{};
  a.M = M; a.N = N; a.K = K;
  *cfg = (M > 0 && N > 0 && K > 0) ? pick_cfg(a, es) : -1;
  if (*cfg < 0) return 1;
  const long tiles = tiles_of(*cfg, M, N);
  const int nk = (int)((long long)K * es / 128);
  // once split, keep doubling while the grid still fits one round of 256 workgroups: a
  // long K then streams in shorter runs per compute unit
  int sp = 1;
  while (sp < SPLIT_MAX && (tiles * sp < SPLIT_MIN_TILES || (sp > 1 && tiles * sp * 2 <= 256)) &&
         nk % (2 * sp) == 0 && nk / (2 * sp) >= SPLIT_MIN_SLICES)
    sp *= 2;
  return sp;
}

// Sparse tile choice: the dense cost model's rounds of 256 tiles (one workgroup per CU),
// with per-tile loop rates measured at BERT shapes (in dense-equivalent multiply-adds: the
// loop is bound by LDS traffic, mostly the dense activation fragments, not by the MFMAs).
static int pick_sp_cfg(const GemmArgs& a) {
  constexpr double EFF[N_SP_CFGS] = {0.26, 0.25, 0.27, 0.5, 0.45};
  constexpr double FIXED_US = 3.5, CUS = 256, RATE = 2 * 3.19e6;
  int best = 0;
  double best_us = -1;
  for (int c = 0; c < N_SP_CFGS; ++c) {
    const PipeCfg& p = SP_CFGS[c];
    const double tiles = (double)((a.M + p.bm - 1) / p.bm) * ((a.N + p.bn - 1) / p.bn);
    const double us = std::ceil(tiles / CUS) * ((double)p.bm * p.bn * a.K / (RATE * EFF[c]) + FIXED_US);
    if (best_us < 0 || us < best_us) {
      best_us = us;
      best = c;
    }
  }
  return best;
}

static bool sparse_ok(int dtype, const GemmArgs& a) {
  return (dtype == DT_F16 || dtype == DT_BF16) && a.K % 128 == 0 && a.splits == 1 && !a.ln_g &&
         (a.epi == EPI_BIAS || a.epi == EPI_BIAS_GELU || a.epi == EPI_BIAS_RESID ||
          a.epi == EPI_QKV_SPLIT);
}

int gemm_sparse_tile_configs() { return N_SP_CFGS; }

static hipError_t launch_gemm_sparse(int dtype, int cfg, const GemmArgs& a, hipStream_t stream) {
  if (!sparse_ok(dtype, a) || cfg < 0 || cfg >= N_SP_CFGS) return hipErrorInvalidValue;
  return dtype == DT_F16 ? run_epi_sp<f16>(cfg, a, stream) : run_epi_sp<bf16>(cfg, a, stream);
}

hipError_t launch_gemm(int dtype, const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  if (a.splits != 1) return hipErrorInvalidValue;   // splits need an explicit configuration
  if (a.w_idx) return launch_gemm_sparse(dtype, pick_sp_cfg(a), a, stream);
  if (a.ln_g && (dtype == DT_I8 || dtype == DT_F32)) return hipErrorInvalidValue;
  switch (dtype) {
    case DT_I8: return run_epi_i8(pick_cfg(a, 1), a, stream);
    case DT_F16: {
      hipError_t err;
      if (launch_rows<f16>(a, stream, &err)) return err;
      if (a.ln_g) return hipErrorInvalidValue;
      return run_epi<f16>(pick_cfg(a, 2), a, stream);
    }
    case DT_BF16: {
      hipError_t err;
      if (launch_rows<bf16>(a, stream, &err)) return err;
      if (a.ln_g) return hipErrorInvalidValue;
      return run_epi<bf16>(pick_cfg(a, 2), a, stream);
    }
    case DT_F32: return run_epi<float>(pick_cfg(a, 4), a, stream);
    default: return hipErrorInvalidValue;
  }
}

int gemm_tile_configs() { return N_PIPE_CFGS; }

// Explicit configuration (tuning and tests): cfg in [-1, N_PIPE_CFGS).
hipError_t launch_gemm_cfg(int dtype, int cfg, const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  if (a.w_idx) return launch_gemm_sparse(dtype, cfg, a, stream);   // cfg: SP_CFGS entry
  if (cfg < -1 || cfg >= N_PIPE_CFGS) return hipErrorInvalidValue;
  const int es = dtype_size(dtype);
  if (cfg >= 0 && (a.K * es) % 128) return hipErrorInvalidValue;
  if (a.splits < 1 || (a.splits > 1 && (cfg < 0 || ((long long)a.K * es / 128) % a.splits)))
    return hipErrorInvalidValue;
  if (a.splits > 1 && a.epi != EPI_PARTIAL) return hipErrorInvalidValue;
  if (a.part16 && (a.epi != EPI_PARTIAL || dtype != DT_F16)) return hipErrorInvalidValue;
  switch (dtype) {
    case DT_I8: return run_epi_i8(cfg, a, stream);
    case DT_F16: return run_epi<f16>(cfg, a, stream);
    case DT_BF16: return run_epi<bf16>(cfg, a, stream);
    case DT_F32: return run_epi<float>(cfg, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tel
