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
#include "device.h"
#include "launch.h"

namespace tel {

template <typename T> struct EpiArgs {
  const float* bias;
  const T* resid;
  T* C;
  int M, N, heads;
};

template <int EPI, typename T>
__device__ __forceinline__ void epilogue_store(const EpiArgs<T>& e, int m, int n, f32x4 acc) {
  const float4 b = *reinterpret_cast<const float4*>(e.bias + n);
  float v[4] = {acc[0] + b.x, acc[1] + b.y, acc[2] + b.z, acc[3] + b.w};
  Vec4<T> out;
  size_t idx;
  if constexpr (EPI == EPI_BIAS_GELU) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = gelu_erf(v[i]);
  }
  if constexpr (EPI == EPI_BIAS_RESID) {
    const Vec4<T> r = *reinterpret_cast<const Vec4<T>*>(e.resid + (size_t)m * e.N + n);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += to_f32(r.v[i]);
  }
  if constexpr (EPI == EPI_QKV_SPLIT) {
    // [3][heads][M][d]: the attention kernel reads each head's Q, K and V as
    // contiguous [tokens][d] blocks.
    const int H = e.N / 3, d = H / e.heads;
    const int which = n / H, rem = n - which * H, hh = rem / d, c = rem - hh * d;
    idx = (((size_t)which * e.heads + hh) * e.M + m) * d + c;
  } else {
    idx = (size_t)m * e.N + n;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) out.v[i] = from_f32<T>(v[i]);
  *reinterpret_cast<Vec4<T>*>(e.C + idx) = out;
}

template <typename T, int BM, int BN, int BK, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM* WN * 64) void gemm_nt_kernel(const T* __restrict__ A,
                                                              const T* __restrict__ W, int K,
                                                              EpiArgs<T> e) {
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

#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int n = n0 + wn * TN + i * 16 + lg * 4;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = m0 + wm * TM + j * 16 + lr;
      if (m < M && n < N) epilogue_store<EPI, T>(e, m, n, acc[i][j]);
    }
  }
#undef TEL_GEMM_FETCH
#undef TEL_GEMM_STASH
}

// ------------------------------------------------------------------ dispatch
template <typename T, int BM, int BN, int WM, int WN>
static hipError_t run_cfg(const GemmArgs& a, hipStream_t stream) {
  constexpr int BK = 128 / sizeof(T);   // 128-byte k slices
  EpiArgs<T> e{a.bias, (const T*)a.resid, (T*)a.C, a.M, a.N, a.heads};
  const int grid = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const T* A = (const T*)a.A;
  const T* W = (const T*)a.W;
  switch (a.epi) {
    case EPI_BIAS:
      gemm_nt_kernel<T, BM, BN, BK, WM, WN, EPI_BIAS><<<grid, WM * WN * 64, 0, stream>>>(A, W, a.K, e);
      break;
    case EPI_BIAS_GELU:
      gemm_nt_kernel<T, BM, BN, BK, WM, WN, EPI_BIAS_GELU><<<grid, WM * WN * 64, 0, stream>>>(A, W, a.K, e);
      break;
    case EPI_BIAS_RESID:
      gemm_nt_kernel<T, BM, BN, BK, WM, WN, EPI_BIAS_RESID><<<grid, WM * WN * 64, 0, stream>>>(A, W, a.K, e);
      break;
    case EPI_QKV_SPLIT:
      gemm_nt_kernel<T, BM, BN, BK, WM, WN, EPI_QKV_SPLIT><<<grid, WM * WN * 64, 0, stream>>>(A, W, a.K, e);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Tile choice per shape (the GEMM-configuration tuning of the Kuaishou article, Fig. 11):
// the largest tile that still gives at least one workgroup per compute unit (256).
template <typename T>
static hipError_t run_typed(const GemmArgs& a, hipStream_t stream) {
  auto tiles = [&](int bm, int bn) { return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
  if (tiles(128, 128) >= 256) return run_cfg<T, 128, 128, 2, 2>(a, stream);
  if (tiles(128, 64) >= 256) return run_cfg<T, 128, 64, 2, 2>(a, stream);
  return run_cfg<T, 64, 64, 2, 2>(a, stream);
}

hipError_t launch_gemm(int dtype, const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  switch (dtype) {
    case DT_F16: return run_typed<f16>(a, stream);
    case DT_BF16: return run_typed<bf16>(a, stream);
    case DT_F32: return run_typed<float>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tel
