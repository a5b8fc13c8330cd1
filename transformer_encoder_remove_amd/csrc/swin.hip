// Shifted-window attention (the Swin talk "大規模なビジュアル モデル…": section 1, window
// attention with a cyclic window shift and a relative position bias; section 2, the fMHA
// module that takes the mask and the bias as tensors; section 3, the bias-table lookup
// moved to preprocessing and the fMHA kernel for inference).
//
// One workgroup per (head, run of WIN_PER_WG windows): 4 wavefronts x 16 queries cover a
// window of up to 64 tokens (7 x 7 = 49 here; the 15 padded queries are computed and
// dropped). K [64][d] and
// V^T [d][64] of the window are staged in LDS; S^T = K Q^T and O^T += V^T P^T on 16x16
// MFMAs with one query per lane, exactly as in the variable-length kernel. The
// relative-position bias comes pre-expanded, pre-scaled and padded ([heads][N][64],
// -inf in the padding columns, so padded keys need no test); the shift mask is computed
// from the region ids of the query and the key (no mask tensor is read).
#include <math.h>

#include "device.h"
#include "launch.h"

namespace tel {

constexpr int WIN_TOK = 64;   // tokens per window, padded
constexpr int WIN_PER_WG = 4; // windows one workgroup walks through, one head

// Q fragments and the 16-byte K / V vectors of one window, held in registers: the next
// window's are requested while the current one is computed.
template <typename T, int D> struct WinRegs {
  using MF = Mfma<T>;
  static constexpr int KPL = MF::KPL, KMF = 4 * KPL, NKS = (D + KMF - 1) / KMF;
  static constexpr int VEC = 16 / sizeof(T), VPRK = D / VEC, NVEC = WIN_TOK * VPRK;
  static constexpr int PER = (NVEC + 255) / 256;
  typedef T vec __attribute__((ext_vector_type(VEC)));
  typename MF::frag q[NKS];
  vec k[PER], v[PER];

  __device__ __forceinline__ void load(const T* qkv, size_t hs, int heads, int h, int start,
                                       int N, int D_, int tid, int qc, int lg) {
    const T* Qh = qkv + (size_t)h * hs + (size_t)start * D;
    const T* Kh = qkv + (size_t)(heads + h) * hs + (size_t)start * D;
    const T* Vh = qkv + (size_t)(2 * heads + h) * hs + (size_t)start * D;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = tid + 256 * p;
      if (NVEC % 256 == 0 || idx < NVEC) {
        const int r = idx / VPRK, c = idx - r * VPRK;
        const size_t off = (size_t)min(r, N - 1) * D + c * VEC;
        k[p] = *reinterpret_cast<const vec*>(Kh + off);
        v[p] = *reinterpret_cast<const vec*>(Vh + off);
      }
    }
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int d0 = s * KMF + lg * KPL;
      q[s] = (d0 < D) ? *reinterpret_cast<const typename MF::frag*>(Qh + (size_t)qc * D + d0)
                      : typename MF::frag{};
    }
    (void)D_;
  }
  template <int LDK, int LDV>
  __device__ __forceinline__ void stage(T* sK, T* sVt, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = tid + 256 * p;
      if (NVEC % 256 == 0 || idx < NVEC) {
        const int r = idx / VPRK, c = idx - r * VPRK;
        *reinterpret_cast<vec*>(&sK[r * LDK + c * VEC]) = k[p];
#pragma unroll
        for (int e = 0; e < VEC; ++e) sVt[(c * VEC + e) * LDV + r] = v[p][e];
      }
    }
  }
};

// One window of one head, K and V^T staged in LDS: scores with the lane's bias values and
// the shift mask, softmax, O^T += V^T P^T, output of the lane's query.
template <typename T, int D, int LDK, int LDV>
__device__ __forceinline__ void window_block(const T* sK, const T* sVt, const int* sReg,
                                             const typename Mfma<T>::frag* qf,
                                             const float (&bias)[WIN_TOK / 16][4], bool masked,
                                             int N, int qi, int qc, float scale_log2, int lr,
                                             int lg, T* out) {
  using MF = Mfma<T>;
  typedef typename MF::frag frag;
  constexpr int KPL = MF::KPL, KMF = 4 * KPL;
  constexpr int NKS = (D + KMF - 1) / KMF;
  constexpr int NCB = D / 16;
  constexpr int NJ = WIN_TOK / 16;
  const int qreg = masked ? sReg[qc] : 0;
  f32x4 sc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    sc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int d0 = s * KMF + lg * KPL;
      const frag kf = (d0 < D) ? *reinterpret_cast<const frag*>(&sK[(j * 16 + lr) * LDK + d0])
                               : frag{};
      sc[j] = MF::mma(kf, qf[s], sc[j]);
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = j * 16 + lg * 4 + i;
      float s = sc[j][i] * scale_log2 + bias[j][i];       // -inf for padded keys
      if (masked && key < N && sReg[key] != qreg) s = -INFINITY;
      sc[j][i] = s;
      mx = fmaxf(mx, s);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));   // finite: a token always sees itself
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = exp2f(sc[j][i] - mx);
      sc[j][i] = p;
      psum += p;
    }
  psum += __shfl_xor(psum, 16, 64);
  psum += __shfl_xor(psum, 32, 64);

  f32x4 o[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  // O^T += V^T P^T; k element e of step t is the lane's score f = t*KPL + e (key
  // 16*(f/4) + 4*lg + f%4); 16-bit P enters as hi + lo parts.
#pragma unroll
  for (int t = 0; t < WIN_TOK / KMF; ++t) {
    T pv[KPL], pl[KPL];
#pragma unroll
    for (int e = 0; e < KPL; ++e) {
      const int f = t * KPL + e;
      pv[e] = from_f32<T>(sc[f / 4][f % 4]);
      pl[e] = from_f32<T>(sc[f / 4][f % 4] - to_f32(pv[e]));
    }
    frag pb, pbl;
    __builtin_memcpy(&pb, pv, sizeof(frag));
    __builtin_memcpy(&pbl, pl, sizeof(frag));
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const T* vrow = &sVt[(c * 16 + lr) * LDV];
      frag va;
      if constexpr (KPL == 8) {
        T tmp[8];
        const int k0 = 16 * (2 * t) + 4 * lg, k1 = k0 + 16;
        __builtin_memcpy(tmp, vrow + k0, 4 * sizeof(T));
        __builtin_memcpy(tmp + 4, vrow + k1, 4 * sizeof(T));
        __builtin_memcpy(&va, tmp, sizeof(frag));
      } else {
        va = vrow[16 * (t / 4) + 4 * lg + (t % 4)];
      }
      o[c] = MF::mma(va, pb, o[c]);
      if constexpr (KPL > 1) o[c] = MF::mma(va, pbl, o[c]);
    }
  }
  if (qi < N) {
    const float inv_l = 1.f / psum;
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      Vec4<T> w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w.v[i] = from_f32<T>(o[c][i] * inv_l);
      *reinterpret_cast<Vec4<T>*>(out + c * 16 + 4 * lg) = w;
    }
  }
}

// Grid (ceil(windows / WIN_PER_WG), heads); 4 wavefronts x 16 queries cover a window of up
// to 64 tokens (49 here; the padded queries are computed and dropped). The lane's bias
// values (its query row against the 64 key slots) are the same in every window of the
// head, so they are loaded once; each window's K and V^T are staged in LDS from the
// register ring while the next window's Q, K, V are in flight.
template <typename T, int D>
__global__ __launch_bounds__(256) void window_attention_kernel(const T* __restrict__ qkv,
                                                               T* __restrict__ ctx,
                                                               const float* __restrict__ bias_exp,
                                                               SwinGeom g, int total_tokens,
                                                               int heads, float scale_log2,
                                                               int windows) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int LDK = D + VEC;
  constexpr int LDV = WIN_TOK + (sizeof(T) == 4 ? 1 : 4);
  constexpr int NJ = WIN_TOK / 16;
  static_assert(D % 16 == 0 && D % VEC == 0, "head_dim");

  __shared__ __attribute__((aligned(16))) T sK[WIN_TOK * LDK];
  __shared__ __attribute__((aligned(16))) T sVt[D * LDV];
  __shared__ int sReg[WIN_TOK];                      // shift-mask region of every key

  const int h = blockIdx.y, w0 = blockIdx.x * WIN_PER_WG;
  const int N = g.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int qi = wave * 16 + lr, qc = min(qi, N - 1);
  const size_t hs = (size_t)total_tokens * D;
  const int nWy = g.nW / g.nWx;

  float bias[NJ][4];
  {
    const float* brow = bias_exp + ((size_t)h * N + qc) * WIN_TOK;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float4 b = *reinterpret_cast<const float4*>(brow + j * 16 + lg * 4);
      bias[j][0] = b.x; bias[j][1] = b.y; bias[j][2] = b.z; bias[j][3] = b.w;
    }
  }
  WinRegs<T, D> r0, r1;
  r0.load(qkv, hs, heads, h, w0 * N, N, D, tid, qc, lg);
#pragma unroll
  for (int i = 0; i < WIN_PER_WG; ++i) {
    const int win = w0 + i;
    if (win >= windows) break;                       // uniform across the workgroup
    WinRegs<T, D>& cur = (i % 2 == 0) ? r0 : r1;
    WinRegs<T, D>& nxt = (i % 2 == 0) ? r1 : r0;
    // Only windows in the last window row or column straddle a region border (the
    // shifted image splits each axis at L - M and L - s, and only the last window spans
    // them), so the mask test is skipped everywhere else; where it applies, the 64 key
    // regions are computed once into LDS.
    const int wimg = win % g.nW, wy = wimg / g.nWx, wx = wimg - wy * g.nWx;
    const bool masked = g.s > 0 && (wy == nWy - 1 || wx == g.nWx - 1);
    __syncthreads();                                 // the previous window's reads are done
    cur.template stage<LDK, LDV>(sK, sVt, tid);
    if (masked && tid < WIN_TOK) sReg[tid] = g.region(wimg, min(tid, N - 1));
    if (i + 1 < WIN_PER_WG && win + 1 < windows)
      nxt.load(qkv, hs, heads, h, (win + 1) * N, N, D, tid, qc, lg);
    __syncthreads();
    T* out = ctx + (size_t)(win * N + qi) * (heads * D) + h * D;
    window_block<T, D, LDK, LDV>(sK, sVt, sReg, cur.q, bias, masked, N, qi, qc, scale_log2, lr,
                                 lg, out);
  }
}

bool window_attention_supported(int dtype, int head_dim, int N) {
  if (dtype != DT_F16 && dtype != DT_BF16 && dtype != DT_F32) return false;
  if (N < 1 || N > WIN_TOK) return false;
  return head_dim == 16 || head_dim == 32 || head_dim == 64;
}

template <typename T, int D>
static void run_win(const void* qkv, void* ctx, const float* bias, const SwinGeom& g, int windows,
                    int heads, hipStream_t stream) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  window_attention_kernel<T, D><<<dim3((windows + WIN_PER_WG - 1) / WIN_PER_WG, heads), 256, 0,
                                  stream>>>((const T*)qkv, (T*)ctx, bias, g, windows * g.N,
                                            heads, scale_log2, windows);
}

template <typename T>
static bool run_win_d(int d, const void* qkv, void* ctx, const float* bias, const SwinGeom& g,
                      int windows, int heads, hipStream_t stream) {
  switch (d) {
    case 16: run_win<T, 16>(qkv, ctx, bias, g, windows, heads, stream); return true;
    case 32: run_win<T, 32>(qkv, ctx, bias, g, windows, heads, stream); return true;
    case 64: run_win<T, 64>(qkv, ctx, bias, g, windows, heads, stream); return true;
  }
  return false;
}

hipError_t launch_window_attention(int dtype, const void* qkv, void* ctx, const float* bias_exp,
                                   const SwinGeom& geom, int windows, int heads, int head_dim,
                                   hipStream_t stream) {
  if (windows == 0) return hipSuccess;
  bool ok = false;
  switch (dtype) {
    case DT_F16: ok = run_win_d<f16>(head_dim, qkv, ctx, bias_exp, geom, windows, heads, stream); break;
    case DT_BF16: ok = run_win_d<bf16>(head_dim, qkv, ctx, bias_exp, geom, windows, heads, stream); break;
    case DT_F32: ok = run_win_d<float>(head_dim, qkv, ctx, bias_exp, geom, windows, heads, stream); break;
  }
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

// ------------------------------------------------------------------ bias-table expansion
// Preprocessing, once per block: bias_exp[h][p][q] = table[(py_p - py_q + M - 1) * (2M - 1)
// + (px_p - px_q + M - 1)][h] * log2(e), for q < N; -inf in the padding columns.
template <typename T>
__global__ void expand_rel_bias_kernel(const T* __restrict__ table, float* __restrict__ out,
                                       int M, int heads) {
  const int N = M * M;
  const int total = heads * N * WIN_TOK;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < total; i += gridDim.x * 256) {
    const int q = i % WIN_TOK, p = (i / WIN_TOK) % N, h = i / (WIN_TOK * N);
    float v = -INFINITY;
    if (q < N) {
      const int dy = p / M - q / M + M - 1, dx = p % M - q % M + M - 1;
      v = to_f32(table[(size_t)(dy * (2 * M - 1) + dx) * heads + h]) * 1.4426950408889634f;
    }
    out[i] = v;
  }
}

hipError_t launch_expand_rel_bias(int dtype, const void* table, float* bias_exp, int M, int heads,
                                  hipStream_t stream) {
  const int total = heads * M * M * WIN_TOK;
  const int grid = (total + 255) / 256;
  switch (dtype) {
    case DT_F16: expand_rel_bias_kernel<f16><<<grid, 256, 0, stream>>>((const f16*)table, bias_exp, M, heads); break;
    case DT_BF16: expand_rel_bias_kernel<bf16><<<grid, 256, 0, stream>>>((const bf16*)table, bias_exp, M, heads); break;
    case DT_F32: expand_rel_bias_kernel<float><<<grid, 256, 0, stream>>>((const float*)table, bias_exp, M, heads); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tel
