// The two halves of the shifted-window block (Swin-T stage 1: channels 96, 3 heads, hidden
// 384) each as one kernel whose intermediates stay on chip. Both keep their weight matrices
// in LDS for a persistent workgroup and take 16 token rows per wavefront at a time.
#include <math.h>

#include <algorithm>

#include "device.h"
#include "launch.h"
#include "rows.h"

namespace tel {

// ------------------------------------------------------------------ fused MLP
// The shifted-window block's MLP half in one pass over the tokens (the Swin talk "大規模な
// ビジュアル モデル…", section 3: LayerNorm, fc1 + bias + GELU and fc2 + bias + residual
// are each fused there; here they are one kernel):
//   y[m] = x1[m] + W2 GELU(W1 LN2(x1[m]) + b1) + b2,  C = 96 channels, hidden 384.
// Both weight matrices sit in LDS for the whole (persistent) workgroup, each wavefront takes
// 16 token rows at a time, and fc1's outputs, GELU applied and rounded to the storage type
// (as the separate fc1 kernel stores them), stay in registers as fc2's MFMA operand: the 384
// hidden values per token never reach memory (2 x 384 x 2 bytes per token of HBM traffic
// saved against fc1 and fc2 as two kernels).
//
// fc1 leaves lane (lr, lg) with hidden columns 16 i + 4 lg + q (q = 0..3) of its token row
// lr, for each 16-column block i. fc2's k-step s (32 hidden columns) takes the lane's own
// values of blocks 2 s and 2 s + 1 as its B fragment as they stand: MFMA k index 8 lg + e of
// the step is hidden column 32 s + 4 lg + e for e < 4 and 32 s + 16 + 4 lg + (e - 4) for
// e >= 4. W2 is staged in LDS with its columns in that order (whole groups of 4 move), so
// its A fragment is one 16-byte read, and the product is the plain sum over all 384 columns.
constexpr int MLP_C = 96, MLP_F = 384;
constexpr int MLP_LDW1 = MLP_C + 8, MLP_LDW2 = MLP_F + 8;   // fp16 per staged row

__device__ __forceinline__ int mlp_w2_col(int k) {   // LDS column of hidden column k
  const int s = k >> 5, r = k & 31;
  return s * 32 + (r < 16 ? 8 * (r >> 2) + (r & 3) : 8 * ((r - 16) >> 2) + 4 + (r & 3));
}

template <typename T, int NTH>
__global__ __launch_bounds__(NTH) void swin_mlp_kernel(const T* __restrict__ X1, T* __restrict__ Y,
                                                       const T* __restrict__ W1,
                                                       const float* __restrict__ b1,
                                                       const T* __restrict__ W2,
                                                       const float* __restrict__ b2,
                                                       const float* __restrict__ ln_g,
                                                       const float* __restrict__ ln_b,
                                                       float ln_eps, int M) {
  using MF = Mfma<T>;
  typedef typename MF::frag frag;
  constexpr int KS1 = MLP_C / 32, NF1 = MLP_F / 16, KS2 = MLP_F / 32, NF2 = MLP_C / 16;
  constexpr int NW = NTH / 64;
  __shared__ __attribute__((aligned(16))) T sW1[MLP_F * MLP_LDW1];
  __shared__ __attribute__((aligned(16))) T sW2[MLP_C * MLP_LDW2];
  __shared__ __attribute__((aligned(16))) float sB1[MLP_F];
  __shared__ __attribute__((aligned(16))) float sG[MLP_C];
  __shared__ __attribute__((aligned(16))) float sB[MLP_C];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  for (int idx = tid; idx < MLP_F * (MLP_C / 8); idx += NTH) {   // W1 rows, 16-byte vectors
    const int r = idx / (MLP_C / 8), c = idx - r * (MLP_C / 8);
    *reinterpret_cast<u32x4*>(sW1 + r * MLP_LDW1 + c * 8) =
        *reinterpret_cast<const u32x4*>(W1 + (size_t)r * MLP_C + c * 8);
  }
  for (int idx = tid; idx < MLP_C * (MLP_F / 4); idx += NTH) {   // W2, permuted groups of 4
    const int r = idx / (MLP_F / 4), g4 = idx - r * (MLP_F / 4);
    *reinterpret_cast<u32x2*>(sW2 + r * MLP_LDW2 + mlp_w2_col(4 * g4)) =
        *reinterpret_cast<const u32x2*>(W2 + (size_t)r * MLP_F + 4 * g4);
  }
  for (int k = tid; k < MLP_F; k += NTH) sB1[k] = b1[k];
  for (int k = tid; k < MLP_C; k += NTH) {
    sG[k] = ln_g[k];
    sB[k] = ln_b[k];
  }
  __syncthreads();
  // LN2's gamma / beta from LDS (lanes of one lg read the same words: broadcasts), which
  // leaves the registers for a third wavefront per SIMD
  auto gb = [&](int t, int j, float& g, float& b) {
    g = sG[t * 32 + lg * 8 + j];
    b = sB[t * 32 + lg * 8 + j];
  };
  const SwinGeom no_geom{};
  const int stride = gridDim.x * NW * 16;
  for (int rb = (blockIdx.x * NW + wave) * 16; rb < M; rb += stride) {
    frag a[KS1];
    rows_load<T, KS1, ROWS_PLAIN>(a, X1, M, rb, lr, lg, no_geom);
    rows_layernorm<T, KS1>(a, gb, ln_eps);
    // fc1 + bias + GELU, 6 hidden blocks at a time, into fc2's B fragments
    frag h[KS2];
#pragma unroll
    for (int g = 0; g < NF1 / 6; ++g) {
      typename MF::acc acc[6];
#pragma unroll
      for (int i = 0; i < 6; ++i) acc[i] = typename MF::acc{};
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < KS1; ++t)
#pragma unroll
        for (int i = 0; i < 6; ++i) {
          const frag w = *reinterpret_cast<const frag*>(
              sW1 + ((g * 6 + i) * 16 + lr) * MLP_LDW1 + t * 32 + lg * 8);
          acc[i] = MF::mma(w, a[t], acc[i]);
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        const int blk = g * 6 + i;
        const float4 bb = *reinterpret_cast<const float4*>(sB1 + blk * 16 + lg * 4);
        const float bv[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          h[blk >> 1][(blk & 1) * 4 + q] = from_f32<T>(gelu_erf(acc[i][q] + bv[q]));
      }
    }
    // fc2 + bias + residual
    typename MF::acc o[NF2];
#pragma unroll
    for (int i = 0; i < NF2; ++i) o[i] = typename MF::acc{};
#pragma unroll
    for (int s2 = 0; s2 < KS2; ++s2)
#pragma unroll
      for (int i = 0; i < NF2; ++i) {
        const frag w = *reinterpret_cast<const frag*>(sW2 + (i * 16 + lr) * MLP_LDW2 + s2 * 32 +
                                                      lg * 8);
        o[i] = MF::mma(w, h[s2], o[i]);
      }
    const int m = rb + lr;
    if (m < M) {   // + bias + residual (the row it normalised), 4 columns per lane and block
#pragma unroll
      for (int i = 0; i < NF2; ++i) {
        const int n = i * 16 + lg * 4;
        const float4 b4 = *reinterpret_cast<const float4*>(b2 + n);
        const Vec4<T> r = *reinterpret_cast<const Vec4<T>*>(X1 + (size_t)m * MLP_C + n);
        Vec4<T> out;
        out.v[0] = from_f32<T>(o[i][0] + b4.x + to_f32(r.v[0]));
        out.v[1] = from_f32<T>(o[i][1] + b4.y + to_f32(r.v[1]));
        out.v[2] = from_f32<T>(o[i][2] + b4.z + to_f32(r.v[2]));
        out.v[3] = from_f32<T>(o[i][3] + b4.w + to_f32(r.v[3]));
        *reinterpret_cast<Vec4<T>*>(Y + (size_t)m * MLP_C + n) = out;
      }
    }
  }
}

// ------------------------------------------------------------------ fused attention half
// The shifted-window block's attention half in one pass over the windows (Swin-T stage 1:
// C 96, 3 heads of 32, 7 x 7 windows), x1 = x + proj(WindowAttention(LN1(x))) with the cyclic
// shift and the window partition / reverse folded into the row gathers:
//  * each wavefront takes 16 of a window's (up to 64) token rows, gathered from the image
//    with the shift (row r of the window order reads image row src(r)), and applies LN1;
//  * per head, its Q, K, V columns (6 blocks of 16 of the 288 projection outputs, W_qkv in
//    LDS) are computed and rounded to fp16 as the separate QKV kernel stores them; K and V^T
//    of the window go to LDS, Q stays in registers;
//  * scores with the relative-position bias and the shift mask, softmax and P V exactly as
//    the window-attention kernel computes them; the context, normalised and rounded to fp16,
//    stays in registers;
//  * proj (W_proj in LDS) + bias + residual, each row written back to its image row.
// Q, K, V and the context never reach memory. Layouts: a lane ends the projection with 4
// consecutive columns 16 i + 4 lg + q of its token row; for a head's 32 columns (blocks 2 h and
// 2 h + 1) its 8 values are taken as the 8 elements of lane group lg of a 32-deep MFMA operand
// (element e: column 4 lg + e, or 16 + 4 lg + e - 4), for Q as it stands and for K as stored
// (one 16-byte LDS row segment), so Q . K sums over the head's 32 channels in that order. The
// context comes out in the same per-lane form (channel blocks c = 0, 1 of the head), and W_proj
// is staged with its input columns in that order (mlp_w2_col), so the proj product needs no
// lane exchange either. Two windows at a time per workgroup (wavefronts 0-3, 4-7).
constexpr int SA_C = 96, SA_HEADS = 3, SA_D = 32, SA_TOK = 64, SA_LDW = SA_C + 8;

template <int NG>
__global__ __launch_bounds__(NG * 256) void swin_attn_half_kernel(
    const f16* __restrict__ X, f16* __restrict__ X1, const f16* __restrict__ Wqkv,
    const float* __restrict__ bqkv, const float* __restrict__ bias_exp,
    const f16* __restrict__ Wproj, const float* __restrict__ bproj,
    const float* __restrict__ ln_g, const float* __restrict__ ln_b, float ln_eps, SwinGeom g,
    int windows) {
  using MF = Mfma<f16>;
  typedef MF::frag frag;
  constexpr int LDK = SA_D + 8, LDV = SA_TOK + 4, NJ = SA_TOK / 16;
  constexpr int NT = NG * 256;
  __shared__ __attribute__((aligned(16))) f16 sW[3 * SA_C * SA_LDW];
  __shared__ __attribute__((aligned(16))) f16 sP[SA_C * SA_LDW];
  __shared__ __attribute__((aligned(16))) float sBq[3 * SA_C];
  __shared__ __attribute__((aligned(16))) float sG[SA_C], sBt[SA_C];
  __shared__ __attribute__((aligned(16))) f16 sK[NG][SA_HEADS][SA_TOK * LDK];
  __shared__ __attribute__((aligned(16))) f16 sVt[NG][SA_HEADS][SA_D * LDV];
  __shared__ int sReg[NG][SA_TOK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int gi = wave >> 2, gw = wave & 3, gt = tid & 255;   // window group, its wave / thread
  for (int idx = tid; idx < 3 * SA_C * (SA_C / 8); idx += NT) {   // W_qkv rows
    const int r = idx / (SA_C / 8), c = idx - r * (SA_C / 8);
    *reinterpret_cast<u32x4*>(sW + r * SA_LDW + c * 8) =
        *reinterpret_cast<const u32x4*>(Wqkv + (size_t)r * SA_C + c * 8);
  }
  for (int idx = tid; idx < SA_C * (SA_C / 4); idx += NT) {   // W_proj, permuted groups of 4
    const int r = idx / (SA_C / 4), g4 = idx - r * (SA_C / 4);
    *reinterpret_cast<u32x2*>(sP + r * SA_LDW + mlp_w2_col(4 * g4)) =
        *reinterpret_cast<const u32x2*>(Wproj + (size_t)r * SA_C + 4 * g4);
  }
  for (int k = tid; k < 3 * SA_C; k += NT) sBq[k] = bqkv[k];
  for (int k = tid; k < SA_C; k += NT) {
    sG[k] = ln_g[k];
    sBt[k] = ln_b[k];
  }
  __syncthreads();
  auto gb = [&](int t, int j, float& gg, float& bb) {
    gg = sG[t * 32 + lg * 8 + j];
    bb = sBt[t * 32 + lg * 8 + j];
  };
  const int N = g.N;
  const int p = gw * 16 + lr, pc = min(p, N - 1);   // the lane's token of the window
  // window-local coordinates, computed once: the lane's token, and (first wavefront of a
  // group) key token gt's for the shift-mask regions
  const int py = pc / g.M, px = pc - py * g.M;
  const int kc = min(gt, N - 1), ky = kc / g.M, kx = kc - ky * g.M;
  const int img = g.Hs * g.Ws;
  // image row of the lane's token in image b, window (wy, wx): the cyclic shift folded in
  auto token_row = [&](int b, int wy, int wx, int ty, int tx) {
    int y = wy * g.M + ty + g.s, x = wx * g.M + tx + g.s;
    if (y >= g.Hs) y -= g.Hs;
    if (x >= g.Ws) x -= g.Ws;
    return (size_t)b * img + (size_t)y * g.Ws + x;
  };
  auto region = [&](int wy, int wx, int ty, int tx) {   // as SwinGeom::region
    const int Y = wy * g.M + ty, X = wx * g.M + tx;
    const int ry = Y < g.Hs - g.M ? 0 : (Y < g.Hs - g.s ? 1 : 2);
    const int rx = X < g.Ws - g.M ? 0 : (X < g.Ws - g.s ? 1 : 2);
    return 3 * ry + rx;
  };
  // log2(e) / sqrt(32) in float32, the value the window-attention launch computes on the host
  constexpr float scale_log2 = 0x1.0527dcp-2f;
  // the lane's query row of the bias table, every head: the same in every window
  float bias[SA_HEADS][NJ][4];
#pragma unroll
  for (int h = 0; h < SA_HEADS; ++h) {
    const float* brow = bias_exp + ((size_t)h * N + pc) * SA_TOK;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float4 b = *reinterpret_cast<const float4*>(brow + j * 16 + lg * 4);
      bias[h][j][0] = b.x; bias[h][j][1] = b.y; bias[h][j][2] = b.z; bias[h][j][3] = b.w;
    }
  }
  const int step = gridDim.x * NG;
  const int iters = (windows + step - 1) / step;
  // the lane's token row of window w, gathered from the image (cyclic shift included)
  auto load_rows = [&](int w, frag (&buf)[3]) {
    const int b = w / g.nW, wi = w - b * g.nW, wy = wi / g.nWx, wx = wi - wy * g.nWx;
    const f16* src = X + token_row(b, wy, wx, py, px) * SA_C + lg * 8;
#pragma unroll
    for (int t = 0; t < 3; ++t) buf[t] = *reinterpret_cast<const frag*>(src + t * 32);
  };
  frag nxt[3];
  load_rows(min(blockIdx.x * NG + gi, windows - 1), nxt);
  for (int it = 0; it < iters; ++it) {   // the same count of barriers in every wavefront
    const int win = it * step + blockIdx.x * NG + gi;
    const bool on = win < windows;
    const int wc = on ? win : windows - 1;
    const int wb = wc / g.nW, wimg = wc - wb * g.nW, wy = wimg / g.nWx, wx = wimg - wy * g.nWx;
    // only the last window row and column straddle a region border
    const bool masked = g.s > 0 && ((wy + 1) * g.nWx == g.nW || wx == g.nWx - 1);
    frag a[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) a[t] = nxt[t];
    if (it + 1 < iters) load_rows(min(win + step, windows - 1), nxt);   // next window's rows
    rows_layernorm<f16, 3>(a, gb, ln_eps);
    // Q, K, V of every head: projection blocks 2h, 2h+1 (Q), 6+2h, 7+2h (K), 12+2h, 13+2h (V);
    // Q stays in registers, K and V^T go to LDS, all three heads before one barrier
    frag qf_h[SA_HEADS];
    __syncthreads();   // the previous window's reads of sK / sVt / sReg are done
#pragma unroll
    for (int h = 0; h < SA_HEADS; ++h) {
      f32x4 acc[6];
#pragma unroll
      for (int i = 0; i < 6; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int i = 0; i < 6; ++i) {
          const int blk = (i >> 1) * 6 + 2 * h + (i & 1);
          const frag w = *reinterpret_cast<const frag*>(sW + (blk * 16 + lr) * SA_LDW + t * 32 + lg * 8);
          acc[i] = MF::mma(w, a[t], acc[i]);
        }
      f16 qkv[3][8];
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        const int blk = (i >> 1) * 6 + 2 * h + (i & 1);
        const float4 bb = *reinterpret_cast<const float4*>(sBq + blk * 16 + lg * 4);
        const float bv[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) qkv[i >> 1][(i & 1) * 4 + q] = from_f32<f16>(acc[i][q] + bv[q]);
      }
      __builtin_memcpy(&qf_h[h], qkv[0], 16);
      u32x4 kbits;
      __builtin_memcpy(&kbits, qkv[1], 16);
      *reinterpret_cast<u32x4*>(&sK[gi][h][p * LDK + 8 * lg]) = kbits;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int d = q < 4 ? 4 * lg + q : 16 + 4 * lg + (q - 4);
        sVt[gi][h][d * LDV + p] = qkv[2][q];
      }
    }
    if (masked && gt < SA_TOK) sReg[gi][gt] = region(wy, wx, ky, kx);
    __syncthreads();
    const int qreg = masked ? sReg[gi][pc] : 0;
    frag ctx[SA_HEADS];
#pragma unroll
    for (int h = 0; h < SA_HEADS; ++h) {
      // scores S^T = K Q^T over the head's 32 channels (4 key blocks of 16)
      f32x4 sc[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const frag kf = *reinterpret_cast<const frag*>(&sK[gi][h][(j * 16 + lr) * LDK + lg * 8]);
        sc[j] = MF::mma(kf, qf_h[h], f32x4{0.f, 0.f, 0.f, 0.f});
      }
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = j * 16 + lg * 4 + i;
          float sv = sc[j][i] * scale_log2 + bias[h][j][i];   // -inf for padded keys
          if (masked && key < N && sReg[gi][key] != qreg) sv = -INFINITY;
          sc[j][i] = sv;
          mx = fmaxf(mx, sv);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));   // finite: a token always sees itself
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pe = exp2f(sc[j][i] - mx);
          sc[j][i] = pe;
          psum += pe;
        }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      // O^T += V^T P^T (P as hi + lo parts), as the window-attention kernel does
      f32x4 o[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int t = 0; t < SA_TOK / 32; ++t) {
        f16 pv[8], pl[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int f = t * 8 + q;
          pv[q] = from_f32<f16>(sc[f / 4][f % 4]);
          pl[q] = from_f32<f16>(sc[f / 4][f % 4] - to_f32(pv[q]));
        }
        frag pb, pbl;
        __builtin_memcpy(&pb, pv, 16);
        __builtin_memcpy(&pbl, pl, 16);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const f16* vrow = &sVt[gi][h][(c * 16 + lr) * LDV];
          f16 tmp[8];
          const int k0 = 16 * (2 * t) + 4 * lg, k1 = k0 + 16;
          __builtin_memcpy(tmp, vrow + k0, 8);
          __builtin_memcpy(tmp + 4, vrow + k1, 8);
          frag va;
          __builtin_memcpy(&va, tmp, 16);
          o[c] = MF::mma(va, pb, o[c]);
          o[c] = MF::mma(va, pbl, o[c]);
        }
      }
      const float inv_l = 1.f / psum;
      f16 cv[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        cv[q] = from_f32<f16>(o[0][q] * inv_l);
        cv[4 + q] = from_f32<f16>(o[1][q] * inv_l);
      }
      __builtin_memcpy(&ctx[h], cv, 16);
    }
    // proj + bias + residual, window reverse and unshift in the store
    f32x4 pa[SA_C / 16];
#pragma unroll
    for (int i = 0; i < SA_C / 16; ++i) pa[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < SA_HEADS; ++h)
#pragma unroll
      for (int i = 0; i < SA_C / 16; ++i) {
        const frag w = *reinterpret_cast<const frag*>(sP + (i * 16 + lr) * SA_LDW + h * 32 + lg * 8);
        pa[i] = MF::mma(w, ctx[h], pa[i]);
      }
    if (on && p < N) {   // + bias + residual, stored at the token's image row
      const size_t row = token_row(wb, wy, wx, py, px) * SA_C;
#pragma unroll
      for (int i = 0; i < SA_C / 16; ++i) {
        const int n = i * 16 + lg * 4;
        const float4 b4 = *reinterpret_cast<const float4*>(bproj + n);
        const Vec4<f16> r = *reinterpret_cast<const Vec4<f16>*>(X + row + n);
        Vec4<f16> out;
        out.v[0] = from_f32<f16>(pa[i][0] + b4.x + to_f32(r.v[0]));
        out.v[1] = from_f32<f16>(pa[i][1] + b4.y + to_f32(r.v[1]));
        out.v[2] = from_f32<f16>(pa[i][2] + b4.z + to_f32(r.v[2]));
        out.v[3] = from_f32<f16>(pa[i][3] + b4.w + to_f32(r.v[3]));
        *reinterpret_cast<Vec4<f16>*>(X1 + row + n) = out;
      }
    }
  }
}

bool swin_attn_half_supported(int dtype, int channels, int heads, int window_tokens) {
  return dtype == DT_F16 && channels == SA_C && heads == SA_HEADS && window_tokens >= 1 &&
         window_tokens <= SA_TOK;
}

hipError_t launch_swin_attn_half(const void* x, void* x1, const void* w_qkv, const float* b_qkv,
                                 const float* bias_exp, const void* w_proj, const float* b_proj,
                                 const float* ln_g, const float* ln_b, float eps,
                                 const SwinGeom& geom, int windows, hipStream_t stream) {
  if (windows == 0) return hipSuccess;
  constexpr int NG = 2;
  const int grid = std::min((windows + NG - 1) / NG, 256);   // one workgroup per compute unit
  swin_attn_half_kernel<NG><<<grid, NG * 256, 0, stream>>>(
      (const f16*)x, (f16*)x1, (const f16*)w_qkv, b_qkv, bias_exp, (const f16*)w_proj, b_proj,
      ln_g, ln_b, eps, geom, windows);
  return hipGetLastError();
}

bool swin_mlp_supported(int dtype, int channels, int hidden) {
  return dtype == DT_F16 && channels == MLP_C && hidden == MLP_F;
}

hipError_t launch_swin_mlp(int dtype, const void* x1, void* y, const void* w1, const float* b1,
                           const void* w2, const float* b2, const float* ln_g, const float* ln_b,
                           float eps, int M, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  constexpr int NTH = 768;   // 12 wavefronts: three per SIMD on the one workgroup per unit
  const int blocks = (M + NTH / 4 - 1) / (NTH / 4);   // 16 rows per wavefront
  const int grid = std::min(blocks, 256);              // one workgroup per compute unit (LDS)
  switch (dtype) {
    case DT_F16:
      swin_mlp_kernel<f16, NTH><<<grid, NTH, 0, stream>>>((const f16*)x1, (f16*)y, (const f16*)w1,
                                                          b1, (const f16*)w2, b2, ln_g, ln_b, eps, M);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tel
