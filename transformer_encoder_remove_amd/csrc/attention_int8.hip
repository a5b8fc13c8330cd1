// Variable-length multi-head attention with both products on int8 codes (the Swin talk
// "大規模なビジュアル モデル…", section 3, INT8 paragraph: every matrix multiplication in
// int8, INT8 outputs where no value is needed). Steps per (sequence b, head h, query i),
// keys of sequence b only:
//   S = q . k over int8 codes, exact int32 (v_mfma_i32_16x16x64_i8);
//   t = float32(S) * a2, a2 = s_q s_k / sqrt(d) * log2 e (base-2 scores);
//   m = max over the sequence's keys of t (a first pass over the keys);
//   p = 2^(t - m) in (0, 1]; P codes r = rne(127 p) in [0, 127];
//   ctx = s_v * (sum_j r v_j) / (sum_j r), both sums exact int32.
// The exact maximum comes first so that no code depends on the order the key blocks are
// visited in. Output: the context as the storage type (fp16), or directly as the int8
// codes of that fp16 value at the O projection's input scale.
//
// Input: Q, K, V codes head-split as [3][heads][T][D] int8 (the int8 QKV epilogue's layout).
// Workgroup = QB / 16 wavefronts = QB queries of one (sequence, head), QB = 128 up to head_dim
// 64 and 64 above (8 or 4 wavefronts; each staged K/V block serves all of them); grid =
// (ceil(max_len / QB), heads, batch); wavefronts whose queries all lie past the sequence end
// stage K/V and meet every barrier but skip the arithmetic. Per 64-key block, K [64][D] and
// V^T [D][64] are staged in LDS; a sequence of up to 128 keys has both blocks staged at once
// and its scores kept in registers (one pass). Each
// wavefront computes S^T = K Q^T for its 16 queries, so a lane holds the scores of one query
// for 16 keys (keys 16 j + 4 lg + i, j, i = 0..3). For P V the MFMA k index e of lane group lg
// is mapped to key 16 (e / 4) + 4 lg + e % 4, the keys that lane already holds, so its 16 P
// codes are its B fragment as they stand; V^T is staged with that key order, so the A
// fragment is one 16-byte LDS read.
#include <math.h>

#include "device.h"
#include "launch.h"

namespace tel {

constexpr int A8_KB = 64;
template <int D> constexpr int a8_qb() { return D <= 64 ? 128 : 64; }

// LDS column of key `key` (0..63) in the permuted V^T rows: lane group g = (key % 16) / 4
// reads columns 16 g .. 16 g + 15, holding keys 4 g + 16 jj + i at column 16 g + 4 jj + i.
__device__ __forceinline__ int a8_vcol(int key) {
  return ((key & 15) >> 2) * 16 + (key >> 4) * 4 + (key & 3);
}

template <int D, bool CODES, int QB = a8_qb<D>()>
__global__ __launch_bounds__(QB * 4) void attn_int8_kernel(const int8_t* __restrict__ qkv,
                                                        void* __restrict__ out,
                                                        const int32_t* __restrict__ cu,
                                                        int total_tokens, int heads,
                                                        const float* __restrict__ scales) {
  using MF = Mfma<int8_t>;
  typedef MF::frag frag;                            // 16 int8 codes per lane
  constexpr int NKS = (D + 63) / 64;                // 64-deep k steps of q . k
  constexpr int NCB = D / 16;                       // 16-channel blocks of the output
  constexpr int LDK = (D < 64 ? 64 : D) + 16;       // bytes per staged K row
  constexpr int LDV = 2 * A8_KB + 16;               // bytes per staged V^T row (two blocks)
  static_assert(D % 16 == 0, "head_dim");
  // room for two key blocks: a sequence of up to 128 keys is staged once (one pass)
  __shared__ __attribute__((aligned(16))) int8_t sK[2 * A8_KB * LDK];
  __shared__ __attribute__((aligned(16))) int8_t sVt[D * LDV];

  const int b = blockIdx.z, h = blockIdx.y;
  const int start = cu[b], L = cu[b + 1] - start;
  constexpr int NT = QB * 4;                        // threads
  const int q0 = blockIdx.x * QB;
  if (q0 >= L) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const size_t hs = (size_t)total_tokens * D;
  const int8_t* Qh = qkv + (size_t)h * hs + (size_t)start * D;
  const int8_t* Kh = qkv + (size_t)(heads + h) * hs + (size_t)start * D;
  const int8_t* Vh = qkv + (size_t)(2 * heads + h) * hs + (size_t)start * D;
  const float a2 = scales[0], s_v = scales[1];

  const int qi = q0 + wave * 16 + lr;
  const int qc = min(qi, L - 1);
  const bool wave_on = q0 + wave * 16 < L;          // some query of this wavefront is valid
  frag qf[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    const int d0 = s * 64 + lg * 16;
    qf[s] = d0 < D ? *reinterpret_cast<const frag*>(Qh + (size_t)qc * D + d0) : frag{};
  }
  // K (and V) of a 64-key block: 16-byte vectors, thread tid owns vectors tid + NT p;
  // rows past the sequence end are clamped to its last key (their scores are masked)
  constexpr int VPR = D / 16, NVEC = A8_KB * VPR, PER = (NVEC + NT - 1) / NT;
  // stage key block kb0 into LDS block slot `slot` (K rows slot * 64.., V^T columns slot * 64..)
  auto stage_k = [&](int kb0, int slot) {
    int8_t* dK = sK + slot * A8_KB * LDK;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = tid + NT * p;
      if (NVEC % NT == 0 || idx < NVEC) {
        const int r = idx / VPR, c = idx - r * VPR;
        *reinterpret_cast<u32x4*>(&dK[r * LDK + c * 16]) =
            *reinterpret_cast<const u32x4*>(Kh + (size_t)min(kb0 + r, L - 1) * D + c * 16);
      }
    }
    if constexpr (D < 64) {   // zero the k padding of the rows once per block
      for (int r = tid; r < A8_KB; r += NT)
#pragma unroll
        for (int c = D; c < 64; c += 16)
          *reinterpret_cast<u32x4*>(&dK[r * LDK + c]) = u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto stage_v = [&](int kb0, int slot) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = tid + NT * p;
      if (NVEC % NT == 0 || idx < NVEC) {
        const int r = idx / VPR, c = idx - r * VPR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(Vh + (size_t)min(kb0 + r, L - 1) * D + c * 16);
        int8_t e[16];
        __builtin_memcpy(e, &v, 16);
        const int col = slot * A8_KB + a8_vcol(r);
#pragma unroll
        for (int k = 0; k < 16; ++k) sVt[(c * 16 + k) * LDV + col] = e[k];
      }
    }
  };
  // scores of the block staged in slot `slot` in base 2, -inf for keys past the end
  auto scores = [&](int kb0, int slot, float (&t)[4][4]) {
    const int8_t* sKb = sK + slot * A8_KB * LDK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      MF::acc s = MF::acc{0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < NKS; ++k) {
        const frag kf = *reinterpret_cast<const frag*>(&sKb[(j * 16 + lr) * LDK + k * 64 + lg * 16]);
        s = MF::mma(kf, qf[k], s);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb0 + j * 16 + lg * 4 + i;
        t[j][i] = key < L ? (float)s[i] * a2 : -INFINITY;
      }
    }
  };

  auto row_max = [&](float (&t)[4][4], float m) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, t[j][i]);
    return m;
  };
  MF::acc o[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) o[c] = MF::acc{0, 0, 0, 0};
  int lsum = 0;
  // P codes of one block's scores and their P V contribution (V^T of `slot`), exact int32
  auto pv = [&](float (&t)[4][4], float m, int slot) {
    int8_t r[16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(t[j][i] - m);                    // 0 for masked keys
        const int code = (int)fminf(__builtin_rintf(p * 127.0f), 127.0f);
        r[4 * j + i] = (int8_t)code;
        lsum += code;
      }
    frag pf;
    __builtin_memcpy(&pf, r, 16);
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const frag vf = *reinterpret_cast<const frag*>(&sVt[(c * 16 + lr) * LDV + slot * A8_KB + lg * 16]);
      o[c] = MF::mma(vf, pf, o[c]);
    }
  };
  float m = -INFINITY;
  if (L <= 2 * A8_KB) {
    // up to 128 keys: both blocks staged at once, scores kept in registers, one pass
    const bool two = L > A8_KB;
    stage_k(0, 0);
    stage_v(0, 0);
    if (two) {
      stage_k(A8_KB, 1);
      stage_v(A8_KB, 1);
    }
    __syncthreads();
    if (wave_on) {
      float t0[4][4], t1[4][4];
      scores(0, 0, t0);
      m = row_max(t0, m);
      if (two) {
        scores(A8_KB, 1, t1);
        m = row_max(t1, m);
      }
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      pv(t0, m, 0);
      if (two) pv(t1, m, 1);
    }
  } else {
    // pass 1: the exact row maximum over all keys of the sequence
    for (int kb0 = 0; kb0 < L; kb0 += A8_KB) {
      __syncthreads();
      stage_k(kb0, 0);
      __syncthreads();
      if (wave_on) {
        float t[4][4];
        scores(kb0, 0, t);
        m = row_max(t, m);
      }
    }
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    // pass 2: P codes and P V
    for (int kb0 = 0; kb0 < L; kb0 += A8_KB) {
      __syncthreads();
      stage_k(kb0, 0);
      stage_v(kb0, 0);
      __syncthreads();
      if (wave_on) {
        float t[4][4];
        scores(kb0, 0, t);
        pv(t, m, 0);
      }
    }
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);

  if (qi < L) {
    const size_t base = (size_t)(start + qi) * (heads * D) + h * D;
    const float inv_l = s_v / (float)lsum;
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      // O^T block c: lane holds channels c * 16 + 4 lg + i of query qi
      if constexpr (CODES) {
        const float inv = scales[2];
        int8_t q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = (float)(f16)((float)o[c][i] * inv_l);
          q[i] = (int8_t)fminf(fmaxf(__builtin_rintf(v * inv), -127.f), 127.f);
        }
        uint32_t packed;
        __builtin_memcpy(&packed, q, 4);
        *reinterpret_cast<uint32_t*>(reinterpret_cast<int8_t*>(out) + base + c * 16 + 4 * lg) = packed;
      } else {
        Vec4<f16> w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w.v[i] = (f16)((float)o[c][i] * inv_l);
        *reinterpret_cast<Vec4<f16>*>(reinterpret_cast<f16*>(out) + base + c * 16 + 4 * lg) = w;
      }
    }
  }
}

bool attention_int8_supported(int head_dim) {
  return head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128;
}

template <int D>
static void run_attn8(const int8_t* qkv, void* out, bool codes, const int32_t* cu, int batch,
                      int total, int max_len, int heads, const float* scales, hipStream_t st) {
  constexpr int QB = a8_qb<D>();
  const dim3 grid((max_len + QB - 1) / QB, heads, batch);
  if (codes)
    attn_int8_kernel<D, true><<<grid, QB * 4, 0, st>>>(qkv, out, cu, total, heads, scales);
  else
    attn_int8_kernel<D, false><<<grid, QB * 4, 0, st>>>(qkv, out, cu, total, heads, scales);
}

hipError_t launch_attention_int8(const int8_t* qkv, void* out, int out_codes, const int32_t* cu,
                                 int batch, int total, int max_len, int heads, int head_dim,
                                 const float* scales, hipStream_t stream) {
  if (total == 0 || max_len == 0) return hipSuccess;
  switch (head_dim) {
    case 16: run_attn8<16>(qkv, out, out_codes, cu, batch, total, max_len, heads, scales, stream); break;
    case 32: run_attn8<32>(qkv, out, out_codes, cu, batch, total, max_len, heads, scales, stream); break;
    case 64: run_attn8<64>(qkv, out, out_codes, cu, batch, total, max_len, heads, scales, stream); break;
    case 128: run_attn8<128>(qkv, out, out_codes, cu, batch, total, max_len, heads, scales, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tel
