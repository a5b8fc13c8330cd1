// Variable-length multi-head self-attention over packed sequences, one fused kernel
// (the fMHA of the Swin talk "大規模なビジュアル モデル…", section 3: batched GEMM, softmax
// and batched GEMM in one kernel, with the head transposes folded into its loads and
// stores). Padding never enters: a query of sequence b reads only the keys
// cu[b] .. cu[b+1]-1 (Kuaishou "如何让Transformer在GPU上跑得更快", Fig. 10).
//
// Input: Q, K, V head-split as [3][heads][T][D] (the QKV GEMM's epilogue layout), so a
// head's keys are one contiguous [len][D] block. Output: ctx [T][heads * D].
//
// Workgroup = QB / 16 wavefronts = QB queries of one (sequence, head), QB = 128 for 16-bit
// types up to head_dim 64 (8 wavefronts: each K/V block is loaded once for up to 128 queries)
// and 64 otherwise; grid = (ceil(max_len / QB), heads, batch), workgroups past a sequence's
// end exit at once, and wavefronts whose queries all lie past it skip the arithmetic (they
// still stage K/V and meet every barrier).
// K and V blocks travel through a two-block register ring: Q and the first two key
// blocks are requested together at the start, and each later block two blocks ahead of
// its use, so the memory latency is paid about once per workgroup. Per 64-key block:
//  * K [64][D] and V^T [D][64] are staged in LDS from those registers;
//  * each wavefront computes S^T = K Q^T for its 16 queries with 16x16 MFMAs, so that
//    every lane holds scores of ONE query (column l % 16) for 16 keys;
//  * online softmax in base 2: the row max and row sum need only the lane's own 16
//    values plus two cross-lane butterflies (xor 16, xor 32);
//  * O^T += V^T P^T with P^T taken straight from the score registers (no LDS round
//    trip): the MFMA k index is mapped to the keys each lane already holds, and the
//    V^T fragment is read with the same mapping; 16-bit P is split into hi + lo parts;
//  * O^T keeps one query per lane as well, so the rescale by exp2(m_old - m_new) and
//    the final 1/l are per-lane scalars.
#include <math.h>

#include <type_traits>

#include "device.h"
#include "launch.h"

namespace tel {

constexpr int ATT_KB = 64;   // keys per LDS block
// read-ahead workgroups when asked for (16,384 threads: a sweep at a 128-token BERT-large
// stack found 8,192 and 32,768 or more slower)
constexpr int ATT_AHEAD_BLOCKS = 32;
constexpr int KV_THREADS = 256;   // threads that stage K/V (KvRegs' layout)

// Scores, online-softmax update and O update for one 64-key block staged in LDS.
template <typename T, int D, int LDK, int LDV, bool PSPLIT>
__device__ __forceinline__ void attn_block(const T* sK, const T* sVt,
                                           const typename Mfma<T>::frag* qf, f32x4* o,
                                           float& m_run, float& l_run, int kb0, int L,
                                           float scale_log2, int lr, int lg) {
  using MF = Mfma<T>;
  typedef typename MF::frag frag;
  constexpr int KPL = MF::KPL, KMF = 4 * KPL;
  constexpr int NKS = (D + KMF - 1) / KMF;
  constexpr int NCB = D / 16;
  constexpr int NJ = ATT_KB / 16;

  // scores S^T[key][query] for 4 sub-blocks of 16 keys
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
      const int key = kb0 + j * 16 + lg * 4 + i;
      const float s = key < L ? sc[j][i] * scale_log2 : -INFINITY;
      sc[j][i] = s;
      mx = fmaxf(mx, s);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float m_new = fmaxf(m_run, mx);       // finite: key 0 of the sequence is valid
  const float alpha = exp2f(m_run - m_new);
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = exp2f(sc[j][i] - m_new);
      sc[j][i] = p;
      psum += p;
    }
  psum += __shfl_xor(psum, 16, 64);
  psum += __shfl_xor(psum, 32, 64);
  l_run = l_run * alpha + psum;
  m_run = m_new;
#pragma unroll
  for (int c = 0; c < NCB; ++c) o[c] *= alpha;

  // O^T[c][q] += sum_key V^T[c][key] * P^T[key][q]; MFMA k element e of step t is the
  // lane's score f = t*KPL + e, i.e. key 16*(f/4) + 4*lg + f%4.
  // PSPLIT (bf16, and fp16 when the int8 codes of the output are written): P is split
  // into P_hi + P_lo (both representable), two MFMAs per step, so P enters the product
  // with ~2x the significant bits of one 16-bit value: bf16 keeps only 8 of them, and
  // downstream int8 codes flip far less often. Plain fp16 rounds P once (11 bits).
#pragma unroll
  for (int t = 0; t < ATT_KB / KMF; ++t) {
    T pv[KPL], pl[KPL];
#pragma unroll
    for (int e = 0; e < KPL; ++e) {
      const int f = t * KPL + e;
      pv[e] = from_f32<T>(sc[f / 4][f % 4]);
      pl[e] = PSPLIT ? from_f32<T>(sc[f / 4][f % 4] - to_f32(pv[e])) : pv[e];
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
        const int f = t;
        va = vrow[16 * (f / 4) + 4 * lg + (f % 4)];
      }
      o[c] = MF::mma(va, pb, o[c]);
      if constexpr (KPL > 1 && PSPLIT) o[c] = MF::mma(va, pbl, o[c]);
    }
  }
}

// 16-byte K and V vectors of one 64-key block held in registers. 16-bit types with an even
// number of vectors per thread (head_dim 64, 128): thread tid owns, in chunk c = tid % VPRK,
// the key rows 2 rp and 2 rp + 1 of row pair rp = tid / VPRK + (256 / VPRK) * pp, so that the
// transposed V can be stored as 4-byte pairs of consecutive keys (half the LDS stores of
// one element at a time); otherwise thread tid owns vectors tid + 256 p (key row idx / VPRK,
// chunk idx % VPRK). Rows past the sequence end are clamped to its last key (their scores
// are masked).
template <typename T, int D> struct KvRegs {
  static constexpr int VEC = 16 / sizeof(T), VPRK = D / VEC, NVEC = ATT_KB * VPRK;
  static constexpr int PER = (NVEC + 255) / 256;
  static constexpr bool PAIRS = sizeof(T) == 2 && PER % 2 == 0 && NVEC % 256 == 0;
  typedef T vec __attribute__((ext_vector_type(VEC)));
  vec k[PER], v[PER];

  __device__ __forceinline__ static void slot(int tid, int p, int& r, int& c) {
    if constexpr (PAIRS) {
      c = tid % VPRK;
      r = 2 * (tid / VPRK + (256 / VPRK) * (p >> 1)) + (p & 1);
    } else {
      const int idx = tid + 256 * p;
      r = idx / VPRK;
      c = idx - r * VPRK;
    }
  }

  __device__ __forceinline__ void load(const T* Kh, const T* Vh, int kb0, int L, int tid) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      if (NVEC % 256 == 0 || tid + 256 * p < NVEC) {
        int r, c;
        slot(tid, p, r, c);
        const size_t off = (size_t)min(kb0 + r, L - 1) * D + c * VEC;
        k[p] = *reinterpret_cast<const vec*>(Kh + off);
        v[p] = *reinterpret_cast<const vec*>(Vh + off);
      }
    }
  }
  // K row-major [key][d] (stride LDK), V transposed [d][key] (stride LDV)
  template <int LDK, int LDV>
  __device__ __forceinline__ void store(T* sK, T* sVt, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      if (NVEC % 256 == 0 || tid + 256 * p < NVEC) {
        int r, c;
        slot(tid, p, r, c);
        *reinterpret_cast<vec*>(&sK[r * LDK + c * VEC]) = k[p];
        if constexpr (PAIRS) {
          if (p & 1) {   // rows r - 1, r: one 4-byte store per transposed element pair
            static_assert(LDV % 2 == 0, "4-byte aligned key pairs");
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              T two[2] = {v[p - 1][e], v[p][e]};
              uint32_t w;
              __builtin_memcpy(&w, two, 4);
              *reinterpret_cast<uint32_t*>(&sVt[(c * VEC + e) * LDV + r - 1]) = w;
            }
          }
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) sVt[(c * VEC + e) * LDV + r] = v[p][e];
        }
      }
    }
  }
};

template <typename T, int D, bool PSPLIT, int QB>
__global__ __launch_bounds__(QB * 4) void attn_varlen_kernel(const T* __restrict__ qkv,
                                                          T* __restrict__ ctx,
                                                          const int32_t* __restrict__ cu,
                                                          int total_tokens, int heads,
                                                          float scale_log2,
                                                          int8_t* __restrict__ ctxq,
                                                          const float* __restrict__ qinv,
                                                          float* __restrict__ amax, int batch,
                                                          const void* ahead,
                                                          size_t ahead_bytes) {
  using MF = Mfma<T>;
  typedef typename MF::frag frag;
  constexpr int KPL = MF::KPL, KMF = 4 * KPL;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int LDK = D + VEC;
  constexpr int LDV = ATT_KB + (sizeof(T) == 4 ? 1 : 4);
  constexpr int NKS = (D + KMF - 1) / KMF;
  constexpr int NCB = D / 16;
  constexpr int NJ = ATT_KB / 16;
  static_assert(D % 16 == 0 && D % VEC == 0, "head_dim");

  __shared__ __attribute__((aligned(16))) T sK[ATT_KB * LDK];
  __shared__ __attribute__((aligned(16))) T sVt[D * LDV];
  __shared__ unsigned int amax_lds[2];   // with amax: workgroup max-abs, counter

  if ((int)blockIdx.z >= batch) {   // read-ahead workgroups (z past the batch): no barrier yet
    read_ahead(ahead, ahead_bytes,
               ((blockIdx.z - batch) * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x,
               (gridDim.z - batch) * gridDim.y * gridDim.x);
    return;
  }
  const int b = blockIdx.z, h = blockIdx.y;
  const int start = cu[b], L = cu[b + 1] - start;
  const int q0 = blockIdx.x * QB;
  if (q0 >= L) return;
  if (amax && threadIdx.x == 0) amax_lds[0] = amax_lds[1] = 0u;   // before the first barrier

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const size_t hs = (size_t)total_tokens * D;
  const T* Qh = qkv + (size_t)h * hs + (size_t)start * D;
  const T* Kh = qkv + (size_t)(heads + h) * hs + (size_t)start * D;
  const T* Vh = qkv + (size_t)(2 * heads + h) * hs + (size_t)start * D;

  // Every global load that does not depend on a result is issued here, so the
  // workgroup pays one memory latency for Q and the first two key blocks together;
  // later blocks are fetched two blocks ahead of their use.
  KvRegs<T, D> kv0, kv1;
  const bool stager = tid < KV_THREADS;
  if (stager) kv0.load(Kh, Vh, 0, L, tid);
  if (stager && ATT_KB < L) kv1.load(Kh, Vh, ATT_KB, L, tid);

  const int qi = q0 + wave * 16 + lr;
  const int qc = min(qi, L - 1);
  const bool wave_on = q0 + wave * 16 < L;    // some query of this wavefront is valid
  frag qf[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    const int d0 = s * KMF + lg * KPL;
    qf[s] = (d0 < D) ? *reinterpret_cast<const frag*>(Qh + (size_t)qc * D + d0) : frag{};
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one 64-key block: stage the registers in LDS, refill them with the block two ahead,
  // then scores, online softmax and O update
#define TEL_ATT_BLOCK(KV, kb0)                                                              \
  do {                                                                                      \
    __syncthreads();                        /* the previous block's LDS reads are done */   \
    if (stager) KV.template store<LDK, LDV>(sK, sVt, tid);                                  \
    if (stager && (kb0) + 2 * ATT_KB < L) KV.load(Kh, Vh, (kb0) + 2 * ATT_KB, L, tid);      \
    __syncthreads();                                                                        \
    if (wave_on)                                                                            \
      attn_block<T, D, LDK, LDV, PSPLIT>(sK, sVt, qf, o, m_run, l_run, (kb0), L, scale_log2, \
                                         lr, lg);                                           \
  } while (0)

  for (int kb0 = 0; kb0 < L; kb0 += 2 * ATT_KB) {
    TEL_ATT_BLOCK(kv0, kb0);
    if (kb0 + ATT_KB < L) TEL_ATT_BLOCK(kv1, kb0 + ATT_KB);
  }
#undef TEL_ATT_BLOCK

  float am = 0.f;   // with amax: this lane's max-abs of its stored context values
  if (qi < L) {
    const float inv_l = 1.f / l_run;
    const size_t base = (size_t)(start + qi) * (heads * D) + h * D;
    if (ctxq) {
      // int8 layer: only the int8 codes of the stored-type context feed the next GEMM,
      // code = clamp(rne(float(T(ctx)) * inv), -127, 127), as the quantise kernel computes
      const float inv = *qinv;
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        int8_t q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float r = __builtin_rintf(to_f32(from_f32<T>(o[c][i] * inv_l)) * inv);
          q[i] = (int8_t)fminf(fmaxf(r, -127.f), 127.f);
        }
        uint32_t packed;
        __builtin_memcpy(&packed, q, 4);
        *reinterpret_cast<uint32_t*>(ctxq + base + c * 16 + 4 * lg) = packed;
      }
    } else {
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        Vec4<T> w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w.v[i] = from_f32<T>(o[c][i] * inv_l);
        *reinterpret_cast<Vec4<T>*>(ctx + base + c * 16 + 4 * lg) = w;
        if (amax) {
#pragma unroll
          for (int i = 0; i < 4; ++i) am = fmaxf(am, fabsf(to_f32(w.v[i])));
        }
      }
    }
  }
  // the max-abs of the stored context, for a dynamically scaled int8 O projection
  if (amax) wg_atomic_max(am, amax, amax_lds, QB / 16);
}

bool attention_supported(int dtype, int head_dim) {
  if (dtype != DT_F16 && dtype != DT_BF16 && dtype != DT_F32) return false;
  return head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128;
}

template <typename T, int D>
static hipError_t run_attn(const void* qkv, void* ctx, const int32_t* cu, int batch, int total,
                           int max_len, int heads, int8_t* ctxq, const float* qinv,
                           bool psplit, float* amax, const void* ahead, size_t ahead_bytes,
                           hipStream_t stream) {
  // 128 queries per workgroup where the registers allow two such workgroups per compute
  // unit (16-bit types, head_dim <= 64), else 64
  constexpr int QB = (sizeof(T) == 2 && D <= 64) ? 128 : 64;
  const int gx = (max_len + QB - 1) / QB;
  // read-ahead: extra z slices holding about ATT_AHEAD_BLOCKS workgroups (none where the
  // grid's z extent would pass its limit: the read-ahead only saves time)
  int extra_z = ahead_bytes ? (ATT_AHEAD_BLOCKS + gx * heads - 1) / (gx * heads) : 0;
  if (batch + extra_z > 65535) extra_z = 0;
  const dim3 grid(gx, heads, batch + extra_z);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  if (ctxq || psplit || !std::is_same<T, f16>::value)   // P split (see attn_block)
    attn_varlen_kernel<T, D, true, QB><<<grid, QB * 4, 0, stream>>>(
        (const T*)qkv, (T*)ctx, cu, total, heads, scale_log2, ctxq, qinv, amax, batch, ahead,
        ahead_bytes);
  else
    attn_varlen_kernel<T, D, false, QB><<<grid, QB * 4, 0, stream>>>(
        (const T*)qkv, (T*)ctx, cu, total, heads, scale_log2, ctxq, qinv, amax, batch, ahead,
        ahead_bytes);
  return hipGetLastError();
}

template <typename T>
static hipError_t run_attn_d(const void* qkv, void* ctx, const int32_t* cu, int batch, int total,
                             int max_len, int heads, int d, int8_t* ctxq, const float* qinv,
                             bool ps, float* amax, const void* ah, size_t ahb,
                             hipStream_t stream) {
  switch (d) {
    case 16: return run_attn<T, 16>(qkv, ctx, cu, batch, total, max_len, heads, ctxq, qinv, ps, amax, ah, ahb, stream);
    case 32: return run_attn<T, 32>(qkv, ctx, cu, batch, total, max_len, heads, ctxq, qinv, ps, amax, ah, ahb, stream);
    case 64: return run_attn<T, 64>(qkv, ctx, cu, batch, total, max_len, heads, ctxq, qinv, ps, amax, ah, ahb, stream);
    case 128: return run_attn<T, 128>(qkv, ctx, cu, batch, total, max_len, heads, ctxq, qinv, ps, amax, ah, ahb, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention(int dtype, const void* qkv, void* ctx, const int32_t* cu, int batch,
                            int total, int max_len, int heads, int head_dim, hipStream_t stream,
                            int8_t* ctxq, const float* qinv, bool psplit, float* amax,
                            const void* ahead, size_t ahead_bytes) {
  if (total == 0 || max_len == 0) return hipSuccess;
  if (ctxq && !qinv) return hipErrorInvalidValue;
  if (amax && ctxq) return hipErrorInvalidValue;   // the max-abs is of the stored context
  if (ahead_bytes < 16) ahead_bytes = 0;
  if (ahead_bytes && (!ahead || (uintptr_t)ahead % 16)) return hipErrorInvalidValue;
  switch (dtype) {
    case DT_F16:
      return run_attn_d<f16>(qkv, ctx, cu, batch, total, max_len, heads, head_dim, ctxq, qinv, psplit, amax, ahead, ahead_bytes, stream);
    case DT_BF16:
      return run_attn_d<bf16>(qkv, ctx, cu, batch, total, max_len, heads, head_dim, ctxq, qinv, psplit, amax, ahead, ahead_bytes, stream);
    case DT_F32:
      return run_attn_d<float>(qkv, ctx, cu, batch, total, max_len, heads, head_dim, ctxq, qinv, psplit, amax, ahead, ahead_bytes, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tel
