// C ABI of libtel.so (declared in include/tel.h): host-side argument validation,
// packed-weight and workspace layouts, and the launch sequence of each entry point.
// Nothing here allocates device memory; every buffer belongs to the caller.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cstdlib>
#include <mutex>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "launch.h"
#include "tel.h"

using namespace tel;

namespace {

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) & ~(ALIGN - 1); }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool aligned256(const void* p) { return ((uintptr_t)p & 255u) == 0; }
inline hipStream_t as_stream(void* s) { return (hipStream_t)s; }
inline int status_of(hipError_t e) { return e == hipSuccess ? TEL_OK : TEL_EDEVICE; }
inline bool float_type(int dt) { return dt == DT_F32 || dt == DT_F16 || dt == DT_BF16; }

#define TEL_TRY(expr)                         \
  do {                                        \
    hipError_t e_ = (expr);                   \
    if (e_ != hipSuccess) return TEL_EDEVICE; \
  } while (0)

// ------------------------------------------------------------------ packed layer layout
// Activation-scale table of an int8 layer (float32): [0..3] s_a of the QKV, O, FFN1, FFN2
// inputs, [4..7] their 1 / s_a; int8 attention: [8..10] 1 / s of the Q, K, V codes the QKV
// epilogue writes, then the attention kernel's [11] s_q s_k / sqrt(d) * log2 e, [12] s_v,
// [13] 1 / s_a of the O projection's input (= [5]).
constexpr int ACT_FLOATS = 16;
// Storage-type weights first (GEMM operands, [N][K] as given), then float32 vectors.
// An int8 layer stores int8 weight codes instead, followed by the per-row weight scales,
// the per-column dequantisation scales and the activation scales s_a[4], inv_a[4].
struct LayerLayout {
  size_t w_qkv, w_o, w_1, w_2;
  size_t wi_qkv, wi_o, wi_1, wi_2;   // 2:4 layers: index words of the compressed weights
  size_t b_qkv, b_o, ln1_g, ln1_b, b_1, b_2, ln2_g, ln2_b;
  size_t sw_qkv, sw_o, sw_1, sw_2, dq_qkv, dq_o, dq_1, dq_2, act;
  size_t total;
};

bool desc_ok(const tel_encoder_desc* d) {
  if (!d) return false;
  if (d->hidden <= 0 || d->heads <= 0 || d->ffn <= 0) return false;
  if (d->hidden % d->heads) return false;
  if (!(d->ln_eps >= 0.f)) return false;
  return true;
}

int desc_supported(const tel_encoder_desc* d) {
  if (!desc_ok(d)) return TEL_EINVAL;
  if (!float_type(d->dtype)) return TEL_EUNSUPPORTED;
  if (d->int8_gemm < 0 || d->int8_gemm > 2) return TEL_EINVAL;
  if (d->int8_gemm && (d->dtype != DT_F16 || d->hidden % 16 || d->ffn % 16)) return TEL_EUNSUPPORTED;
  if (d->int8_gemm == 2 && !attention_int8_supported(d->hidden / d->heads)) return TEL_EUNSUPPORTED;
  if (d->dynamic_scales < 0 || d->dynamic_scales > 1) return TEL_EINVAL;
  if (d->dynamic_scales && d->int8_gemm != 1) return TEL_EUNSUPPORTED;
  if (d->sparse_2of4 && (d->int8_gemm || (d->dtype != DT_F16 && d->dtype != DT_BF16) ||
                         d->hidden % 128 || d->ffn % 128))
    return TEL_EUNSUPPORTED;
  if (d->hidden % 8 || d->ffn % 8) return TEL_EUNSUPPORTED;
  if (!attention_supported(d->dtype, d->hidden / d->heads)) return TEL_EUNSUPPORTED;
  if (!layernorm_supported(d->dtype, d->hidden)) return TEL_EUNSUPPORTED;
  return TEL_OK;
}

LayerLayout layer_layout(const tel_encoder_desc* d) {
  const size_t H = d->hidden, F = d->ffn, es = d->int8_gemm ? 1 : dtype_size(d->dtype);
  LayerLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes); return r; };
  if (d->sparse_2of4) {   // kept values [N][K/2] and index words [N][K/16]
    L.w_qkv = take(3 * H * H / 2 * es);
    L.w_o = take(H * H / 2 * es);
    L.w_1 = take(F * H / 2 * es);
    L.w_2 = take(H * F / 2 * es);
    L.wi_qkv = take(3 * H * H / 16 * 2);
    L.wi_o = take(H * H / 16 * 2);
    L.wi_1 = take(F * H / 16 * 2);
    L.wi_2 = take(H * F / 16 * 2);
  } else {
    L.w_qkv = take(3 * H * H * es);
    L.w_o = take(H * H * es);
    L.w_1 = take(F * H * es);
    L.w_2 = take(H * F * es);
  }
  L.b_qkv = take(3 * H * 4);
  L.b_o = take(H * 4);
  L.ln1_g = take(H * 4);
  L.ln1_b = take(H * 4);
  L.b_1 = take(F * 4);
  L.b_2 = take(H * 4);
  L.ln2_g = take(H * 4);
  L.ln2_b = take(H * 4);
  if (d->int8_gemm) {
    L.sw_qkv = take(3 * H * 4);
    L.sw_o = take(H * 4);
    L.sw_1 = take(F * 4);
    L.sw_2 = take(H * 4);
    L.dq_qkv = take(3 * H * 4);
    L.dq_o = take(H * 4);
    L.dq_1 = take(F * 4);
    L.dq_2 = take(H * 4);
    L.act = take(ACT_FLOATS * 4);
  }
  L.total = o;
  return L;
}

// ------------------------------------------------------------------ layer workspace
// A bf16 layer keeps its pre-LayerNorm sums and its residual stream (h1) in float32:
// bf16 keeps 8 significant bits, and rounding those two values to bf16 alone costs more
// than the 2e-2 absolute error budget at |y| ~ 4; fp16 and fp32 layers keep them in
// their storage type. When few tokens leave most compute units idle, the output
// projection and FFN2 run split over k instead: float32 (int32 for int8 operands)
// partial sums that the reduce-LayerNorm kernel adds with bias and residual.
constexpr int DYN_STATS = 5;   // dynamic scales: max-abs statistics per layer

struct LayerWs {
  size_t qkv, ctx, pre, part, h1, h1f, f, total;
  size_t xq, ctxq, h1q;   // int8 layer: codes of the inputs of the QKV, O and FFN1 GEMMs
  size_t fq, dyn;         // dynamic scales: codes of the GELU output, the four max-abs
};

inline bool f32_stream(const tel_encoder_desc* d) { return d->dtype == DT_BF16; }
inline int gemm_dtype(const tel_encoder_desc* d) { return d->int8_gemm ? (int)DT_I8 : d->dtype; }

// Rows of partial sums the layer needs for T tokens: the k-split plans of the output
// projection and FFN2 at every token count up to T (fewer tokens may mean more splits),
// so a workspace sized for T also serves any smaller batch.
size_t partial_rows_uncached(const tel_encoder_desc* d, size_t T) {
  if (d->dynamic_scales) return 0;   // that layer never splits over k
  const int dt = gemm_dtype(d), H = d->hidden, F = d->ffn;
  auto need = [&](size_t t) {
    int cfg, p16;
    const int sp = std::max(gemm_partial_plan(dt, (int)t, H, H, &cfg, &p16),
                            gemm_partial_plan(dt, (int)t, H, F, &cfg, &p16));
    return sp > 1 ? (size_t)sp * t : 0;
  };
  // Plans change only where a tile count does, i.e. just past a multiple of some tile
  // height (32, 64, 96, 128 or 192 rows: all multiples of 32), so the largest need inside each
  // run of equal plans is at its top, a multiple of 32 (or T itself).
  size_t rows = need(T);
  for (size_t t = 32; t < T; t += 32) rows = std::max(rows, need(t));
  return rows;
}

// The workspace layout is computed on every layer call; remember the last answer per
// thread so a stack of layers at one token count pays for the plan scan once.
size_t partial_rows(const tel_encoder_desc* d, size_t T) {
  struct Key { int dt, H, F, dyn; size_t T; size_t rows; };
  thread_local Key last{-1, 0, 0, 0, 0, 0};
  const int dt = gemm_dtype(d);
  if (last.dt == dt && last.H == d->hidden && last.F == d->ffn && last.dyn == d->dynamic_scales &&
      last.T == T)
    return last.rows;
  const size_t rows = partial_rows_uncached(d, T);
  last = Key{dt, d->hidden, d->ffn, d->dynamic_scales, T, rows};
  return rows;
}

LayerWs layer_ws(const tel_encoder_desc* d, size_t T) {
  const size_t H = d->hidden, F = d->ffn, es = dtype_size(d->dtype);
  LayerWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes); return r; };
  // dynamic scales: the four max-abs values first (documented: bytes 0..15 of the workspace):
  // two regions of 8 folded maxima (DynLink), then from byte 128 each region's five
  // statistics of AMAX_SLOTS copies (amax_raise)
  if (d->dynamic_scales) w.dyn = take((32 + 2 * DYN_STATS * AMAX_STAT_FLOATS) * 4);
  w.qkv = take(3 * T * H * es);
  w.ctx = take(T * H * es);
  w.pre = take(T * H * (f32_stream(d) ? 4 : es));
  w.part = take(partial_rows(d, T) * H * 4);
  w.h1 = take(T * H * es);
  w.h1f = f32_stream(d) ? take(T * H * 4) : 0;
  // int8 layer: GELU output as codes (static scales), or as fp16 values and then codes
  // (dynamic scales: the scale needs the whole tensor's max-abs first)
  w.f = take(T * F * (d->int8_gemm && !d->dynamic_scales ? 1 : es));
  if (d->int8_gemm) {
    w.xq = take(T * H);
    w.ctxq = take(T * H);
    w.h1q = take(T * H);
  }
  if (d->dynamic_scales) w.fq = take(T * F);
  w.total = o;
  return w;
}

struct StackWs {
  size_t cu, po, xa, xb, qa, qb, dbg, layer, total;   // qa, qb: int8 stack, codes of xa / xb
};                                                    // dbg: TEL_DEBUG length-check result

StackWs stack_ws(const tel_encoder_desc* d, int batch, int max_seq) {
  const size_t T = (size_t)batch * max_seq, H = d->hidden, es = dtype_size(d->dtype);
  StackWs s;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes); return r; };
  s.cu = take(((size_t)batch + 1) * 4);
  s.po = take(T * 4);
  s.xa = take(T * H * es);
  s.xb = take(T * H * es);
  s.qa = d->int8_gemm ? take(T * H) : 0;
  s.qb = d->int8_gemm ? take(T * H) : 0;
  s.dbg = take(4);
  s.layer = take(layer_ws(d, T).total);
  s.total = o;
  return s;
}

// Codes shared between consecutive int8 layers of a stack: xq_in holds this layer's input
// codes (made by the previous layer's LN2), xq_out receives the output's codes at the next
// layer's input scale *next_qinv. All null: quantise the input here, no codes out.
struct Int8Link {
  const int8_t* xq_in = nullptr;
  int8_t* xq_out = nullptr;
  const float* next_qinv = nullptr;
};

// Int8 layer with dynamic activation scales ("揭秘Transformer模型…", section 3.3: the
// quantisation parameters follow the data at inference time): each GEMM input is stored as
// fp16 by its producer, its max-abs over the batch is reduced on the device (raised by
// the producer for ctx, h1 and the GELU output; a pass of its own for the layer input), the
// quantise kernel takes 127 / max-abs as its inverse scale, and the GEMM epilogue forms the
// dequantisation scale (max-abs / 127) * s_w[n] per column. The layer never splits over k.
//
// Each max-abs is a statistic of AMAX_SLOTS copies that its producer's workgroups raise
// (amax_raise: one address per copy, so the atomics do not queue on one), and the quantise
// kernel that reads it folds the copies and stores the value for the GEMM's epilogue.
// In a stack, layer i uses region i % 2 of W.dyn: folded values [0..3] its four maxima,
// [4] the max-abs of its output, whose statistic its LN2 raises and layer i + 1 takes as
// its input statistic (DynLink), so only the first layer reads its input for the max-abs.
struct DynLink {
  int parity = 0;         // region of this layer
  bool in_from_prev = false;   // input max-abs left by the previous layer's LN2
  bool out_to_next = false;    // raise this layer's output max-abs for the next layer
};

int layer_forward_int8_dynamic(const tel_encoder_desc* d, const char* P, const void* x, void* y,
                               const int32_t* cu, int batch, int T, int max_len, char* ws,
                               hipStream_t st, const DynLink& link = DynLink{}) {
  const LayerLayout L = layer_layout(d);
  const LayerWs W = layer_ws(d, (size_t)T);
  const int H = d->hidden, F = d->ffn, nh = d->heads;
  auto F32 = [&](size_t off) { return (const float*)(P + off); };
  float* const dyn = (float*)(ws + W.dyn);
  float* amax = dyn + 8 * link.parity;   // folded values
  auto stat = [&](int parity, int g) {
    return dyn + 32 + ((size_t)parity * DYN_STATS + g) * AMAX_STAT_FLOATS;
  };
  const float* x_stat = link.in_from_prev ? stat(1 - link.parity, 4) : stat(link.parity, 0);
  float* x_amax = link.in_from_prev ? dyn + 8 * (1 - link.parity) + 4 : amax + 0;
  int8_t* xq = (int8_t*)(ws + W.xq);
  int8_t* ctxq = (int8_t*)(ws + W.ctxq);
  int8_t* h1q = (int8_t*)(ws + W.h1q);
  int8_t* fq = (int8_t*)(ws + W.fq);
  void* qkv = ws + W.qkv;
  void* ctx = ws + W.ctx;
  void* pre = ws + W.pre;
  void* h1 = ws + W.h1;
  void* f = ws + W.f;
  // this layer's five statistics start at 0: cleared by a kernel (not a memset: graph
  // capture), or, inside a stack, by the quantise kernel of the layer input, which reads the
  // other region's statistic (the previous layer's LN2 maximum) and so saves a launch
  if (!link.in_from_prev) TEL_TRY(launch_clear_amax(stat(link.parity, 0), DYN_STATS, st));
  // the layer input's max-abs has its own pass; ctx's, h1's and the GELU output's are raised
  // by the kernels that store them (attention, LN1, the FFN1 epilogue)
  auto quantize = [&](const void* a, size_t n, int8_t* q, int g) {
    return launch_quantize_act(DT_F16, a, q, n, nullptr, 0.f, st, stat(link.parity, g),
                               amax + g);
  };
  if (!link.in_from_prev)
    TEL_TRY(launch_absmax(DT_F16, x, (size_t)T * H, stat(link.parity, 0), st, true));
  TEL_TRY(launch_quantize_act(DT_F16, x, xq, (size_t)T * H, nullptr, 0.f, st, x_stat, x_amax,
                              link.in_from_prev ? stat(link.parity, 0) : nullptr,
                              link.in_from_prev ? DYN_STATS : 0));
  GemmArgs g{EPI_QKV_SPLIT, xq, P + L.w_qkv, F32(L.b_qkv), nullptr, qkv, T, 3 * H, H, nh};
  g.dq = F32(L.sw_qkv);
  g.dyn_amax = x_amax;
  TEL_TRY(launch_gemm(DT_I8, g, st));
  // P split as in the static int8 layer: ctx's codes follow P's rounding closely
  TEL_TRY(launch_attention(DT_F16, qkv, ctx, cu, batch, T, max_len, nh, H / nh, st, nullptr,
                           nullptr, true, stat(link.parity, 1)));
  TEL_TRY(quantize(ctx, (size_t)T * H, ctxq, 1));
  g = GemmArgs{EPI_BIAS_RESID, ctxq, P + L.w_o, F32(L.b_o), x, pre, T, H, H, nh};
  g.dq = F32(L.sw_o);
  g.dyn_amax = amax + 1;
  TEL_TRY(launch_gemm(DT_I8, g, st));
  TEL_TRY(launch_layernorm_amax(pre, h1, stat(link.parity, 2), F32(L.ln1_g), F32(L.ln1_b), T, H,
                                d->ln_eps, st));
  TEL_TRY(quantize(h1, (size_t)T * H, h1q, 2));
  g = GemmArgs{EPI_BIAS_GELU_AMAX, h1q, P + L.w_1, F32(L.b_1), nullptr, f, T, F, H, nh};
  g.dq = F32(L.sw_1);
  g.dyn_amax = amax + 2;
  g.out_amax = stat(link.parity, 3);
  TEL_TRY(launch_gemm(DT_I8, g, st));
  TEL_TRY(quantize(f, (size_t)T * F, fq, 3));
  g = GemmArgs{EPI_BIAS_RESID, fq, P + L.w_2, F32(L.b_2), h1, pre, T, H, F, nh};
  g.dq = F32(L.sw_2);
  g.dyn_amax = amax + 3;
  TEL_TRY(launch_gemm(DT_I8, g, st));
  if (link.out_to_next)
    TEL_TRY(launch_layernorm_amax(pre, y, stat(link.parity, 4), F32(L.ln2_g), F32(L.ln2_b), T, H,
                                  d->ln_eps, st));
  else
    TEL_TRY(launch_layernorm(DT_F16, DT_F16, pre, y, nullptr, F32(L.ln2_g), F32(L.ln2_b), T, H,
                             d->ln_eps, st));
  return TEL_OK;
}

// Int8 layer ([SW] section 3, INT8: quantise -> INT8 GEMM -> INT32 -> dequantise; bias,
// residual and LayerNorm stay floating point; attention runs in fp16 on the dequantised
// Q, K, V). Codes are produced where the value is made: the attention kernel for ctx, the
// LayerNorm for h1 (and, in a stack, LN2 for the next layer's input), the FFN1 epilogue for
// the GELU output; only a stack's first input goes through the quantise kernel.
int layer_forward_int8(const tel_encoder_desc* d, const char* P, const void* x, void* y,
                       const int32_t* cu, int batch, int T, int max_len, char* ws,
                       hipStream_t st, const Int8Link& link = Int8Link{}) {
  if (d->dynamic_scales)
    return layer_forward_int8_dynamic(d, P, x, y, cu, batch, T, max_len, ws, st);
  const LayerLayout L = layer_layout(d);
  const LayerWs W = layer_ws(d, (size_t)T);
  const int H = d->hidden, F = d->ffn, nh = d->heads;
  auto F32 = [&](size_t off) { return (const float*)(P + off); };
  const float* inv = F32(L.act) + 4;
  const bool attn8 = d->int8_gemm == 2;
  const int8_t* xq = link.xq_in ? link.xq_in : (const int8_t*)(ws + W.xq);
  int8_t* ctxq = (int8_t*)(ws + W.ctxq);
  int8_t* h1q = (int8_t*)(ws + W.h1q);
  int8_t* fq = (int8_t*)(ws + W.f);
  void* qkv = ws + W.qkv;
  void* ctx = ws + W.ctx;
  void* pre = ws + W.pre;
  void* part = ws + W.part;
  void* h1 = ws + W.h1;
  int cfg_o, cfg_2, p16;   // int8 partials are int32 (p16 stays 0)
  const int sp_o = gemm_partial_plan(DT_I8, T, H, H, &cfg_o, &p16);
  const int sp_2 = gemm_partial_plan(DT_I8, T, H, F, &cfg_2, &p16);

  if (!link.xq_in)
    TEL_TRY(launch_quantize_act(DT_F16, x, (int8_t*)(ws + W.xq), (size_t)T * H, inv + 0, 0.f, st));
  GemmArgs g{EPI_QKV_SPLIT, xq, P + L.w_qkv, F32(L.b_qkv), nullptr, qkv, T, 3 * H, H, nh};
  g.dq = F32(L.dq_qkv);
  if (attn8) {   // int8 attention: the QKV epilogue writes the codes of Q, K and V
    g.out_i8 = 1;
    g.qinv = F32(L.act) + 8;
  }
  TEL_TRY(launch_gemm(DT_I8, g, st));
  // attention writes the int8 codes of its fp16 output directly (the O projection's input)
  if (attn8)
    TEL_TRY(launch_attention_int8((const int8_t*)qkv, ctxq, 1, cu, batch, T, max_len, nh, H / nh,
                                  F32(L.act) + 11, st));
  else
    TEL_TRY(launch_attention(DT_F16, qkv, ctx, cu, batch, T, max_len, nh, H / nh, st, ctxq,
                             inv + 1));
  // output projection + dequantise + bias + residual (stored fp16), LayerNorm and the
  // int8 codes of h1; split over k (int32 partials, all of that in the reduce kernel)
  // when few tokens leave the GPU idle
  if (sp_o > 1) {
    g = GemmArgs{EPI_PARTIAL, ctxq, P + L.w_o, nullptr, nullptr, part, T, H, H, nh};
    g.splits = sp_o;
    TEL_TRY(launch_gemm_cfg(DT_I8, cfg_o, g, st));
    const LnReduceArgs r{part, sp_o, F32(L.dq_o), F32(L.b_o), x, DT_F16, h1, DT_F16, nullptr,
                         h1q, inv + 2, F32(L.ln1_g), F32(L.ln1_b), T, H, d->ln_eps, 1};
    TEL_TRY(launch_layernorm_reduce(r, st));
  } else {
    g = GemmArgs{EPI_BIAS_RESID, ctxq, P + L.w_o, F32(L.b_o), x, pre, T, H, H, nh};
    g.dq = F32(L.dq_o);
    TEL_TRY(launch_gemm(DT_I8, g, st));
    TEL_TRY(launch_layernorm_q8(pre, h1, h1q, inv + 2, F32(L.ln1_g), F32(L.ln1_b), T, H,
                                d->ln_eps, st));
  }
  g = GemmArgs{EPI_BIAS_GELU, h1q, P + L.w_1, F32(L.b_1), nullptr, fq, T, F, H, nh};
  g.dq = F32(L.dq_1);
  g.qinv = inv + 3;
  g.out_i8 = 1;
  TEL_TRY(launch_gemm(DT_I8, g, st));
  if (sp_2 > 1) {
    g = GemmArgs{EPI_PARTIAL, fq, P + L.w_2, nullptr, nullptr, part, T, H, F, nh};
    g.splits = sp_2;
    TEL_TRY(launch_gemm_cfg(DT_I8, cfg_2, g, st));
    const LnReduceArgs r{part, sp_2, F32(L.dq_2), F32(L.b_2), h1, DT_F16, y, DT_F16, nullptr,
                         link.xq_out, link.next_qinv, F32(L.ln2_g), F32(L.ln2_b), T, H,
                         d->ln_eps, 1};
    TEL_TRY(launch_layernorm_reduce(r, st));
  } else {
    g = GemmArgs{EPI_BIAS_RESID, fq, P + L.w_2, F32(L.b_2), h1, pre, T, H, F, nh};
    g.dq = F32(L.dq_2);
    TEL_TRY(launch_gemm(DT_I8, g, st));
    if (link.xq_out)
      TEL_TRY(launch_layernorm_q8(pre, y, link.xq_out, link.next_qinv, F32(L.ln2_g),
                                  F32(L.ln2_b), T, H, d->ln_eps, st));
    else
      TEL_TRY(launch_layernorm(DT_F16, DT_F16, pre, y, nullptr, F32(L.ln2_g), F32(L.ln2_b), T,
                               H, d->ln_eps, st));
  }
  return TEL_OK;
}

// Weights read ahead by extra workgroups of the layer's short kernels (see the weight
// prefetch below): with `on`, FFN1's during the attention and FFN2's during the first
// reduce-LayerNorm, and `next`'s QKV and output-projection weights (when not null) during
// the second.
struct LayerPrefetch {
  bool on = false;
  const char* next = nullptr;
};

int layer_forward(const tel_encoder_desc* d, const char* P, const void* x, void* y,
                  const int32_t* cu, int batch, int T, int max_len, char* ws, hipStream_t st,
                  const LayerPrefetch& pf = LayerPrefetch()) {
  if (T == 0) return TEL_OK;
  if (d->int8_gemm) return layer_forward_int8(d, P, x, y, cu, batch, T, max_len, ws, st);
  const LayerLayout L = layer_layout(d);
  const LayerWs W = layer_ws(d, (size_t)T);
  const int H = d->hidden, F = d->ffn, nh = d->heads, dt = d->dtype;
  void* qkv = ws + W.qkv;
  void* ctx = ws + W.ctx;
  void* pre = ws + W.pre;
  void* part = ws + W.part;
  void* h1 = ws + W.h1;
  void* f = ws + W.f;
  const bool f32s = f32_stream(d);
  float* h1f = f32s ? (float*)(ws + W.h1f) : nullptr;
  auto F32 = [&](size_t off) { return (const float*)(P + off); };
  // 2:4 layers: compressed weights on the sparse MFMA, never split over k
  const bool sparse = d->sparse_2of4 != 0;
  auto IDX = [&](size_t off) { return sparse ? (const uint16_t*)(P + off) : nullptr; };
  int cfg_o, cfg_2, p16_o = 0, p16_2 = 0;
  const int sp_o = sparse ? 1 : gemm_partial_plan(dt, T, H, H, &cfg_o, &p16_o);
  const int sp_2 = sparse ? 1 : gemm_partial_plan(dt, T, H, F, &cfg_2, &p16_2);

  GemmArgs g{};
  // QKV projection + bias, written head-split for the attention kernel
  g = GemmArgs{EPI_QKV_SPLIT, x, P + L.w_qkv, F32(L.b_qkv), nullptr, qkv, T, 3 * H, H, nh};
  g.w_idx = IDX(L.wi_qkv);
  TEL_TRY(launch_gemm(dt, g, st));
  // with the read-ahead: FFN1's weights during the attention
  TEL_TRY(launch_attention(dt, qkv, ctx, cu, batch, T, max_len, nh, H / nh, st, nullptr,
                           nullptr, false, nullptr, pf.on ? P + L.w_1 : nullptr,
                           pf.on ? L.w_2 - L.w_1 : 0));
  const int pre_dt = f32s ? (int)DT_F32 : dt;
  // output projection + bias + residual, then LayerNorm; split over k (float32 partials;
  // bias + residual + LayerNorm in the reduce kernel) when the plan says the split pays
  if (sp_o > 1) {
    g = GemmArgs{EPI_PARTIAL, ctx, P + L.w_o, nullptr, nullptr, part, T, H, H, nh};
    g.splits = sp_o;
    g.part16 = p16_o;
    TEL_TRY(launch_gemm_cfg(dt, cfg_o, g, st));
    LnReduceArgs r{part, sp_o, nullptr, F32(L.b_o), x, dt, h1, dt, h1f, nullptr, nullptr,
                   F32(L.ln1_g), F32(L.ln1_b), T, H, d->ln_eps, 0};
    r.part16 = p16_o;
    if (pf.on) {   // FFN2's weights
      r.prefetch = P + L.w_2;
      r.prefetch_bytes = L.b_qkv - L.w_2;
    }
    TEL_TRY(launch_layernorm_reduce(r, st));
  } else {
    g = GemmArgs{EPI_BIAS_RESID, ctx, P + L.w_o, F32(L.b_o), x, pre, T, H, H, nh, 0, f32s};
    g.w_idx = IDX(L.wi_o);
    TEL_TRY(launch_gemm(dt, g, st));
    TEL_TRY(launch_layernorm(pre_dt, dt, pre, h1, h1f, F32(L.ln1_g), F32(L.ln1_b), T, H,
                             d->ln_eps, st));
  }
  // FFN: bias + GELU, then bias + residual, then LayerNorm (FFN2 split as above)
  g = GemmArgs{EPI_BIAS_GELU, h1, P + L.w_1, F32(L.b_1), nullptr, f, T, F, H, nh};
  g.w_idx = IDX(L.wi_1);
  TEL_TRY(launch_gemm(dt, g, st));
  const void* res2 = f32s ? (const void*)h1f : h1;
  if (sp_2 > 1) {
    g = GemmArgs{EPI_PARTIAL, f, P + L.w_2, nullptr, nullptr, part, T, H, F, nh};
    g.splits = sp_2;
    g.part16 = p16_2;
    TEL_TRY(launch_gemm_cfg(dt, cfg_2, g, st));
    LnReduceArgs r{part, sp_2, nullptr, F32(L.b_2), res2, f32s ? (int)DT_F32 : dt, y, dt,
                   nullptr, nullptr, nullptr, F32(L.ln2_g), F32(L.ln2_b), T, H, d->ln_eps, 0};
    r.part16 = p16_2;
    if (pf.next) {   // the next layer's QKV and output-projection weights
      r.prefetch = pf.next + L.w_qkv;
      r.prefetch_bytes = L.w_1 - L.w_qkv;
    }
    TEL_TRY(launch_layernorm_reduce(r, st));
  } else {
    g = GemmArgs{EPI_BIAS_RESID, f, P + L.w_2, F32(L.b_2), res2, pre, T, H, F, nh, f32s, f32s};
    g.w_idx = IDX(L.wi_2);
    TEL_TRY(launch_gemm(dt, g, st));
    TEL_TRY(launch_layernorm(pre_dt, dt, pre, y, nullptr, F32(L.ln2_g), F32(L.ln2_b), T, H,
                             d->ln_eps, st));
  }
  return TEL_OK;
}

// ------------------------------------------------------------------ shifted-window block
int swin_supported(const tel_swin_desc* d) {
  if (!d) return TEL_EINVAL;
  if (d->batch <= 0 || d->height <= 0 || d->width <= 0 || d->channels <= 0 || d->heads <= 0 ||
      d->window <= 0 || d->mlp_hidden <= 0 || d->shift < 0 || !(d->ln_eps >= 0.f))
    return TEL_EINVAL;
  if (d->channels % d->heads || d->height % d->window || d->width % d->window ||
      d->shift >= d->window)
    return TEL_EINVAL;
  if ((long long)d->batch * d->height * d->width > INT32_MAX / 4) return TEL_EUNSUPPORTED;
  if (d->dtype != DT_F16 && d->dtype != DT_F32) return TEL_EUNSUPPORTED;
  if (d->channels % 8 || d->mlp_hidden % 8) return TEL_EUNSUPPORTED;
  if (!layernorm_supported(d->dtype, d->channels)) return TEL_EUNSUPPORTED;
  if (!window_attention_supported(d->dtype, d->channels / d->heads, d->window * d->window))
    return TEL_EUNSUPPORTED;
  return TEL_OK;
}

SwinGeom swin_geom(const tel_swin_desc* d) {
  SwinGeom g;
  g.Hs = d->height;
  g.Ws = d->width;
  g.M = d->window;
  g.s = d->shift;
  g.nWx = d->width / d->window;
  g.nW = (d->height / d->window) * g.nWx;
  g.N = d->window * d->window;
  return g;
}

// Which halves of the block run as one kernel each (TEL_SWIN_FUSED_*): both need the
// skinny-kernel shapes (C 96 here) in fp16; the attention half also 3 heads and windows of
// at most 64 tokens.
int swin_fused_stages(const tel_swin_desc* d) {
  const int C = d->channels, F = d->mlp_hidden, dt = d->dtype;
  if (!gemm_rows_supported(dt, 3 * C, C) || !gemm_rows_supported(dt, F, C)) return 0;
  int f = 0;
  if (swin_attn_half_supported(dt, C, d->heads, d->window * d->window)) f |= TEL_SWIN_FUSED_ATTN;
  if (swin_mlp_supported(dt, C, F)) f |= TEL_SWIN_FUSED_MLP;
  return f;
}

struct SwinLayout {
  size_t w_qkv, w_proj, w_1, w_2;
  size_t ln1_g, ln1_b, b_qkv, b_proj, ln2_g, ln2_b, b_1, b_2, bias;
  size_t total;
};

SwinLayout swin_layout(const tel_swin_desc* d) {
  const size_t C = d->channels, F = d->mlp_hidden, es = dtype_size(d->dtype);
  const size_t N = (size_t)d->window * d->window;
  SwinLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes); return r; };
  L.w_qkv = take(3 * C * C * es);
  L.w_proj = take(C * C * es);
  L.w_1 = take(F * C * es);
  L.w_2 = take(C * F * es);
  L.ln1_g = take(C * 4);
  L.ln1_b = take(C * 4);
  L.b_qkv = take(3 * C * 4);
  L.b_proj = take(C * 4);
  L.ln2_g = take(C * 4);
  L.ln2_b = take(C * 4);
  L.b_1 = take(F * 4);
  L.b_2 = take(C * 4);
  L.bias = take((size_t)d->heads * N * 64 * 4);
  L.total = o;
  return L;
}

struct SwinWs {
  size_t zw, qkv, ctx, x1, h, f, total;
};

SwinWs swin_ws(const tel_swin_desc* d) {
  const size_t T = (size_t)d->batch * d->height * d->width;
  const size_t C = d->channels, F = d->mlp_hidden, es = dtype_size(d->dtype);
  SwinWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes); return r; };
  w.zw = take(T * C * es);
  w.qkv = take(3 * T * C * es);
  w.ctx = take(T * C * es);
  w.x1 = take(T * C * es);
  w.h = take(T * C * es);
  w.f = take(T * F * es);
  w.total = o;
  return w;
}

}  // namespace

extern "C" {

const char* tel_status_str(int s) {
  switch (s) {
    case TEL_OK: return "TEL_OK";
    case TEL_EINVAL: return "TEL_EINVAL: invalid argument";
    case TEL_EUNSUPPORTED: return "TEL_EUNSUPPORTED: unsupported shape or type";
    case TEL_EWORKSPACE: return "TEL_EWORKSPACE: buffer too small";
    case TEL_EDEVICE: return "TEL_EDEVICE: HIP runtime error";
  }
  return "unknown tel_status";
}

const char* tel_version(void) { return "tel 0.1 (gfx950)"; }

int tel_build_offsets(const int32_t* seq_lens, int batch, int max_seq, int32_t* cu_seqlens,
                      int32_t* padding_offset, void* stream) {
  if (!seq_lens || !cu_seqlens || !padding_offset) return TEL_EINVAL;
  if (batch <= 0 || max_seq <= 0) return TEL_EINVAL;
  if ((long long)batch * max_seq > INT32_MAX) return TEL_EUNSUPPORTED;
  return status_of(launch_offsets(seq_lens, batch, max_seq, cu_seqlens, padding_offset,
                                  as_stream(stream)));
}

int tel_remove_padding(const void* x_pad, void* x_packed, const int32_t* padding_offset,
                       int total_tokens, int width, int dtype, void* stream) {
  if (total_tokens < 0 || width <= 0) return TEL_EINVAL;
  if (!float_type(dtype) && dtype != DT_I8) return TEL_EINVAL;
  if (total_tokens == 0) return TEL_OK;
  if (!x_pad || !x_packed || !padding_offset) return TEL_EINVAL;
  if (!aligned16(x_pad) || !aligned16(x_packed)) return TEL_EINVAL;
  const long long row_bytes = (long long)width * dtype_size(dtype);
  if (row_bytes % 16) return TEL_EUNSUPPORTED;
  return status_of(launch_remove_padding(x_pad, x_packed, padding_offset, total_tokens,
                                         (int)row_bytes, as_stream(stream)));
}

int tel_rebuild_padding(const void* x_packed, void* x_pad, const int32_t* cu_seqlens, int batch,
                        int max_seq, int width, int dtype, void* stream) {
  if (batch <= 0 || max_seq <= 0 || width <= 0) return TEL_EINVAL;
  if (!float_type(dtype) && dtype != DT_I8) return TEL_EINVAL;
  if (!x_packed || !x_pad || !cu_seqlens) return TEL_EINVAL;
  if (!aligned16(x_pad) || !aligned16(x_packed)) return TEL_EINVAL;
  const long long row_bytes = (long long)width * dtype_size(dtype);
  if (row_bytes % 16) return TEL_EUNSUPPORTED;
  return status_of(launch_rebuild_padding(x_packed, x_pad, cu_seqlens, batch, max_seq,
                                          (int)row_bytes, as_stream(stream)));
}

int tel_build_offsets_mask(const uint8_t* mask, int batch, int max_seq, int32_t* cu_seqlens,
                           int32_t* padding_offset, void* stream) {
  if (!mask || !cu_seqlens || !padding_offset) return TEL_EINVAL;
  if (batch <= 0 || max_seq <= 0) return TEL_EINVAL;
  if ((long long)batch * max_seq > INT32_MAX) return TEL_EUNSUPPORTED;
  return status_of(launch_offsets_mask(mask, batch, max_seq, cu_seqlens, padding_offset,
                                       as_stream(stream)));
}

int tel_rebuild_padding_mask(const void* x_packed, void* x_pad, const uint8_t* mask,
                             const int32_t* padding_offset, int total_tokens, int batch,
                             int max_seq, int width, int dtype, void* stream) {
  if (batch <= 0 || max_seq <= 0 || width <= 0 || total_tokens < 0) return TEL_EINVAL;
  if ((long long)total_tokens > (long long)batch * max_seq) return TEL_EINVAL;
  if (!float_type(dtype) && dtype != DT_I8) return TEL_EINVAL;
  if (!x_pad || !mask || (total_tokens > 0 && (!x_packed || !padding_offset))) return TEL_EINVAL;
  if (!aligned16(x_pad) || (x_packed && !aligned16(x_packed))) return TEL_EINVAL;
  const long long row_bytes = (long long)width * dtype_size(dtype);
  if (row_bytes % 16) return TEL_EUNSUPPORTED;
  return status_of(launch_rebuild_padding_mask(x_packed, x_pad, mask, padding_offset,
                                               total_tokens, batch, max_seq, (int)row_bytes,
                                               as_stream(stream)));
}

size_t tel_encoder_packed_size(const tel_encoder_desc* d) {
  if (desc_supported(d) != TEL_OK) return 0;
  return layer_layout(d).total;
}

int tel_encoder_prepare(const tel_encoder_desc* d, const tel_encoder_weights* w, void* packed,
                        size_t packed_bytes, void* stream) {
  const int sup = desc_supported(d);
  if (sup != TEL_OK) return sup;
  if (!w || !packed || !aligned256(packed)) return TEL_EINVAL;
  const void* ptrs[] = {w->w_qkv, w->b_qkv, w->w_o, w->b_o, w->ln1_g, w->ln1_b,
                        w->w_1, w->b_1, w->w_2, w->b_2, w->ln2_g, w->ln2_b};
  for (const void* p : ptrs)
    if (!p) return TEL_EINVAL;
  const LayerLayout L = layer_layout(d);
  if (packed_bytes < L.total) return TEL_EWORKSPACE;
  const size_t H = d->hidden, F = d->ffn, es = dtype_size(d->dtype);
  char* P = (char*)packed;
  hipStream_t st = as_stream(stream);
  const int dt = d->dtype;
  if (d->int8_gemm && d->dynamic_scales) {   // weights only: activation scales at run time
    TEL_TRY(launch_quantize_weight(dt, w->w_qkv, (int8_t*)(P + L.w_qkv), (float*)(P + L.sw_qkv),
                                   nullptr, 0.f, 3 * H, H, st));
    TEL_TRY(launch_quantize_weight(dt, w->w_o, (int8_t*)(P + L.w_o), (float*)(P + L.sw_o), nullptr,
                                   0.f, H, H, st));
    TEL_TRY(launch_quantize_weight(dt, w->w_1, (int8_t*)(P + L.w_1), (float*)(P + L.sw_1), nullptr,
                                   0.f, F, H, st));
    TEL_TRY(launch_quantize_weight(dt, w->w_2, (int8_t*)(P + L.w_2), (float*)(P + L.sw_2), nullptr,
                                   0.f, H, F, st));
  } else if (d->int8_gemm) {
    float sa[4], inv[4];
    for (int i = 0; i < 4; ++i) {
      const float a = w->act_amax[i];
      if (!(a > 0.f) || !(a < 3.0e38f)) return TEL_EINVAL;   // positive and finite
      sa[i] = a / 127.0f;
      inv[i] = 127.0f / a;
    }
    float act[ACT_FLOATS] = {sa[0], sa[1], sa[2], sa[3], inv[0], inv[1], inv[2], inv[3]};
    if (d->int8_gemm == 2) {   // int8 attention: Q, K, V code scales and the kernel's constants
      float sqkv[3];
      for (int i = 0; i < 3; ++i) {
        const float a = w->attn_amax[i];
        if (!(a > 0.f) || !(a < 3.0e38f)) return TEL_EINVAL;
        sqkv[i] = a / 127.0f;
        act[8 + i] = 127.0f / a;
      }
      const int hd = d->hidden / d->heads;
      act[11] = ((sqkv[0] * sqkv[1]) / sqrtf((float)hd)) * 1.4426950408889634f;
      act[12] = sqkv[2];
      act[13] = inv[1];
    }
    TEL_TRY(launch_store_f32((float*)(P + L.act), act, ACT_FLOATS, st));
    TEL_TRY(launch_quantize_weight(dt, w->w_qkv, (int8_t*)(P + L.w_qkv), (float*)(P + L.sw_qkv),
                                   (float*)(P + L.dq_qkv), sa[0], 3 * H, H, st));
    TEL_TRY(launch_quantize_weight(dt, w->w_o, (int8_t*)(P + L.w_o), (float*)(P + L.sw_o),
                                   (float*)(P + L.dq_o), sa[1], H, H, st));
    TEL_TRY(launch_quantize_weight(dt, w->w_1, (int8_t*)(P + L.w_1), (float*)(P + L.sw_1),
                                   (float*)(P + L.dq_1), sa[2], F, H, st));
    TEL_TRY(launch_quantize_weight(dt, w->w_2, (int8_t*)(P + L.w_2), (float*)(P + L.sw_2),
                                   (float*)(P + L.dq_2), sa[3], H, F, st));
  } else if (d->sparse_2of4) {   // prune 2:4 and compress into the sparse MFMA operand form
    TEL_TRY(launch_prune_2of4(dt, w->w_qkv, P + L.w_qkv, (uint16_t*)(P + L.wi_qkv), 3 * H, H, st));
    TEL_TRY(launch_prune_2of4(dt, w->w_o, P + L.w_o, (uint16_t*)(P + L.wi_o), H, H, st));
    TEL_TRY(launch_prune_2of4(dt, w->w_1, P + L.w_1, (uint16_t*)(P + L.wi_1), F, H, st));
    TEL_TRY(launch_prune_2of4(dt, w->w_2, P + L.w_2, (uint16_t*)(P + L.wi_2), H, F, st));
  } else {
    TEL_TRY(hipMemcpyAsync(P + L.w_qkv, w->w_qkv, 3 * H * H * es, hipMemcpyDeviceToDevice, st));
    TEL_TRY(hipMemcpyAsync(P + L.w_o, w->w_o, H * H * es, hipMemcpyDeviceToDevice, st));
    TEL_TRY(hipMemcpyAsync(P + L.w_1, w->w_1, F * H * es, hipMemcpyDeviceToDevice, st));
    TEL_TRY(hipMemcpyAsync(P + L.w_2, w->w_2, H * F * es, hipMemcpyDeviceToDevice, st));
  }
  TEL_TRY(launch_widen_f32(dt, w->b_qkv, (float*)(P + L.b_qkv), 3 * H, st));
  TEL_TRY(launch_widen_f32(dt, w->b_o, (float*)(P + L.b_o), H, st));
  TEL_TRY(launch_widen_f32(dt, w->ln1_g, (float*)(P + L.ln1_g), H, st));
  TEL_TRY(launch_widen_f32(dt, w->ln1_b, (float*)(P + L.ln1_b), H, st));
  TEL_TRY(launch_widen_f32(dt, w->b_1, (float*)(P + L.b_1), F, st));
  TEL_TRY(launch_widen_f32(dt, w->b_2, (float*)(P + L.b_2), H, st));
  TEL_TRY(launch_widen_f32(dt, w->ln2_g, (float*)(P + L.ln2_g), H, st));
  TEL_TRY(launch_widen_f32(dt, w->ln2_b, (float*)(P + L.ln2_b), H, st));
  return TEL_OK;
}

size_t tel_encoder_workspace_size(const tel_encoder_desc* d, int max_tokens) {
  if (desc_supported(d) != TEL_OK || max_tokens < 0) return 0;
  return layer_ws(d, (size_t)max_tokens).total;
}

int tel_encoder_layer_forward(const tel_encoder_desc* d, const void* packed, const void* x,
                              void* y, const int32_t* cu_seqlens, int batch, int total_tokens,
                              int max_len, void* workspace, size_t ws_bytes, void* stream) {
  const int sup = desc_supported(d);
  if (sup != TEL_OK) return sup;
  if (batch <= 0 || total_tokens < 0 || max_len < 0) return TEL_EINVAL;
  if (total_tokens == 0) return TEL_OK;
  if (max_len == 0) return TEL_EINVAL;
  if (!packed || !x || !y || !cu_seqlens || !workspace) return TEL_EINVAL;
  if (!aligned256(packed) || !aligned256(workspace) || !aligned16(x) || !aligned16(y))
    return TEL_EINVAL;
  if (x == y) return TEL_EINVAL;
  if (ws_bytes < layer_ws(d, (size_t)total_tokens).total) return TEL_EWORKSPACE;
  return layer_forward(d, (const char*)packed, x, y, cu_seqlens, batch, total_tokens, max_len,
                       (char*)workspace, as_stream(stream));
}

int tel_encoder_layer_forward_noalloc(const tel_encoder_desc* d, const void* packed,
                                      const void* x, void* y, const int32_t* cu_seqlens,
                                      int batch, int total_tokens, int max_len, void* stream) {
  const int sup = desc_supported(d);
  if (sup != TEL_OK) return sup;
  if (batch <= 0 || total_tokens < 0 || max_len < 0) return TEL_EINVAL;
  if (total_tokens == 0) return TEL_OK;
  if (max_len == 0) return TEL_EINVAL;
  if (!packed || !x || !y || !cu_seqlens) return TEL_EINVAL;
  if (!aligned256(packed) || !aligned16(x) || !aligned16(y)) return TEL_EINVAL;
  if (x == y) return TEL_EINVAL;
  if (layer_ws(d, (size_t)total_tokens).total > TEL_NOALLOC_SCRATCH_BYTES) return TEL_EWORKSPACE;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (noalloc_scratch(&ws, &ws_bytes) != hipSuccess) return TEL_EDEVICE;
  return layer_forward(d, (const char*)packed, x, y, cu_seqlens, batch, total_tokens, max_len,
                       (char*)ws, as_stream(stream));
}

int tel_encoder_calibrate(const tel_encoder_desc* d, const void* packed, const void* x, void* y,
                          const int32_t* cu_seqlens, int batch, int total_tokens, int max_len,
                          float* amax, void* workspace, size_t ws_bytes, void* stream) {
  if (d && d->int8_gemm) return TEL_EINVAL;
  if (!amax) return TEL_EINVAL;
  const int r = tel_encoder_layer_forward(d, packed, x, y, cu_seqlens, batch, total_tokens,
                                          max_len, workspace, ws_bytes, stream);
  if (r != TEL_OK || total_tokens == 0) return r;
  const LayerWs W = layer_ws(d, (size_t)total_tokens);
  const size_t T = total_tokens, H = d->hidden, F = d->ffn;
  const char* ws = (const char*)workspace;
  const int dt = d->dtype;
  hipStream_t st = as_stream(stream);
  // inputs of the QKV, O, FFN1 and FFN2 GEMMs: x, ctx, h1 and the GELU output; then the
  // Q, K and V parts of the projection (head-split: three contiguous [heads][T][d] blocks)
  const size_t es = dtype_size(dt);
  TEL_TRY(launch_absmax(dt, x, T * H, amax + 0, st));
  TEL_TRY(launch_absmax(dt, ws + W.ctx, T * H, amax + 1, st));
  TEL_TRY(launch_absmax(dt, ws + W.h1, T * H, amax + 2, st));
  TEL_TRY(launch_absmax(dt, ws + W.f, T * F, amax + 3, st));
  for (int i = 0; i < 3; ++i)
    TEL_TRY(launch_absmax(dt, ws + W.qkv + i * T * H * es, T * H, amax + 4 + i, st));
  return TEL_OK;
}

size_t tel_encoder_forward_workspace_size(const tel_encoder_desc* d, int batch, int max_seq) {
  if (desc_supported(d) != TEL_OK || batch <= 0 || max_seq <= 0) return 0;
  return stack_ws(d, batch, max_seq).total;
}

// ------------------------------------------------------------------ weight prefetch
// A deep stack at few tokens (BERT-large, 24 layers, one 128-token sequence: 25 MB of
// weights per layer against 0.25 MB of activations) is bound by fetching weights: the
// stack's 605 MB do not stay in the 256 MB memory-side cache between forwards, and each
// GEMM pulls its weights from HBM through its few workgroups. There, the layer's short
// kernels (using few compute units at these token counts) carry extra workgroups that read
// weights a later GEMM needs, once, into that cache: the attention FFN1's, the first
// reduce-LayerNorm (after the output projection) FFN2's, the second one (end of the layer)
// the next layer's QKV and output-projection weights, about 8 MB each at BERT-large. Used
// when the weights cannot all stay cached and dominate what a layer reads (few tokens, where
// the plan splits those GEMMs over k and the reduce kernels run); float layers only.
namespace {
constexpr size_t PREFETCH_MIN_STACK_BYTES = size_t(160) << 20;
std::mutex g_prefetch_mu;
int g_prefetch_on = -1;           // -1: read TEL_PREFETCH once (on unless it is "0")

bool prefetch_on_locked() {
  if (g_prefetch_on < 0) {
    const char* e = getenv("TEL_PREFETCH");
    g_prefetch_on = (e && e[0] == '0') ? 0 : 1;
  }
  return g_prefetch_on == 1;
}

bool prefetch_on() {
  std::lock_guard<std::mutex> lk(g_prefetch_mu);
  return prefetch_on_locked();
}

bool prefetch_wanted(const tel_encoder_desc* d, int n_layers, int total_tokens) {
  if (n_layers < 2 || total_tokens <= 0 || d->int8_gemm || d->sparse_2of4) return false;
  const size_t packed = tel_encoder_packed_size(d);
  if ((size_t)n_layers * packed < PREFETCH_MIN_STACK_BYTES) return false;
  const size_t act = (size_t)total_tokens * d->hidden * dtype_size(d->dtype);
  return act * 8 < packed && prefetch_on();
}
}  // namespace

int tel_weight_prefetch(int enable) {
  std::lock_guard<std::mutex> lk(g_prefetch_mu);
  const int prev = prefetch_on_locked() ? 1 : 0;
  if (enable >= 0) g_prefetch_on = enable ? 1 : 0;
  return prev;
}

// Named ranges on the host timeline around a forward and each of its layers (shown by
// rocprofv3 --marker-trace; a call into the marker library otherwise).
namespace {
struct MarkerRange {
  explicit MarkerRange(const char* name) { roctxRangePushA(name); }
  ~MarkerRange() { roctxRangePop(); }
  MarkerRange(const MarkerRange&) = delete;
  MarkerRange& operator=(const MarkerRange&) = delete;
};
const char* const LAYER_NAMES[] = {"tel layer 0", "tel layer 1", "tel layer 2", "tel layer 3",
                                   "tel layer 4", "tel layer 5", "tel layer 6", "tel layer 7",
                                   "tel layer 8", "tel layer 9", "tel layer 10", "tel layer 11",
                                   "tel layer 12", "tel layer 13", "tel layer 14", "tel layer 15",
                                   "tel layer 16", "tel layer 17", "tel layer 18", "tel layer 19",
                                   "tel layer 20", "tel layer 21", "tel layer 22", "tel layer 23"};
constexpr int N_LAYER_NAMES = sizeof(LAYER_NAMES) / sizeof(LAYER_NAMES[0]);
}  // namespace

// The whole forward (offsets, remove padding, layers, rebuild) enqueued on stream st;
// arguments already validated.
static int forward_enqueue(const tel_encoder_desc* d, const void* const* packed_layers,
                           int n_layers, const void* x_pad, void* y_pad,
                           const int32_t* seq_lens, int batch, int max_seq, int total_tokens,
                           int max_len, void* workspace, hipStream_t st) {
  const StackWs S = stack_ws(d, batch, max_seq);
  // the layer workspace is laid out for batch * max_seq tokens; a layer at total_tokens
  // (<= batch * max_seq) re-derives its offsets from its own token count and must fit
  if (layer_ws(d, (size_t)total_tokens).total > S.total - S.layer) return TEL_EWORKSPACE;
  char* ws = (char*)workspace;
  int32_t* cu = (int32_t*)(ws + S.cu);
  int32_t* po = (int32_t*)(ws + S.po);
  void* xa = ws + S.xa;
  void* xb = ws + S.xb;
  const int row_bytes = d->hidden * dtype_size(d->dtype);
  if (batch <= 1024) {   // one launch for both (padding_offset not needed afterwards)
    TEL_TRY(launch_offsets_remove_padding(seq_lens, batch, max_seq, cu, x_pad, xa,
                                          total_tokens, row_bytes, st));
  } else {
    TEL_TRY(launch_offsets(seq_lens, batch, max_seq, cu, po, st));
    TEL_TRY(launch_remove_padding(x_pad, xa, po, total_tokens, row_bytes, st));
  }
  int8_t* qa = (int8_t*)(ws + S.qa);
  int8_t* qb = (int8_t*)(ws + S.qb);
  const size_t act_off = d->int8_gemm ? layer_layout(d).act : 0;
  const bool pf = prefetch_wanted(d, n_layers, total_tokens);
  MarkerRange fwd("tel encoder forward");
  for (int i = 0; i < n_layers; ++i) {
    MarkerRange layer(i < N_LAYER_NAMES ? LAYER_NAMES[i] : "tel layer");
    int r;
    if (d->int8_gemm && !d->dynamic_scales && total_tokens > 0) {
      // each LN2 writes the codes of its output at the next layer's input scale
      Int8Link link;
      link.xq_in = i > 0 ? qa : nullptr;
      if (i + 1 < n_layers) {
        link.xq_out = qb;
        link.next_qinv = (const float*)((const char*)packed_layers[i + 1] + act_off) + 4;
      }
      r = layer_forward_int8(d, (const char*)packed_layers[i], xa, xb, cu, batch, total_tokens,
                             max_len, ws + S.layer, st, link);
      int8_t* tq = qa;
      qa = qb;
      qb = tq;
    } else if (d->int8_gemm && d->dynamic_scales && total_tokens > 0) {
      // each LN2 raises the max-abs statistic of its output for the next layer's input scale
      DynLink dl;
      dl.parity = i & 1;
      dl.in_from_prev = i > 0;
      dl.out_to_next = i + 1 < n_layers;
      r = layer_forward_int8_dynamic(d, (const char*)packed_layers[i], xa, xb, cu, batch,
                                     total_tokens, max_len, ws + S.layer, st, dl);
    } else {
      LayerPrefetch lp;
      lp.on = pf;
      lp.next = pf && i + 1 < n_layers ? (const char*)packed_layers[i + 1] : nullptr;
      r = layer_forward(d, (const char*)packed_layers[i], xa, xb, cu, batch, total_tokens,
                        max_len, ws + S.layer, st, lp);
    }
    if (r != TEL_OK) return r;
    void* t = xa;
    xa = xb;
    xb = t;
  }
  TEL_TRY(launch_rebuild_padding(xa, y_pad, cu, batch, max_seq, row_bytes, st));
  return TEL_OK;
}

// ------------------------------------------------------------------ forward graph cache
// A forward is ~7 launches per layer; replaying them as one HIP graph removes the host's
// per-launch cost, which matters when the caller's host is slow to enqueue. Measured on the
// encoder workloads here the host keeps ahead of the GPU (graph and eager steps within 1 %),
// so the cache is off unless asked for. Graphs are captured on an internal stream
// (capture is not allowed on the legacy default stream) the first time a given set of
// arguments is seen, and launched on the caller's stream afterwards. The key holds every
// argument the launches depend on (pointers, sizes, device); buffer contents and weights
// are read when the graph runs, so reusing buffers is safe. The forward records no memset
// or host work, only kernels.
namespace {
struct GraphEntry {
  std::vector<uintptr_t> key;
  hipGraphExec_t exec;
};
std::mutex g_graph_mu;
std::vector<GraphEntry> g_graphs;                 // most recently used last
std::vector<hipStream_t> g_capture_streams;       // per device, created on first use
int g_graphs_on = -1;                              // -1: read TEL_GRAPHS once
constexpr size_t GRAPH_CACHE_MAX = 8;

bool debug_checks() {   // read on every call, so a process can switch it on and off
  const char* e = getenv("TEL_DEBUG");
  return e && e[0] == '1';
}

bool graphs_on_locked() {
  if (g_graphs_on < 0) {
    const char* e = getenv("TEL_GRAPHS");
    g_graphs_on = (e && e[0] == '1') ? 1 : 0;
  }
  return g_graphs_on == 1;
}
}  // namespace

int tel_graph_cache(int enable) {
  std::lock_guard<std::mutex> lk(g_graph_mu);
  const int prev = graphs_on_locked() ? 1 : 0;
  if (enable >= 0) g_graphs_on = enable ? 1 : 0;
  return prev;
}

int tel_encoder_forward(const tel_encoder_desc* d, const void* const* packed_layers, int n_layers,
                        const void* x_pad, void* y_pad, const int32_t* seq_lens, int batch,
                        int max_seq, int total_tokens, int max_len, void* workspace,
                        size_t ws_bytes, void* stream) {
  const int sup = desc_supported(d);
  if (sup != TEL_OK) return sup;
  if (batch <= 0 || max_seq <= 0 || n_layers < 0 || total_tokens < 0 || max_len < 0)
    return TEL_EINVAL;
  if ((long long)batch * max_seq > INT32_MAX) return TEL_EUNSUPPORTED;
  if (total_tokens > batch * max_seq || max_len > max_seq) return TEL_EINVAL;
  if (total_tokens > 0 && max_len == 0) return TEL_EINVAL;
  if (!x_pad || !y_pad || !seq_lens || !workspace || (n_layers > 0 && !packed_layers))
    return TEL_EINVAL;
  for (int i = 0; i < n_layers; ++i)
    if (!packed_layers[i] || !aligned256(packed_layers[i])) return TEL_EINVAL;
  if (!aligned256(workspace) || !aligned16(x_pad) || !aligned16(y_pad)) return TEL_EINVAL;
  if (x_pad == y_pad) return TEL_EINVAL;
  const StackWs S = stack_ws(d, batch, max_seq);
  if (ws_bytes < S.total) return TEL_EWORKSPACE;
  hipStream_t st = as_stream(stream);
  if (debug_checks()) {
    // TEL_DEBUG=1: the caller's obligations on the lengths checked on the device before any
    // kernel reads the padded batch (a synchronisation of `stream`, in this mode only)
    int32_t* flag = (int32_t*)((char*)workspace + S.dbg);
    int32_t bad = 0;
    TEL_TRY(launch_check_lengths(seq_lens, batch, max_seq, total_tokens, max_len, flag, st));
    TEL_TRY(hipMemcpyAsync(&bad, flag, 4, hipMemcpyDeviceToHost, st));
    TEL_TRY(hipStreamSynchronize(st));
    if (bad) return TEL_EINVAL;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TEL_EDEVICE;
  std::unique_lock<std::mutex> lk(g_graph_mu);
  if (!graphs_on_locked()) {
    lk.unlock();
    return forward_enqueue(d, packed_layers, n_layers, x_pad, y_pad, seq_lens, batch, max_seq,
                           total_tokens, max_len, workspace, st);
  }
  std::vector<uintptr_t> key = {(uintptr_t)dev, (uintptr_t)d->hidden, (uintptr_t)d->heads,
                                (uintptr_t)d->ffn, (uintptr_t)d->dtype, (uintptr_t)d->int8_gemm,
                                (uintptr_t)d->sparse_2of4, (uintptr_t)d->dynamic_scales,
                                (uintptr_t)n_layers, (uintptr_t)x_pad, (uintptr_t)y_pad,
                                (uintptr_t)seq_lens, (uintptr_t)batch, (uintptr_t)max_seq,
                                (uintptr_t)total_tokens, (uintptr_t)max_len,
                                (uintptr_t)workspace,
                                (uintptr_t)prefetch_wanted(d, n_layers, total_tokens)};
  uint32_t eps_bits;
  memcpy(&eps_bits, &d->ln_eps, 4);
  key.push_back(eps_bits);
  for (int i = 0; i < n_layers; ++i) key.push_back((uintptr_t)packed_layers[i]);
  for (size_t i = 0; i < g_graphs.size(); ++i) {
    if (g_graphs[i].key == key) {
      GraphEntry e = g_graphs[i];
      g_graphs.erase(g_graphs.begin() + i);
      g_graphs.push_back(e);
      return status_of(hipGraphLaunch(e.exec, st));
    }
  }
  if ((int)g_capture_streams.size() <= dev) g_capture_streams.resize(dev + 1, nullptr);
  if (!g_capture_streams[dev] &&
      hipStreamCreateWithFlags(&g_capture_streams[dev], hipStreamNonBlocking) != hipSuccess)
    return TEL_EDEVICE;
  hipStream_t cs = g_capture_streams[dev];
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) return TEL_EDEVICE;
  const int r = forward_enqueue(d, packed_layers, n_layers, x_pad, y_pad, seq_lens, batch,
                                max_seq, total_tokens, max_len, workspace, cs);
  hipGraph_t graph = nullptr;
  const hipError_t ce = hipStreamEndCapture(cs, &graph);
  if (r != TEL_OK || ce != hipSuccess || !graph) {
    if (graph) hipGraphDestroy(graph);
    return r != TEL_OK ? r : TEL_EDEVICE;
  }
  hipGraphExec_t exec = nullptr;
  const hipError_t ie = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  hipGraphDestroy(graph);
  if (ie != hipSuccess || !exec) return TEL_EDEVICE;
  if (g_graphs.size() >= GRAPH_CACHE_MAX) {
    // the evicted graph may still be running on some stream: let the device drain first
    if (hipDeviceSynchronize() != hipSuccess) return TEL_EDEVICE;
    hipGraphExecDestroy(g_graphs.front().exec);
    g_graphs.erase(g_graphs.begin());
  }
  g_graphs.push_back(GraphEntry{key, exec});
  return status_of(hipGraphLaunch(exec, st));
}

int tel_gemm_tile_configs(void) { return gemm_tile_configs(); }

int tel_gemm_ex(int epilogue, int dtype, int tile_config, const void* A, const void* W,
                const float* bias, const void* resid, void* C, int M, int N, int K, int heads,
                void* stream) {
  if (!float_type(dtype)) return TEL_EUNSUPPORTED;
  if (M < 0 || N <= 0 || K <= 0) return TEL_EINVAL;
  if (epilogue < TEL_EPI_BIAS || epilogue > TEL_EPI_QKV_SPLIT) return TEL_EINVAL;
  if (tile_config < -2 || tile_config >= gemm_tile_configs()) return TEL_EINVAL;
  if (M == 0) return TEL_OK;
  if (!A || !W || !bias || !C) return TEL_EINVAL;
  if (epilogue == TEL_EPI_BIAS_RESID && !resid) return TEL_EINVAL;
  if (!aligned16(A) || !aligned16(W) || !aligned16(bias) || !aligned16(C)) return TEL_EINVAL;
  if (resid && !aligned16(resid)) return TEL_EINVAL;
  if (K % 8 || N % 4) return TEL_EUNSUPPORTED;
  if (tile_config >= 0 && ((long long)K * dtype_size(dtype)) % 128) return TEL_EUNSUPPORTED;
  if (epilogue == TEL_EPI_QKV_SPLIT) {
    if (heads <= 0 || N % 3 || (N / 3) % heads || ((N / 3) / heads) % 4) return TEL_EUNSUPPORTED;
  }
  GemmArgs g{epilogue, A, W, bias, resid, C, M, N, K, heads};
  const hipStream_t st = as_stream(stream);
  return status_of(tile_config == -2 ? launch_gemm(dtype, g, st)
                                     : launch_gemm_cfg(dtype, tile_config, g, st));
}

int tel_gemm(int epilogue, int dtype, const void* A, const void* W, const float* bias,
             const void* resid, void* C, int M, int N, int K, int heads, void* stream) {
  return tel_gemm_ex(epilogue, dtype, -2, A, W, bias, resid, C, M, N, K, heads, stream);
}

int tel_prune_2of4(const void* w, void* values, uint16_t* index, int N, int K, int dtype,
                   void* stream) {
  if (dtype != DT_F16 && dtype != DT_BF16) return TEL_EUNSUPPORTED;
  if (N < 0 || K <= 0) return TEL_EINVAL;
  if (K % 16) return TEL_EUNSUPPORTED;
  if (N == 0) return TEL_OK;
  if (!w || !values || !index || !aligned16(w) || !aligned16(values) || ((uintptr_t)index & 1u))
    return TEL_EINVAL;
  return status_of(launch_prune_2of4(dtype, w, values, index, N, K, as_stream(stream)));
}

int tel_gemm_2of4_tile_configs(void) { return gemm_sparse_tile_configs(); }

int tel_gemm_2of4(int epilogue, int dtype, int tile_config, const void* A, const void* values,
                  const uint16_t* index, const float* bias, const void* resid, void* C, int M,
                  int N, int K, int heads, void* stream) {
  if (dtype != DT_F16 && dtype != DT_BF16) return TEL_EUNSUPPORTED;
  if (M < 0 || N <= 0 || K <= 0) return TEL_EINVAL;
  if (epilogue < TEL_EPI_BIAS || epilogue > TEL_EPI_QKV_SPLIT) return TEL_EINVAL;
  if (tile_config < -2 || tile_config == -1 || tile_config >= gemm_sparse_tile_configs())
    return TEL_EINVAL;
  if (K % 128 || N % 4) return TEL_EUNSUPPORTED;
  if (epilogue == TEL_EPI_QKV_SPLIT &&
      (heads <= 0 || N % 3 || (N / 3) % heads || ((N / 3) / heads) % 4))
    return TEL_EUNSUPPORTED;
  if (M == 0) return TEL_OK;
  if (!A || !values || !index || !bias || !C) return TEL_EINVAL;
  if (epilogue == TEL_EPI_BIAS_RESID && !resid) return TEL_EINVAL;
  if (!aligned16(A) || !aligned16(values) || !aligned16(index) || !aligned16(bias) ||
      !aligned16(C) || (resid && !aligned16(resid)))
    return TEL_EINVAL;
  GemmArgs g{epilogue, A, values, bias, resid, C, M, N, K, heads};
  g.w_idx = index;
  const hipStream_t st = as_stream(stream);
  return status_of(tile_config == -2 ? launch_gemm(dtype, g, st)
                                     : launch_gemm_cfg(dtype, tile_config, g, st));
}

int tel_quantize_i8(const void* x, int8_t* q, size_t n, float inv_scale, int dtype,
                    void* stream) {
  if (!float_type(dtype)) return TEL_EUNSUPPORTED;
  if (!(inv_scale > 0.f) || !(inv_scale < 3.0e38f)) return TEL_EINVAL;
  if (n == 0) return TEL_OK;
  if (!x || !q || !aligned16(x) || ((uintptr_t)q & 7u)) return TEL_EINVAL;
  return status_of(launch_quantize_act(dtype, x, q, n, nullptr, inv_scale, as_stream(stream)));
}

int tel_quantize_weight_i8(const void* w, int8_t* q, float* scales, int N, int K, int dtype,
                           void* stream) {
  if (!float_type(dtype)) return TEL_EUNSUPPORTED;
  if (N < 0 || K <= 0) return TEL_EINVAL;
  if (N == 0) return TEL_OK;
  if (!w || !q || !scales) return TEL_EINVAL;
  return status_of(launch_quantize_weight(dtype, w, q, scales, nullptr, 0.f, N, K,
                                          as_stream(stream)));
}

int tel_gemm_i8_i32(const int8_t* A, const int8_t* B, int32_t* C, int M, int N, int K,
                    void* stream) {
  if (M < 0 || N <= 0 || K <= 0) return TEL_EINVAL;
  if (M == 0) return TEL_OK;
  if (!A || !B || !C || !aligned16(A) || !aligned16(B) || !aligned16(C)) return TEL_EINVAL;
  if (K % 16 || N % 4) return TEL_EUNSUPPORTED;
  GemmArgs g{EPI_RAW_I32, A, B, nullptr, nullptr, C, M, N, K, 1};
  return status_of(launch_gemm(DT_I8, g, as_stream(stream)));
}

int tel_gemm_i8(int epilogue, const int8_t* A, const int8_t* W, const float* dq,
                const float* bias, const void* resid, void* C, const float* qinv, int out_int8,
                int M, int N, int K, int heads, void* stream) {
  if (M < 0 || N <= 0 || K <= 0) return TEL_EINVAL;
  if (epilogue < TEL_EPI_BIAS || epilogue > TEL_EPI_QKV_SPLIT) return TEL_EINVAL;
  if (out_int8 && epilogue != TEL_EPI_BIAS_GELU && epilogue != TEL_EPI_QKV_SPLIT) return TEL_EINVAL;
  if (M == 0) return TEL_OK;
  if (!A || !W || !dq || !bias || !C || (out_int8 && !qinv)) return TEL_EINVAL;
  if (epilogue == TEL_EPI_BIAS_RESID && !resid) return TEL_EINVAL;
  if (!aligned16(A) || !aligned16(W) || !aligned16(dq) || !aligned16(bias) || !aligned16(C))
    return TEL_EINVAL;
  if (resid && !aligned16(resid)) return TEL_EINVAL;
  if (K % 16 || N % 4) return TEL_EUNSUPPORTED;
  if (epilogue == TEL_EPI_QKV_SPLIT &&
      (heads <= 0 || N % 3 || (N / 3) % heads || ((N / 3) / heads) % 4))
    return TEL_EUNSUPPORTED;
  GemmArgs g{epilogue, A, W, bias, resid, C, M, N, K, heads};
  g.dq = dq;
  g.qinv = qinv;
  g.out_i8 = out_int8 ? 1 : 0;
  return status_of(launch_gemm(DT_I8, g, as_stream(stream)));
}

size_t tel_swin_packed_size(const tel_swin_desc* d) {
  if (swin_supported(d) != TEL_OK) return 0;
  return swin_layout(d).total;
}

int tel_swin_prepare(const tel_swin_desc* d, const tel_swin_weights* w, void* packed,
                     size_t packed_bytes, void* stream) {
  const int sup = swin_supported(d);
  if (sup != TEL_OK) return sup;
  if (!w || !packed || !aligned256(packed)) return TEL_EINVAL;
  const void* ptrs[] = {w->ln1_g, w->ln1_b, w->w_qkv, w->b_qkv, w->rpb_table, w->w_proj,
                        w->b_proj, w->ln2_g, w->ln2_b, w->w_1, w->b_1, w->w_2, w->b_2};
  for (const void* p : ptrs)
    if (!p) return TEL_EINVAL;
  const SwinLayout L = swin_layout(d);
  if (packed_bytes < L.total) return TEL_EWORKSPACE;
  const size_t C = d->channels, F = d->mlp_hidden, es = dtype_size(d->dtype);
  const int dt = d->dtype;
  char* P = (char*)packed;
  hipStream_t st = as_stream(stream);
  TEL_TRY(hipMemcpyAsync(P + L.w_qkv, w->w_qkv, 3 * C * C * es, hipMemcpyDeviceToDevice, st));
  TEL_TRY(hipMemcpyAsync(P + L.w_proj, w->w_proj, C * C * es, hipMemcpyDeviceToDevice, st));
  TEL_TRY(hipMemcpyAsync(P + L.w_1, w->w_1, F * C * es, hipMemcpyDeviceToDevice, st));
  TEL_TRY(hipMemcpyAsync(P + L.w_2, w->w_2, C * F * es, hipMemcpyDeviceToDevice, st));
  TEL_TRY(launch_widen_f32(dt, w->ln1_g, (float*)(P + L.ln1_g), C, st));
  TEL_TRY(launch_widen_f32(dt, w->ln1_b, (float*)(P + L.ln1_b), C, st));
  TEL_TRY(launch_widen_f32(dt, w->b_qkv, (float*)(P + L.b_qkv), 3 * C, st));
  TEL_TRY(launch_widen_f32(dt, w->b_proj, (float*)(P + L.b_proj), C, st));
  TEL_TRY(launch_widen_f32(dt, w->ln2_g, (float*)(P + L.ln2_g), C, st));
  TEL_TRY(launch_widen_f32(dt, w->ln2_b, (float*)(P + L.ln2_b), C, st));
  TEL_TRY(launch_widen_f32(dt, w->b_1, (float*)(P + L.b_1), F, st));
  TEL_TRY(launch_widen_f32(dt, w->b_2, (float*)(P + L.b_2), C, st));
  TEL_TRY(launch_expand_rel_bias(dt, w->rpb_table, (float*)(P + L.bias), d->window, d->heads, st));
  return TEL_OK;
}

int tel_swin_fused_stages(const tel_swin_desc* d) {
  if (swin_supported(d) != TEL_OK) return 0;
  return swin_fused_stages(d);
}

size_t tel_swin_workspace_size(const tel_swin_desc* d) {
  if (swin_supported(d) != TEL_OK) return 0;
  return swin_ws(d).total;
}

int tel_window_attention_forward(const tel_swin_desc* d, const void* packed, const void* x,
                                 void* y, int flags, void* workspace, size_t ws_bytes,
                                 void* stream) {
  const int sup = swin_supported(d);
  if (sup != TEL_OK) return sup;
  // flags: TEL_SWIN_ATTN_ONLY, or one stage alone (TEL_SWIN_ONE_STAGE(k), k = 0..4) on the
  // workspace buffers a whole block leaves behind
  const int stage = (flags >> 8) - 1;
  if (flags & ~(TEL_SWIN_ATTN_ONLY | (0xf << 8))) return TEL_EINVAL;
  if (stage >= 5 || (stage >= 0 && (flags & TEL_SWIN_ATTN_ONLY))) return TEL_EINVAL;
  auto run = [stage](int k) { return stage < 0 || stage == k; };
  if (!packed || !x || !y || !workspace) return TEL_EINVAL;
  if (!aligned256(packed) || !aligned256(workspace) || !aligned16(x) || !aligned16(y))
    return TEL_EINVAL;
  if (x == y) return TEL_EINVAL;
  const SwinWs W = swin_ws(d);
  if (ws_bytes < W.total) return TEL_EWORKSPACE;
  const SwinLayout L = swin_layout(d);
  const SwinGeom g = swin_geom(d);
  const int T = d->batch * d->height * d->width, C = d->channels, F = d->mlp_hidden;
  const int nh = d->heads, dt = d->dtype;
  const char* P = (const char*)packed;
  char* ws = (char*)workspace;
  auto F32 = [&](size_t off) { return (const float*)(P + off); };
  hipStream_t st = as_stream(stream);
  void* zw = ws + W.zw;
  void* qkv = ws + W.qkv;
  void* ctx = ws + W.ctx;
  void* x1 = (flags & TEL_SWIN_ATTN_ONLY) ? y : (void*)(ws + W.x1);
  void* hh = ws + W.h;
  void* f = ws + W.f;
  // LN1 + roll(-s) + window partition, one gather: on the QKV GEMM's input rows when the
  // skinny kernel serves these shapes (no LN1 tensor at all), else a gather LayerNorm
  const bool fuse_ln = gemm_rows_supported(dt, 3 * C, C) && gemm_rows_supported(dt, F, C);
  GemmArgs a{EPI_QKV_SPLIT, zw, P + L.w_qkv, F32(L.b_qkv), nullptr, qkv, T, 3 * C, C, nh};
  if (fuse_ln) {
    a.A = x;
    a.ln_g = F32(L.ln1_g);
    a.ln_b = F32(L.ln1_b);
    a.ln_eps = d->ln_eps;
    a.ln_gather = 1;
    a.geom = g;
  } else if (run(0)) {
    TEL_TRY(launch_layernorm_gather(dt, x, zw, F32(L.ln1_g), F32(L.ln1_b), T, C, d->ln_eps, g,
                                    st));
  }
  const int fused = swin_fused_stages(d);
  if (fused & TEL_SWIN_FUSED_ATTN) {
    // the attention half in one kernel (stage 0); stages 1 and 2 have nothing left to do
    if (run(0))
      TEL_TRY(launch_swin_attn_half(x, x1, P + L.w_qkv, F32(L.b_qkv), F32(L.bias),
                                    P + L.w_proj, F32(L.b_proj), F32(L.ln1_g), F32(L.ln1_b),
                                    d->ln_eps, g, d->batch * g.nW, st));
  } else {
    if (run(0)) TEL_TRY(launch_gemm(dt, a, st));
    if (run(1))
      TEL_TRY(launch_window_attention(dt, qkv, ctx, F32(L.bias), g, d->batch * g.nW, nh, C / nh,
                                      st));
    // proj + bias, window reverse + roll(+s) + residual in the epilogue
    a = GemmArgs{EPI_SWIN_SCATTER, ctx, P + L.w_proj, F32(L.b_proj), x, x1, T, C, C, nh};
    a.geom = g;
    if (run(2)) TEL_TRY(launch_gemm(dt, a, st));
  }
  if (flags & TEL_SWIN_ATTN_ONLY) return TEL_OK;
  if (fused & TEL_SWIN_FUSED_MLP) {
    // the MLP half in one kernel (stage 3); stage 4 has nothing left to do
    if (run(3))
      TEL_TRY(launch_swin_mlp(dt, x1, y, P + L.w_1, F32(L.b_1), P + L.w_2, F32(L.b_2),
                              F32(L.ln2_g), F32(L.ln2_b), d->ln_eps, T, st));
    return TEL_OK;
  }
  // LN2 on fc1's input rows (or a LayerNorm kernel), fc1 + bias + GELU
  a = GemmArgs{EPI_BIAS_GELU, hh, P + L.w_1, F32(L.b_1), nullptr, f, T, F, C, nh};
  if (fuse_ln) {
    a.A = x1;
    a.ln_g = F32(L.ln2_g);
    a.ln_b = F32(L.ln2_b);
    a.ln_eps = d->ln_eps;
  } else if (run(3)) {
    TEL_TRY(launch_layernorm(dt, dt, x1, hh, nullptr, F32(L.ln2_g), F32(L.ln2_b), T, C,
                             d->ln_eps, st));
  }
  if (run(3)) TEL_TRY(launch_gemm(dt, a, st));
  a = GemmArgs{EPI_BIAS_RESID, f, P + L.w_2, F32(L.b_2), x1, y, T, C, F, nh};
  if (run(4)) TEL_TRY(launch_gemm(dt, a, st));
  return TEL_OK;
}

int tel_window_partition_layernorm(const void* x, void* y, const float* gamma, const float* beta,
                                   int batch, int height, int width, int channels, int window,
                                   int shift, float eps, int dtype, void* stream) {
  if (batch <= 0 || height <= 0 || width <= 0 || channels <= 0 || window <= 0 || shift < 0 ||
      !(eps >= 0.f))
    return TEL_EINVAL;
  if (height % window || width % window || shift >= window) return TEL_EINVAL;
  if (!layernorm_supported(dtype, channels)) return TEL_EUNSUPPORTED;
  if ((long long)batch * height * width > INT32_MAX / 4) return TEL_EUNSUPPORTED;
  if (!x || !y || !gamma || !beta) return TEL_EINVAL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(gamma) || !aligned16(beta)) return TEL_EINVAL;
  if (x == y) return TEL_EINVAL;
  tel_swin_desc d{};
  d.height = height;
  d.width = width;
  d.window = window;
  d.shift = shift;
  return status_of(launch_layernorm_gather(dtype, x, y, gamma, beta, batch * height * width,
                                           channels, eps, swin_geom(&d), as_stream(stream)));
}

int tel_attention_int8(const int8_t* qkv_codes, void* out, int out_codes, const float* scales,
                       const int32_t* cu_seqlens, int batch, int total_tokens, int max_len,
                       int heads, int head_dim, void* stream) {
  if (batch <= 0 || total_tokens < 0 || max_len < 0 || heads <= 0 || head_dim <= 0)
    return TEL_EINVAL;
  if (!attention_int8_supported(head_dim)) return TEL_EUNSUPPORTED;
  if (total_tokens == 0) return TEL_OK;
  if (max_len == 0) return TEL_EINVAL;
  if (!qkv_codes || !out || !scales || !cu_seqlens) return TEL_EINVAL;
  if (!aligned16(qkv_codes) || !aligned16(out) || ((uintptr_t)scales & 3u)) return TEL_EINVAL;
  return status_of(launch_attention_int8(qkv_codes, out, out_codes ? 1 : 0, cu_seqlens, batch,
                                         total_tokens, max_len, heads, head_dim, scales,
                                         as_stream(stream)));
}

int tel_patch_merging(const void* x, void* y, const float* gamma, const float* beta,
                      const void* w_red, int batch, int height, int width, int channels,
                      float eps, int dtype, void* stream) {
  if (batch <= 0 || height <= 0 || width <= 0 || channels <= 0 || !(eps >= 0.f))
    return TEL_EINVAL;
  if (height % 2 || width % 2) return TEL_EINVAL;
  if (!patch_merging_supported(dtype, channels)) return TEL_EUNSUPPORTED;
  if ((long long)batch * height * width > INT32_MAX / 4) return TEL_EUNSUPPORTED;
  if (!x || !y || !gamma || !beta || !w_red) return TEL_EINVAL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(gamma) || !aligned16(beta) || !aligned16(w_red))
    return TEL_EINVAL;
  if (x == y) return TEL_EINVAL;
  const int M = batch * (height / 2) * (width / 2);
  GemmArgs a{EPI_PLAIN, x, w_red, nullptr, nullptr, y, M, 2 * channels, 4 * channels, 1};
  a.ln_g = gamma;
  a.ln_b = beta;
  a.ln_eps = eps;
  a.ln_merge = 1;
  a.geom.Hs = height;
  a.geom.Ws = width;
  return status_of(launch_gemm(dtype, a, as_stream(stream)));
}

int tel_attention_varlen(const void* qkv_split, void* ctx, const int32_t* cu_seqlens, int batch,
                         int total_tokens, int max_len, int heads, int head_dim, int dtype,
                         void* stream) {
  if (batch <= 0 || total_tokens < 0 || max_len < 0 || heads <= 0 || head_dim <= 0)
    return TEL_EINVAL;
  if (!attention_supported(dtype, head_dim)) return TEL_EUNSUPPORTED;
  if (total_tokens == 0) return TEL_OK;
  if (max_len == 0) return TEL_EINVAL;
  if (!qkv_split || !ctx || !cu_seqlens) return TEL_EINVAL;
  if (!aligned16(qkv_split) || !aligned16(ctx)) return TEL_EINVAL;
  return status_of(launch_attention(dtype, qkv_split, ctx, cu_seqlens, batch, total_tokens,
                                    max_len, heads, head_dim, as_stream(stream)));
}

int tel_gemm_partial(int dtype, int tile_config, int splits, const void* A, const void* W,
                     void* partials, int partial_bytes, int M, int N, int K, void* stream) {
  if (!float_type(dtype) && dtype != DT_I8) return TEL_EUNSUPPORTED;
  if (M < 0 || N <= 0 || K <= 0 || splits < 1) return TEL_EINVAL;
  if (partial_bytes != 4 && partial_bytes != 2) return TEL_EINVAL;
  if (partial_bytes == 2 && dtype != DT_F16) return TEL_EUNSUPPORTED;
  if (tile_config < -1 || tile_config >= gemm_tile_configs()) return TEL_EINVAL;
  if (M == 0) return TEL_OK;
  if (!A || !W || !partials) return TEL_EINVAL;
  if (!aligned16(A) || !aligned16(W) || !aligned16(partials)) return TEL_EINVAL;
  const long long kb = (long long)K * dtype_size(dtype);
  if (K % (dtype == DT_I8 ? 16 : 8) || N % 4) return TEL_EUNSUPPORTED;
  if (tile_config >= 0 && kb % 128) return TEL_EUNSUPPORTED;
  if (splits > 1 && (tile_config < 0 || (kb / 128) % splits)) return TEL_EUNSUPPORTED;
  GemmArgs g{EPI_PARTIAL, A, W, nullptr, nullptr, partials, M, N, K, 1};
  g.splits = splits;
  g.part16 = partial_bytes == 2;
  return status_of(launch_gemm_cfg(dtype, tile_config, g, as_stream(stream)));
}

int tel_gemm_partial_plan(int dtype, int M, int N, int K, int* tile_config, int* splits,
                          int* partial_bytes) {
  if (!tile_config || !splits || !partial_bytes) return TEL_EINVAL;
  if (!float_type(dtype) && dtype != DT_I8) return TEL_EUNSUPPORTED;
  if (M < 0 || N <= 0 || K <= 0) return TEL_EINVAL;
  int p16 = 0;
  *splits = gemm_partial_plan(dtype, M, N, K, tile_config, &p16);
  *partial_bytes = p16 ? 2 : 4;
  return TEL_OK;
}

int tel_layernorm_reduce(const void* partials, int splits, int partial_bytes, const float* dq,
                         const float* bias, const void* resid, int resid_dtype, void* y,
                         int out_dtype, float* y32, int8_t* yq, const float* qinv,
                         const float* gamma, const float* beta, int rows, int width, float eps,
                         int round_pre, void* stream) {
  if (rows < 0 || width <= 0 || splits < 1 || splits > 8 || !(eps >= 0.f)) return TEL_EINVAL;
  if (partial_bytes != 4 && partial_bytes != 2) return TEL_EINVAL;
  if (partial_bytes == 2 && (out_dtype != DT_F16 || dq)) return TEL_EUNSUPPORTED;
  const bool combo = (resid_dtype == DT_F16 && out_dtype == DT_F16) ||
                     (resid_dtype == DT_BF16 && out_dtype == DT_BF16) ||
                     (resid_dtype == DT_F32 && (out_dtype == DT_BF16 || out_dtype == DT_F32));
  if (!combo || !layernorm_supported(out_dtype, width)) return TEL_EUNSUPPORTED;
  if (rows == 0) return TEL_OK;
  if (!partials || !bias || !resid || !y || !gamma || !beta || (yq && !qinv)) return TEL_EINVAL;
  for (const void* q : {partials, (const void*)bias, resid, (const void*)y, (const void*)gamma,
                        (const void*)beta})
    if (!aligned16(q)) return TEL_EINVAL;
  if ((dq && !aligned16(dq)) || (y32 && !aligned16(y32)) || (yq && ((uintptr_t)yq % 8)))
    return TEL_EINVAL;
  LnReduceArgs a{partials, splits, dq, bias, resid, resid_dtype, y, out_dtype, y32, yq,
                 qinv, gamma, beta, rows, width, eps, round_pre ? 1 : 0};
  a.part16 = partial_bytes == 2;
  return status_of(launch_layernorm_reduce(a, as_stream(stream)));
}

int tel_layernorm(const void* x, void* y, const float* gamma, const float* beta, int rows,
                  int width, float eps, int dtype, void* stream) {
  if (rows < 0 || width <= 0 || !(eps >= 0.f)) return TEL_EINVAL;
  if (!layernorm_supported(dtype, width)) return TEL_EUNSUPPORTED;
  if (rows == 0) return TEL_OK;
  if (!x || !y || !gamma || !beta) return TEL_EINVAL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(gamma) || !aligned16(beta)) return TEL_EINVAL;
  return status_of(launch_layernorm(dtype, dtype, x, y, nullptr, gamma, beta, rows, width, eps,
                                    as_stream(stream)));
}

}  // extern "C"
