// Host-side launchers of the library's kernels (internal; the public ABI is include/tel.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device.h"

namespace tel {

enum DType { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_I8 = 3 };
enum Epi {
  EPI_BIAS = 0, EPI_BIAS_GELU = 1, EPI_BIAS_RESID = 2, EPI_QKV_SPLIT = 3, EPI_RAW_I32 = 4,
  EPI_SWIN_SCATTER = 5,  // bias + residual, row m written to image row geom.src_row(m)
  EPI_PARTIAL = 6,       // raw 32-bit accumulators (float32, or int32 for int8 operands) of
                         // k-split s at C + s * M * N, or those sums rounded to fp16
                         // (GemmArgs::part16, fp16 operands); a reduce kernel finishes the sum
  EPI_PLAIN = 7,         // C = A W^T in the storage type, no bias (skinny kernel only)
  EPI_BIAS_GELU_AMAX = 8 // int8 operands, fp16 output: EPI_BIAS_GELU that also raises the
                         // max-abs statistic out_amax (amax_raise) by its stored outputs
};

inline int dtype_size(int dt) { return dt == DT_F32 ? 4 : dt == DT_I8 ? 1 : 2; }

// offsets.hip
hipError_t launch_offsets(const int32_t* lens, int batch, int max_seq, int32_t* cu,
                          int32_t* padding_offset, hipStream_t stream);
// Offsets from a 0/1 mask [batch][max_seq] (holes allowed); padding_offset capacity
// batch * max_seq, its first batch entries also scratch for the per-sequence counts.
hipError_t launch_offsets_mask(const uint8_t* mask, int batch, int max_seq, int32_t* cu,
                               int32_t* padding_offset, hipStream_t stream);
// Debug check of a forward's lengths (one workgroup): out[0] = bit 0 some length outside
// [0, max_seq], bit 1 sum != total, bit 2 max > max_len; 0 when all hold.
hipError_t launch_check_lengths(const int32_t* lens, int batch, int max_seq, long long total,
                                int max_len, int32_t* out, hipStream_t stream);
// padding.hip (row_bytes % 16 == 0)
// Rebuild for the mask form: rows with mask 0 zeroed, packed row t to row t + po[t].
hipError_t launch_rebuild_padding_mask(const void* x_packed, void* x_pad, const uint8_t* mask,
                                       const int32_t* po, int total_tokens, int batch,
                                       int max_seq, int row_bytes, hipStream_t stream);
hipError_t launch_remove_padding(const void* x_pad, void* x_packed, const int32_t* padding_offset,
                                 int total_tokens, int row_bytes, hipStream_t stream);
hipError_t launch_rebuild_padding(const void* x_packed, void* x_pad, const int32_t* cu, int batch,
                                  int max_seq, int row_bytes, hipStream_t stream);
// Offsets (cu only) and padding removal in one launch; batch <= 1024, else
// hipErrorInvalidValue (use launch_offsets + launch_remove_padding).
hipError_t launch_offsets_remove_padding(const int32_t* lens, int batch, int max_seq,
                                        int32_t* cu, const void* x_pad, void* x_packed,
                                        int total_tokens, int row_bytes, hipStream_t stream);

// gemm.hip
struct GemmArgs {
  int epi;
  const void* A;        // [M][K]
  const void* W;        // [N][K]
  const float* bias;    // [N] float32
  const void* resid;    // [M][N] (EPI_BIAS_RESID)
  void* C;
  int M, N, K;
  int heads;            // EPI_QKV_SPLIT
  int resid_f32 = 0;    // EPI_BIAS_RESID, bf16 operands only: residual is float32
  int out_f32 = 0;      // EPI_BIAS_RESID, bf16 operands only: output is float32
  const float* dq = nullptr;    // int8 operands: per-column dequantisation scale [N]
  const float* dyn_amax = nullptr;  // int8 operands, dynamic activation scale: dq holds the
                                    // weight scales s_w and the activation scale is
                                    // *dyn_amax / 127 (1 when 0), applied per column
  const float* qinv = nullptr;  // int8 output: device scalar 1 / scale (EPI_BIAS_GELU), or
                                // three of them, for Q, K and V (EPI_QKV_SPLIT)
  int out_i8 = 0;               // int8 operands, EPI_BIAS_GELU / EPI_QKV_SPLIT: int8 codes
  float* out_amax = nullptr;    // EPI_BIAS_GELU_AMAX: max-abs statistic raised by |stored
                                // output| (AMAX_SLOTS copies, each >= 0 before)
  SwinGeom geom{};              // EPI_SWIN_SCATTER
  int splits = 1;               // pipelined kernel only: K split over this many workgroups
  int part16 = 0;               // EPI_PARTIAL, fp16 operands: partial sums stored as fp16
  // LayerNorm applied to each row of A before the product (skinny kernel only, see
  // gemm_rows_supported): A row r is LN(A[r]) * ln_g + ln_b, read from row geom.src_row(r)
  // when ln_gather is set (the shifted-window partition)
  const float* ln_g = nullptr;
  const float* ln_b = nullptr;
  float ln_eps = 0.f;
  int ln_gather = 0;
  // patch merging (skinny kernel, with ln_g): A row r is the concatenation of the four
  // image rows geom.merge_src(r, k), k = 0..3, of the Hs x Ws image in geom
  int ln_merge = 0;
  // 2:4-sparse weights (f16/bf16, K % 128 == 0): W holds the kept values [N][K/2] and
  // w_idx the 16-bit index words [N][K/16] (the form launch_prune_2of4 writes)
  const uint16_t* w_idx = nullptr;
};
// The (dtype, N, K) the skinny row kernel serves (the shifted-window block's projections).
bool gemm_rows_supported(int dtype, int N, int K);
// Patch merging of an image of `channels` channels runs on the skinny kernel (N = 2C, K = 4C).
bool patch_merging_supported(int dtype, int channels);
// The shifted-window block's attention half fused (LN1 + shift + partition, QKV, window
// attention with the bias table and shift mask, proj + reverse + unshift + residual), for
// fp16, channels 96, 3 heads and windows of up to 64 tokens; bias_exp as for
// launch_window_attention.
bool swin_attn_half_supported(int dtype, int channels, int heads, int window_tokens);
hipError_t launch_swin_attn_half(const void* x, void* x1, const void* w_qkv, const float* b_qkv,
                                 const float* bias_exp, const void* w_proj, const float* b_proj,
                                 const float* ln_g, const float* ln_b, float eps,
                                 const SwinGeom& geom, int windows, hipStream_t stream);
// The shifted-window block's MLP half fused (LN2, fc1 + bias + GELU, fc2 + bias + residual:
// y = x1 + W2 GELU(W1 LN(x1) + b1) + b2), for channels 96 and hidden 384, fp16.
bool swin_mlp_supported(int dtype, int channels, int hidden);
hipError_t launch_swin_mlp(int dtype, const void* x1, void* y, const void* w1, const float* b1,
                           const void* w2, const float* b2, const float* ln_g, const float* ln_b,
                           float eps, int M, hipStream_t stream);
hipError_t launch_gemm(int dtype, const GemmArgs& a, hipStream_t stream);
// Explicit tile configuration: -1 = register-staged kernel, 0.. = pipelined tile table.
hipError_t launch_gemm_cfg(int dtype, int cfg, const GemmArgs& a, hipStream_t stream);
int gemm_tile_configs();
int gemm_sparse_tile_configs();   // tile table of the 2:4-sparse kernel
// Tile configuration and number of k-splits for a partial-sum GEMM (EPI_PARTIAL) of this
// shape; returns the splits (>= 1), sets *cfg, and *part16 = 1 when the partial sums are
// to be stored as fp16 (fp16 operands only), else 0.
int gemm_partial_plan(int dtype, int M, int N, int K, int* cfg, int* part16);

// attention.hip
bool attention_supported(int dtype, int head_dim);
// ctxq != nullptr: write only the int8 codes of the stored-type output (scale *qinv);
// psplit: P enters P V split into two 16-bit parts also for fp16 values (the int8 layers,
// whose codes of the context are sensitive to P's rounding; always so for bf16 and codes).
// amax (context stored, no codes): raise the max-abs statistic amax (AMAX_SLOTS copies,
// amax_raise; each >= 0 before) by |stored context|.
// ahead (16-byte aligned): extra workgroups read [ahead, ahead + ahead_bytes) once into the
// cache for a later kernel (read_ahead).
hipError_t launch_attention(int dtype, const void* qkv, void* ctx, const int32_t* cu, int batch,
                            int total, int max_len, int heads, int head_dim, hipStream_t stream,
                            int8_t* ctxq = nullptr, const float* qinv = nullptr,
                            bool psplit = false, float* amax = nullptr,
                            const void* ahead = nullptr, size_t ahead_bytes = 0);

// attention_int8.hip: attention on int8 Q, K, V codes ([3][heads][T][D]); scales (device):
// [0] = s_q s_k / sqrt(D) * log2 e, [1] = s_v, [2] = 1 / (input scale of the O projection);
// out = fp16 context (out_codes 0) or its int8 codes at scales[2] (out_codes 1).
bool attention_int8_supported(int head_dim);
hipError_t launch_attention_int8(const int8_t* qkv, void* out, int out_codes, const int32_t* cu,
                                 int batch, int total, int max_len, int heads, int head_dim,
                                 const float* scales, hipStream_t stream);

// layernorm.hip: y = LN(x) in type dtype_out from x in type dtype_in; when y_f32 is not
// null the same result is also written there in float32.
bool layernorm_supported(int dtype, int width);
// LayerNorm of a sum finished here: x = sum_s part[s] (float32; int32 times dq[n] when dq is
// set) + bias[n] + resid[row][n], optionally rounded to the output type first (the int8
// layer's stored pre-LayerNorm values); writes y (dtype_out), optionally y32 (float32 copy)
// and yq (int8 codes of the stored y, scale device scalar *qinv).
struct LnReduceArgs {
  const void* part; int nsplit; const float* dq; const float* bias;
  const void* resid; int resid_dt;
  void* y; int out_dt; float* y32; int8_t* yq; const float* qinv;
  const float* gamma; const float* beta; int rows, width; float eps; int round_pre;
  int part16 = 0;   // partial sums stored as fp16 (out type fp16 only), else 32-bit
  // optional: extra workgroups read [prefetch, prefetch + prefetch_bytes) (16-byte aligned)
  // once and discard it, bringing weights a later kernel needs into the memory-side cache
  const void* prefetch = nullptr;
  size_t prefetch_bytes = 0;
};
hipError_t launch_layernorm_reduce(const LnReduceArgs& a, hipStream_t stream);
hipError_t launch_layernorm(int dtype_in, int dtype_out, const void* x, void* y, float* y_f32,
                            const float* gamma, const float* beta, int rows, int width, float eps,
                            hipStream_t stream);
// LayerNorm of the shifted-window gather: y[r] = LN(x[geom.src_row(r)]).
hipError_t launch_layernorm_gather(int dtype, const void* x, void* y, const float* gamma,
                                   const float* beta, int rows, int width, float eps,
                                   const SwinGeom& geom, hipStream_t stream);
// fp16 LayerNorm that also raises the max-abs statistic amax (AMAX_SLOTS copies,
// amax_raise; each must hold a non-negative value, e.g. 0, beforehand) by its
// (fp16-rounded) output.
hipError_t launch_layernorm_amax(const void* x, void* y, float* amax, const float* gamma,
                                 const float* beta, int rows, int width, float eps,
                                 hipStream_t stream);
// fp16 LayerNorm that also writes the int8 codes of its (fp16-rounded) output.
hipError_t launch_layernorm_q8(const void* x, void* y, int8_t* yq, const float* qinv,
                               const float* gamma, const float* beta, int rows, int width,
                               float eps, hipStream_t stream);

// swin.hip: window attention with relative-position bias and shift mask over window-
// order Q, K, V in the [3][heads][T][d] layout; bias_exp [heads][N][64] float32 (already
// times log2 e, -inf in columns >= N). total_tokens = images * nW * N.
bool window_attention_supported(int dtype, int head_dim, int N);
hipError_t launch_window_attention(int dtype, const void* qkv_split, void* ctx,
                                   const float* bias_exp, const SwinGeom& geom, int windows,
                                   int heads, int head_dim, hipStream_t stream);
// bias_exp[h][p][q] = table[idx(p, q)][h] * log2(e) for q < N = M * M, -inf for q >= N.
hipError_t launch_expand_rel_bias(int dtype, const void* table, float* bias_exp, int M, int heads,
                                  hipStream_t stream);

// sparse.hip: 2:4 magnitude pruning of W [N][K] (K % 16 == 0) into kept values [N][K/2]
// and 16-bit index words [N][K/16] (two largest |w| of every group of four along k, ties to
// the lower k; group g of a word in bits 4g..4g+3, first position in the low two bits).
hipError_t launch_prune_2of4(int dtype, const void* w, void* values, uint16_t* index, int N,
                             int K, hipStream_t stream);

// noalloc.hip: device address (on the current device) and size of the library-owned
// scratch array of tel_encoder_layer_forward_noalloc; looked up once per device.
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

// prepare.hip
hipError_t launch_widen_f32(int dtype, const void* src, float* dst, int n, hipStream_t stream);
hipError_t launch_store_f32(float* dst, const float* vals, int n, hipStream_t stream);
// quant.hip: per-row weight quantisation W[N][K] -> codes [N][K], scales [N]; optional
// per-column dequantisation scales dq[n] = act_scale * s_w[n] (dq may be null).
hipError_t launch_quantize_weight(int dtype, const void* w, int8_t* q, float* s_w, float* dq,
                                  float act_scale, int N, int K, hipStream_t stream);
// q[i] = clamp(rne(float(x[i]) * inv), -127, 127); inv is a device scalar when inv_dev is
// not null, else the host value inv_host. Dynamic scales: amax_stat is a max-abs statistic
// (AMAX_SLOTS copies), a = its folded value, inv = 127 / a (1 when a is 0), and a is stored
// to *amax_out (for the GEMM epilogue that dequantises). The n_zero statistics
// zero + i * AMAX_STAT_FLOATS (n_zero <= 8, none of them amax_stat) are cleared by the
// kernel, for maxima later kernels of the stream raise.
hipError_t launch_quantize_act(int dtype, const void* x, int8_t* q, size_t n, const float* inv_dev,
                               float inv_host, hipStream_t stream,
                               const float* amax_stat = nullptr, float* amax_out = nullptr,
                               float* zero = nullptr, int n_zero = 0);
// *out = max(*out, max |x[i]|) (calibration statistic; out is a device float >= 0); with
// stat, out is a max-abs statistic of AMAX_SLOTS copies raised by amax_raise instead.
hipError_t launch_absmax(int dtype, const void* x, size_t n, float* out, hipStream_t stream,
                         bool stat = false);
// Clears n max-abs statistics stats + i * AMAX_STAT_FLOATS (every copy) with a kernel.
hipError_t launch_clear_amax(float* stats, int n, hipStream_t stream);

}  // namespace tel
