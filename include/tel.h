/*
 * tel.h - C ABI of libtel.so: inference forward of a Transformer encoder layer with
 * padding removal and fused kernels, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow these web pages (cited by title and figure/section):
 *   [KS]  Kuaishou heterogeneous-computing article "GPU底层优化 | 如何让Transformer在GPU上
 *         跑得更快？" (How to make Transformer run faster on GPU): Fig. 6 (fused
 *         self-attention and FFN kernels), Fig. 7 (FP16 precision per kernel), Fig. 8
 *         (memory management), Fig. 9 (padding removal with an offset mask, padded and
 *         packed sequences convertible both ways), Fig. 10 (which kernels can run
 *         without padding), Fig. 11 (GEMM configuration).
 *   [SW]  NVIDIA talk on Swin Transformer "大規模なビジュアル モデルを使用してトレーニングと
 *         推論を高速化するにはどうすればよいですか?" (How to accelerate training and inference
 *         of large visual models): section 1 (attention, multi-head, BERT as a stack of
 *         encoders, window attention, window shift, relative position bias); section 3
 *         (inference: preprocessing done once, GEMM + bias / + activation epilogues,
 *         separating the bias from a GEMM whose post-op is LayerNorm, hand-written
 *         LayerNorm and shift-window-partition kernels, fMHA, QKV GEMM+bias with
 *         re-laid-out weights, INT8 GEMM with INT32 accumulation and dequantisation).
 *
 * Conventions (every entry point):
 *   - Pointers are DEVICE pointers unless marked [host]. The caller owns every buffer
 *     (inputs, outputs, packed weights, workspace); the library never allocates or
 *     frees device memory. The one exception is the fixed scratch array of
 *     tel_encoder_layer_forward_noalloc, part of the library's image on each GPU.
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call only enqueues
 *     work on it and returns; there is no hidden synchronisation. Buffers must stay
 *     valid until the stream has consumed them. Outputs must not alias inputs.
 *   - Return value: a tel_status. Arguments are validated on the host before any
 *     launch; on failure nothing is enqueued. TEL_EDEVICE reports a launch error from
 *     the HIP runtime.
 *   - Layouts are row-major. Weights use the nn.Linear layout W[out][in]. Activation
 *     and weight storage type is TEL_F32, TEL_F16 or TEL_BF16; accumulation,
 *     softmax, LayerNorm statistics and GELU are float32.
 *   - Caller obligations not checked on the device: 0 <= seq_lens[b] <= max_seq,
 *     total_tokens == sum(seq_lens), max_len >= max(seq_lens). With the environment
 *     variable TEL_DEBUG=1 (read on every call), tel_encoder_forward checks all three on the device
 *     before any kernel reads the padded batch and returns TEL_EINVAL when one fails; that
 *     check synchronises the caller's stream (this mode only).
 *   - Thread safety: calls on different streams may run concurrently; there is no
 *     global mutable state except the graph cache (mutex-guarded) and the scratch array
 *     of tel_encoder_layer_forward_noalloc (see there).
 */
#ifndef TEL_H
#define TEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TEL_OK = 0,
  TEL_EINVAL = 1,        /* null/misaligned pointer, negative or inconsistent size      */
  TEL_EUNSUPPORTED = 2,  /* valid but unsupported shape or type (e.g. head_dim 48)      */
  TEL_EWORKSPACE = 3,    /* workspace or packed buffer smaller than required            */
  TEL_EDEVICE = 4        /* the HIP runtime reported an error                           */
} tel_status;

typedef enum { TEL_F32 = 0, TEL_F16 = 1, TEL_BF16 = 2, TEL_I8 = 3 } tel_dtype;

/* Human-readable name of a status code (static string). */
const char* tel_status_str(int status);
/* Library version string (static). */
const char* tel_version(void);

/* ------------------------------------------------------------------ offsets, padding */

/* Offset mask of padding removal ([KS] Fig. 9).
 *   seq_lens        [batch] int32, valid length of each right-padded sequence.
 *   cu_seqlens      [batch+1] int32 out: exclusive prefix sum, cu[0] = 0, cu[b+1] = cu[b] + len[b].
 *   padding_offset  [>= total tokens] int32 out: for packed token t of sequence b,
 *                   padding_offset[t] = b * max_seq - cu[b], so its padded row is
 *                   t + padding_offset[t].
 * batch >= 1, max_seq >= 1. Two launches (a single-workgroup scan, then a fill). */
int tel_build_offsets(const int32_t* seq_lens, int batch, int max_seq, int32_t* cu_seqlens,
                      int32_t* padding_offset, void* stream);

/* Padding removal ([KS] Figs. 9-10): x_packed[t][:] = x_pad[t + padding_offset[t]][:].
 *   x_pad [batch*max_seq][width], x_packed [total_tokens][width], element type `dtype`
 *   (TEL_F32/F16/BF16). width * element size must be a multiple of 16 bytes and both
 *   pointers 16-byte aligned. total_tokens == 0 is a no-op. */
int tel_remove_padding(const void* x_pad, void* x_packed, const int32_t* padding_offset,
                       int total_tokens, int width, int dtype, void* stream);

/* Padding rebuild ([KS] Fig. 9), inverse of tel_remove_padding:
 *   x_pad[b*max_seq + i][:] = x_packed[cu[b] + i][:] for i < len[b], and 0 for the pad rows.
 *   Same type/alignment rules as tel_remove_padding. */
int tel_rebuild_padding(const void* x_packed, void* x_pad, const int32_t* cu_seqlens,
                        int batch, int max_seq, int width, int dtype, void* stream);

/* The offset mask in its general form ([KS] Fig. 9: tokens removed wherever the mask says,
 * holes allowed). mask [batch][max_seq] uint8 (device; 0 = padding, anything else = valid).
 * Packed order: sequence by sequence, positions increasing.
 *   cu_seqlens[b+1] = cu_seqlens[b] + (valid positions of sequence b), cu_seqlens[0] = 0;
 *   padding_offset[t] = b*max_seq + s - t for the packed token t at position s of sequence b,
 *   so tel_remove_padding gathers the valid rows unchanged and cu_seqlens feeds the layer.
 * padding_offset: capacity batch*max_seq int32 (the first batch entries also serve as
 * scratch during the call; T = cu_seqlens[batch] entries hold the result). The caller learns
 * T (and the longest sequence) from the mask or by reading cu_seqlens back.
 * batch >= 1, max_seq >= 1, batch*max_seq < 2^31 (else TEL_EUNSUPPORTED). Three launches
 * (per-sequence counts, the tiled scan of tel_build_offsets, per-sequence compaction). */
int tel_build_offsets_mask(const uint8_t* mask, int batch, int max_seq, int32_t* cu_seqlens,
                           int32_t* padding_offset, void* stream);

/* Padding rebuild for the mask form, inverse of tel_remove_padding with the offsets of
 * tel_build_offsets_mask: x_pad[t + padding_offset[t]][:] = x_packed[t][:] for t < total_tokens,
 * and 0 for every row whose mask byte is 0. x_pad [batch*max_seq][width]; type and alignment
 * rules as tel_remove_padding; total_tokens == 0 zeroes every masked row only. */
int tel_rebuild_padding_mask(const void* x_packed, void* x_pad, const uint8_t* mask,
                             const int32_t* padding_offset, int total_tokens, int batch,
                             int max_seq, int width, int dtype, void* stream);

/* ------------------------------------------------------------------ encoder layer */

/* Post-LN BERT encoder layer ([SW] section 1; [KS] Fig. 6):
 *   qkv = x W_qkv^T + b_qkv ; ctx = MHA(qkv) within each sequence, scale 1/sqrt(head_dim)
 *   h1  = LN(ctx W_o^T + b_o + x) ; f = GELU(h1 W_1^T + b_1)   (exact erf GELU)
 *   y   = LN(f W_2^T + b_2 + h1)  ; LN: biased variance, eps = ln_eps. */
typedef struct {
  int hidden;      /* H, multiple of 8                                         */
  int heads;       /* H % heads == 0; head_dim = H / heads in {16, 32, 64, 128} */
  int ffn;         /* F, multiple of 8                                         */
  int dtype;       /* storage type of activations and weights                 */
  int int8_gemm;   /* 1: the four projection GEMMs run in int8 (dtype TEL_F16; H and F
                      multiples of 16); 2: attention's two products in int8 as well
                      (tel_attention_int8); see the int8 section below               */
  float ln_eps;
  int sparse_2of4; /* 1: the four projection matrices are pruned 2:4 when prepared and run
                      on the sparse MFMA (dtype TEL_F16 or TEL_BF16, not int8_gemm; H and F
                      multiples of 128); see the 2:4 section below                   */
  int dynamic_scales; /* 1 (int8_gemm == 1 only): dynamic activation scales ("揭秘Transformer
                         模型：速度优化与量化技术", section 3.3, dynamic quantisation): each int8
                         GEMM's activation scale is max-abs / 127 of that GEMM's fp16 input over
                         the batch being run, reduced on the device; act_amax is ignored.
                         After tel_encoder_layer_forward the first 16 bytes of its workspace
                         hold the four max-abs values it used (float32: the QKV, O, FFN1 and
                         FFN2 inputs); the layer never splits a GEMM over k              */
} tel_encoder_desc;

/* Canonical weights of one layer, storage type desc->dtype, device pointers:
 * W_qkv [3H][H] with rows [Q heads | K heads | V heads], b_qkv [3H], W_o [H][H], b_o [H],
 * ln1 gamma/beta [H], W_1 [F][H], b_1 [F], W_2 [H][F], b_2 [H], ln2 gamma/beta [H]. */
typedef struct {
  const void *w_qkv, *b_qkv, *w_o, *b_o, *ln1_g, *ln1_b;
  const void *w_1, *b_1, *w_2, *b_2, *ln2_g, *ln2_b;
  /* [host] int8 only: calibration max-abs of the inputs of the QKV, O, FFN1 and FFN2
   * GEMMs (static per-tensor activation scales a/127). Ignored otherwise. */
  float act_amax[4];
  /* [host] int8_gemm == 2 only: calibration max-abs of the Q, K and V parts of the QKV
   * projection (the static scales of the codes attention multiplies). Ignored otherwise. */
  float attn_amax[3];
} tel_encoder_weights;

/* Bytes of the packed (preprocessed) form of one layer's weights. 0 on a bad desc. */
size_t tel_encoder_packed_size(const tel_encoder_desc* desc);

/* One-time preprocessing of one layer's weights ([SW] section 3: work that needs doing
 * once is done ahead of inference): copies weights into the GEMM operand layout, widens
 * biases and LayerNorm parameters to float32, and for int8 quantises the weights per
 * output channel (codes rne(W / s) clamped to +-127, s = max|W[n,:]| / 127) and stores
 * the per-column dequantisation scales. `packed` (>= tel_encoder_packed_size bytes,
 * 256-byte aligned) is written on `stream`. */
int tel_encoder_prepare(const tel_encoder_desc* desc, const tel_encoder_weights* w,
                        void* packed, size_t packed_bytes, void* stream);

/* Workspace bytes tel_encoder_layer_forward needs for up to max_tokens packed tokens. */
size_t tel_encoder_workspace_size(const tel_encoder_desc* desc, int max_tokens);

/* One layer on packed tokens: x [total_tokens][H] -> y [total_tokens][H].
 * cu_seqlens [batch+1] from tel_build_offsets; max_len [host] >= longest sequence.
 * workspace: >= tel_encoder_workspace_size(desc, total_tokens) bytes, 256-byte aligned. */
int tel_encoder_layer_forward(const tel_encoder_desc* desc, const void* packed,
                              const void* x, void* y, const int32_t* cu_seqlens, int batch,
                              int total_tokens, int max_len, void* workspace,
                              size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): tel_encoder_layer_forward with the
 * workspace taken from a scratch array the library owns, one per GPU, of
 * TEL_NOALLOC_SCRATCH_BYTES, held until the process ends. Nothing is allocated or freed
 * by the call; the caller still passes inputs, output and packed weights as for
 * tel_encoder_layer_forward (same arguments, same results).
 *   Limit: tel_encoder_workspace_size(desc, total_tokens) must not exceed
 *   TEL_NOALLOC_SCRATCH_BYTES (64 MiB: e.g. a BERT-base fp16 layer up to 4,241 tokens),
 *   else TEL_EWORKSPACE and nothing is enqueued.
 *   Every call on one GPU uses that GPU's one array, which keeps the last call's contents:
 *   calls that can overlap on the same GPU (different streams, or host threads without
 *   ordering) race on it and must be serialised by the caller. The first call on a device
 *   looks up the array's address there (hipGetSymbolAddress; TEL_EDEVICE on failure). */
#define TEL_NOALLOC_SCRATCH_BYTES (64u << 20)
int tel_encoder_layer_forward_noalloc(const tel_encoder_desc* desc, const void* packed,
                                      const void* x, void* y, const int32_t* cu_seqlens,
                                      int batch, int total_tokens, int max_len, void* stream);

/* Post-training calibration of the int8 variant's static activation scales: runs one
 * floating-point layer (desc->int8_gemm == 0) exactly as tel_encoder_layer_forward and
 * raises amax[0..6] (device float[7], caller-initialised, e.g. to 0) to the max-abs of
 * the inputs of its QKV, O, FFN1 and FFN2 GEMMs (x, attention output, h1, GELU output)
 * and of the Q, K and V parts of its QKV projection ([4..6]). Calls accumulate, so a stack
 * is calibrated layer by layer on one or more batches; [0..3] become
 * tel_encoder_weights.act_amax of the int8 layer, [4..6] its attn_amax. */
int tel_encoder_calibrate(const tel_encoder_desc* desc, const void* packed, const void* x,
                          void* y, const int32_t* cu_seqlens, int batch, int total_tokens,
                          int max_len, float* amax, void* workspace, size_t ws_bytes,
                          void* stream);

/* Workspace bytes of tel_encoder_forward for a batch of `batch` x `max_seq`. */
size_t tel_encoder_forward_workspace_size(const tel_encoder_desc* desc, int batch, int max_seq);

/* Whole stack on a padded batch ([KS] Figs. 9-10): offsets, padding removal, n_layers
 * layers on the packed tokens, padding rebuild (pad rows of y_pad are 0).
 *   packed_layers [host] array of n_layers device pointers (tel_encoder_prepare output).
 *   x_pad, y_pad [batch][max_seq][H]; seq_lens [batch] int32 (device).
 *   total_tokens, max_len [host]: sum and max of seq_lens. */
int tel_encoder_forward(const tel_encoder_desc* desc, const void* const* packed_layers,
                        int n_layers, const void* x_pad, void* y_pad, const int32_t* seq_lens,
                        int batch, int max_seq, int total_tokens, int max_len,
                        void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ shifted-window block
 * Swin-style block ([SW] section 1: attention inside non-overlapping M x M windows, a
 * cyclic window shift, a relative position bias; section 3: the bias lookup moved to
 * preprocessing, a fused shift-window-partition kernel, fMHA), pre-LN:
 *   Z  = LN1(X); Zs = roll(Z, -s) (both image axes); windows row-major, tokens row-major
 *   A  = per window and head: softmax(q k^T / sqrt(d) + B_h + mask) v, heads concatenated,
 *        then W_proj + b_proj; B_h[p][q] = table[(py_p - py_q + M - 1) * (2M - 1) +
 *        (px_p - px_q + M - 1)][h]; mask excludes key q for query p unless both lie in
 *        the same region of the shifted frame (per axis [0, L-M), [L-M, L-s), [L-s, L))
 *   X1 = X + roll(window_reverse(A), +s);  Y = X1 + W_2 GELU(W_1 LN2(X1) + b_1) + b_2
 * Tokens are in row-major image order: x, y [batch][height * width][channels].
 * Supported: dtype TEL_F16 or TEL_F32; channels, mlp_hidden multiples of 8; head_dim in
 * {16, 32, 64}; window * window <= 64; height, width multiples of window; 0 <= shift < window. */
typedef struct {
  int batch, height, width, channels, heads, window, shift, mlp_hidden;
  int dtype;
  float ln_eps;
} tel_swin_desc;

/* Device pointers, storage type desc->dtype: ln1/ln2 gamma, beta [C]; W_qkv [3C][C] (rows
 * [Q heads | K heads | V heads]), b_qkv [3C]; rpb_table [(2M-1)^2][heads]; W_proj [C][C],
 * b_proj [C]; W_1 [F][C], b_1 [F]; W_2 [C][F], b_2 [C]. */
typedef struct {
  const void *ln1_g, *ln1_b, *w_qkv, *b_qkv, *rpb_table, *w_proj, *b_proj;
  const void *ln2_g, *ln2_b, *w_1, *b_1, *w_2, *b_2;
} tel_swin_weights;

/* tel_window_attention_forward flag: stop after X1 = X + attention branch (y := X1). */
#define TEL_SWIN_ATTN_ONLY 1
/* tel_window_attention_forward flag for per-kernel measurement: run stage k alone, reading and
 * writing the workspace buffers exactly as the whole block does (k = 0: LN1 + shift + window
 * partition + QKV; 1: window attention; 2: proj + window reverse + unshift + residual; 3: LN2 +
 * fc1 + GELU; 4: fc2 + residual, which writes y; where tel_swin_fused_stages says so, stage 0
 * is the whole attention half and writes X1 while stages 1 and 2 do nothing, and stage 3 is the
 * whole MLP half and writes y while stage 4 does nothing). Stage k
 * reads what stages < k wrote into the same workspace, so a whole-block call on that workspace
 * must come first; running the five stages in order equals one whole-block call. Not
 * combinable with TEL_SWIN_ATTN_ONLY (TEL_EINVAL). */
#define TEL_SWIN_ONE_STAGE(k) (((k) + 1) << 8)

size_t tel_swin_packed_size(const tel_swin_desc* desc);
/* One-time preprocessing: weights copied, vectors widened to float32, and the bias table
 * expanded to [heads][M*M][64] float32 (times log2 e, -inf padding). packed: 256-byte
 * aligned, >= tel_swin_packed_size bytes. */
int tel_swin_prepare(const tel_swin_desc* desc, const tel_swin_weights* w, void* packed,
                     size_t packed_bytes, void* stream);
size_t tel_swin_workspace_size(const tel_swin_desc* desc);
/* [host] Which halves of the block run as one kernel each (the Swin talk "大規模なビジュアル
 * モデル…", section 3, fuses the steps within each half; here each half is one pass whose
 * intermediates never reach memory): TEL_SWIN_FUSED_ATTN, the attention half (LN1 + shift +
 * partition, QKV, window attention, proj + reverse + unshift + residual), for fp16, channels
 * 96, 3 heads, windows of at most 64 tokens; TEL_SWIN_FUSED_MLP, the MLP half (LN2, fc1 + bias
 * + GELU, fc2 + bias + residual), for fp16, channels 96, mlp_hidden 384 (Swin-T stage 1).
 * 0 for an unsupported descriptor. No device work. */
#define TEL_SWIN_FUSED_ATTN 1
#define TEL_SWIN_FUSED_MLP 2
int tel_swin_fused_stages(const tel_swin_desc* desc);
/* The block on x -> y (flags 0), or the attention half only (TEL_SWIN_ATTN_ONLY).
 * Workspace: 256-byte aligned, >= tel_swin_workspace_size bytes. x and y must differ. */
int tel_window_attention_forward(const tel_swin_desc* desc, const void* packed, const void* x,
                                 void* y, int flags, void* workspace, size_t ws_bytes,
                                 void* stream);

/* ------------------------------------------------------------------ kernel-level entry points
 * The same kernels the layer uses, exposed so that tests and per-kernel measurements can
 * localise a result to one kernel. */

/* GEMM epilogue selector for tel_gemm. */
typedef enum {
  TEL_EPI_BIAS = 0,        /* C = A W^T + b                                               */
  TEL_EPI_BIAS_GELU = 1,   /* C = GELU(A W^T + b)                                         */
  TEL_EPI_BIAS_RESID = 2,  /* C = A W^T + b + R       (R [M][N])                          */
  TEL_EPI_QKV_SPLIT = 3    /* C = A W^T + b written head-split as [3][heads][M][N/(3*heads)] */
} tel_epilogue;

/* C = epilogue(A [M][K] x W[N][K]^T), storage type `dtype`, float32 accumulation; bias is
 * float32 [N]; resid (TEL_EPI_BIAS_RESID) has C's type and shape; `heads` is used by
 * TEL_EPI_QKV_SPLIT only. K % 8 == 0, N % 4 == 0, 16-byte aligned pointers. */
int tel_gemm(int epilogue, int dtype, const void* A, const void* W, const float* bias,
             const void* resid, void* C, int M, int N, int K, int heads, void* stream);

/* Number of entries in the GEMM tile table (tile_config 0 .. n-1 of tel_gemm_ex). */
int tel_gemm_tile_configs(void);

/* tel_gemm with an explicit tile configuration, for tuning and tests:
 *   -2 = automatic (the choice tel_gemm makes), -1 = register-staged 64x64 kernel (any K with
 *   K % 8 == 0), 0 .. n-1 = entries of the pipelined tile table (K * element size must be
 *   a multiple of 128 bytes). Other arguments as tel_gemm. */
int tel_gemm_ex(int epilogue, int dtype, int tile_config, const void* A, const void* W,
                const float* bias, const void* resid, void* C, int M, int N, int K, int heads,
                void* stream);

/* Variable-length multi-head attention ([SW] section 3, fMHA: batched GEMM, softmax and
 * batched GEMM in one kernel). qkv_split [3][heads][total_tokens][head_dim] (the
 * TEL_EPI_QKV_SPLIT layout); ctx [total_tokens][heads*head_dim]; query i of sequence b
 * attends to keys cu[b] .. cu[b+1]-1 only; scale 1/sqrt(head_dim). */
int tel_attention_varlen(const void* qkv_split, void* ctx, const int32_t* cu_seqlens, int batch,
                         int total_tokens, int max_len, int heads, int head_dim, int dtype,
                         void* stream);

/* ------------------------------------------------------------------ 2:4 sparse weights
 * [TRT], the paragraphs on sparsity of the Ampere architecture: weak connections are
 * pruned, removing about half of the weights, and the matrix hardware skips their work.
 * Here: fine-grained 2:4 structured sparsity along the input dimension k, by magnitude,
 * executed on gfx950's sparse MFMA (v_smfmac_f32_16x16x64_{f16,bf16}). */

/* Prune W [N][K] (type dtype: TEL_F16 or TEL_BF16) 2:4 and write it compressed: in every
 * group of four consecutive k of a row the two weights of largest |w| are kept (ties to the
 * lower k); values [N][K/2] receive them in increasing k; index [N][K/16] receives one
 * 16-bit word per 16 k with group g's two positions (0..3) in bits 4g..4g+3, the first in
 * the low two bits. K % 16 == 0; w and values 16-byte aligned, index 2-byte aligned. */
int tel_prune_2of4(const void* w, void* values, uint16_t* index, int N, int K, int dtype,
                   void* stream);

/* Number of entries in the 2:4-sparse GEMM's tile table (tile_config of tel_gemm_2of4). */
int tel_gemm_2of4_tile_configs(void);

/* C = epilogue(A W^T) with W given in the compressed 2:4 form of tel_prune_2of4 (values,
 * index), i.e. the product with the pruned matrix; epilogues, bias, resid, heads and the
 * storage type as tel_gemm (TEL_F16 or TEL_BF16). K % 128 == 0, N % 4 == 0, 16-byte aligned
 * pointers. tile_config: -2 automatic, else 0 .. tel_gemm_2of4_tile_configs() - 1. */
int tel_gemm_2of4(int epilogue, int dtype, int tile_config, const void* A, const void* values,
                  const uint16_t* index, const float* bias, const void* resid, void* C, int M,
                  int N, int K, int heads, void* stream);

/* ------------------------------------------------------------------ int8 GEMM variant
 * [SW] section 3, INT8 quantisation: inputs and weights are quantised to INT8, the GEMM
 * accumulates in INT32 and the result is dequantised; bias, residual and LayerNorm stay
 * floating point. Here: symmetric codes in [-127, 127], round half to even; weights per
 * output channel (s[n] = max_k |W[n][k]| / 127, 1 for a zero row), activations per tensor
 * with static scales s_a = amax / 127 from calibration (tel_encoder_weights.act_amax).
 * With desc->int8_gemm = 1 an encoder layer quantises the inputs of its QKV, O, FFN1 and
 * FFN2 GEMMs, runs them on int8 MFMA with int32 accumulation and dequantises in the
 * epilogue (acc * s_a * s[n] + bias); attention runs in fp16 on the dequantised Q, K, V.
 * Every code is taken from the fp16-rounded value: code = clamp(rne(float(x) * 127/amax)). */

/* q[i] = clamp(rne(float(x[i]) * inv_scale), -127, 127) for i < n; x of type dtype,
 * 16-byte aligned; q 8-byte aligned; inv_scale [host] > 0 and finite. */
int tel_quantize_i8(const void* x, int8_t* q, size_t n, float inv_scale, int dtype, void* stream);

/* Per-output-channel weight quantisation of W [N][K] (type dtype): scales[n] =
 * max_k |W[n][k]| / 127 (1 if the row is zero), q[n][k] = clamp(rne(W[n][k] / scales[n]),
 * -127, 127), float32 arithmetic with correctly rounded division. */
int tel_quantize_weight_i8(const void* w, int8_t* q, float* scales, int N, int K, int dtype,
                           void* stream);

/* C[m][n] = sum_k A[m][k] * B[n][k], exact int32 accumulation of int8 codes (the int8
 * layer's GEMM without its epilogue). K % 16 == 0, N % 4 == 0, 16-byte aligned pointers.
 * |C| <= K * 127^2 must fit in int32 (K <= 133,143). */
int tel_gemm_i8_i32(const int8_t* A, const int8_t* B, int32_t* C, int M, int N, int K,
                    void* stream);

/* One GEMM of the int8 layer with its epilogue ([SW] section 3, INT8: INT8 GEMM, INT32
 * accumulation, dequantised outputs): acc[m][n] = sum_k A[m][k] * W[n][k] over int8 codes,
 * exact in int32, then v = acc * dq[n] + bias[n] (float32 arithmetic; dq[n] = activation
 * scale * weight scale of column n) and the epilogue of tel_gemm: TEL_EPI_BIAS, _BIAS_GELU,
 * _BIAS_RESID (resid fp16 [M][N]) or _QKV_SPLIT. C is fp16 ([M][N], or the head-split
 * layout), except out_int8 != 0 (TEL_EPI_BIAS_GELU or TEL_EPI_QKV_SPLIT): C receives int8
 * codes clamp(rne(float(fp16(v)) * qinv), -127, 127), qinv a device scalar (GELU) or three,
 * one each for the Q, K and V columns (head split, int8 attention). A [M][K], W [N][K];
 * K % 16 == 0, N % 4 == 0, 16-byte aligned pointers. */
int tel_gemm_i8(int epilogue, const int8_t* A, const int8_t* W, const float* dq,
                const float* bias, const void* resid, void* C, const float* qinv, int out_int8,
                int M, int N, int K, int heads, void* stream);

/* Attention with both products on int8 codes ([SW] section 3, INT8 paragraph: all matrix
 * multiplications in int8), the attention of an int8_gemm == 2 layer. qkv_codes
 * [3][heads][total_tokens][head_dim] int8 (codes of Q, K, V at scales s_q, s_k, s_v);
 * scales: device float[3] = {s_q * s_k / sqrt(head_dim) * log2(e), s_v, 1 / s_o}. Per query
 * i of sequence b and head h, keys of sequence b only: S = q . k exact in int32; t = S *
 * scales[0] (float32); p = 2^(t - max_j t) in float32; P codes r = rne(127 p); ctx = s_v *
 * (sum_j r v_j) / (sum_j r), both sums exact int32. out: ctx [total_tokens][heads *
 * head_dim] fp16 (out_codes 0), or the int8 codes clamp(rne(float(fp16(ctx)) / s_o), +-127)
 * (out_codes 1). head_dim in {16, 32, 64, 128}; qkv_codes and out 16-byte aligned. */
int tel_attention_int8(const int8_t* qkv_codes, void* out, int out_codes, const float* scales,
                       const int32_t* cu_seqlens, int batch, int total_tokens, int max_len,
                       int heads, int head_dim, void* stream);

/* Shifted-window partition with LayerNorm, one gather ([SW] section 3, the hand-written
 * shift-window-partition kernel): y row r (window order: images, windows row-major,
 * tokens row-major in a window) = LN(x image row ((wy*M + py + s) mod H, (wx*M + px + s)
 * mod W)) * gamma + beta. x, y [batch * height * width][channels]. */
int tel_window_partition_layernorm(const void* x, void* y, const float* gamma, const float* beta,
                                   int batch, int height, int width, int channels, int window,
                                   int shift, float eps, int dtype, void* stream);

/* Patch merging, the downsampling between two Swin stages ([SW] section 1: stages with a
 * downsampling step between them, halving the resolution; section 3, INT8 paragraph: the
 * PatchMerge GEMM). One kernel: the 2 x 2 gather, a LayerNorm over the 4C gathered
 * features and the linear map 4C -> 2C (no bias):
 *   v(i, j) = [x(2i, 2j), x(2i+1, 2j), x(2i, 2j+1), x(2i+1, 2j+1)]     (4 * channels values)
 *   y(i, j) = (LN(v(i, j)) * gamma + beta) W_red^T
 * x [batch][height * width][channels] (row-major image order), y [batch][(height/2) *
 * (width/2)][2 * channels], W_red [2 * channels][4 * channels] of type dtype; gamma, beta
 * float32 [4 * channels]. height and width even; dtype TEL_F16 or TEL_BF16; channels 96
 * (Swin-T's stage 1 -> stage 2), else TEL_EUNSUPPORTED. 16-byte aligned pointers, x != y. */
int tel_patch_merging(const void* x, void* y, const float* gamma, const float* beta,
                      const void* w_red, int batch, int height, int width, int channels,
                      float eps, int dtype, void* stream);

/* y[r][:] = LN(x[r][:]) * gamma + beta over rows of width `width` (float32 gamma/beta). */
int tel_layernorm(const void* x, void* y, const float* gamma, const float* beta, int rows,
                  int width, float eps, int dtype, void* stream);

/* Graph cache of tel_encoder_forward, for callers whose host is slow to enqueue (off by
 * default; the environment variable TEL_GRAPHS=1 turns it on at load). With it on, the
 * first call with a given set of arguments (device,
 * descriptor, layer pointers, buffers, sizes) records the forward's kernels as one HIP graph
 * on an internal stream, and every call replays that graph on the caller's stream: one
 * launch instead of ~10 per layer. Buffer contents (inputs, lengths, weights) are read when
 * the graph runs, so refilling buffers between calls is safe; at most 8 graphs are kept (the
 * eviction of the oldest waits for the device to drain). enable: 1 on, 0 off, -1 query only;
 * returns the previous setting. Thread-safe. */
int tel_graph_cache(int enable);

/* Weight read-ahead of tel_encoder_forward (on by default; the environment variable
 * TEL_PREFETCH=0 turns it off at load). For float stacks whose weights cannot all stay in
 * the GPU's 256 MB memory-side cache and dominate what a layer reads (n_layers x packed size
 * >= 160 MiB and packed size > 8 x the layer's activation bytes, e.g. a 24-layer BERT-large
 * over 128 tokens), the two reduce-LayerNorm kernels of each k-split layer carry extra
 * workgroups that read weights the next GEMMs use, once, so that those GEMMs find them
 * cached: the layer's FFN weights after the output projection, the next layer's QKV and
 * output-projection weights at the end of the layer. A scheduling aid of this library, not
 * a step of the layer: same stream, no extra launch, and outputs bit-identical with and
 * without. enable: 1 on, 0 off, -1 query only; returns the previous setting.
 * Thread-safe. */
int tel_weight_prefetch(int enable);

/* Split-k GEMM without epilogue: the first half of a layer's output projection and FFN2,
 * whose add-bias + residual + LayerNorm epilogue ([SW] section 3, the fused
 * add-bias-residual-LayerNorm) tel_layernorm_reduce finishes.
 *   partials[s][m][n] = sum over k in split s of A[m][k] * W[n][k]
 * A [M][K], W [N][K] of type dtype (TEL_F16, TEL_BF16, TEL_F32, or TEL_I8 codes); with
 * partial_bytes 4 the partials are float32 for float operands and exact int32 for TEL_I8;
 * with partial_bytes 2 (TEL_F16 only, else TEL_EUNSUPPORTED) each partial sum is rounded to
 * fp16. splits * M * N values written.
 * K is cut into `splits` equal runs of whole 128-byte slices. tile_config as in tel_gemm_ex
 * except -2 (no automatic choice here: see tel_gemm_partial_plan); splits > 1 needs
 * tile_config >= 0 and (K * element size / 128) % splits == 0. K % 8 == 0 (16 for int8),
 * N % 4 == 0, 16-byte aligned pointers. */
int tel_gemm_partial(int dtype, int tile_config, int splits, const void* A, const void* W,
                     void* partials, int partial_bytes, int M, int N, int K, void* stream);

/* [host] The tile configuration, number of k-splits and partial-sum width (4: float32 /
 * int32, 2: fp16) the encoder layer uses for a partial GEMM of this shape. splits > 1 when
 * the unsplit tile grid has fewer than about 100 workgroups (few tokens): the smallest
 * power of two (at most 8) that reaches that many, then doubled while the grid still fits
 * one round of 256 workgroups, keeping at least 8 k-slices of 128 bytes per split, 32-bit
 * partials (partial_bytes 4; fp16 partials are never planned). The layer
 * runs its output projection and FFN2 split (tel_gemm_partial + tel_layernorm_reduce)
 * exactly when splits > 1. No device work. */
int tel_gemm_partial_plan(int dtype, int M, int N, int K, int* tile_config, int* splits,
                          int* partial_bytes);

/* LayerNorm of a split GEMM's unfinished sum ([KS] Fig. 11 and [SW] section 3: add-bias,
 * residual and LayerNorm fused after the GEMM):
 *   x[r][n] = sum_s partials[s][r][n] (int32 partials: times dq[n]; fp16 partials added in
 *             float32) + bias[n] + resid[r][n]
 *   x rounded to out_dtype first when round_pre != 0 (the int8 layer's stored values)
 *   y[r][:] = LN(x[r][:]) * gamma + beta, written as out_dtype; also as float32 to y32
 *   and as int8 codes clamp(rne(float(y) * *qinv), +-127) to yq when those are non-null.
 * partials [splits][rows][width]: partial_bytes 4: float32 (dq == NULL) or int32 (dq !=
 * NULL); partial_bytes 2: fp16 (dq == NULL and out_dtype TEL_F16, else TEL_EUNSUPPORTED);
 * 1 <= splits <= 8; bias, dq,
 * gamma, beta float32 [width]; resid [rows][width] of resid_dtype. (resid_dtype,
 * out_dtype) in {(F16, F16), (BF16, BF16), (F32, BF16), (F32, F32)}; qinv a device scalar. */
int tel_layernorm_reduce(const void* partials, int splits, int partial_bytes, const float* dq,
                         const float* bias, const void* resid, int resid_dtype, void* y,
                         int out_dtype, float* y32, int8_t* yq, const float* qinv,
                         const float* gamma, const float* beta, int rows, int width, float eps,
                         int round_pre, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TEL_H */
