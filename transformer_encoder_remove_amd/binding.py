"""ctypes binding of libtel.so: one Python function per C entry point, same names.

Argument marshalling only: torch tensors become device pointers, torch's current HIP
stream becomes the `stream` argument, and a non-zero status raises TelError. Every
step of the computation runs in the library's HIP kernels; nothing here computes.
The library must have been built (``python transformer_encoder_remove_amd/build.py``);
importing this module fails loudly when it is missing.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtel.so")

TEL_OK, TEL_EINVAL, TEL_EUNSUPPORTED, TEL_EWORKSPACE, TEL_EDEVICE = range(5)
TEL_F32, TEL_F16, TEL_BF16, TEL_I8 = range(4)
TEL_EPI_BIAS, TEL_EPI_BIAS_GELU, TEL_EPI_BIAS_RESID, TEL_EPI_QKV_SPLIT = range(4)

DTYPE_CODE = {torch.float32: TEL_F32, torch.float16: TEL_F16, torch.bfloat16: TEL_BF16,
              torch.int8: TEL_I8}
CODE_DTYPE = {v: k for k, v in DTYPE_CODE.items()}

# Every symbol include/tel.h declares (checked by the CPU tests).
EXPORTS = (
    "tel_status_str", "tel_version", "tel_build_offsets", "tel_remove_padding",
    "tel_rebuild_padding", "tel_encoder_packed_size", "tel_encoder_prepare",
    "tel_encoder_workspace_size", "tel_encoder_layer_forward", "tel_encoder_calibrate",
    "tel_encoder_forward_workspace_size", "tel_encoder_forward", "tel_gemm",
    "tel_gemm_tile_configs", "tel_gemm_ex", "tel_attention_varlen", "tel_quantize_i8",
    "tel_quantize_weight_i8", "tel_gemm_i8_i32", "tel_layernorm", "tel_swin_packed_size",
    "tel_swin_prepare", "tel_swin_workspace_size", "tel_swin_fused_stages",
    "tel_window_attention_forward",
    "tel_window_partition_layernorm", "tel_gemm_partial", "tel_gemm_partial_plan",
    "tel_layernorm_reduce", "tel_graph_cache", "tel_weight_prefetch", "tel_gemm_i8",
    "tel_prune_2of4",
    "tel_gemm_2of4_tile_configs", "tel_gemm_2of4", "tel_build_offsets_mask",
    "tel_rebuild_padding_mask", "tel_encoder_layer_forward_noalloc", "tel_patch_merging",
    "tel_attention_int8",
)
TEL_NOALLOC_SCRATCH_BYTES = 64 << 20
TEL_SWIN_ATTN_ONLY = 1


def TEL_SWIN_ONE_STAGE(k: int) -> int:
    """tel_window_attention_forward flag: stage k (0..4) of the block alone."""
    return (k + 1) << 8


class TelError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python transformer_encoder_remove_amd/build.py`")
lib = ctypes.CDLL(LIB_PATH)

P = ctypes.c_void_p
I = ctypes.c_int
SZ = ctypes.c_size_t
F = ctypes.c_float


class tel_encoder_desc(ctypes.Structure):
    _fields_ = [("hidden", I), ("heads", I), ("ffn", I), ("dtype", I), ("int8_gemm", I),
                ("ln_eps", F), ("sparse_2of4", I), ("dynamic_scales", I)]


class tel_swin_desc(ctypes.Structure):
    _fields_ = [(n, I) for n in ("batch", "height", "width", "channels", "heads", "window",
                                 "shift", "mlp_hidden", "dtype")] + [("ln_eps", F)]


_SWIN_WNAMES = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "rpb_table", "w_proj", "b_proj", "ln2_g",
                "ln2_b", "w_1", "b_1", "w_2", "b_2")


class tel_swin_weights(ctypes.Structure):
    _fields_ = [(n, P) for n in _SWIN_WNAMES]


class tel_encoder_weights(ctypes.Structure):
    _fields_ = [(n, P) for n in ("w_qkv", "b_qkv", "w_o", "b_o", "ln1_g", "ln1_b",
                                 "w_1", "b_1", "w_2", "b_2", "ln2_g", "ln2_b")] + \
               [("act_amax", F * 4), ("attn_amax", F * 3)]


_SIG = {
    "tel_status_str": (ctypes.c_char_p, [I]),
    "tel_version": (ctypes.c_char_p, []),
    "tel_build_offsets": (I, [P, I, I, P, P, P]),
    "tel_remove_padding": (I, [P, P, P, I, I, I, P]),
    "tel_rebuild_padding": (I, [P, P, P, I, I, I, I, P]),
    "tel_encoder_packed_size": (SZ, [ctypes.POINTER(tel_encoder_desc)]),
    "tel_encoder_prepare": (I, [ctypes.POINTER(tel_encoder_desc),
                                ctypes.POINTER(tel_encoder_weights), P, SZ, P]),
    "tel_encoder_workspace_size": (SZ, [ctypes.POINTER(tel_encoder_desc), I]),
    "tel_encoder_layer_forward": (I, [ctypes.POINTER(tel_encoder_desc), P, P, P, P, I, I, I, P,
                                      SZ, P]),
    "tel_encoder_layer_forward_noalloc": (I, [ctypes.POINTER(tel_encoder_desc), P, P, P, P, I,
                                              I, I, P]),
    "tel_encoder_calibrate": (I, [ctypes.POINTER(tel_encoder_desc), P, P, P, P, I, I, I, P, P, SZ,
                                  P]),
    "tel_encoder_forward_workspace_size": (SZ, [ctypes.POINTER(tel_encoder_desc), I, I]),
    "tel_encoder_forward": (I, [ctypes.POINTER(tel_encoder_desc), ctypes.POINTER(P), I, P, P, P,
                                I, I, I, I, P, SZ, P]),
    "tel_gemm": (I, [I, I, P, P, P, P, P, I, I, I, I, P]),
    "tel_gemm_tile_configs": (I, []),
    "tel_gemm_ex": (I, [I, I, I, P, P, P, P, P, I, I, I, I, P]),
    "tel_attention_varlen": (I, [P, P, P, I, I, I, I, I, I, P]),
    "tel_layernorm": (I, [P, P, P, P, I, I, F, I, P]),
    "tel_patch_merging": (I, [P, P, P, P, P, I, I, I, I, F, I, P]),
    "tel_attention_int8": (I, [P, P, I, P, P, I, I, I, I, I, P]),
    "tel_quantize_i8": (I, [P, P, SZ, F, I, P]),
    "tel_quantize_weight_i8": (I, [P, P, P, I, I, I, P]),
    "tel_gemm_i8_i32": (I, [P, P, P, I, I, I, P]),
    "tel_swin_packed_size": (SZ, [ctypes.POINTER(tel_swin_desc)]),
    "tel_swin_prepare": (I, [ctypes.POINTER(tel_swin_desc), ctypes.POINTER(tel_swin_weights), P,
                             SZ, P]),
    "tel_swin_workspace_size": (SZ, [ctypes.POINTER(tel_swin_desc)]),
    "tel_swin_fused_stages": (I, [ctypes.POINTER(tel_swin_desc)]),
    "tel_window_attention_forward": (I, [ctypes.POINTER(tel_swin_desc), P, P, P, I, P, SZ, P]),
    "tel_window_partition_layernorm": (I, [P, P, P, P, I, I, I, I, I, I, F, I, P]),
    "tel_gemm_partial": (I, [I, I, I, P, P, P, I, I, I, I, P]),
    "tel_gemm_partial_plan": (I, [I, I, I, I, ctypes.POINTER(I), ctypes.POINTER(I),
                                  ctypes.POINTER(I)]),
    "tel_layernorm_reduce": (I, [P, I, I, P, P, P, I, P, I, P, P, P, P, P, I, I, F, I, P]),
    "tel_graph_cache": (I, [I]),
    "tel_weight_prefetch": (I, [I]),
    "tel_gemm_i8": (I, [I, P, P, P, P, P, P, P, I, I, I, I, I, P]),
    "tel_prune_2of4": (I, [P, P, P, I, I, I, P]),
    "tel_gemm_2of4_tile_configs": (I, []),
    "tel_gemm_2of4": (I, [I, I, I, P, P, P, P, P, P, I, I, I, I, P]),
    "tel_build_offsets_mask": (I, [P, I, I, P, P, P]),
    "tel_rebuild_padding_mask": (I, [P, P, P, P, I, I, I, I, I, P]),
}
for _name, (_res, _args) in _SIG.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


# ------------------------------------------------------------------ marshalling helpers
def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.numel() and not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr() if t.numel() else None


def _stream(stream) -> int | None:
    if stream is None:
        if not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, status: int):
    if status != TEL_OK:
        raise TelError(fn, status, lib.tel_status_str(status).decode())


def dtype_code(t: torch.dtype) -> int:
    return DTYPE_CODE[t]


def _i32(name: str, *ts):
    """Lengths, offsets and cu_seqlens are int32 on the C side: refuse other integer types
    rather than let the library read them as int32."""
    for t in ts:
        if t is not None and t.dtype != torch.int32:
            raise TypeError(f"{name}: expected an int32 tensor, got {t.dtype}")


def _act(name: str, desc, *ts):
    """Activations of an encoder call have the descriptor's storage type."""
    for t in ts:
        if t is not None and DTYPE_CODE.get(t.dtype) != desc.dtype:
            raise TypeError(f"{name}: tensor of {t.dtype} does not match the descriptor's "
                            f"storage type {CODE_DTYPE.get(desc.dtype)}")


# ------------------------------------------------------------------ entry points
def tel_version() -> str:
    return lib.tel_version().decode()


def tel_status_str(status: int) -> str:
    return lib.tel_status_str(status).decode()


def tel_build_offsets(seq_lens, max_seq: int, cu_seqlens, padding_offset, stream=None):
    _i32("tel_build_offsets", seq_lens, cu_seqlens, padding_offset)
    _check("tel_build_offsets", lib.tel_build_offsets(
        _ptr(seq_lens), seq_lens.numel(), max_seq, _ptr(cu_seqlens), _ptr(padding_offset),
        _stream(stream)))


def tel_remove_padding(x_pad, x_packed, padding_offset, total_tokens: int, stream=None):
    width = x_pad.shape[-1]
    _i32("tel_remove_padding", padding_offset)
    _check("tel_remove_padding", lib.tel_remove_padding(
        _ptr(x_pad), _ptr(x_packed), _ptr(padding_offset), total_tokens, width,
        dtype_code(x_pad.dtype), _stream(stream)))


def tel_rebuild_padding(x_packed, x_pad, cu_seqlens, stream=None):
    B, S, W = x_pad.shape
    _i32("tel_rebuild_padding", cu_seqlens)
    _check("tel_rebuild_padding", lib.tel_rebuild_padding(
        _ptr(x_packed), _ptr(x_pad), _ptr(cu_seqlens), B, S, W, dtype_code(x_pad.dtype),
        _stream(stream)))


def tel_build_offsets_mask(mask, cu_seqlens, padding_offset, stream=None):
    """mask [B, S] uint8/bool device tensor; cu_seqlens [B+1], padding_offset [>= B*S] int32."""
    B, S = mask.shape
    _i32("tel_build_offsets_mask", cu_seqlens, padding_offset)
    _check("tel_build_offsets_mask", lib.tel_build_offsets_mask(
        _ptr(mask), B, S, _ptr(cu_seqlens), _ptr(padding_offset), _stream(stream)))


def tel_rebuild_padding_mask(x_packed, x_pad, mask, padding_offset, total_tokens: int,
                             stream=None):
    B, S, W = x_pad.shape
    _i32("tel_rebuild_padding_mask", padding_offset)
    _check("tel_rebuild_padding_mask", lib.tel_rebuild_padding_mask(
        _ptr(x_packed), _ptr(x_pad), _ptr(mask), _ptr(padding_offset), total_tokens, B, S, W,
        dtype_code(x_pad.dtype), _stream(stream)))


def make_encoder_desc(hidden, heads, ffn, dtype: torch.dtype, eps=1e-5, int8_gemm=False,
                      sparse_2of4=False, dynamic_scales=False):
    """int8_gemm: False/0, True/1 (int8 GEMMs) or 2 (int8 GEMMs and int8 attention);
    dynamic_scales: int8 activation scales from each batch's own max-abs (int8_gemm 1)."""
    return tel_encoder_desc(hidden, heads, ffn, dtype_code(dtype), int(int8_gemm), eps,
                            int(sparse_2of4), int(dynamic_scales))


def tel_encoder_packed_size(desc) -> int:
    return lib.tel_encoder_packed_size(ctypes.byref(desc))


def tel_encoder_workspace_size(desc, max_tokens: int) -> int:
    return lib.tel_encoder_workspace_size(ctypes.byref(desc), max_tokens)


def tel_encoder_forward_workspace_size(desc, batch: int, max_seq: int) -> int:
    return lib.tel_encoder_forward_workspace_size(ctypes.byref(desc), batch, max_seq)


_WNAMES = ("w_qkv", "b_qkv", "w_o", "b_o", "ln1_g", "ln1_b", "w_1", "b_1", "w_2", "b_2",
           "ln2_g", "ln2_b")


def tel_encoder_prepare(desc, weights: dict, packed, act_amax=(0.0, 0.0, 0.0, 0.0),
                        attn_amax=(0.0, 0.0, 0.0), stream=None):
    """weights: dict of device tensors (storage type) named as in tel_encoder_weights."""
    w = tel_encoder_weights(*[_ptr(weights[n]) for n in _WNAMES], (F * 4)(*act_amax),
                            (F * 3)(*attn_amax))
    _check("tel_encoder_prepare", lib.tel_encoder_prepare(
        ctypes.byref(desc), ctypes.byref(w), _ptr(packed), packed.numel() * packed.element_size(),
        _stream(stream)))


def tel_encoder_layer_forward(desc, packed, x, y, cu_seqlens, total_tokens: int, max_len: int,
                              workspace, stream=None):
    _i32("tel_encoder_layer_forward", cu_seqlens)
    _act("tel_encoder_layer_forward", desc, x, y)
    _check("tel_encoder_layer_forward", lib.tel_encoder_layer_forward(
        ctypes.byref(desc), _ptr(packed), _ptr(x), _ptr(y), _ptr(cu_seqlens),
        cu_seqlens.numel() - 1, total_tokens, max_len, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def tel_encoder_layer_forward_noalloc(desc, packed, x, y, cu_seqlens, total_tokens: int,
                                      max_len: int, stream=None):
    _i32("tel_encoder_layer_forward_noalloc", cu_seqlens)
    _act("tel_encoder_layer_forward_noalloc", desc, x, y)
    _check("tel_encoder_layer_forward_noalloc", lib.tel_encoder_layer_forward_noalloc(
        ctypes.byref(desc), _ptr(packed), _ptr(x), _ptr(y), _ptr(cu_seqlens),
        cu_seqlens.numel() - 1, total_tokens, max_len, _stream(stream)))


def tel_encoder_calibrate(desc, packed, x, y, cu_seqlens, total_tokens: int, max_len: int, amax,
                          workspace, stream=None):
    _i32("tel_encoder_calibrate", cu_seqlens)
    _act("tel_encoder_calibrate", desc, x, y)
    _check("tel_encoder_calibrate", lib.tel_encoder_calibrate(
        ctypes.byref(desc), _ptr(packed), _ptr(x), _ptr(y), _ptr(cu_seqlens),
        cu_seqlens.numel() - 1, total_tokens, max_len, _ptr(amax), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def tel_encoder_forward(desc, packed_layers: list, x_pad, y_pad, seq_lens, total_tokens: int,
                        max_len: int, workspace, stream=None):
    B, S, _ = x_pad.shape
    arr = (P * max(1, len(packed_layers)))(*[_ptr(p) for p in packed_layers])
    _i32("tel_encoder_forward", seq_lens)
    _act("tel_encoder_forward", desc, x_pad, y_pad)
    _check("tel_encoder_forward", lib.tel_encoder_forward(
        ctypes.byref(desc), arr, len(packed_layers), _ptr(x_pad), _ptr(y_pad), _ptr(seq_lens),
        B, S, total_tokens, max_len, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def tel_gemm(epilogue: int, A, W, bias, C, resid=None, heads: int = 1, stream=None):
    M, K = A.shape
    N = W.shape[0]
    _check("tel_gemm", lib.tel_gemm(
        epilogue, dtype_code(A.dtype), _ptr(A), _ptr(W), _ptr(bias), _ptr(resid), _ptr(C),
        M, N, K, heads, _stream(stream)))


def tel_prune_2of4(w, values, index, stream=None):
    """values [N][K/2] (w's dtype), index [N][K/16] (int16 tensor holding the 16-bit words)."""
    N, K = w.shape
    _check("tel_prune_2of4", lib.tel_prune_2of4(
        _ptr(w), _ptr(values), _ptr(index), N, K, dtype_code(w.dtype), _stream(stream)))


def tel_gemm_2of4_tile_configs() -> int:
    return lib.tel_gemm_2of4_tile_configs()


def tel_gemm_2of4(epilogue: int, A, values, index, bias, C, resid=None, heads: int = 1,
                  tile_config: int = -2, stream=None):
    M, K = A.shape
    N = values.shape[0]
    _check("tel_gemm_2of4", lib.tel_gemm_2of4(
        epilogue, dtype_code(A.dtype), tile_config, _ptr(A), _ptr(values), _ptr(index),
        _ptr(bias), _ptr(resid), _ptr(C), M, N, K, heads, _stream(stream)))


def tel_gemm_tile_configs() -> int:
    return lib.tel_gemm_tile_configs()


def tel_gemm_ex(epilogue: int, tile_config: int, A, W, bias, C, resid=None, heads: int = 1,
                stream=None):
    M, K = A.shape
    N = W.shape[0]
    _check("tel_gemm_ex", lib.tel_gemm_ex(
        epilogue, dtype_code(A.dtype), tile_config, _ptr(A), _ptr(W), _ptr(bias), _ptr(resid),
        _ptr(C), M, N, K, heads, _stream(stream)))


def tel_attention_varlen(qkv_split, ctx, cu_seqlens, total_tokens: int, max_len: int,
                         heads: int, head_dim: int, stream=None):
    _i32("tel_attention_varlen", cu_seqlens)
    _check("tel_attention_varlen", lib.tel_attention_varlen(
        _ptr(qkv_split), _ptr(ctx), _ptr(cu_seqlens), cu_seqlens.numel() - 1, total_tokens,
        max_len, heads, head_dim, dtype_code(ctx.dtype), _stream(stream)))


def tel_attention_int8(qkv_codes, out, scales, cu_seqlens, total_tokens: int, max_len: int,
                       heads: int, head_dim: int, stream=None):
    """qkv_codes int8 [3*heads*T*head_dim]; out fp16 [T, heads*head_dim] (the context) or
    int8 (its codes at scales[2]); scales float32 device [3]."""
    _i32("tel_attention_int8", cu_seqlens)
    _check("tel_attention_int8", lib.tel_attention_int8(
        _ptr(qkv_codes), _ptr(out), int(out.dtype == torch.int8), _ptr(scales), _ptr(cu_seqlens),
        cu_seqlens.numel() - 1, total_tokens, max_len, heads, head_dim, _stream(stream)))


def tel_patch_merging(x, y, gamma, beta, w_red, height: int, width: int, eps: float,
                      stream=None):
    """x [B, height*width, C] -> y [B, (height/2)*(width/2), 2C]; gamma, beta float32 [4C];
    w_red [2C, 4C] of x's type."""
    B, L, C = x.shape
    _check("tel_patch_merging", lib.tel_patch_merging(
        _ptr(x), _ptr(y), _ptr(gamma), _ptr(beta), _ptr(w_red), B, height, width, C, eps,
        dtype_code(x.dtype), _stream(stream)))


def tel_layernorm(x, y, gamma, beta, eps: float, stream=None):
    rows, width = x.shape
    _check("tel_layernorm", lib.tel_layernorm(
        _ptr(x), _ptr(y), _ptr(gamma), _ptr(beta), rows, width, eps, dtype_code(x.dtype),
        _stream(stream)))


def tel_quantize_i8(x, q, inv_scale: float, stream=None):
    _check("tel_quantize_i8", lib.tel_quantize_i8(
        _ptr(x), _ptr(q), x.numel(), inv_scale, dtype_code(x.dtype), _stream(stream)))


def tel_quantize_weight_i8(w, q, scales, stream=None):
    N, K = w.shape
    _check("tel_quantize_weight_i8", lib.tel_quantize_weight_i8(
        _ptr(w), _ptr(q), _ptr(scales), N, K, dtype_code(w.dtype), _stream(stream)))


def tel_graph_cache(enable: int = -1) -> int:
    """Turn tel_encoder_forward's graph cache on (1) or off (0); -1 queries. Returns the
    previous setting."""
    return lib.tel_graph_cache(enable)


def tel_weight_prefetch(enable: int = -1) -> int:
    """Turn tel_encoder_forward's weight read-ahead on (1) or off (0); -1 queries. Returns
    the previous setting."""
    return lib.tel_weight_prefetch(enable)


def tel_gemm_partial_plan(dtype: int, M: int, N: int, K: int) -> tuple[int, int, int]:
    """(tile_config, splits, partial_bytes) the encoder layer uses for a partial GEMM of
    this shape; partial_bytes 4 = float32 (int32 for int8), 2 = fp16."""
    cfg, sp, pb = I(), I(), I()
    _check("tel_gemm_partial_plan", lib.tel_gemm_partial_plan(
        dtype, M, N, K, ctypes.byref(cfg), ctypes.byref(sp), ctypes.byref(pb)))
    return cfg.value, sp.value, pb.value


def tel_gemm_partial(tile_config: int, splits: int, A, W, partials, stream=None):
    """partials float32 / int32 (4-byte partial sums) or float16 (fp16 partial sums)."""
    M, K = A.shape
    N = W.shape[0]
    _check("tel_gemm_partial", lib.tel_gemm_partial(
        dtype_code(A.dtype), tile_config, splits, _ptr(A), _ptr(W), _ptr(partials),
        partials.element_size(), M, N, K, _stream(stream)))


def tel_layernorm_reduce(partials, splits: int, bias, resid, y, gamma, beta, eps: float,
                         dq=None, y32=None, yq=None, qinv=None, round_pre: bool = False,
                         stream=None):
    rows, width = y.shape
    _check("tel_layernorm_reduce", lib.tel_layernorm_reduce(
        _ptr(partials), splits, partials.element_size(), _ptr(dq), _ptr(bias), _ptr(resid),
        dtype_code(resid.dtype),
        _ptr(y), dtype_code(y.dtype), _ptr(y32), _ptr(yq), _ptr(qinv), _ptr(gamma), _ptr(beta),
        rows, width, eps, int(round_pre), _stream(stream)))


def tel_gemm_i8(epilogue: int, A, W, dq, bias, C, resid=None, qinv=None, out_int8=False,
                heads: int = 1, stream=None):
    """One int8-layer GEMM with its epilogue (A, W int8 codes; C fp16, or int8 codes)."""
    M, K = A.shape
    N = W.shape[0]
    _check("tel_gemm_i8", lib.tel_gemm_i8(
        epilogue, _ptr(A), _ptr(W), _ptr(dq), _ptr(bias), _ptr(resid), _ptr(C), _ptr(qinv),
        int(out_int8), M, N, K, heads, _stream(stream)))


def tel_gemm_i8_i32(A, B, C, stream=None):
    M, K = A.shape
    N = B.shape[0]
    _check("tel_gemm_i8_i32", lib.tel_gemm_i8_i32(_ptr(A), _ptr(B), _ptr(C), M, N, K,
                                                  _stream(stream)))


def make_swin_desc(batch, height, width, channels, heads, window, shift, mlp_hidden,
                   dtype: torch.dtype, eps=1e-5):
    return tel_swin_desc(batch, height, width, channels, heads, window, shift, mlp_hidden,
                         dtype_code(dtype), eps)


def tel_swin_packed_size(desc) -> int:
    return lib.tel_swin_packed_size(ctypes.byref(desc))


def tel_swin_workspace_size(desc) -> int:
    return lib.tel_swin_workspace_size(ctypes.byref(desc))


TEL_SWIN_FUSED_ATTN, TEL_SWIN_FUSED_MLP = 1, 2


def tel_swin_fused_stages(desc) -> int:
    """Bit mask: TEL_SWIN_FUSED_ATTN (stage 0 is the whole attention half, stages 1-2 empty),
    TEL_SWIN_FUSED_MLP (stage 3 is the whole MLP half, stage 4 empty)."""
    return lib.tel_swin_fused_stages(ctypes.byref(desc))


def tel_swin_prepare(desc, weights: dict, packed, stream=None):
    w = tel_swin_weights(*[_ptr(weights[n]) for n in _SWIN_WNAMES])
    _check("tel_swin_prepare", lib.tel_swin_prepare(
        ctypes.byref(desc), ctypes.byref(w), _ptr(packed), packed.numel() * packed.element_size(),
        _stream(stream)))


def tel_window_attention_forward(desc, packed, x, y, workspace, flags: int = 0, stream=None):
    _check("tel_window_attention_forward", lib.tel_window_attention_forward(
        ctypes.byref(desc), _ptr(packed), _ptr(x), _ptr(y), flags, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def tel_window_partition_layernorm(x, y, gamma, beta, batch, height, width, window, shift,
                                   eps: float, stream=None):
    C = x.shape[-1]
    _check("tel_window_partition_layernorm", lib.tel_window_partition_layernorm(
        _ptr(x), _ptr(y), _ptr(gamma), _ptr(beta), batch, height, width, C, window, shift, eps,
        dtype_code(x.dtype), _stream(stream)))


# ------------------------------------------------------------------ allocation helpers
def alloc_bytes(nbytes: int, device="cuda") -> torch.Tensor:
    """A caller-owned device buffer of at least nbytes (torch's allocator aligns to 512 B)."""
    return torch.empty(max(1, nbytes), dtype=torch.uint8, device=device)
