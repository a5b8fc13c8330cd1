"""Oracle: int8-GEMM variant of the encoder layer (quantise -> int8 GEMM -> int32 -> dequantise).

Test infrastructure only (see oracle/__init__.py). Page keys as listed there.

[SW] section 3, INT8 quantisation paragraph: inputs and weights are quantised to
INT8, the product is accumulated in INT32, and a dequantisation step returns
FP32/FP16 values; in FasterTransformer's int8 flow every GEMM has a quantise
node before it and a dequantise node after it, while bias, residual and
LayerNorm stay in floating point. Readings where the page is silent:
  * symmetric codes in [-127, 127], round-half-to-even, clamp;
  * weights per output channel: s_w[n] = max_k |W[n, k]| / 127 (1 if the row is 0);
  * activations per tensor with a static scale from calibration (PTQ, named on
    the page): a = max-abs of that GEMM's input on a calibration batch,
    s = a / 127, inv = 127 / a, both float32;
  * the GEMM output is INT32 (the INT8-output form is a later variant);
  * QK^T and PV stay in floating point on the dequantised Q, K, V;
  * the layer's activations are fp16: each dequantised GEMM result (with its bias,
    and residual where there is one), the attention output and the LayerNorm output
    is stored as fp16, as the workload defines the int8 GEMMs as dequantised to fp16
    before softmax and LayerNorm (the page keeps bias, residual and LayerNorm in
    FP16/FP32 after the dequantise node).
Where a floating-point value decides a code, the decision is taken in float32
exactly as stated here (from the stored fp16 activation), so that both
implementations make the same decision.
"""
from __future__ import annotations

import math

import numpy as np

from . import encoder as enc

__all__ = ["quantize_weight", "quantize_act", "int8_matmul", "dequantize", "calibrate",
           "calibrate_attention", "act_scale", "attention_int8", "encoder_layer_int8",
           "encoder_stack_int8"]


def _rne_clamp(v32: np.ndarray) -> np.ndarray:
    return np.clip(np.rint(v32), -127, 127).astype(np.int8)


def quantize_weight(w: np.ndarray):
    """Per-output-channel symmetric int8 weights: returns (Wq int8 [N, K], s_w float32 [N]).

    s_w[n] = max_k |W[n,k]| / 127 in float32 (1 when the row is all zero);
    Wq = clamp(rne(W / s_w[n]), -127, 127) with the division in float32.
    """
    w32 = np.asarray(w, dtype=np.float32)
    amax = np.abs(w32).max(axis=1)
    s = np.where(amax > 0, amax / np.float32(127.0), np.float32(1.0)).astype(np.float32)
    q = _rne_clamp((w32 / s[:, None]).astype(np.float32))
    return q, s


def act_scale(amax: float):
    """Per-tensor activation scale from a calibration max-abs: (s, inv) in float32."""
    a = np.float32(amax)
    if not a > 0:
        return np.float32(1.0), np.float32(1.0)
    return np.float32(a / np.float32(127.0)), np.float32(np.float32(127.0) / a)


def quantize_act(x_storage: np.ndarray, inv: np.float32) -> np.ndarray:
    """q = clamp(rne(float32(x) * inv), -127, 127): one float32 multiply, then
    round-half-to-even. ``x_storage`` holds the stored (e.g. fp16) activation."""
    x32 = np.asarray(x_storage, dtype=np.float32)
    return _rne_clamp((x32 * np.float32(inv)).astype(np.float32))


def int8_matmul(q: np.ndarray, wq: np.ndarray) -> np.ndarray:
    """acc[t, n] = sum_k q[t, k] * Wq[n, k], exact in int64."""
    return np.asarray(q, np.int64) @ np.asarray(wq, np.int64).T


def dequantize(acc: np.ndarray, s_a: np.float32, s_w: np.ndarray, bias) -> np.ndarray:
    """y = acc * (s_a * s_w[n]) + b[n]; the scale product is formed in float32,
    the rest in float64."""
    scale = (np.float32(s_a) * np.asarray(s_w, np.float32)).astype(np.float32)
    return np.asarray(acc, np.float64) * scale.astype(np.float64) + np.asarray(bias, np.float64)


def calibrate(x: np.ndarray, cu_seqlens, w: dict, heads: int, eps: float) -> list:
    """Max-abs of the inputs of the four GEMMs (QKV, O, FFN1, FFN2) in a float64 run of
    the floating-point layer on a calibration batch (static PTQ scales)."""
    _, mid = enc.encoder_layer(x, cu_seqlens, w, heads, eps, return_intermediates=True)
    return [float(np.abs(np.asarray(x, np.float64)).max()), float(np.abs(mid["ctx"]).max()),
            float(np.abs(mid["h1"]).max()), float(np.abs(mid["f"]).max())]


def calibrate_attention(x: np.ndarray, cu_seqlens, w: dict, heads: int, eps: float) -> list:
    """Max-abs of the Q, K and V parts of the QKV projection in a float64 run of the
    floating-point layer on a calibration batch (the static scales of int8 attention)."""
    _, mid = enc.encoder_layer(x, cu_seqlens, w, heads, eps, return_intermediates=True)
    H = mid["qkv"].shape[1] // 3
    return [float(np.abs(mid["qkv"][:, i * H:(i + 1) * H]).max()) for i in range(3)]


def attention_int8(qkv_storage: np.ndarray, cu_seqlens, heads: int, attn_amax: list):
    """Multi-head attention with both products on int8 codes ([SW] section 3, INT8
    paragraph: all matrix multiplications in int8). Reading of the steps the page leaves
    open, per sequence b, head h and query i (keys j of sequence b only):
      * Q, K, V codes from the stored (fp16) projection at static per-tensor scales
        s_q, s_k, s_v (calibration max-abs / 127), the quantize_act rule;
      * S[i, j] = sum_c q[i, c] k[j, c], exact integers;
      * t[i, j] = float32(S) * a2 with a2 = float32(float32(s_q * s_k) / sqrt(d)) *
        log2(e), one float32 multiply (scores in base 2);
      * p[i, j] = 2^(t[i, j] - max_j t[i, j]) in float32, in (0, 1];
      * P codes r[i, j] = rne(127 p[i, j]) in [0, 127] (fixed scale 1/127);
      * ctx[i, h d + c] = s_v * (sum_j r[i, j] v[j, c]) / (sum_j r[i, j]): both sums exact
        integers (the largest p gives r = 127, so the denominator is >= 127).
    Decisions that turn floats into codes are taken in float32, as the kernel takes them.
    Returns ctx [T, H] in float64 (not rounded)."""
    qkv = np.asarray(qkv_storage)
    T, H3 = qkv.shape
    H = H3 // 3
    d = H // heads
    f32 = np.float32
    sc = [act_scale(a) for a in attn_amax]
    q = quantize_act(qkv[:, :H], sc[0][1]).astype(np.int64)
    k = quantize_act(qkv[:, H:2 * H], sc[1][1]).astype(np.int64)
    v = quantize_act(qkv[:, 2 * H:], sc[2][1]).astype(np.int64)
    a2 = f32(f32(f32(sc[0][0] * sc[1][0]) / f32(math.sqrt(d))) * f32(1.4426950408889634))
    out = np.zeros((T, H), np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if s1 == s0:
            continue
        for h in range(heads):
            cs = slice(h * d, (h + 1) * d)
            S = q[s0:s1, cs] @ k[s0:s1, cs].T                       # exact
            t = S.astype(f32) * a2
            p = np.exp2((t - t.max(axis=1, keepdims=True)).astype(f32)).astype(f32)
            r = np.clip(np.rint((p * f32(127.0)).astype(f32)), 0, 127).astype(np.int64)
            num = r @ v[s0:s1, cs]                                  # exact
            out[s0:s1, cs] = float(sc[2][0]) * num / r.sum(axis=1, keepdims=True)
    return out


def encoder_layer_int8(x: np.ndarray, cu_seqlens, w: dict, heads: int, eps: float,
                       amax: list, storage=np.float16, attn_amax=None, dynamic=False,
                       dyn_amax=None, dyn_trace=None):
    """Post-LN encoder layer with the four projection GEMMs in int8.

    ``w`` holds the floating-point weights; they are quantised here per
    quantize_weight. ``amax`` are the four calibration max-abs values.
    ``storage`` is the type every activation is stored in (fp16): the dequantised
    QKV, the attention output, the two pre-LayerNorm sums, h1 and the GELU output.
    With ``attn_amax`` (the Q, K, V max-abs of calibrate_attention) attention runs on
    int8 codes too (attention_int8); the QKV projection's fp16 value is then only the
    value its codes are taken from.
    With ``dynamic`` the activation scales are not static ([P5] section 3.3, dynamic
    quantisation: the quantisation parameters follow the data at inference time): each
    GEMM's scale comes from the max-abs of that GEMM's stored input over the batch being
    run (amax is then unused). ``dyn_amax`` optionally gives those four maxima instead of
    computing them (a caller that must take the same scale decision as another
    implementation feeds that implementation's maxima); ``dyn_trace`` (a list) receives the
    maxima this run found, in GEMM order. The returned output is not rounded.
    """
    scales = None if dynamic else [act_scale(a) for a in amax]

    def st(a):
        return np.asarray(a, np.float64).astype(storage).astype(np.float64)

    def qlinear(a, wname, bname, g):
        wq, sw = quantize_weight(w[wname])
        a_st = np.asarray(a, np.float64).astype(storage)
        if dynamic:
            a_run = float(np.abs(a_st.astype(np.float64)).max())
            s, inv = act_scale(dyn_amax[g] if dyn_amax is not None else a_run)
        else:
            s, inv = scales[g]
        if dynamic and dyn_trace is not None:
            dyn_trace.append(a_run)
        q = quantize_act(a_st, inv)
        return dequantize(int8_matmul(q, wq), s, sw, w[bname])

    x = np.asarray(x, np.float64)
    qkv = st(qlinear(x, "w_qkv", "b_qkv", 0))
    if attn_amax is not None:
        ctx = st(attention_int8(qkv.astype(storage), cu_seqlens, heads, attn_amax))
    else:
        ctx = st(enc.attention(qkv, cu_seqlens, heads))
    h1 = st(enc.layer_norm(st(qlinear(ctx, "w_o", "b_o", 1) + x), w["ln1_g"], w["ln1_b"], eps))
    f = st(enc.gelu(qlinear(h1, "w_1", "b_1", 2)))
    return enc.layer_norm(st(qlinear(f, "w_2", "b_2", 3) + h1), w["ln2_g"], w["ln2_b"], eps)


def encoder_stack_int8(x, cu_seqlens, layers: list, amaxes: list, heads: int, eps: float,
                       storage=np.float16, attn_amaxes=None, dynamic=False):
    """Layers in order, each with its own calibration max-abs list (and, for int8
    attention, its own Q/K/V max-abs list); the output of every layer is rounded to
    ``storage`` as the stored activation."""
    y = np.asarray(x, np.float64)
    if amaxes is None:
        amaxes = [None] * len(layers)
    for i, (w, a) in enumerate(zip(layers, amaxes)):
        aa = attn_amaxes[i] if attn_amaxes is not None else None
        y = encoder_layer_int8(y, cu_seqlens, w, heads, eps, a, storage, attn_amax=aa,
                               dynamic=dynamic)
        y = y.astype(storage).astype(np.float64)
    return y
