"""Oracle: post-LN Transformer encoder layer over padding-removed sequences (float64).

Test infrastructure only (see oracle/__init__.py). Page keys as listed there.

Padding removal is exact: the layer applied to the packed valid tokens equals the
same layer applied to the padded batch with padded keys excluded, on the valid
rows ([KS] Figs. 9-10). So each function below is the plain definition of its
step, in float64, with library matmuls.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

__all__ = [
    "offsets", "remove_padding", "rebuild_padding", "offsets_from_mask", "remove_padding_mask",
    "rebuild_padding_mask", "linear", "softmax", "attention",
    "layer_norm", "gelu", "encoder_layer", "encoder_stack", "encoder_forward",
]


def offsets(lens, max_seq: int):
    """Offset mask of padding removal ([KS] Fig. 9).

    Reading of the lost figure: an exclusive prefix sum of the valid lengths gives
    ``cu_seqlens`` (cu[0] = 0, cu[b+1] = cu[b] + lens[b]); for packed token t of
    sequence b, ``padding_offset[t] = b * max_seq - cu[b]`` so that the token's row
    in the padded [B*S] layout is ``t + padding_offset[t]``.
    Returns (cu_seqlens[B+1], padding_offset[T]) as int64.
    """
    lens = np.asarray(lens, dtype=np.int64)
    if lens.ndim != 1 or (lens < 0).any() or (lens > max_seq).any():
        raise ValueError("lengths must be a 1-D array with 0 <= len <= max_seq")
    B = lens.shape[0]
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    po = np.empty(int(cu[-1]), dtype=np.int64)
    for b in range(B):
        po[cu[b]:cu[b + 1]] = b * max_seq - cu[b]
    return cu, po


def remove_padding(x_pad: np.ndarray, lens) -> np.ndarray:
    """Packed rows: the valid prefix of every sequence, concatenated in batch order
    ([KS] Fig. 9). x_pad is [B, S, W]; the result is [T, W] with T = sum(lens)."""
    lens = np.asarray(lens, dtype=np.int64)
    parts = [x_pad[b, :lens[b]] for b in range(x_pad.shape[0])]
    if not parts:
        return np.zeros((0, x_pad.shape[-1]), dtype=x_pad.dtype)
    return np.concatenate(parts, axis=0)


def rebuild_padding(x_packed: np.ndarray, lens, max_seq: int) -> np.ndarray:
    """Inverse of remove_padding ([KS] Fig. 9): scatter packed rows back to
    [B, S, W]; every padded row is zero (a reading: the pages do not say)."""
    lens = np.asarray(lens, dtype=np.int64)
    B = lens.shape[0]
    out = np.zeros((B, max_seq, x_packed.shape[-1]), dtype=x_packed.dtype)
    t = 0
    for b in range(B):
        out[b, :lens[b]] = x_packed[t:t + lens[b]]
        t += lens[b]
    return out


def offsets_from_mask(mask):
    """Offset mask of padding removal in its general form ([KS] Fig. 9: tokens are removed
    where the mask says so, wherever they sit): mask [B, S], nonzero = valid, holes
    allowed. Packed order is sequence by sequence, positions increasing. cu[b+1] = cu[b] +
    (valid positions of b); the packed token t that sits at position s of sequence b has
    padding_offset[t] = b * S + s - t, so its padded row is t + padding_offset[t] as in
    offsets() (to which this reduces for right-padded masks).
    Returns (cu_seqlens[B+1], padding_offset[T]) as int64."""
    m = np.asarray(mask) != 0
    if m.ndim != 2:
        raise ValueError("mask must be [B, S]")
    B, S = m.shape
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(m.sum(axis=1))
    rows = np.flatnonzero(m.reshape(-1)).astype(np.int64)   # b * S + s, b-major, s increasing
    return cu, rows - np.arange(rows.shape[0], dtype=np.int64)


def remove_padding_mask(x_pad: np.ndarray, mask) -> np.ndarray:
    """Packed rows of a [B, S, W] batch: its valid positions in packed order."""
    m = np.asarray(mask) != 0
    B, S, W = x_pad.shape
    return x_pad.reshape(B * S, W)[np.flatnonzero(m.reshape(-1))]


def rebuild_padding_mask(x_packed: np.ndarray, mask) -> np.ndarray:
    """Inverse of remove_padding_mask: packed rows back to their positions, every position
    the mask marks invalid zero."""
    m = np.asarray(mask) != 0
    B, S = m.shape
    out = np.zeros((B * S, x_packed.shape[-1]), dtype=x_packed.dtype)
    out[np.flatnonzero(m.reshape(-1))] = x_packed
    return out.reshape(B, S, -1)


def linear(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """y = x W^T + b with W in [out, in] layout, float64."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T + np.asarray(b, np.float64)


def softmax(s: np.ndarray) -> np.ndarray:
    """Row softmax over the last axis, max-subtracted, float64."""
    s = np.asarray(s, np.float64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention(qkv: np.ndarray, cu_seqlens, heads: int) -> np.ndarray:
    """Multi-head scaled-dot-product self-attention over packed sequences.

    [SW] section 1 defines the head: query and key give the attention map through
    softmax, which weights the values; several heads side by side form multi-head
    attention. Scale 1/sqrt(head_dim) (a reading: the pages give none). qkv is
    [T, 3H] with columns [Q | K | V], head h owning columns h*d..h*d+d-1 of each;
    queries of sequence b attend to the keys of sequence b only ([KS] Fig. 10).
    Returns ctx[T, H] with head h in columns h*d..h*d+d-1.
    """
    qkv = np.asarray(qkv, np.float64)
    T, threeH = qkv.shape
    H = threeH // 3
    d = H // heads
    ctx = np.zeros((T, H), dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for b in range(len(cu) - 1):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        if r1 == r0:
            continue
        for h in range(heads):
            q = qkv[r0:r1, h * d:(h + 1) * d]
            k = qkv[r0:r1, H + h * d:H + (h + 1) * d]
            v = qkv[r0:r1, 2 * H + h * d:2 * H + (h + 1) * d]
            p = softmax(q @ k.T / math.sqrt(d))
            ctx[r0:r1, h * d:(h + 1) * d] = p @ v
    return ctx


def layer_norm(x: np.ndarray, gamma, beta, eps: float) -> np.ndarray:
    """LayerNorm over the last axis: mean, then the biased variance of the centred
    values (two passes), (x - mean) / sqrt(var + eps) * gamma + beta."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    xc = x - mu
    var = (xc * xc).mean(axis=-1, keepdims=True)
    return xc / np.sqrt(var + eps) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def gelu(x: np.ndarray) -> np.ndarray:
    """GELU in its exact form, x * Phi(x) = x/2 * (1 + erf(x / sqrt(2)))."""
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def encoder_layer(x: np.ndarray, cu_seqlens, w: dict, heads: int, eps: float,
                  return_intermediates: bool = False):
    """One post-LN BERT encoder layer on packed tokens x[T, H].

    Steps ([SW] section 1 for attention, [KS] Fig. 6 for the fused blocks):
      qkv = x W_qkv^T + b_qkv
      ctx = multi-head attention over each sequence's own tokens
      h1  = LN(ctx W_o^T + b_o + x; ln1)
      f   = GELU(h1 W_1^T + b_1)
      y   = LN(f W_2^T + b_2 + h1; ln2)
    """
    x = np.asarray(x, np.float64)
    qkv = linear(x, w["w_qkv"], w["b_qkv"])
    ctx = attention(qkv, cu_seqlens, heads)
    h1 = layer_norm(linear(ctx, w["w_o"], w["b_o"]) + x, w["ln1_g"], w["ln1_b"], eps)
    f = gelu(linear(h1, w["w_1"], w["b_1"]))
    y = layer_norm(linear(f, w["w_2"], w["b_2"]) + h1, w["ln2_g"], w["ln2_b"], eps)
    if return_intermediates:
        return y, dict(qkv=qkv, ctx=ctx, h1=h1, f=f)
    return y


def encoder_stack(x: np.ndarray, cu_seqlens, layers: list, heads: int, eps: float,
                  round_to=None) -> np.ndarray:
    """Apply the layers in order to packed tokens. ``round_to`` (a NumPy dtype or a
    callable) optionally rounds each layer's output to the storage type, as a
    stack that stores activations between layers does."""
    y = np.asarray(x, np.float64)
    for w in layers:
        y = encoder_layer(y, cu_seqlens, w, heads, eps)
        if round_to is not None:
            y = (round_to(y) if callable(round_to) else y.astype(round_to)).astype(np.float64)
    return y


def encoder_forward(x_pad: np.ndarray, lens, layers: list, heads: int, eps: float,
                    round_to=None) -> np.ndarray:
    """Whole path on a padded batch: remove padding, the layer stack, rebuild
    padding ([KS] Figs. 9-10). Returns y_pad[B, S, H] (float64), pads zero."""
    S = x_pad.shape[1]
    cu, _ = offsets(lens, S)
    xp = remove_padding(np.asarray(x_pad, np.float64), lens)
    y = encoder_stack(xp, cu, layers, heads, eps, round_to=round_to)
    return rebuild_padding(y, lens, S)
