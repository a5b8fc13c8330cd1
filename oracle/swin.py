"""Oracle: Swin-style shifted-window attention block with relative-position bias (float64).

Test infrastructure only (see oracle/__init__.py). Page keys as listed there.

[SW] section 1: attention is computed only inside non-overlapping windows; a
cyclic window shift covers the window borders; a relative position bias adds
position information; a block is window operations (shift, partition, reverse),
attention, and an FFN. [SW] section 3 moves the bias-table lookup to a one-time
preprocessing step. The page names these operations without formulas; the
readings taken (the standard shifted-window definitions) are:
  * pre-LN block: X1 = X + WindowAttention(LN1(X)); Y = X1 + FFN(LN2(X1));
  * shift: roll by -s on both image axes before the partition, +s after the reverse;
  * windows row-major inside each image, images outermost; tokens row-major in a window;
  * Bias_h[p, q] = table[(py_p - py_q + M - 1) * (2M - 1) + (px_p - px_q + M - 1), h];
  * shift mask: in the shifted frame each axis splits into [0, L-M), [L-M, L-s), [L-s, L);
    a query attends to a key only when both fall in the same pair of ranges
    (excluded keys get -inf, i.e. weight exactly 0); no mask when s = 0.
"""
from __future__ import annotations

import math

import numpy as np

from . import encoder as enc

__all__ = ["cyclic_shift", "window_partition", "window_reverse", "relative_position_index",
           "region_ids", "window_mask", "window_attention", "swin_block", "patch_merge_gather",
           "patch_merging", "stage_shifts", "swin_stage", "swin_two_stages"]


def cyclic_shift(img: np.ndarray, s: int) -> np.ndarray:
    """out[b, y, x] = img[b, (y + s) mod Hs, (x + s) mod Ws] (a roll by -s), img [B, Hs, Ws, C]."""
    return np.roll(img, shift=(-s, -s), axis=(1, 2))


def window_partition(img: np.ndarray, M: int) -> np.ndarray:
    """[B, Hs, Ws, C] -> [B * nW, M*M, C]; window w = wy * (Ws/M) + wx, token p = py * M + px."""
    B, Hs, Ws, C = img.shape
    t = img.reshape(B, Hs // M, M, Ws // M, M, C).transpose(0, 1, 3, 2, 4, 5)
    return t.reshape(B * (Hs // M) * (Ws // M), M * M, C)


def window_reverse(win: np.ndarray, M: int, B: int, Hs: int, Ws: int) -> np.ndarray:
    """Inverse of window_partition: [B * nW, M*M, C] -> [B, Hs, Ws, C]."""
    C = win.shape[-1]
    t = win.reshape(B, Hs // M, Ws // M, M, M, C).transpose(0, 1, 3, 2, 4, 5)
    return t.reshape(B, Hs, Ws, C)


def relative_position_index(M: int) -> np.ndarray:
    """idx[p, q] = (py_p - py_q + M - 1) * (2M - 1) + (px_p - px_q + M - 1), shape [M*M, M*M]."""
    py, px = np.divmod(np.arange(M * M), M)
    dy = py[:, None] - py[None, :] + M - 1
    dx = px[:, None] - px[None, :] + M - 1
    return dy * (2 * M - 1) + dx


def region_ids(Hs: int, Ws: int, M: int, s: int) -> np.ndarray:
    """Region id of each position of the shifted frame, [Hs, Ws]; all zero when s = 0."""
    def axis(L):
        c = np.arange(L)
        if s == 0:
            return np.zeros(L, dtype=np.int64)
        return np.where(c < L - M, 0, np.where(c < L - s, 1, 2))
    return 3 * axis(Hs)[:, None] + axis(Ws)[None, :]


def window_mask(Hs: int, Ws: int, M: int, s: int) -> np.ndarray:
    """Additive mask [nW, M*M, M*M]: 0 where query and key share a region, -inf otherwise."""
    reg = window_partition(region_ids(Hs, Ws, M, s)[None, :, :, None], M)[:, :, 0]
    same = reg[:, :, None] == reg[:, None, :]
    return np.where(same, 0.0, -np.inf)


def window_attention(zw: np.ndarray, w: dict, heads: int, M: int, mask: np.ndarray | None):
    """Multi-head attention inside each window with relative-position bias and
    optional shift mask. zw is [nWin, M*M, C] (nWin a multiple of the mask's nW);
    returns the projected output [nWin, M*M, C]."""
    nWin, N, C = zw.shape
    d = C // heads
    qkv = enc.linear(zw.reshape(-1, C), w["w_qkv"], w["b_qkv"]).reshape(nWin, N, 3, heads, d)
    q, k, v = (qkv[:, :, i].transpose(0, 2, 1, 3) for i in range(3))  # [nWin, nh, N, d]
    table = np.asarray(w["rpb_table"], np.float64)
    bias = table[relative_position_index(M)].transpose(2, 0, 1)       # [nh, N, N]
    s = q @ k.transpose(0, 1, 3, 2) / math.sqrt(d) + bias[None]
    if mask is not None:
        nW = mask.shape[0]
        s = s.reshape(nWin // nW, nW, heads, N, N) + mask[None, :, None]
        s = s.reshape(nWin, heads, N, N)
    o = enc.softmax(s) @ v                                            # [nWin, nh, N, d]
    o = o.transpose(0, 2, 1, 3).reshape(nWin * N, C)
    return enc.linear(o, w["w_proj"], w["b_proj"]).reshape(nWin, N, C)


def swin_block(x: np.ndarray, w: dict, Hs: int, Ws: int, heads: int, M: int, s: int,
               eps: float, return_attn_only: bool = False) -> np.ndarray:
    """Shifted-window block on x[B, Hs*Ws, C] (tokens in row-major image order).

    LN1 -> roll(-s) -> partition -> window attention (+bias, +mask) -> reverse ->
    roll(+s) -> residual -> LN2 -> fc1 + GELU -> fc2 -> residual.
    With return_attn_only the result is X1 = X + attention branch.
    """
    x = np.asarray(x, np.float64)
    B, L, C = x.shape
    z = enc.layer_norm(x, w["ln1_g"], w["ln1_b"], eps).reshape(B, Hs, Ws, C)
    zs = cyclic_shift(z, s) if s else z
    mask = window_mask(Hs, Ws, M, s) if s else None
    a = window_attention(window_partition(zs, M), w, heads, M, mask)
    a = window_reverse(a, M, B, Hs, Ws)
    a = cyclic_shift(a, -s) if s else a
    x1 = x + a.reshape(B, L, C)
    if return_attn_only:
        return x1
    hid = enc.gelu(enc.linear(enc.layer_norm(x1, w["ln2_g"], w["ln2_b"], eps).reshape(-1, C),
                              w["w_1"], w["b_1"]))
    return x1 + enc.linear(hid, w["w_2"], w["b_2"]).reshape(B, L, C)


# ------------------------------------------------------------------ stages and downsampling
# [SW] section 1: the network is a sequence of stages with a downsampling step between
# them, so the resolution halves from stage to stage (a resolution pyramid); section 3,
# INT8 paragraph, names that step's GEMM (PatchMerge). The page gives no formula; the
# reading taken is the standard Swin patch merging:
#   * every 2 x 2 neighbourhood of the image becomes one token whose 4C features are the
#     four tokens' features concatenated in the order (row offset, column offset) =
#     (0, 0), (1, 0), (0, 1), (1, 1);
#   * a LayerNorm over the 4C features, then a linear map 4C -> 2C without bias;
#   * inside a stage, blocks alternate regular windows (shift 0) and shifted windows.

MERGE_ORDER = ((0, 0), (1, 0), (0, 1), (1, 1))   # (row offset, column offset) of part k


def patch_merge_gather(x: np.ndarray, Hs: int, Ws: int) -> np.ndarray:
    """[B, Hs*Ws, C] (row-major image order) -> [B, (Hs/2)*(Ws/2), 4C]: output token (i, j)
    holds the features of image tokens (2i + dy, 2j + dx) for (dy, dx) in MERGE_ORDER."""
    B, L, C = x.shape
    if Hs % 2 or Ws % 2 or L != Hs * Ws:
        raise ValueError("patch merging needs an even image height and width")
    img = np.asarray(x).reshape(B, Hs, Ws, C)
    parts = [img[:, dy::2, dx::2] for dy, dx in MERGE_ORDER]
    return np.concatenate(parts, axis=-1).reshape(B, (Hs // 2) * (Ws // 2), 4 * C)


def patch_merging(x: np.ndarray, w: dict, Hs: int, Ws: int, eps: float) -> np.ndarray:
    """Downsampling between stages: y = LN(gather(x); norm_g, norm_b) W_red^T, with W_red
    [2C, 4C] and no bias. Returns [B, (Hs/2)*(Ws/2), 2C]."""
    v = patch_merge_gather(np.asarray(x, np.float64), Hs, Ws)
    B, L2, C4 = v.shape
    z = enc.layer_norm(v.reshape(-1, C4), w["norm_g"], w["norm_b"], eps)
    return (z @ np.asarray(w["w_red"], np.float64).T).reshape(B, L2, -1)


def stage_shifts(n_blocks: int, Hs: int, Ws: int, M: int) -> list:
    """Shift of each block of a stage: 0 for even blocks, M // 2 for odd ones; 0 throughout
    when one window covers the image (nothing to shift)."""
    s = M // 2 if min(Hs, Ws) > M else 0
    return [0 if i % 2 == 0 else s for i in range(n_blocks)]


def swin_stage(x: np.ndarray, blocks: list, Hs: int, Ws: int, heads: int, M: int,
               eps: float) -> np.ndarray:
    """The blocks of one stage in order on x [B, Hs*Ws, C], shifts as stage_shifts."""
    for w, s in zip(blocks, stage_shifts(len(blocks), Hs, Ws, M)):
        x = swin_block(x, w, Hs, Ws, heads, M, s, eps)
    return x


def swin_two_stages(x: np.ndarray, stage1: list, merge: dict, stage2: list, Hs: int, Ws: int,
                    heads1: int, heads2: int, M: int, eps: float) -> np.ndarray:
    """Stage 1 at Hs x Ws, patch merging, stage 2 at (Hs/2) x (Ws/2) with twice the
    channels; every tensor between the pieces stays float64 (no storage rounding)."""
    x = swin_stage(x, stage1, Hs, Ws, heads1, M, eps)
    x = patch_merging(x, merge, Hs, Ws, eps)
    return swin_stage(x, stage2, Hs // 2, Ws // 2, heads2, M, eps)
