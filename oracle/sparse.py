"""Oracle: 2:4 structured-sparse projection weights.

Test infrastructure only (see oracle/__init__.py). Page keys as listed there.

[TRT], the paragraphs on sparsity of the Ampere architecture: connections that do not
contribute to the network's result are pruned, which removes about half of the
weights, and the hardware skips the work they would have needed. Readings where the
page is silent:
  * the pattern is the fine-grained structured one such sparse matrix units execute:
    in every group of four consecutive weights along the input dimension k of an
    output row, two are kept and two are zero ("2:4");
  * magnitude pruning: the two weights of largest |w| in a group are kept; among equal
    magnitudes the lower k is kept first (a deterministic order);
  * the sparse layer is the dense layer with its four projection matrices pruned:
    products, biases, attention, GELU and LayerNorm are unchanged.
Compressed form (how the library stores a pruned matrix; written out here so that its
encoding is checked bit for bit): values[n][K/2] hold the two kept weights of every
group in increasing k; index[n][K/16] are 16-bit words, one per 16 consecutive k, in
which group g (k = 16 w + 4 g .. 16 w + 4 g + 3) occupies bits 4g .. 4g+3: bits 4g, 4g+1
give the position (0..3) of its first kept weight and bits 4g+2, 4g+3 that of its second.
"""
from __future__ import annotations

import numpy as np

from . import encoder as enc

__all__ = ["prune_2of4", "keep_positions", "compress_2of4", "decompress_2of4",
           "prune_layer_weights", "SPARSE_WEIGHTS"]

# the four projection matrices of an encoder layer, pruned by the sparse variant
SPARSE_WEIGHTS = ("w_qkv", "w_o", "w_1", "w_2")


def keep_positions(w: np.ndarray) -> np.ndarray:
    """Positions (0..3, increasing) of the two kept weights of every group of four along
    the last axis: [..., K] -> [..., K/4, 2]. Order of preference: larger |w| first, then
    lower position."""
    w = np.asarray(w, np.float64)
    assert w.shape[-1] % 4 == 0, "K must be a multiple of 4"
    g = np.abs(w.reshape(*w.shape[:-1], w.shape[-1] // 4, 4))
    order = np.argsort(-g, axis=-1, kind="stable")   # stable: ties keep the lower position
    return np.sort(order[..., :2], axis=-1)


def prune_2of4(w: np.ndarray) -> np.ndarray:
    """w with the two smaller-magnitude weights of every group of four (along k) zeroed."""
    w = np.asarray(w, np.float64)
    pos = keep_positions(w)
    groups = w.reshape(*w.shape[:-1], w.shape[-1] // 4, 4)
    keep = np.zeros(groups.shape, bool)
    np.put_along_axis(keep, pos, True, axis=-1)
    return np.where(keep, groups, 0.0).reshape(w.shape)


def compress_2of4(w: np.ndarray):
    """(values [N][K/2] float64, index [N][K/16] uint16) of the pruned matrix; K % 16 == 0."""
    w = np.asarray(w, np.float64)
    N, K = w.shape
    assert K % 16 == 0, "K must be a multiple of 16"
    pos = keep_positions(w)                                    # [N, K/4, 2]
    groups = w.reshape(N, K // 4, 4)
    values = np.take_along_axis(groups, pos, axis=-1).reshape(N, K // 2)
    nib = (pos[..., 0] | (pos[..., 1] << 2)).astype(np.int64)  # [N, K/4], 4 bits a group
    nib = nib.reshape(N, K // 16, 4)
    words = nib[..., 0] | (nib[..., 1] << 4) | (nib[..., 2] << 8) | (nib[..., 3] << 12)
    return values, words.astype(np.uint16)


def decompress_2of4(values: np.ndarray, index: np.ndarray, K: int) -> np.ndarray:
    """Dense [N][K] matrix from the compressed form (zeros where nothing is kept)."""
    values = np.asarray(values, np.float64)
    index = np.asarray(index).astype(np.int64)
    N = values.shape[0]
    out = np.zeros((N, K))
    for n in range(N):
        for wd in range(K // 16):
            word = int(index[n, wd])
            for g in range(4):
                p0 = (word >> (4 * g)) & 3
                p1 = (word >> (4 * g + 2)) & 3
                base = 16 * wd + 4 * g
                v = 8 * wd + 2 * g
                out[n, base + p0] += values[n, v]
                out[n, base + p1] += values[n, v + 1]
    return out


def prune_layer_weights(w: dict) -> dict:
    """One encoder layer's weights with its four projection matrices pruned 2:4 (biases,
    LayerNorm parameters unchanged); the sparse layer is encoder.encoder_layer on these."""
    out = dict(w)
    for k in SPARSE_WEIGHTS:
        out[k] = prune_2of4(w[k])
    return out


def linear_2of4(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """x W^T + b with W pruned 2:4."""
    return enc.linear(x, prune_2of4(w), b)
