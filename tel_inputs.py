"""Seeded synthetic inputs for the encoder-layer and shifted-window workloads.

This module holds random draws and storage-type rounding only. It contains no
step of the layer's arithmetic, so both the CPU oracle's callers (tests, the
benchmark's CPU leg) and the GPU path's callers can use it without sharing any
of the method.

Workloads (sizes as named below):
  * tiny               post-LN encoder layer, fp32, batch 2, lengths {5, 8} padded to 8,
                       hidden 64, 4 heads, FFN 256
  * bert_base          12 layers, fp16, batch 32, max_seq 128, lengths U{32..128},
                       hidden 768, 12 heads, FFN 3072
  * bert_large_latency 24 layers, fp16, batch 1, seq 128 all valid, hidden 1024, 16 heads,
                       FFN 4096
  * bert_large_tput    24 layers, fp16, batch 64, max_seq 384, lengths U{64..384}
  * bert_base_int8     bert_base shape, int8 GEMMs
  * swin_t_stage1      shifted-window block, fp16, batch 64, 56x56 tokens, C 96, 3 heads,
                       window 7, shift 3, MLP 384

Draw recipe: weights N(0, 0.02), activations N(0, 1), relative-position-bias
table N(0, 0.02). Biases are 0, LayerNorm gamma 1 and beta 0 unless
``variant=True``, which draws biases N(0, 0.02), gamma 1 + N(0, 0.1) and
beta N(0, 0.1) so that every epilogue term is exercised. Pad rows of the
padded input are random too: they must not influence any valid output.
Values are rounded once to the storage type ("f32", "f16" or "bf16"; bf16 is
returned as float32 arrays holding bf16-representable values).
"""
from __future__ import annotations

import numpy as np

ENCODER_CONFIGS = {
    "tiny": dict(batch=2, max_seq=8, lens=[5, 8], hidden=64, heads=4, ffn=256,
                 layers=1, dtype="f32", seed=0),
    "bert_base": dict(batch=32, max_seq=128, len_range=(32, 128), hidden=768, heads=12,
                      ffn=3072, layers=12, dtype="f16", seed=1),
    "bert_large_latency": dict(batch=1, max_seq=128, lens=[128], hidden=1024, heads=16,
                               ffn=4096, layers=24, dtype="f16", seed=2),
    "bert_large_tput": dict(batch=64, max_seq=384, len_range=(64, 384), hidden=1024,
                            heads=16, ffn=4096, layers=24, dtype="f16", seed=3),
    "bert_base_int8": dict(batch=32, max_seq=128, len_range=(32, 128), hidden=768, heads=12,
                           ffn=3072, layers=12, dtype="f16", seed=4, int8=True),
    # the same int8 batch with dynamic activation scales (from each batch's own max-abs)
    "bert_base_int8_dyn": dict(batch=32, max_seq=128, len_range=(32, 128), hidden=768,
                               heads=12, ffn=3072, layers=12, dtype="f16", seed=4, int8=True,
                               dynamic=True),
    # the same int8 batch with attention's two products on int8 codes as well
    "bert_base_int8_attn": dict(batch=32, max_seq=128, len_range=(32, 128), hidden=768,
                                heads=12, ffn=3072, layers=12, dtype="f16", seed=4, int8=2),
    # BERT-base with its projection matrices pruned 2:4 (same batch and weights as bert_base)
    "bert_base_sparse": dict(batch=32, max_seq=128, len_range=(32, 128), hidden=768, heads=12,
                             ffn=3072, layers=12, dtype="f16", seed=1, sparse=True),
}

SWIN_CONFIGS = {
    "swin_t_stage1": dict(batch=64, height=56, width=56, channels=96, heads=3, window=7,
                          shift=3, mlp=384, dtype="f16", seed=5),
}

# Swin-T's first two stages with the downsampling between them: stage 1 (56 x 56, C 96,
# 3 heads) and stage 2 (28 x 28, C 192, 6 heads), two blocks each (regular, then shifted
# windows), window 7, MLP ratio 4; patch merging 4C = 384 -> 2C = 192.
SWIN_STAGES = {
    "swin_t_stage12": dict(batch=64, height=56, width=56, channels=96, heads=(3, 6), window=7,
                           blocks=(2, 2), mlp_ratio=4, dtype="f16", seed=6),
}

LN_EPS = 1e-5


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float values to the nearest bfloat16 (ties to even); returns float32."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = ((u + 0x7FFF + lsb) >> 16) << 16
    out = u.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(f), f, out)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the storage type once: f32 -> float32, f16 -> float16, bf16 -> float32."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# ----------------------------------------------------------------------------- encoder
def encoder_lengths(cfg: dict, seed: int | None = None) -> np.ndarray:
    """Valid length of every sequence (int32, right padding up to max_seq)."""
    if "lens" in cfg:
        return np.asarray(cfg["lens"], dtype=np.int32)
    rng = np.random.default_rng([cfg["seed"] if seed is None else seed, 0])
    lo, hi = cfg["len_range"]
    return rng.integers(lo, hi + 1, size=cfg["batch"]).astype(np.int32)


# Stress shape for the offsets kernel alone: many sequences, T near 2^24 valid tokens.
OFFSETS_STRESS = dict(batch=65536, max_seq=512, seed=123)


# Stress shape for the padding and LayerNorm kernels alone: ~0.4 GB of packed rows.
PADDING_STRESS = dict(batch=1024, max_seq=512, hidden=768, seed=124)


def padding_stress_lengths(cfg: dict = PADDING_STRESS) -> np.ndarray:
    """lens ~ U{0..max_seq} for the padding stress shape (int32)."""
    rng = np.random.default_rng(cfg["seed"])
    return rng.integers(0, cfg["max_seq"] + 1, size=cfg["batch"]).astype(np.int32)


def offsets_stress_lengths(cfg: dict = OFFSETS_STRESS) -> np.ndarray:
    """lens ~ U{0..max_seq} for the offsets stress shape (int32)."""
    rng = np.random.default_rng(cfg["seed"])
    return rng.integers(0, cfg["max_seq"] + 1, size=cfg["batch"]).astype(np.int32)


def encoder_input(cfg: dict, seed: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """(lens[B] int32, x_pad[B, S, H]) with x ~ N(0, 1) everywhere, pads included."""
    s = cfg["seed"] if seed is None else seed
    lens = encoder_lengths(cfg, s)
    rng = np.random.default_rng([s, 1])
    x = rng.standard_normal((cfg["batch"], cfg["max_seq"], cfg["hidden"]))
    return lens, to_storage(x, cfg["dtype"])


def encoder_layer_weights(cfg: dict, layer: int, variant: bool = False,
                          seed: int | None = None) -> dict:
    """Weights of one layer in nn.Linear layout: W[out, in]; W_qkv rows are [Q; K; V].

    Each layer has its own generator, so any layer can be drawn on its own.
    """
    s = cfg["seed"] if seed is None else seed
    H, F, dt = cfg["hidden"], cfg["ffn"], cfg["dtype"]
    rng = np.random.default_rng([s, 2, layer])
    w = {
        "w_qkv": rng.standard_normal((3 * H, H)) * 0.02,
        "w_o": rng.standard_normal((H, H)) * 0.02,
        "w_1": rng.standard_normal((F, H)) * 0.02,
        "w_2": rng.standard_normal((H, F)) * 0.02,
    }
    if variant:
        rv = np.random.default_rng([s, 3, layer])
        w.update({
            "b_qkv": rv.standard_normal(3 * H) * 0.02,
            "b_o": rv.standard_normal(H) * 0.02,
            "ln1_g": 1.0 + rv.standard_normal(H) * 0.1,
            "ln1_b": rv.standard_normal(H) * 0.1,
            "b_1": rv.standard_normal(F) * 0.02,
            "b_2": rv.standard_normal(H) * 0.02,
            "ln2_g": 1.0 + rv.standard_normal(H) * 0.1,
            "ln2_b": rv.standard_normal(H) * 0.1,
        })
    else:
        w.update({
            "b_qkv": np.zeros(3 * H), "b_o": np.zeros(H),
            "ln1_g": np.ones(H), "ln1_b": np.zeros(H),
            "b_1": np.zeros(F), "b_2": np.zeros(H),
            "ln2_g": np.ones(H), "ln2_b": np.zeros(H),
        })
    return {k: to_storage(v, dt) for k, v in w.items()}


def custom_encoder_config(batch, max_seq, lens, hidden, heads, ffn, dtype="f16", seed=0,
                          layers=1) -> dict:
    """A config dict of the same form as ENCODER_CONFIGS for ad-hoc shapes."""
    return dict(batch=batch, max_seq=max_seq, lens=list(lens), hidden=hidden, heads=heads,
                ffn=ffn, layers=layers, dtype=dtype, seed=seed)


# ----------------------------------------------------------------------------- swin
def swin_input(cfg: dict, seed: int | None = None) -> np.ndarray:
    """x[B, Hs*Ws, C] ~ N(0, 1), tokens in row-major image order."""
    s = cfg["seed"] if seed is None else seed
    rng = np.random.default_rng([s, 1])
    x = rng.standard_normal((cfg["batch"], cfg["height"] * cfg["width"], cfg["channels"]))
    return to_storage(x, cfg["dtype"])


def swin_block_weights(cfg: dict, variant: bool = False, seed: int | None = None) -> dict:
    """Weights of one shifted-window block; rpb_table is [(2M-1)^2, heads]."""
    s = cfg["seed"] if seed is None else seed
    C, F, nh, M = cfg["channels"], cfg["mlp"], cfg["heads"], cfg["window"]
    rng = np.random.default_rng([s, 2])
    w = {
        "w_qkv": rng.standard_normal((3 * C, C)) * 0.02,
        "rpb_table": rng.standard_normal(((2 * M - 1) ** 2, nh)) * 0.02,
        "w_proj": rng.standard_normal((C, C)) * 0.02,
        "w_1": rng.standard_normal((F, C)) * 0.02,
        "w_2": rng.standard_normal((C, F)) * 0.02,
    }
    if variant:
        rv = np.random.default_rng([s, 3])
        w.update({
            "ln1_g": 1.0 + rv.standard_normal(C) * 0.1, "ln1_b": rv.standard_normal(C) * 0.1,
            "b_qkv": rv.standard_normal(3 * C) * 0.02, "b_proj": rv.standard_normal(C) * 0.02,
            "ln2_g": 1.0 + rv.standard_normal(C) * 0.1, "ln2_b": rv.standard_normal(C) * 0.1,
            "b_1": rv.standard_normal(F) * 0.02, "b_2": rv.standard_normal(C) * 0.02,
        })
    else:
        w.update({
            "ln1_g": np.ones(C), "ln1_b": np.zeros(C), "b_qkv": np.zeros(3 * C),
            "b_proj": np.zeros(C), "ln2_g": np.ones(C), "ln2_b": np.zeros(C),
            "b_1": np.zeros(F), "b_2": np.zeros(C),
        })
    return {k: to_storage(v, cfg["dtype"]) for k, v in w.items()}


def custom_swin_config(batch, height, width, channels, heads, window, shift, mlp,
                       dtype="f16", seed=0) -> dict:
    return dict(batch=batch, height=height, width=width, channels=channels, heads=heads,
                window=window, shift=shift, mlp=mlp, dtype=dtype, seed=seed)


# ----------------------------------------------------------------------------- int8 gemm
def int8_operands(M: int, N: int, K: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Random int8 operands A[M, K], B[N, K] with codes in [-127, 127]."""
    rng = np.random.default_rng([seed, 7])
    a = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    b = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    return a, b


def swin_stage_block_config(cfg: dict, stage: int, shift: int) -> dict:
    """The block config (as SWIN_CONFIGS entries) of stage 0 or 1 of a SWIN_STAGES entry."""
    f = 2 ** stage
    C = cfg["channels"] * f
    return dict(batch=cfg["batch"], height=cfg["height"] // f, width=cfg["width"] // f,
                channels=C, heads=cfg["heads"][stage], window=cfg["window"], shift=shift,
                mlp=C * cfg["mlp_ratio"], dtype=cfg["dtype"], seed=cfg["seed"])


def swin_stage_weights(cfg: dict, variant: bool = False):
    """(stage-1 block weights, patch-merging weights, stage-2 block weights) of a
    SWIN_STAGES entry; every block draws from its own seed tuple."""
    s = cfg["seed"]
    out = []
    for stage in range(2):
        blocks = []
        for i in range(cfg["blocks"][stage]):
            bc = swin_stage_block_config(cfg, stage, 0)
            blocks.append(swin_block_weights(bc, variant, seed=1000 * s + 100 * stage + i))
        out.append(blocks)
    return out[0], patch_merge_weights(cfg["channels"], variant, seed=s), out[1]


def patch_merge_weights(C: int, variant: bool = False, seed: int = 0, dtype: str = "f16") -> dict:
    """norm_g, norm_b [4C] (1 and 0, or 1 + N(0, 0.1) and N(0, 0.1) with variant) and
    w_red [2C, 4C] ~ N(0, 0.02), rounded to the storage type."""
    rng = np.random.default_rng([seed, 7])
    w = {"w_red": rng.standard_normal((2 * C, 4 * C)) * 0.02,
         "norm_g": np.ones(4 * C), "norm_b": np.zeros(4 * C)}
    if variant:
        w["norm_g"] = 1.0 + rng.standard_normal(4 * C) * 0.1
        w["norm_b"] = rng.standard_normal(4 * C) * 0.1
    return {k: to_storage(v, dtype) for k, v in w.items()}
