"""Pins of oracle/swin.py: a direct image-coordinate brute force, textbook attention in
special cases, index-map identities and the mask layout. CPU only."""
import math

import numpy as np
import pytest
import torch

import tel_inputs as ti
from oracle import encoder as enc
from oracle import swin
from tests.test_oracle_encoder import golden_rows
from tests import brute

EPS = ti.LN_EPS


@pytest.mark.parametrize("Hs,M,s", [(6, 3, 1), (6, 3, 0), (4, 2, 1), (6, 2, 1)])
def test_block_matches_direct_brute_force(Hs, M, s):
    cfg = ti.custom_swin_config(2, Hs, Hs, 8, 2, M, s, 16, dtype="f32", seed=Hs * 10 + M + s)
    x = ti.swin_input(cfg)
    w = ti.swin_block_weights(cfg, variant=True)
    y = swin.swin_block(x, w, Hs, Hs, 2, M, s, EPS)
    ref = brute.swin_block_direct(x, w, Hs, Hs, 2, M, s, EPS)
    assert np.abs(y - ref).max() <= 1e-10


def test_index_maps_are_inverse():
    rng = np.random.default_rng(0)
    img = rng.standard_normal((2, 14, 21, 3))
    assert np.array_equal(swin.window_reverse(swin.window_partition(img, 7), 7, 2, 14, 21), img)
    assert np.array_equal(swin.cyclic_shift(swin.cyclic_shift(img, 3), -3), img)
    sh = swin.cyclic_shift(img, 3)
    assert sh[1, 0, 0, 2] == img[1, 3, 3, 2] and sh[0, 13, 20, 1] == img[0, 2, 2, 1]
    win = swin.window_partition(img, 7)                           # window 1 = (wy 0, wx 1)
    assert win.shape == (12, 49, 3)
    assert np.array_equal(win[1, 8], img[0, 1, 8])                # token p=8 -> (py 1, px 1)


def test_relative_position_index():
    idx = swin.relative_position_index(7)
    assert idx.shape == (49, 49) and idx.min() == 0 and idx.max() == 168
    assert (np.diag(idx) == 6 * 13 + 6).all()                     # zero offset -> table centre
    assert idx[0, 48] == 0 and idx[48, 0] == 168


def test_relative_position_index_golden():
    """The 2x2-window index table worked by hand (tests/golden/relative_position_index_window2.txt)."""
    want = np.array(golden_rows("relative_position_index_window2.txt"), dtype=np.int64)
    assert np.array_equal(swin.relative_position_index(2), want)


def test_shift_mask_golden():
    """Masked windows of the Swin-T stage-1 grid (tests/golden/swin_shift_mask_56_7_3.txt)."""
    grid = np.array(golden_rows("swin_shift_mask_56_7_3.txt"), dtype=np.int64).astype(bool)
    m = swin.window_mask(56, 56, 7, 3)
    assert np.array_equal(np.isinf(m).any(axis=(1, 2)).reshape(8, 8), grid)


def test_mask_layout_56_7_3():
    m = swin.window_mask(56, 56, 7, 3)
    assert m.shape == (64, 49, 49)
    masked = np.isinf(m).any(axis=(1, 2))
    grid = masked.reshape(8, 8)
    assert masked.sum() == 15                                     # only the last row and column
    assert grid[7].all() and grid[:, 7].all() and not grid[:7, :7].any()
    assert (np.diagonal(m, axis1=1, axis2=2) == 0).all()          # a token always sees itself
    assert not np.isinf(swin.window_mask(56, 56, 7, 0)).any()


def test_no_shift_zero_table_is_plain_window_mha():
    cfg = ti.custom_swin_config(1, 6, 6, 8, 2, 3, 0, 16, dtype="f32", seed=4)
    x = ti.swin_input(cfg)
    w = ti.swin_block_weights(cfg, variant=True)
    w["rpb_table"] = np.zeros_like(w["rpb_table"])
    x1 = swin.swin_block(x, w, 6, 6, 2, 3, 0, EPS, return_attn_only=True)
    z = enc.layer_norm(x, w["ln1_g"], w["ln1_b"], EPS).reshape(1, 6, 6, 8)
    zw = torch.from_numpy(swin.window_partition(z, 3))            # [4, 9, 8]
    mha = torch.nn.MultiheadAttention(8, 2, batch_first=True, dtype=torch.float64)
    mha.load_state_dict({"in_proj_weight": torch.from_numpy(w["w_qkv"].astype(np.float64)),
                         "in_proj_bias": torch.from_numpy(w["b_qkv"].astype(np.float64)),
                         "out_proj.weight": torch.from_numpy(w["w_proj"].astype(np.float64)),
                         "out_proj.bias": torch.from_numpy(w["b_proj"].astype(np.float64))})
    with torch.no_grad():
        a = mha(zw, zw, zw, need_weights=False)[0].numpy()
    ref = x + swin.window_reverse(a, 3, 1, 6, 6).reshape(1, 36, 8)
    assert np.abs(x1 - ref).max() <= 1e-12


def test_single_window_is_global_attention_with_bias():
    """M = Hs = Ws and s = 0: one window covering the image, so the block is global
    attention with an additive bias: torch scaled_dot_product_attention with a float mask."""
    M, C, nh = 4, 8, 2
    d = C // nh
    cfg = ti.custom_swin_config(2, M, M, C, nh, M, 0, 16, dtype="f32", seed=5)
    x = ti.swin_input(cfg).astype(np.float64)
    w = {k: v.astype(np.float64) for k, v in ti.swin_block_weights(cfg, variant=True).items()}
    y = swin.swin_block(x, w, M, M, nh, M, 0, EPS)
    t = lambda a: torch.from_numpy(a)
    F = torch.nn.functional
    z = F.layer_norm(t(x), (C,), t(w["ln1_g"]), t(w["ln1_b"]), EPS)
    qkv = F.linear(z, t(w["w_qkv"]), t(w["b_qkv"])).reshape(2, M * M, 3, nh, d)
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    py, px = np.divmod(np.arange(M * M), M)
    rel = (py[:, None] - py[None] + M - 1) * (2 * M - 1) + (px[:, None] - px[None] + M - 1)
    bias = t(w["rpb_table"][rel].transpose(2, 0, 1))[None]
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=bias).transpose(1, 2).reshape(2, M * M, C)
    x1 = t(x) + F.linear(o, t(w["w_proj"]), t(w["b_proj"]))
    h = F.gelu(F.linear(F.layer_norm(x1, (C,), t(w["ln2_g"]), t(w["ln2_b"]), EPS),
                        t(w["w_1"]), t(w["b_1"])))
    ref = (x1 + F.linear(h, t(w["w_2"]), t(w["b_2"]))).numpy()
    assert np.abs(y - ref).max() <= 1e-12


# ------------------------------------------------------------------ stages, patch merging
def test_patch_merge_gather_golden():
    """tests/golden/patch_merge_order_4x6.txt: the 2 x 2 gather of a 4 x 6 image, by hand."""
    img = np.array([[10 * y + x for x in range(6)] for y in range(4)], np.float64)
    got = swin.patch_merge_gather(img.reshape(1, 24, 1), 4, 6)
    want = np.array([[float(v) for v in r] for r in golden_rows("patch_merge_order_4x6.txt")])
    assert got.shape == (1, 6, 4)
    assert np.array_equal(got[0], want)


def test_patch_merge_gather_is_a_rearrangement():
    """The gather is einops' rearrangement b (h p1) (w p2) c -> b (h w) (p2 p1 c): the
    column offset p2 is the slower of the two offsets in the concatenated features."""
    from einops import rearrange
    rng = np.random.default_rng(3)
    B, Hs, Ws, C = 2, 6, 10, 5
    x = rng.standard_normal((B, Hs * Ws, C))
    want = rearrange(x.reshape(B, Hs, Ws, C), "b (h p1) (w p2) c -> b (h w) (p2 p1 c)", p1=2, p2=2)
    assert np.array_equal(swin.patch_merge_gather(x, Hs, Ws), want)
    with pytest.raises(ValueError):
        swin.patch_merge_gather(x[:, :55], 5, 11)


@pytest.mark.parametrize("Hs,Ws,C", [(4, 6, 3), (8, 8, 4), (2, 2, 8)])
def test_patch_merging_matches_brute_force(Hs, Ws, C):
    rng = np.random.default_rng(Hs * Ws + C)
    x = rng.standard_normal((2, Hs * Ws, C))
    w = ti.patch_merge_weights(C, variant=True, seed=C, dtype="f32")
    y = swin.patch_merging(x, w, Hs, Ws, EPS)
    assert y.shape == (2, (Hs // 2) * (Ws // 2), 2 * C)
    assert np.abs(y - brute.patch_merging_direct(x, w, Hs, Ws, EPS)).max() <= 1e-12


def test_patch_merging_normalises_all_four_parts_together():
    """Parts of very different scale: a LayerNorm per part (or per channel group) would map
    each part to unit variance; over all 4C the small parts stay small."""
    C = 4
    x = np.zeros((1, 4, C))
    x[0, 0] = [1, 2, 3, 4]          # part 0 of the single output token
    x[0, 1:] = 1e-3 * np.arange(12).reshape(3, C)
    w = {"w_red": np.eye(2 * C, 4 * C), "norm_g": np.ones(4 * C), "norm_b": np.zeros(4 * C)}
    v = np.concatenate([x[0, 0], x[0, 2], x[0, 1], x[0, 3]])   # order (0,0), (1,0), (0,1), (1,1)
    z = (v - v.mean()) / np.sqrt(v.var() + EPS)
    assert np.abs(swin.patch_merging(x, w, 2, 2, EPS)[0, 0] - z[:2 * C]).max() <= 1e-12


def test_stage_shifts():
    assert swin.stage_shifts(2, 56, 56, 7) == [0, 3]
    assert swin.stage_shifts(4, 28, 28, 7) == [0, 3, 0, 3]
    assert swin.stage_shifts(2, 7, 7, 7) == [0, 0]          # one window covers the image


def test_two_stages_match_brute_force_composition():
    """Stage 1 (two blocks), patch merging, stage 2 (two blocks) against the direct block
    brute force and the patch-merging brute force chained by hand."""
    B, Hs, M = 1, 8, 2
    c1 = ti.custom_swin_config(B, Hs, Hs, 8, 2, M, 1, 16, dtype="f32", seed=71)
    c2 = ti.custom_swin_config(B, Hs // 2, Hs // 2, 16, 4, M, 1, 32, dtype="f32", seed=72)
    s1 = [ti.swin_block_weights(c1, variant=True, seed=80 + i) for i in range(2)]
    s2 = [ti.swin_block_weights(c2, variant=True, seed=90 + i) for i in range(2)]
    mw = ti.patch_merge_weights(8, variant=True, seed=5, dtype="f32")
    x = ti.swin_input(c1)
    got = swin.swin_two_stages(x, s1, mw, s2, Hs, Hs, 2, 4, M, EPS)
    ref = brute.swin_block_direct(x, s1[0], Hs, Hs, 2, M, 0, EPS)
    ref = brute.swin_block_direct(ref, s1[1], Hs, Hs, 2, M, 1, EPS)
    ref = brute.patch_merging_direct(ref, mw, Hs, Hs, EPS)
    ref = brute.swin_block_direct(ref, s2[0], Hs // 2, Hs // 2, 4, M, 0, EPS)
    ref = brute.swin_block_direct(ref, s2[1], Hs // 2, Hs // 2, 4, M, 1, EPS)
    assert got.shape == (B, (Hs // 2) ** 2, 16)
    assert np.abs(got - ref).max() <= 1e-10
