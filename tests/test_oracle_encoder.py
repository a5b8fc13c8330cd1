"""Pins of oracle/encoder.py against brute force, a textbook library layer, closed forms
and invariants. CPU only."""
import math

import os

import numpy as np
import pytest
import torch

import tel_inputs as ti
from oracle import encoder as enc
from tests import brute

EPS = ti.LN_EPS


# ------------------------------------------------------------------ offsets and padding
def test_offsets_tiny_closed_form():
    cu, po = enc.offsets([5, 8], 8)
    assert cu.tolist() == [0, 5, 13]
    assert po.tolist() == [0] * 5 + [3] * 8


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_rows(name):
    """Whitespace-separated rows of a fixture under tests/golden, comments dropped."""
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


def test_offsets_golden():
    """Hand-worked offset masks (tests/golden/offsets.txt, after [KS] Fig. 9)."""
    cases, cur = [], None
    for tok in golden_rows("offsets.txt"):
        if tok[0] == "case":
            cur = {}
            cases.append(cur)
        else:
            cur[tok[0]] = [int(v) for v in tok[1:]]
    assert len(cases) == 3
    for c in cases:
        cu, po = enc.offsets(c["lens"], c["S"][0])
        assert cu.tolist() == c["cu_seqlens"], c
        assert po.tolist() == c["padding_offset"], c


def test_offsets_brute_force_random():
    rng = np.random.default_rng(11)
    for _ in range(20):
        B = int(rng.integers(1, 9))
        S = int(rng.integers(1, 17))
        lens = rng.integers(0, S + 1, size=B)
        cu, po = enc.offsets(lens, S)
        assert cu[-1] == lens.sum()
        rows = [b * S + i for b in range(B) for i in range(lens[b])]   # padded row of each token
        assert (np.arange(len(po)) + po).tolist() == rows
        for b in range(B):
            assert cu[b] == sum(lens[:b])


def test_offsets_mask_golden():
    """Hand-worked offset masks with holes (tests/golden/offsets_mask.txt, after [KS] Fig. 9)."""
    cases, cur = [], None
    for tok in golden_rows("offsets_mask.txt"):
        if tok[0] == "case":
            cur = {"mask": []}
            cases.append(cur)
        elif tok[0] == "mask":
            cur["mask"].append([int(v) for v in tok[1:]])
        else:
            cur[tok[0]] = [int(v) for v in tok[1:]]
    assert len(cases) == 4
    for c in cases:
        assert all(len(r) == c["S"][0] for r in c["mask"])
        cu, po = enc.offsets_from_mask(np.array(c["mask"]))
        assert cu.tolist() == c["cu_seqlens"], c
        assert po.tolist() == c["padding_offset"], c


def test_offsets_mask_brute_force_and_right_padded_case():
    rng = np.random.default_rng(12)
    for _ in range(30):
        B, S = int(rng.integers(1, 9)), int(rng.integers(1, 17))
        mask = rng.random((B, S)) < rng.random()
        cu, po = enc.offsets_from_mask(mask)
        rows, t, cu_ref = [], 0, [0]           # walk the batch position by position
        for b in range(B):
            for s in range(S):
                if mask[b, s]:
                    rows.append(b * S + s)
                    t += 1
            cu_ref.append(t)
        assert cu.tolist() == cu_ref
        assert (np.arange(len(po)) + po).tolist() == rows
        lens = rng.integers(0, S + 1, size=B)  # a right-padded mask is the lengths form
        right = np.arange(S)[None, :] < lens[:, None]
        for a, b_ in zip(enc.offsets_from_mask(right), enc.offsets(lens, S)):
            assert a.tolist() == b_.tolist()


def test_remove_rebuild_mask_roundtrip():
    rng = np.random.default_rng(13)
    mask = rng.random((4, 7)) < 0.6
    x = rng.standard_normal((4, 7, 5))
    xp = enc.remove_padding_mask(x, mask)
    assert xp.shape == (int(mask.sum()), 5)
    y = enc.rebuild_padding_mask(xp, mask)
    assert np.array_equal(y[mask], x[mask]) and not y[~mask].any()
    assert np.array_equal(enc.remove_padding_mask(y, mask), xp)


def test_layer_with_holes_matches_masked_padded_layer():
    """A layer on the packed tokens of a mask with holes equals, on the valid positions,
    the textbook layer over the padded batch with those keys masked out: the pure-Python
    brute force and torch's nn.TransformerEncoderLayer with src_key_padding_mask."""
    B, S, H, nh, F = 3, 7, 32, 2, 64
    rng = np.random.default_rng(14)
    mask = rng.random((B, S)) < 0.6
    mask[:, 3] = True                                  # no sequence fully masked
    cfg = ti.custom_encoder_config(B, S, [S] * B, H, nh, F, dtype="f32", seed=15)
    _, x = ti.encoder_input(cfg)
    w = ti.encoder_layer_weights(cfg, 0, variant=True)
    cu, _ = enc.offsets_from_mask(mask)
    y = enc.encoder_layer(enc.remove_padding_mask(x.astype(np.float64), mask), cu, w, nh, EPS)
    ref = brute.encoder_layer_padded(x, [S] * B, w, nh, EPS, mask=mask.tolist())
    assert np.abs(ref[mask] - y).max() <= 1e-10
    layer = _torch_layer(w, H, nh, F)
    with torch.no_grad():
        t = layer(torch.from_numpy(x.astype(np.float64)),
                  src_key_padding_mask=torch.from_numpy(~mask)).numpy()
    assert np.abs(t[mask] - y).max() <= 1e-10


def test_offsets_reject_bad_lengths():
    with pytest.raises(ValueError):
        enc.offsets([3, 9], 8)
    with pytest.raises(ValueError):
        enc.offsets([-1, 2], 8)


def test_remove_rebuild_roundtrip():
    rng = np.random.default_rng(3)
    for lens in ([5, 8], [0, 3, 0], [1], [4, 4, 4], [0]):
        S, W = 8, 6
        xp = rng.standard_normal((len(lens), S, W))
        packed = enc.remove_padding(xp, lens)
        assert packed.shape == (sum(lens), W)
        rb = enc.rebuild_padding(packed, lens, S)
        for b, L in enumerate(lens):
            assert np.array_equal(rb[b, :L], xp[b, :L])          # valid rows identical
            assert not rb[b, L:].any()                            # pads are zero
        assert np.array_equal(enc.remove_padding(rb, lens), packed)   # remove o rebuild = id


# ------------------------------------------------------------------ small pieces
def test_softmax_rows_sum_to_one():
    s = np.random.default_rng(0).standard_normal((7, 13)) * 30
    p = enc.softmax(s)
    assert np.abs(p.sum(-1) - 1).max() <= 1e-12
    assert (p >= 0).all()


def test_gelu_closed_forms():
    x = np.linspace(-6, 6, 97)
    assert np.allclose(enc.gelu(x) - enc.gelu(-x), x, atol=1e-14, rtol=0)
    assert enc.gelu(np.array([0.0]))[0] == 0.0
    # GELU(1) = Phi(1), the standard normal CDF at 1 (textbook table value)
    assert abs(enc.gelu(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15
    assert abs(enc.gelu(np.array([-1.0]))[0] + 0.15865525393145707) < 1e-15


def test_gelu_normal_cdf_golden():
    """GELU(x) = x * Phi(x) at the table values of tests/golden/normal_cdf.txt."""
    rows = golden_rows("normal_cdf.txt")
    assert len(rows) == 4
    for x, phi in rows:
        x, phi = float(x), float(phi)
        assert abs(enc.gelu(np.array([x]))[0] - x * phi) < 1e-15, x


def test_layernorm_invariants():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64)) * 3 + 2
    y = enc.layer_norm(x, np.ones(64), np.zeros(64), EPS)
    assert np.abs(y.mean(-1)).max() <= 1e-12
    var = x.var(-1)
    assert np.allclose((y * y).mean(-1), var / (var + EPS), atol=1e-12, rtol=0)
    beta = rng.standard_normal(64)
    const = enc.layer_norm(np.full((2, 64), 3.25), rng.standard_normal(64), beta, EPS)
    assert np.allclose(const, beta[None], atol=1e-12, rtol=0)
    twice = enc.layer_norm(y, np.ones(64), np.zeros(64), EPS)
    assert np.allclose(twice, y, atol=1e-4)


def _qkv_for(rng, T, H):
    return rng.standard_normal((T, 3 * H))


def test_attention_identical_keys_give_mean_of_v():
    rng = np.random.default_rng(2)
    H, heads, lens = 16, 2, [3, 5]
    cu, _ = enc.offsets(lens, 5)
    qkv = _qkv_for(rng, 8, H)
    qkv[:, H:2 * H] = rng.standard_normal(H)            # every key identical
    ctx = enc.attention(qkv, cu, heads)
    for b in range(2):
        sl = slice(cu[b], cu[b + 1])
        assert np.allclose(ctx[sl], qkv[sl, 2 * H:].mean(0, keepdims=True), atol=1e-13)


def test_attention_single_token_and_ones():
    rng = np.random.default_rng(4)
    H, heads, lens = 16, 4, [1, 6]
    cu, _ = enc.offsets(lens, 6)
    qkv = _qkv_for(rng, 7, H)
    ctx = enc.attention(qkv, cu, heads)
    assert np.allclose(ctx[0], qkv[0, 2 * H:], atol=1e-15)     # a lone token returns its own V
    qkv[:, 2 * H:] = 1.0
    assert np.allclose(enc.attention(qkv, cu, heads), 1.0, atol=1e-13)


def test_attention_permutation_and_independence():
    rng = np.random.default_rng(5)
    H, heads, lens = 32, 4, [6, 4]
    cu, _ = enc.offsets(lens, 6)
    qkv = _qkv_for(rng, 10, H)
    ctx = enc.attention(qkv, cu, heads)
    perm = np.r_[rng.permutation(6), 6 + rng.permutation(4)]
    assert np.allclose(enc.attention(qkv[perm], cu, heads), ctx[perm], atol=1e-13)
    other = qkv.copy()
    other[6:] = rng.standard_normal((4, 3 * H))               # change sequence 1 only
    assert np.array_equal(enc.attention(other, cu, heads)[:6], ctx[:6])


def test_attention_matches_padded_mask_sdpa():
    """Packed attention equals torch's scaled_dot_product_attention on the padded batch
    with a boolean key mask (a library routine), on valid rows."""
    rng = np.random.default_rng(6)
    H, heads, S, lens = 32, 4, 7, [7, 3, 5]
    d = H // heads
    cu, _ = enc.offsets(lens, S)
    qkv = _qkv_for(rng, sum(lens), H)
    ctx = enc.attention(qkv, cu, heads)
    pad = enc.rebuild_padding(qkv, lens, S)                   # [B, S, 3H]
    t = torch.from_numpy(pad)
    q, k, v = (t[..., i * H:(i + 1) * H].reshape(3, S, heads, d).transpose(1, 2) for i in range(3))
    keymask = torch.tensor([[j < L for j in range(S)] for L in lens])[:, None, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=keymask)
    ref = ref.transpose(1, 2).reshape(3, S, H).numpy()
    assert np.abs(enc.remove_padding(ref, lens) - ctx).max() <= 1e-12


# ------------------------------------------------------------------ whole layer
def _tiny():
    cfg = ti.ENCODER_CONFIGS["tiny"]
    lens, x = ti.encoder_input(cfg)
    return cfg, lens, x


@pytest.mark.parametrize("variant", [False, True])
def test_layer_matches_brute_force_tiny(variant):
    cfg, lens, x = _tiny()
    w = ti.encoder_layer_weights(cfg, 0, variant=variant)
    cu, _ = enc.offsets(lens, cfg["max_seq"])
    y = enc.encoder_layer(enc.remove_padding(x.astype(np.float64), lens), cu, w, cfg["heads"], EPS)
    ref = brute.encoder_layer_padded(x, lens, w, cfg["heads"], EPS)
    assert np.abs(enc.remove_padding(ref, lens) - y).max() <= 1e-10


def _torch_layer(w, H, heads, F):
    layer = torch.nn.TransformerEncoderLayer(H, heads, F, dropout=0.0, activation="gelu",
                                             layer_norm_eps=EPS, batch_first=True,
                                             norm_first=False, dtype=torch.float64)
    sd = {
        "self_attn.in_proj_weight": w["w_qkv"], "self_attn.in_proj_bias": w["b_qkv"],
        "self_attn.out_proj.weight": w["w_o"], "self_attn.out_proj.bias": w["b_o"],
        "linear1.weight": w["w_1"], "linear1.bias": w["b_1"],
        "linear2.weight": w["w_2"], "linear2.bias": w["b_2"],
        "norm1.weight": w["ln1_g"], "norm1.bias": w["ln1_b"],
        "norm2.weight": w["ln2_g"], "norm2.bias": w["ln2_b"],
    }
    layer.load_state_dict({k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in sd.items()})
    layer.train()      # training mode (dropout 0) keeps torch on its plain math path
    return layer


@pytest.mark.parametrize("shape", [
    dict(B=2, S=8, lens=[5, 8], H=64, heads=4, F=256),
    dict(B=3, S=9, lens=[9, 1, 4], H=32, heads=2, F=64),
    dict(B=2, S=6, lens=[6, 3], H=48, heads=3, F=96),
])
def test_layer_matches_torch_transformer_encoder_layer(shape):
    """nn.TransformerEncoderLayer (post-LN, exact GELU) in float64 on the padded batch with
    a key-padding mask is the textbook layer; on valid rows it must equal the packed oracle."""
    cfg = ti.custom_encoder_config(shape["B"], shape["S"], shape["lens"], shape["H"],
                                   shape["heads"], shape["F"], dtype="f32", seed=9)
    lens, x = ti.encoder_input(cfg)
    w = ti.encoder_layer_weights(cfg, 0, variant=True)
    layer = _torch_layer(w, shape["H"], shape["heads"], shape["F"])
    pad_mask = torch.tensor([[j >= L for j in range(shape["S"])] for L in lens])
    with torch.no_grad():
        ref = layer(torch.from_numpy(x.astype(np.float64)), src_key_padding_mask=pad_mask).numpy()
    cu, _ = enc.offsets(lens, shape["S"])
    y = enc.encoder_layer(enc.remove_padding(x.astype(np.float64), lens), cu, w, shape["heads"], EPS)
    assert np.abs(enc.remove_padding(ref, lens) - y).max() <= 1e-10


def test_layer_zero_weights_closed_form():
    """Zero weights and biases, gamma 1, beta 0: Q=K=V=0 so ctx=0, h1 = LN(x); GELU(0)=0 so
    y = LN(LN(x))."""
    cfg, lens, x = _tiny()
    w = {k: np.zeros_like(v) for k, v in ti.encoder_layer_weights(cfg, 0).items()}
    H = cfg["hidden"]
    w["ln1_g"] = np.ones(H); w["ln2_g"] = np.ones(H)
    xp = enc.remove_padding(x.astype(np.float64), lens)
    cu, _ = enc.offsets(lens, cfg["max_seq"])
    y = enc.encoder_layer(xp, cu, w, cfg["heads"], EPS)
    one, zero = np.ones(H), np.zeros(H)
    expect = enc.layer_norm(enc.layer_norm(xp, one, zero, EPS), one, zero, EPS)
    assert np.abs(y - expect).max() <= 1e-12


def test_padded_rows_do_not_matter():
    cfg, lens, x = _tiny()
    w = ti.encoder_layer_weights(cfg, 0, variant=True)
    y1 = enc.encoder_forward(x, lens, [w], cfg["heads"], EPS)
    x2 = x.copy()
    x2[0, lens[0]:] = 1e3                                     # garbage in the pad rows
    y2 = enc.encoder_forward(x2, lens, [w], cfg["heads"], EPS)
    assert np.array_equal(y1, y2)
    assert not y1[0, lens[0]:].any()


def test_stack_equals_repeated_layers():
    cfg, lens, x = _tiny()
    ws = [ti.encoder_layer_weights(cfg, i, variant=True) for i in range(3)]
    cu, _ = enc.offsets(lens, cfg["max_seq"])
    xp = enc.remove_padding(x.astype(np.float64), lens)
    y = xp
    for w in ws:
        y = enc.encoder_layer(y, cu, w, cfg["heads"], EPS)
    assert np.array_equal(enc.encoder_stack(xp, cu, ws, cfg["heads"], EPS), y)
