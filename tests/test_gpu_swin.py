"""GPU parity of the shifted-window block against oracle/swin.py: the partition gather,
the attention half (gather, QKV, window attention with bias and shift mask, scatter with
residual) and the whole block, on small shapes, edge cases and the Swin-T stage-1 batch
(GPU on all 64 images, oracle on a sample of images: images are independent)."""
import numpy as np
import pytest
import torch

import tel_inputs as ti
from oracle import encoder as enc
from oracle import swin
from tests.gpu_helpers import TORCH_DT, assert_close, dev, dev_f32, errors, host

pytestmark = pytest.mark.gpu

tel = pytest.importorskip("transformer_encoder_remove_amd")
EPS = ti.LN_EPS


def gpu_swin(cfg, x, w, flags=0):
    dt = cfg["dtype"]
    desc = tel.make_swin_desc(cfg["batch"], cfg["height"], cfg["width"], cfg["channels"],
                              cfg["heads"], cfg["window"], cfg["shift"], cfg["mlp"], TORCH_DT[dt],
                              EPS)
    n = tel.tel_swin_packed_size(desc)
    assert n > 0
    packed = tel.alloc_bytes(n)
    tel.tel_swin_prepare(desc, {k: dev(v, dt) for k, v in w.items()}, packed)
    xd = dev(x, dt)
    yd = torch.full_like(xd, float("nan"))
    ws = tel.alloc_bytes(tel.tel_swin_workspace_size(desc))
    tel.tel_window_attention_forward(desc, packed, xd, yd, ws, flags=flags)
    torch.cuda.synchronize()
    return host(yd)


def _oracle(cfg, x, w, attn_only=False):
    return swin.swin_block(x, w, cfg["height"], cfg["width"], cfg["heads"], cfg["window"],
                           cfg["shift"], EPS, return_attn_only=attn_only)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("geo", [(14, 14, 7, 3), (56, 56, 7, 3), (12, 8, 4, 2), (7, 7, 7, 0)])
def test_partition_layernorm(dtype, geo):
    Hs, Ws, M, s = geo
    rng = np.random.default_rng(Hs + M)
    B, C = 2, 96
    x = ti.to_storage(rng.standard_normal((B, Hs * Ws, C)) * 2, dtype)
    g = 1 + rng.standard_normal(C) * 0.1
    b = rng.standard_normal(C) * 0.1
    y = torch.full((B * Hs * Ws, C), float("nan"), dtype=TORCH_DT[dtype], device="cuda")
    tel.tel_window_partition_layernorm(dev(x, dtype), y, dev_f32(g), dev_f32(b), B, Hs, Ws, M, s, EPS)
    torch.cuda.synchronize()
    z = enc.layer_norm(x, g.astype(np.float32), b.astype(np.float32), EPS).reshape(B, Hs, Ws, C)
    ref = swin.window_partition(swin.cyclic_shift(z, s) if s else z, M).reshape(-1, C)
    assert_close(host(y), ref, dtype, f"partition LN {geo}")


SMALL = [
    dict(batch=2, height=14, width=14, channels=64, heads=2, window=7, shift=3, mlp=128),
    dict(batch=1, height=14, width=14, channels=64, heads=2, window=7, shift=0, mlp=128),
    dict(batch=2, height=8, width=12, channels=32, heads=2, window=4, shift=2, mlp=64),
    dict(batch=1, height=8, width=8, channels=64, heads=1, window=8, shift=0, mlp=128),   # one window
    dict(batch=2, height=14, width=7, channels=96, heads=6, window=7, shift=3, mlp=96),   # head_dim 16
]


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("shape", SMALL)
def test_block_small(dtype, shape):
    cfg = dict(shape, dtype=dtype, seed=shape["height"] + shape["window"] + shape["shift"])
    x = ti.swin_input(cfg)
    w = ti.swin_block_weights(cfg, variant=True)
    a = gpu_swin(cfg, x, w, flags=tel.TEL_SWIN_ATTN_ONLY)
    assert_close(a, _oracle(cfg, x, w, attn_only=True), dtype, f"attention half {shape}")
    y = gpu_swin(cfg, x, w)
    assert_close(y, _oracle(cfg, x, w), dtype, f"block {shape}")


@pytest.mark.parametrize("variant", [False, True])
def test_swin_t_stage1_sampled_images(variant):
    """Swin-T stage-1 block (64 images, 56x56, C 96, 3 heads, window 7, shift 3, MLP 384)
    on the GPU; the oracle computes a sample of whole images."""
    cfg = ti.SWIN_CONFIGS["swin_t_stage1"]
    x = ti.swin_input(cfg)
    w = ti.swin_block_weights(cfg, variant=variant)
    y = gpu_swin(cfg, x, w).reshape(cfg["batch"], -1, cfg["channels"])
    pick = [0, 13, 63]
    sub = dict(cfg, batch=len(pick))
    ref = _oracle(sub, x[pick], w)
    ma, rel = errors(y[pick], ref)
    print(f"swin_t_stage1 images {pick}: max_abs={ma:.3e} rel_frob={rel:.3e}")
    assert_close(y[pick], ref, "f16", "swin_t_stage1 block")


@pytest.mark.parametrize("shape", [SMALL[0], dict(batch=2, height=14, width=14, channels=96,
                                                   heads=3, window=7, shift=3, mlp=384)])
def test_one_stage_flags_compose_to_the_block(shape):
    """TEL_SWIN_ONE_STAGE(k) for k = 0..4 in order, on a fresh workspace, gives the whole
    block's output bit for bit (the per-kernel timings of the benchmark run the stages this
    way); and the stage that writes y, re-run on the workspace a whole block left behind,
    reproduces it."""
    cfg = dict(shape, dtype="f16", seed=7)
    x = ti.swin_input(cfg)
    w = ti.swin_block_weights(cfg, variant=True)
    desc = tel.make_swin_desc(cfg["batch"], cfg["height"], cfg["width"], cfg["channels"],
                              cfg["heads"], cfg["window"], cfg["shift"], cfg["mlp"], torch.float16,
                              EPS)
    packed = tel.alloc_bytes(tel.tel_swin_packed_size(desc))
    tel.tel_swin_prepare(desc, {k: dev(v, "f16") for k, v in w.items()}, packed)
    xd = dev(x, "f16")
    y_full = torch.full_like(xd, float("nan"))
    ws = tel.alloc_bytes(tel.tel_swin_workspace_size(desc))
    tel.tel_window_attention_forward(desc, packed, xd, y_full, ws)
    y_st = torch.full_like(xd, float("nan"))
    ws2 = tel.alloc_bytes(tel.tel_swin_workspace_size(desc))
    ws2.fill_(0xFF)
    for k in range(5):
        tel.tel_window_attention_forward(desc, packed, xd, y_st, ws2, flags=tel.TEL_SWIN_ONE_STAGE(k))
    # the stage that writes y: fc2 + residual, or the fused MLP half (stage 4 then empty)
    last = 3 if tel.tel_swin_fused_stages(desc) & tel.TEL_SWIN_FUSED_MLP else 4
    y_re = torch.full_like(xd, float("nan"))
    tel.tel_window_attention_forward(desc, packed, xd, y_re, ws,
                                     flags=tel.TEL_SWIN_ONE_STAGE(last))
    torch.cuda.synchronize()
    assert torch.equal(y_st.view(torch.int16), y_full.view(torch.int16))
    assert torch.equal(y_re.view(torch.int16), y_full.view(torch.int16))
    assert torch.isfinite(y_full.float()).all()
