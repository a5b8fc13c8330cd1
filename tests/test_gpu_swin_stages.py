"""GPU parity of the downsampling between Swin stages (patch merging: 2 x 2 gather,
LayerNorm over 4C, 4C -> 2C) and of the stage-1 -> stage-2 pipeline against
oracle/swin.py. Each piece of the pipeline is gated against the oracle fed the GPU's own
input to that piece; the end-to-end error over all five pieces is reported."""
import numpy as np
import pytest
import torch

import tel_inputs as ti
from oracle import swin
from tests.gpu_helpers import (TORCH_DT, assert_close, dev, dev_f32, errors, host,
                               swin_block_gpu, swin_two_stages_gpu)

pytestmark = pytest.mark.gpu

tel = pytest.importorskip("transformer_encoder_remove_amd")
EPS = ti.LN_EPS


def gpu_merge(x, w, H, W, dt):
    B, L, C = x.shape
    y = torch.full((B, (H // 2) * (W // 2), 2 * C), float("nan"), dtype=TORCH_DT[dt], device="cuda")
    tel.tel_patch_merging(dev(x, dt), y, dev_f32(w["norm_g"]), dev_f32(w["norm_b"]),
                          dev(w["w_red"], dt), H, W, EPS)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 2, 2), (2, 4, 6), (1, 14, 10), (3, 56, 56), (64, 56, 56)])
def test_patch_merging_vs_oracle(dt, shape):
    """Ragged row counts (1, 12, 35 merged tokens), several persistent passes (3 images),
    and the whole Swin-T stage-1 output (64 images, 50,176 merged tokens)."""
    B, H, W = shape
    C = 96
    rng = np.random.default_rng(B * 1000 + H * W)
    x = ti.to_storage(rng.standard_normal((B, H * W, C)) * 2, dt)
    w = ti.patch_merge_weights(C, variant=True, seed=H + W, dtype=dt)
    print(f"patch merging {dt} B={B} {H}x{W}", flush=True)
    y = gpu_merge(x, w, H, W, dt)
    ref = swin.patch_merging(x, w, H, W, EPS)
    ma, rel = assert_close(y, ref, dt, f"patch merging {shape}")
    print(f"  max_abs={ma:.3e} rel_frob={rel:.3e}")


def test_patch_merging_validation():
    x = torch.zeros((1, 16, 96), dtype=torch.float16, device="cuda")
    y = torch.zeros((1, 4, 192), dtype=torch.float16, device="cuda")
    g = torch.ones(384, device="cuda")
    wr = torch.zeros((192, 384), dtype=torch.float16, device="cuda")
    with pytest.raises(tel.TelError) as e:                           # odd height
        tel.tel_patch_merging(x, y, g, g, wr, 3, 5, EPS)
    assert e.value.status == tel.TEL_EINVAL
    x64 = torch.zeros((1, 16, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(tel.TelError) as e:                           # channels other than 96
        tel.tel_patch_merging(x64, y, g, g, wr, 4, 4, EPS)
    assert e.value.status == tel.TEL_EUNSUPPORTED


@pytest.mark.parametrize("shift", [0, 3])
def test_stage2_block(shift):
    """A Swin-T stage-2 block (28 x 28, C 192, 6 heads, MLP 768) on two images."""
    cfg = dict(batch=2, height=28, width=28, channels=192, heads=6, window=7, shift=shift,
               mlp=768, dtype="f16", seed=50 + shift)
    x = ti.swin_input(cfg)
    w = ti.swin_block_weights(cfg, variant=True)
    desc, packed, ws = swin_block_gpu(tel, cfg, w)
    xd = dev(x, "f16")
    yd = torch.full_like(xd, float("nan"))
    tel.tel_window_attention_forward(desc, packed, xd, yd, ws)
    torch.cuda.synchronize()
    ref = swin.swin_block(x, w, 28, 28, 6, 7, shift, EPS)
    assert_close(host(yd), ref, "f16", f"stage-2 block shift {shift}")


def test_two_stages_pipeline_sampled_images():
    """Swin-T stages 1 and 2 with the merge between them on all 64 images; the oracle takes
    3 of the images through each piece from the GPU's own input to that piece (gated), and
    through the whole float64 pipeline (reported)."""
    cfg = ti.SWIN_STAGES["swin_t_stage12"]
    x = ti.swin_input(dict(cfg, channels=cfg["channels"]))
    s1, mw, s2 = ti.swin_stage_weights(cfg, variant=True)
    y, ins = swin_two_stages_gpu(tel, cfg, x, s1, mw, s2)
    pick = [0, 31, 63]
    H, W, M = cfg["height"], cfg["width"], cfg["window"]
    pieces = []
    for stage, blocks in ((0, s1), (1, s2)):
        f = 2 ** stage
        for w, s in zip(blocks, swin.stage_shifts(len(blocks), H // f, W // f, M)):
            pieces.append(("block", stage, s, w))
        if stage == 0:
            pieces.append(("merge", 0, 0, mw))
    outs = ins[1:] + [y]
    assert len(pieces) == len(ins) == 5
    for (kind, stage, s, w), xin, xout in zip(pieces, ins, outs):
        f = 2 ** stage
        xi = xin.reshape(cfg["batch"], -1, xin.shape[-1])[pick]
        if kind == "merge":
            ref = swin.patch_merging(xi, w, H, W, EPS)
        else:
            ref = swin.swin_block(xi, w, H // f, W // f, cfg["heads"][stage], M, s, EPS)
        got = xout.reshape(cfg["batch"], -1, xout.shape[-1])[pick]
        ma, rel = assert_close(got, ref, "f16", f"{kind} stage {stage + 1} shift {s}")
        print(f"{kind} stage {stage + 1} shift {s}: max_abs={ma:.3e} rel_frob={rel:.3e}", flush=True)
    ref_all = swin.swin_two_stages(x[pick], s1, mw, s2, H, W, cfg["heads"][0], cfg["heads"][1], M, EPS)
    ma, rel = errors(y.reshape(cfg["batch"], -1, y.shape[-1])[pick], ref_all)
    print(f"whole pipeline vs float64 oracle (reported): max_abs={ma:.3e} rel_frob={rel:.3e}")
    assert rel < 2e-2
