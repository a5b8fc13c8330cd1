"""GPU parity of the int8 layer with dynamic activation scales (tel_encoder_desc.
dynamic_scales: each int8 GEMM's activation scale from its fp16 input's max-abs over the
batch, reduced on the device) against the Q-oracle's dynamic layer.

A dynamic scale is a float decision over a whole tensor: when the GPU's fp16 maximum and the
oracle's float64 one differ by a rounding step, every code near a rounding boundary moves
with it. So, as for every float that decides integers here, both sides take the same
decision: the GPU's four maxima (left in the first 16 bytes of the layer workspace) are
checked against the oracle's own, to fp16 rounding, and then fed to the oracle. Stacks are
gated layer by layer on the GPU's own layer input; the whole stack equals those layers."""
import numpy as np
import pytest
import torch

import tel_inputs as ti
from oracle import encoder as enc
from oracle import int8 as q8
from tests.gpu_helpers import assert_close, dev, host, prepare_layers

pytestmark = pytest.mark.gpu

tel = pytest.importorskip("transformer_encoder_remove_amd")
EPS = ti.LN_EPS


def _desc(cfg):
    return tel.make_encoder_desc(cfg["hidden"], cfg["heads"], cfg["ffn"], torch.float16, EPS,
                                 int8_gemm=1, dynamic_scales=True)


def _layer(desc, packed, xp16, cu, max_len):
    """One dynamic int8 layer on packed tokens; returns (y, the four maxima it used)."""
    T = xp16.shape[0]
    xd = dev(xp16, "f16")
    yd = torch.full_like(xd, float("nan"))
    ws = tel.alloc_bytes(tel.tel_encoder_workspace_size(desc, T))
    tel.tel_encoder_layer_forward(desc, packed, xd, yd, torch.from_numpy(cu.astype(np.int32)).cuda(),
                                  T, max_len, ws)
    torch.cuda.synchronize()
    return host(yd), ws[:16].view(torch.float32).cpu().numpy().astype(np.float64)


def _check_layer(cfg, w, xp16, cu, max_len, what):
    desc = _desc(cfg)
    packed = prepare_layers(tel, desc, [w], "f16")[0]
    y, amax_gpu = _layer(desc, packed, xp16, cu, max_len)
    trace = []
    q8.encoder_layer_int8(xp16.astype(np.float64), cu, w, cfg["heads"], EPS, None, dynamic=True,
                          dyn_trace=trace)
    own = np.array(trace)
    assert amax_gpu[0] == own[0]                              # the input itself: exact
    assert np.all(np.abs(amax_gpu - own) <= 2e-3 * own), (amax_gpu, own)
    ref = q8.encoder_layer_int8(xp16.astype(np.float64), cu, w, cfg["heads"], EPS, None,
                                dynamic=True, dyn_amax=list(amax_gpu))
    ma, rel = assert_close(y, ref, "f16", what)
    print(f"{what}: max_abs={ma:.3e} rel_frob={rel:.3e}; maxima gpu {amax_gpu} oracle {own}")
    return y


@pytest.mark.parametrize("variant", [False, True])
def test_dynamic_int8_bert_base_layer_full_batch(variant):
    cfg = ti.ENCODER_CONFIGS["bert_base_int8_dyn"]
    lens, x = ti.encoder_input(cfg)
    w = ti.encoder_layer_weights(cfg, 0, variant)
    cu, _ = enc.offsets(lens, cfg["max_seq"])
    xp = enc.remove_padding(x, lens)
    _check_layer(cfg, w, xp, cu, int(lens.max()), f"dynamic int8 layer variant={variant}")


@pytest.mark.parametrize("scale", [1.0, 16.0])
def test_dynamic_int8_stack_layer_by_layer(scale):
    """Three layers; the input scaled by 16 as well (static scales calibrated on the
    unscaled batch would clip it; the dynamic ones follow it). Each layer is gated on its
    GPU input; tel_encoder_forward over the three layers equals the layers one by one."""
    cfg = ti.custom_encoder_config(4, 50, [50, 1, 23, 40], 128, 2, 256, dtype="f16", seed=29,
                                   layers=3)
    lens, x = ti.encoder_input(cfg)
    x = ti.to_storage(x.astype(np.float64) * scale, "f16")
    ws = [ti.encoder_layer_weights(cfg, i, variant=True) for i in range(3)]
    cu, _ = enc.offsets(lens, cfg["max_seq"])
    cur = enc.remove_padding(x, lens)
    for i, w in enumerate(ws):
        cur = _check_layer(cfg, w, cur, cu, int(lens.max()), f"dynamic layer {i} x{scale}")
        cur = cur.astype(np.float16)
    desc = _desc(cfg)
    packed = prepare_layers(tel, desc, ws, "f16")
    B, S, _ = x.shape
    xd = dev(x, "f16")
    yd = torch.full_like(xd, float("nan"))
    wsb = tel.alloc_bytes(tel.tel_encoder_forward_workspace_size(desc, B, S))
    tel.tel_encoder_forward(desc, packed, xd, yd, torch.from_numpy(lens.astype(np.int32)).cuda(),
                            int(lens.sum()), int(lens.max()), wsb)
    torch.cuda.synchronize()
    assert np.array_equal(enc.remove_padding(host(yd), lens), cur.astype(np.float64))
