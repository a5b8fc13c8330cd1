"""GPU test of tel_encoder_layer_forward_noalloc (the layer forward whose workspace is the
library's own scratch array): its output equals tel_encoder_layer_forward's, bit for bit,
on two calls in a row, the second with fewer tokens, and a size past the scratch limit is
rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

import tel_inputs as ti
from oracle import encoder as enc
from tests.gpu_helpers import TORCH_DT, assert_close, dev, host, prepare_layers

pytestmark = pytest.mark.gpu

tel = pytest.importorskip("transformer_encoder_remove_amd")
EPS = ti.LN_EPS


def _packed_inputs(cfg, lens, x_pad):
    cu, _ = enc.offsets(lens, x_pad.shape[1])
    xp = enc.remove_padding(x_pad.astype(np.float64), lens)
    return cu, xp


def _run_both(desc, packed, dt, xp, cu, max_len):
    T, H = xp.shape
    x = dev(xp, dt)
    cu_d = torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    y_ref = torch.full_like(x, float("nan"))
    ws = tel.alloc_bytes(tel.tel_encoder_workspace_size(desc, T))
    tel.tel_encoder_layer_forward(desc, packed, x, y_ref, cu_d, T, max_len, ws)
    y = torch.full_like(x, float("nan"))
    tel.tel_encoder_layer_forward_noalloc(desc, packed, x, y, cu_d, T, max_len)
    torch.cuda.synchronize()
    return y, y_ref


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_noalloc_layer_equals_layer_forward_two_calls(dt):
    cfg = dict(ti.ENCODER_CONFIGS["bert_base"], dtype=dt)
    w = ti.encoder_layer_weights(cfg, 0, variant=True)
    desc = tel.make_encoder_desc(cfg["hidden"], cfg["heads"], cfg["ffn"], TORCH_DT[dt], EPS)
    packed = prepare_layers(tel, desc, [w], dt)[0]
    # first call: the full BERT-base batch (T = 2557)
    lens, x_pad = ti.encoder_input(cfg)
    cu, xp = _packed_inputs(cfg, lens, x_pad)
    print(f"noalloc {dt}: call 1, T={xp.shape[0]}", flush=True)
    y, y_ref = _run_both(desc, packed, dt, xp, cu, int(lens.max()))
    assert torch.equal(y, y_ref), "call 1 differs from tel_encoder_layer_forward"
    ref = enc.encoder_layer(ti.to_storage(xp, dt), cu, w, cfg["heads"], EPS)
    assert_close(host(y), ref, dt, "noalloc call 1 vs oracle")
    # second call: a smaller ragged batch on the same scratch (the first call's contents stay)
    small = ti.custom_encoder_config(9, 100, [100, 1, 37, 64, 99, 0, 65, 80, 17], cfg["hidden"],
                                     cfg["heads"], cfg["ffn"], dtype=dt, seed=31)
    lens2, x_pad2 = ti.encoder_input(small)
    cu2, xp2 = _packed_inputs(small, lens2, x_pad2)
    print(f"noalloc {dt}: call 2, T={xp2.shape[0]}", flush=True)
    y2, y2_ref = _run_both(desc, packed, dt, xp2, cu2, int(lens2.max()))
    assert torch.equal(y2, y2_ref), "call 2 differs from tel_encoder_layer_forward"
    ref2 = enc.encoder_layer(ti.to_storage(xp2, dt), cu2, w, cfg["heads"], EPS)
    assert_close(host(y2), ref2, dt, "noalloc call 2 vs oracle")


def test_noalloc_rejects_sizes_past_the_scratch():
    cfg = ti.ENCODER_CONFIGS["bert_base"]
    desc = tel.make_encoder_desc(cfg["hidden"], cfg["heads"], cfg["ffn"], torch.float16, EPS)
    T = 1
    while tel.tel_encoder_workspace_size(desc, T) <= tel.TEL_NOALLOC_SCRATCH_BYTES:
        T *= 2
    x = torch.zeros((T, cfg["hidden"]), dtype=torch.float16, device="cuda")
    y = torch.empty_like(x)
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    packed = tel.alloc_bytes(tel.tel_encoder_packed_size(desc))
    with pytest.raises(tel.TelError) as e:
        tel.tel_encoder_layer_forward_noalloc(desc, packed, x, y, cu, T, T)
    assert e.value.status == tel.TEL_EWORKSPACE
