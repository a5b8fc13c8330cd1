"""TEL_DEBUG=1: tel_encoder_forward checks the caller's obligations on the lengths on the
device (every length in [0, max_seq], their sum = total_tokens, their maximum <= max_len)
before any kernel reads the padded batch, and refuses a batch that breaks one. The check
kernel reads only the lengths, so the bad cases below touch nothing out of bounds."""
import os

import numpy as np
import pytest
import torch

import tel_inputs as ti
from tests.gpu_helpers import TORCH_DT, dev, prepare_layers

pytestmark = pytest.mark.gpu

tel = pytest.importorskip("transformer_encoder_remove_amd")


@pytest.fixture
def debug_mode():
    old = os.environ.get("TEL_DEBUG")
    os.environ["TEL_DEBUG"] = "1"
    yield
    if old is None:
        del os.environ["TEL_DEBUG"]
    else:
        os.environ["TEL_DEBUG"] = old


def _setup():
    cfg = ti.custom_encoder_config(4, 16, [16, 3, 0, 9], 64, 4, 256, dtype="f16", seed=41)
    lens, x_pad = ti.encoder_input(cfg)
    w = ti.encoder_layer_weights(cfg, 0, variant=True)
    desc = tel.make_encoder_desc(64, 4, 256, TORCH_DT["f16"], ti.LN_EPS)
    packed = prepare_layers(tel, desc, [w], "f16")
    x = dev(x_pad, "f16")
    ws = tel.alloc_bytes(tel.tel_encoder_forward_workspace_size(desc, 4, 16))
    return lens, x, desc, packed, ws


def _run(desc, packed, x, lens, T, max_len, ws):
    y = torch.full_like(x, float("nan"))
    tel.tel_encoder_forward(desc, packed, x, y, torch.from_numpy(np.asarray(lens, np.int32)).cuda(),
                            T, max_len, ws)
    torch.cuda.synchronize()
    return y


def test_debug_check_passes_good_lengths(debug_mode):
    lens, x, desc, packed, ws = _setup()
    y_dbg = _run(desc, packed, x, lens, int(lens.sum()), int(lens.max()), ws)
    os.environ["TEL_DEBUG"] = "0"
    y = _run(desc, packed, x, lens, int(lens.sum()), int(lens.max()), ws)
    assert torch.equal(y, y_dbg)


@pytest.mark.parametrize("case", ["len_above_max_seq", "negative_len", "sum_mismatch",
                                  "max_len_too_small"])
def test_debug_check_refuses_bad_lengths(debug_mode, case):
    lens, x, desc, packed, ws = _setup()
    T, max_len = int(lens.sum()), int(lens.max())
    bad = lens.copy()
    if case == "len_above_max_seq":
        bad[1] = 17                                  # max_seq is 16
        T = int(bad.sum())
        max_len = 17
    elif case == "negative_len":
        bad[2] = -1
        T = int(bad.sum())
    elif case == "sum_mismatch":
        T = T - 1
    else:
        max_len = max_len - 1
    print(f"debug check case {case}: lens {bad.tolist()} T {T} max_len {max_len}", flush=True)
    if case == "len_above_max_seq":
        # the host already refuses max_len > max_seq; give it a max_len the host accepts
        max_len = 16
    y = torch.full_like(x, float("nan"))
    with pytest.raises(tel.TelError) as e:
        tel.tel_encoder_forward(desc, packed, x, y, torch.from_numpy(bad).cuda(), T, max_len, ws)
    assert e.value.status == tel.TEL_EINVAL
    torch.cuda.synchronize()
    assert torch.isnan(y).all()                      # nothing after the check ran
