"""tel_encoder_forward's weight read-ahead (extra workgroups of the reduce-LayerNorm kernels
reading the next GEMMs' weights): on a stack deep enough to use it (8 BERT-large layers,
201 MB of packed weights, one 128-token sequence) the output is bit-identical with the
read-ahead on and off, over repeated calls with other GPU work and synchronisations between
them, and through the graph cache; and the stack with it matches the oracle."""
import numpy as np
import pytest
import torch

import tel_inputs as ti
from oracle import encoder as enc
from tests.gpu_helpers import TORCH_DT, assert_close, dev, host, prepare_layers

pytestmark = pytest.mark.gpu

tel = pytest.importorskip("transformer_encoder_remove_amd")

LAYERS = 8


@pytest.fixture
def switches():
    pf, gr = tel.tel_weight_prefetch(-1), tel.tel_graph_cache(-1)
    yield
    tel.tel_weight_prefetch(pf)
    tel.tel_graph_cache(gr)


def _stack(layers, dtype="f16"):
    cfg = dict(ti.ENCODER_CONFIGS["bert_large_latency"], dtype=dtype, layers=layers)
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, i, variant=True) for i in range(layers)]
    desc = tel.make_encoder_desc(cfg["hidden"], cfg["heads"], cfg["ffn"], TORCH_DT[dtype],
                                 ti.LN_EPS)
    packed = prepare_layers(tel, desc, ws, dtype)
    B, S, H = x.shape
    xd = dev(x, dtype)
    yd = torch.empty_like(xd)
    lens_d = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    wsb = tel.alloc_bytes(tel.tel_encoder_forward_workspace_size(desc, B, S))
    T, max_len = int(np.sum(lens)), int(np.max(lens))

    def run():
        yd.fill_(float("nan"))
        tel.tel_encoder_forward(desc, packed, xd, yd, lens_d, T, max_len, wsb)
        torch.cuda.synchronize()
        return yd.clone()

    return cfg, desc, lens, x, ws, run


def test_stack_uses_the_prefetch():
    """The stack under test meets the library's condition for the read-ahead: weights that
    cannot all stay in the 256 MB cache (>= 160 MiB) and dominate what a layer reads
    (packed size > 8 x the activation bytes)."""
    cfg, desc, lens, x, _, _ = _stack(1)
    packed = tel.tel_encoder_packed_size(desc)
    act = int(np.sum(lens)) * cfg["hidden"] * 2
    assert LAYERS * packed >= 160 << 20 and act * 8 < packed


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefetch_on_off_bit_identical(switches, dtype):
    _, _, _, _, _, run = _stack(LAYERS, dtype)
    tel.tel_graph_cache(0)
    tel.tel_weight_prefetch(0)
    ref = run()
    assert torch.isfinite(ref.float()).all()
    tel.tel_weight_prefetch(1)
    for i in range(3):
        y = run()
        torch.randn(1 << 20, device="cuda").sum().item()   # unrelated work in between
        assert torch.equal(y, ref), f"call {i}: the read-ahead changed the output"
    tel.tel_graph_cache(1)
    for i in range(2):
        assert torch.equal(run(), ref), f"graph replay {i}"


def test_prefetch_stack_vs_oracle(switches):
    """The 8-layer stack with the read-ahead on against the oracle's stack, at the fp16
    tolerance (fp16 storage between layers, as in the 12-layer BERT-base test)."""
    tel.tel_graph_cache(0)
    tel.tel_weight_prefetch(1)
    cfg, _, lens, x, ws, run = _stack(LAYERS)
    y = host(run())
    ref = enc.encoder_forward(x, lens, ws, cfg["heads"], ti.LN_EPS)
    assert_close(y, ref, "f16", f"bert_large_latency {LAYERS} layers, read-ahead on")
