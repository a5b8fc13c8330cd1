"""tel_encoder_forward's graph cache: replays of the recorded forward equal the eager
forward bitwise, across several replays with unrelated eager GPU work and synchronisations
in between, and read buffer contents (inputs, lengths) at replay time."""
import numpy as np
import pytest
import torch

import tel_inputs as ti
from tests.gpu_helpers import TORCH_DT, dev, prepare_layers

pytestmark = pytest.mark.gpu

tel = pytest.importorskip("transformer_encoder_remove_amd")


@pytest.fixture
def cache_state():
    prev = tel.tel_graph_cache(-1)
    yield
    tel.tel_graph_cache(prev)


def _setup(name, dtype, layers, int8=False):
    cfg = dict(ti.ENCODER_CONFIGS[name], dtype=dtype, layers=layers)
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, i, variant=True) for i in range(layers)]
    desc = tel.make_encoder_desc(cfg["hidden"], cfg["heads"], cfg["ffn"], TORCH_DT[dtype],
                                 ti.LN_EPS, int8_gemm=int8)
    amax = [[3.0, 2.5, 4.0, 1.5]] * layers if int8 else None
    packed = prepare_layers(tel, desc, ws, dtype, amax)
    B, S, _ = x.shape
    xd = dev(x, dtype)
    yd = torch.empty_like(xd)
    lens_d = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    wsb = tel.alloc_bytes(tel.tel_encoder_forward_workspace_size(desc, B, S))
    T, max_len = int(np.sum(lens)), int(np.max(lens))
    run = lambda: tel.tel_encoder_forward(desc, packed, xd, yd, lens_d, T, max_len, wsb)
    return cfg, lens, x, xd, yd, lens_d, run


@pytest.mark.parametrize("name,dtype,layers,int8", [("bert_base", "f16", 2, False),
                                                      ("bert_large_latency", "f16", 2, False),
                                                      ("bert_base_int8", "f16", 3, True)])
def test_graph_replays_equal_eager(cache_state, name, dtype, layers, int8):
    cfg, lens, x, xd, yd, lens_d, run = _setup(name, dtype, layers, int8)
    tel.tel_graph_cache(0)
    yd.fill_(float("nan"))
    run()
    torch.cuda.synchronize()
    ref = yd.clone()
    tel.tel_graph_cache(1)
    for i in range(4):
        yd.fill_(float("nan"))
        run()
        # unrelated eager work between replays
        junk = torch.randn(1 << 20, device="cuda")
        _ = (junk * 2).sum().item()
        torch.cuda.synchronize()
        assert torch.equal(yd, ref), f"replay {i}"


def test_graph_reads_buffers_at_replay(cache_state):
    """Same buffers and sizes (same graph), new contents: new inputs, and the lengths
    permuted (same total and maximum), give the eager results of the new contents."""
    cfg, lens, x, xd, yd, lens_d, run = _setup("bert_base", "f16", 2)
    tel.tel_graph_cache(1)
    run()                                       # records the graph
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    x2 = ti.to_storage(rng.standard_normal(x.shape), "f16")
    perm = np.asarray(lens)[::-1].copy()
    for new_x, new_lens in ((x2, lens), (x2, perm)):
        xd.copy_(dev(new_x, "f16"))
        lens_d.copy_(torch.from_numpy(np.asarray(new_lens, np.int32)))
        tel.tel_graph_cache(0)
        yd.fill_(float("nan"))
        run()
        torch.cuda.synchronize()
        ref = yd.clone()
        tel.tel_graph_cache(1)
        yd.fill_(float("nan"))
        run()
        torch.cuda.synchronize()
        assert torch.equal(yd, ref)


@pytest.mark.parametrize("name,layers,int8", [("bert_base", 2, False), ("bert_large_latency", 2, False),
                                              ("bert_base_int8_attn", 1, 2)])
def test_graph_replays_match_oracle(cache_state, name, layers, int8):
    """Graph replays of the whole forward against the oracle (not only against eager): every
    replay, with unrelated eager work and refilled outputs between replays, is within the
    fp16 tolerance of the oracle's stack (fp16 stored between layers, as the stack stores).
    The int8 case is one layer: int8 codes that flip at a rounding boundary compound from
    layer to layer, so int8 parity is gated per layer (replay = eager bit for bit above)."""
    from oracle import encoder as enc
    from oracle import int8 as q8
    cfg = dict(ti.ENCODER_CONFIGS[name], layers=layers)
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, i, variant=True) for i in range(layers)]
    cu, _ = enc.offsets(lens, cfg["max_seq"])
    xp = enc.remove_padding(x.astype(np.float64), lens)
    amax = attn = None
    if int8:
        amax, attn, h = [], [], xp
        for w in ws:
            amax.append(q8.calibrate(h, cu, w, cfg["heads"], ti.LN_EPS))
            attn.append(q8.calibrate_attention(h, cu, w, cfg["heads"], ti.LN_EPS))
            h = enc.encoder_layer(h, cu, w, cfg["heads"], ti.LN_EPS)
        ref = q8.encoder_stack_int8(xp, cu, ws, amax, cfg["heads"], ti.LN_EPS, attn_amaxes=attn)
    else:
        ref = enc.encoder_stack(xp, cu, ws, cfg["heads"], ti.LN_EPS, round_to=np.float16)
    desc = tel.make_encoder_desc(cfg["hidden"], cfg["heads"], cfg["ffn"], torch.float16, ti.LN_EPS,
                                 int8_gemm=int8)
    packed = prepare_layers(tel, desc, ws, "f16", amax, attn)
    B, S, _ = x.shape
    xd = dev(x, "f16")
    yd = torch.empty_like(xd)
    lens_d = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    wsb = tel.alloc_bytes(tel.tel_encoder_forward_workspace_size(desc, B, S))
    T, max_len = int(np.sum(lens)), int(np.max(lens))
    tel.tel_graph_cache(1)
    for i in range(3):
        yd.fill_(float("nan"))
        tel.tel_encoder_forward(desc, packed, xd, yd, lens_d, T, max_len, wsb)
        junk = torch.randn(1 << 20, device="cuda")
        _ = (junk * 2).sum().item()
        torch.cuda.synchronize()
        got = enc.remove_padding(yd.float().cpu().numpy().astype(np.float64), lens)
        from tests.gpu_helpers import assert_close
        ma, rel = assert_close(got, ref, "f16", f"graph replay {i} {name}")
        print(f"graph replay {i} {name}: max_abs={ma:.3e} rel_frob={rel:.3e}")
        # pad rows of the rebuilt output are exactly zero
        for b in range(B):
            assert not yd[b, int(lens[b]):].any()


def test_graph_key_tells_static_from_dynamic_scales(cache_state):
    """Two descriptors that differ only in dynamic_scales, on the same packed weights and
    buffers, record two graphs: each replay equals its own eager forward."""
    cfg = dict(ti.ENCODER_CONFIGS["bert_base_int8"], layers=1)
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, 0, variant=True)]
    mk = lambda dyn: tel.make_encoder_desc(cfg["hidden"], cfg["heads"], cfg["ffn"],
                                           torch.float16, ti.LN_EPS, int8_gemm=True,
                                           dynamic_scales=dyn)
    d_static, d_dyn = mk(False), mk(True)
    packed = prepare_layers(tel, d_static, ws, "f16", [[3.0, 2.5, 4.0, 1.5]])
    B, S, _ = x.shape
    xd = dev(x, "f16")
    yd = torch.empty_like(xd)
    lens_d = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    wsb = tel.alloc_bytes(max(tel.tel_encoder_forward_workspace_size(d, B, S)
                              for d in (d_static, d_dyn)))
    T, max_len = int(np.sum(lens)), int(np.max(lens))
    run = lambda d: tel.tel_encoder_forward(d, packed, xd, yd, lens_d, T, max_len, wsb)
    tel.tel_graph_cache(0)
    refs = []
    for d in (d_static, d_dyn):
        yd.fill_(float("nan"))
        run(d)
        torch.cuda.synchronize()
        refs.append(yd.clone())
    assert not torch.equal(refs[0], refs[1])   # the two scale modes give different codes
    tel.tel_graph_cache(1)
    for i in range(3):
        for d, ref in zip((d_static, d_dyn), refs):
            yd.fill_(float("nan"))
            run(d)
            torch.cuda.synchronize()
            assert torch.equal(yd, ref), f"replay {i}, dynamic={d.dynamic_scales}"
