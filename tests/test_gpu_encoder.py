"""GPU parity of the whole path (offsets, padding removal, encoder layers, rebuild) through
tel_encoder_forward, against the float64 oracle, on the seeded workloads."""
import numpy as np
import pytest

import tel_inputs as ti
from oracle import encoder as enc
from tests.gpu_helpers import assert_close, errors, gpu_encoder_forward

pytestmark = pytest.mark.gpu

tel = pytest.importorskip("transformer_encoder_remove_amd")
EPS = ti.LN_EPS


def _oracle(cfg, lens, x, ws):
    return enc.encoder_forward(x, lens, ws, cfg["heads"], EPS)


@pytest.mark.parametrize("variant", [False, True])
def test_tiny_fp32(variant):
    cfg = ti.ENCODER_CONFIGS["tiny"]
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, 0, variant)]
    y = gpu_encoder_forward(tel, cfg, lens, x, ws)
    assert_close(y, _oracle(cfg, lens, x, ws), "f32", "tiny fp32")
    assert not y[0, lens[0]:].any()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("variant", [False, True])
def test_bert_base_one_layer_full_batch(dtype, variant):
    """One BERT-base layer on the full seeded batch (B 32, S 128, lengths U{32..128})."""
    cfg = dict(ti.ENCODER_CONFIGS["bert_base"], dtype=dtype)
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, 0, variant)]
    y = gpu_encoder_forward(tel, cfg, lens, x, ws)
    ref = _oracle(cfg, lens, x, ws)
    assert_close(enc.remove_padding(y, lens), enc.remove_padding(ref, lens), dtype, "bert_base L1")
    for b in range(len(lens)):
        assert not y[b, lens[b]:].any()


@pytest.mark.parametrize("shape", [
    dict(B=3, S=9, lens=[9, 1, 0], H=64, heads=4, F=256),         # empty and single-token sequences
    dict(B=1, S=200, lens=[200], H=256, heads=2, F=512),          # head_dim 128, one sequence
    dict(B=5, S=70, lens=[70, 33, 64, 65, 2], H=128, heads=8, F=384),   # head_dim 16
    dict(B=2, S=40, lens=[40, 17], H=96, heads=3, F=384),         # head_dim 32, H 96
])
@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_edge_shapes(shape, dtype):
    cfg = ti.custom_encoder_config(shape["B"], shape["S"], shape["lens"], shape["H"],
                                   shape["heads"], shape["F"], dtype=dtype, seed=shape["S"], layers=2)
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, i, variant=True) for i in range(2)]
    y = gpu_encoder_forward(tel, cfg, lens, x, ws)
    assert_close(y, _oracle(cfg, lens, x, ws), dtype, f"edge {shape}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bert_base_512_token_sequence(dtype):
    """BERT's longest sequence (512 tokens, eight 64-key blocks and four 128-query
    workgroups per head) beside a 300-token and a one-token sequence, at BERT-base width;
    one layer against the oracle, pads exactly 0."""
    lens = [512, 300, 1]
    cfg = ti.custom_encoder_config(len(lens), 512, lens, 768, 12, 3072, dtype=dtype, seed=512,
                                   layers=1)
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, 0, variant=True)]
    y = gpu_encoder_forward(tel, cfg, lens, x, ws)
    ref = _oracle(cfg, lens, x, ws)
    assert_close(enc.remove_padding(y, lens), enc.remove_padding(ref, lens), dtype, "512 tokens")
    for b in range(len(lens)):
        assert not y[b, lens[b]:].any()


def test_fp16_ffn2_k2048_ragged_two_layers():
    """H 768, F 2048 (FFN2 at K 2048): two layers with non-trivial LayerNorm parameters over
    1434 ragged tokens (empty and one-token sequences, not a multiple of any tile)."""
    lens = [128, 97, 33, 120, 1, 64, 65, 128, 77, 100, 90, 127, 31, 80, 99, 91, 98, 2, 0, 3]
    cfg = ti.custom_encoder_config(len(lens), 128, lens, 768, 12, 2048, dtype="f16", seed=77,
                                   layers=2)
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, i, variant=True) for i in range(2)]
    y = gpu_encoder_forward(tel, cfg, lens, x, ws)
    assert_close(enc.remove_padding(y, lens), enc.remove_padding(_oracle(cfg, lens, x, ws), lens),
                 "f16", "F 2048, 2 layers")


def test_bert_base_12_layers_sampled_sequences():
    """The benchmarked call: 12 BERT-base layers on the full batch. The oracle computes a
    sample of sequences (independent of one another) through the same 12 layers."""
    cfg = ti.ENCODER_CONFIGS["bert_base"]
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, i) for i in range(cfg["layers"])]
    y = gpu_encoder_forward(tel, cfg, lens, x, ws)
    pick = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 7, 31})
    ref = _oracle(cfg, lens[pick], x[pick], ws)
    got = y[pick]
    ma, rel = errors(enc.remove_padding(got, lens[pick]), enc.remove_padding(ref, lens[pick]))
    print(f"bert_base 12 layers, sequences {pick}: max_abs={ma:.3e} rel_frob={rel:.3e}")
    assert_close(enc.remove_padding(got, lens[pick]), enc.remove_padding(ref, lens[pick]), "f16",
                 "bert_base 12 layers")


def test_bert_base_bf16_12_layers_sampled():
    """12 bf16 BERT-base layers on the full batch, sampled sequences. Per layer: the output
    of the GPU's first k+1 layers against the oracle's layer k applied to the GPU's own
    output of the first k layers, within the fp16/bf16 bound. End to end, against the
    float64 oracle of all 12 layers: each layer's output is stored as bf16 (unit roundoff
    u = 2^-8) before the next one reads it, and these independent roundings add up like a
    random walk, so the bound there is sqrt(12) times the per-layer one (max-abs 6.9e-2,
    relative Frobenius 1.7e-2); the measured error is printed."""
    cfg = dict(ti.ENCODER_CONFIGS["bert_base"], dtype="bf16")
    lens, x = ti.encoder_input(cfg)
    nl = cfg["layers"]
    ws = [ti.encoder_layer_weights(cfg, i) for i in range(nl)]
    pick = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 7, 31})
    lp = lens[pick]
    prev = x[pick]
    for k in range(nl):
        y = gpu_encoder_forward(tel, dict(cfg, layers=k + 1), lens, x, ws[:k + 1])[pick]
        ref = enc.encoder_forward(prev, lp, [ws[k]], cfg["heads"], EPS)
        got, want = enc.remove_padding(y, lp), enc.remove_padding(ref, lp)
        assert_close(got, want, "bf16", f"bf16 layer {k} on the GPU's own input")
        prev = y
    ref = enc.encoder_forward(x[pick], lp, ws, cfg["heads"], EPS)
    ma, rel = errors(enc.remove_padding(prev, lp), enc.remove_padding(ref, lp))
    print(f"bf16 12 layers end to end vs float64: max_abs={ma:.3e} rel_frob={rel:.3e}")
    root = np.sqrt(nl)
    assert ma <= 2e-2 * root and rel <= 5e-3 * root, (ma, rel)


def test_bert_large_tput_one_layer_sampled():
    """BERT-large throughput batch (B 64, S 384, lengths U{64..384}), one layer on the GPU for
    the whole batch; the oracle checks a sample of sequences."""
    cfg = ti.ENCODER_CONFIGS["bert_large_tput"]
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, 0, variant=True)]
    y = gpu_encoder_forward(tel, cfg, lens, x, ws)
    pick = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 5, 40})
    ref = _oracle(cfg, lens[pick], x[pick], ws)
    assert_close(enc.remove_padding(y[pick], lens[pick]), enc.remove_padding(ref, lens[pick]),
                 "f16", "bert_large_tput L1")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bert_large_latency_split_layers(dtype):
    """BERT-large latency batch (one sequence of 128 tokens): the output projection and FFN2
    run split over k (partial sums finished by the reduce-LayerNorm kernel). Two layers in
    fp16; one in bf16, whose inter-layer storage rounding alone (8 significant bits at
    |y| ~ 4.5) would take most of the 2e-2 budget in a second layer."""
    nl = 2 if dtype == "f16" else 1
    cfg = dict(ti.ENCODER_CONFIGS["bert_large_latency"], dtype=dtype, layers=nl)
    dt = tel.TEL_F16 if dtype == "f16" else tel.TEL_BF16
    assert tel.tel_gemm_partial_plan(dt, 128, 1024, 1024)[1] > 1
    assert tel.tel_gemm_partial_plan(dt, 128, 1024, 4096)[1] > 1
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, i, variant=True) for i in range(nl)]
    y = gpu_encoder_forward(tel, cfg, lens, x, ws)
    assert_close(y, _oracle(cfg, lens, x, ws), dtype, f"bert_large_latency {nl} layers")


@pytest.mark.parametrize("int8", [False, True])
def test_all_sequences_empty(int8):
    """Every length 0 (T = 0): the stack runs no layer work and the padded output is all
    zeros."""
    cfg = dict(ti.ENCODER_CONFIGS["bert_base"], layers=2)
    lens = np.zeros(4, np.int64)
    x = np.ones((4, 16, cfg["hidden"]), np.float32)
    ws = [ti.encoder_layer_weights(cfg, i) for i in range(2)]
    y = gpu_encoder_forward(tel, dict(cfg, batch=4, max_seq=16), lens, x, ws, int8=int8,
                            act_amax=[[1.0] * 4] * 2)
    assert y.shape == x.shape and not y.any()


def test_deterministic_repeat():
    """Two runs give bitwise-identical outputs (no races in LDS staging)."""
    cfg = dict(ti.ENCODER_CONFIGS["bert_base"], batch=8)
    lens, x = ti.encoder_input(cfg)
    lens, x = lens[:8], x[:8]
    ws = [ti.encoder_layer_weights(cfg, 0, variant=True)]
    y1 = gpu_encoder_forward(tel, cfg, lens, x, ws)
    y2 = gpu_encoder_forward(tel, cfg, lens, x, ws)
    assert np.array_equal(y1, y2)
