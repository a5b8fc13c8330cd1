"""Pins of oracle/int8.py: brute force on tiny inputs, rounding rules, exactness and
error bounds. CPU only."""
import numpy as np

import tel_inputs as ti
from oracle import encoder as enc
from oracle import int8 as q8
from tests import brute

EPS = ti.LN_EPS


def test_weight_quantization_rules():
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((9, 33)) * 0.02).astype(np.float16)
    w[3] = 0
    wq, s = q8.quantize_weight(w)
    assert wq.dtype == np.int8 and s.dtype == np.float32
    assert s[3] == 1.0 and not wq[3].any()
    for n in range(9):
        if n == 3:
            continue
        k = np.abs(w[n].astype(np.float32)).argmax()
        assert abs(int(wq[n, k])) == 127                          # the row's max maps to +-127
        err = np.abs(w[n].astype(np.float64) / np.float64(s[n]) - wq[n])
        assert err.max() <= 0.5 + 1e-5                             # rounding error <= half a step
    assert np.abs(wq.astype(int)).max() <= 127


def test_activation_quantization_ties_and_clamp():
    x = np.array([2.5, 3.5, -2.5, -3.5, 0.5, 1.5, 200.0, -200.0, 0.0], dtype=np.float16)
    q = q8.quantize_act(x, np.float32(1.0))
    assert q.tolist() == [2, 4, -2, -4, 0, 2, 127, -127, 0]        # half to even, clamp at 127


def test_activation_scale():
    s, inv = q8.act_scale(254.0)
    assert s == np.float32(2.0) and inv == np.float32(0.5)
    assert q8.act_scale(0.0) == (1.0, 1.0)


def test_int8_matmul_brute_force_and_bound():
    a, b = ti.int8_operands(5, 7, 40, seed=1)
    acc = q8.int8_matmul(a, b)
    for i in range(5):
        for j in range(7):
            assert acc[i, j] == sum(int(a[i, k]) * int(b[j, k]) for k in range(40))
    worst = q8.int8_matmul(np.full((1, 3072), -127, np.int8), np.full((1, 3072), -127, np.int8))
    assert worst[0, 0] == 3072 * 127 * 127 < 2 ** 31


def test_quantized_linear_is_exact_on_the_grid():
    """When x is an integer multiple of s_a and each weight row an integer multiple of its
    scale, quantise -> int GEMM -> dequantise reproduces x W^T + b."""
    rng = np.random.default_rng(2)
    qx = rng.integers(-127, 128, size=(4, 16))
    qw = rng.integers(-127, 128, size=(6, 16))
    qw[:, 0] = 127                                                # row max is exactly 127 codes
    s_a = np.float32(0.125)
    sw = np.float32(2.0) ** -rng.integers(6, 10, size=6).astype(np.float32)
    x = (qx * s_a).astype(np.float16)
    w = (qw * sw[:, None]).astype(np.float16)
    b = rng.standard_normal(6)
    wq, s = q8.quantize_weight(w)
    assert np.array_equal(wq, qw) and np.array_equal(s, sw)
    y = q8.dequantize(q8.int8_matmul(q8.quantize_act(x, np.float32(1) / s_a), wq), s_a, s, b)
    assert np.abs(y - enc.linear(x, w, b)).max() <= 1e-12


def test_int8_layer_matches_brute_force_tiny():
    cfg = ti.custom_encoder_config(2, 6, [6, 4], 32, 2, 64, dtype="f16", seed=3)
    lens, x = ti.encoder_input(cfg)
    w = ti.encoder_layer_weights(cfg, 0, variant=True)
    cu, _ = enc.offsets(lens, 6)
    xp = enc.remove_padding(x.astype(np.float64), lens)
    amax = q8.calibrate(xp, cu, w, 2, EPS)
    y = q8.encoder_layer_int8(xp, cu, w, 2, EPS, amax)
    ref = brute.encoder_layer_int8_padded(x, lens, w, 2, EPS, amax)
    assert np.abs(enc.remove_padding(ref, lens) - y).max() <= 1e-9


def test_int8_layer_close_to_float_layer():
    cfg = ti.ENCODER_CONFIGS["tiny"]
    cfg = dict(cfg, dtype="f16")
    lens, x = ti.encoder_input(cfg)
    w = ti.encoder_layer_weights(cfg, 0, variant=True)
    cu, _ = enc.offsets(lens, 8)
    xp = enc.remove_padding(x.astype(np.float64), lens)
    amax = q8.calibrate(xp, cu, w, 4, EPS)
    y8 = q8.encoder_layer_int8(xp, cu, w, 4, EPS, amax)
    y = enc.encoder_layer(xp, cu, w, 4, EPS)
    assert np.linalg.norm(y8 - y) / np.linalg.norm(y) < 0.05


def _tiny_int8_case(seed=5, lens=(6, 3, 5), S=6, H=32, heads=2, F=64):
    cfg = ti.custom_encoder_config(len(lens), S, list(lens), H, heads, F, dtype="f16", seed=seed)
    lens, x = ti.encoder_input(cfg)
    return cfg, lens, x


def test_calibrate_matches_brute_force_gemm_inputs():
    """calibrate() returns the max-abs of the four projection GEMMs' inputs over the valid
    tokens only: the layer input, the attention output, the first LayerNorm's output and the
    GELU output, each taken from the pure-Python padded brute force (pad rows excluded).
    Pad rows of x are scaled up so that a statistic taken over padded rows would differ."""
    cfg, lens, x = _tiny_int8_case()
    x = x.astype(np.float64)
    for b, L in enumerate(lens):
        x[b, L:] *= 9.0                                        # pads larger than any valid row
    w = ti.encoder_layer_weights(cfg, 0, variant=True)
    trace = {}
    brute.encoder_layer_padded(x, lens, w, cfg["heads"], EPS, trace=trace)
    want = [max(abs(v) for row in trace[k] for v in row) for k in ("x", "ctx", "h1", "f")]
    cu, _ = enc.offsets(lens, cfg["max_seq"])
    got = q8.calibrate(enc.remove_padding(x, lens), cu, w, cfg["heads"], EPS)
    assert len(got) == 4
    for g, r, name in zip(got, want, ("x", "ctx", "h1", "gelu")):
        assert abs(g - r) <= 1e-12 * max(1.0, r), (name, g, r)
    # the four statistics are distinct quantities here, so a swapped or mis-sourced one
    # (e.g. FFN1's input taken before the LayerNorm) cannot pass
    assert len({round(v, 9) for v in want}) == 4


def _brute_stack_int8(x_pad, lens, layers, amaxes, heads):
    """Two or more int8 layers, each the pure-Python padded brute force, the output of each
    layer stored as fp16 before the next one reads it (pad rows stay zero)."""
    y = np.asarray(x_pad, np.float64)
    for w, a in zip(layers, amaxes):
        y = brute.encoder_layer_int8_padded(y, lens, w, heads, EPS, a)
        for b, L in enumerate(lens):
            y[b, L:] = 0.0
        y = y.astype(np.float16).astype(np.float64)
    return y


def test_int8_stack_matches_two_layer_brute_force():
    cfg, lens, x = _tiny_int8_case(seed=7)
    heads = cfg["heads"]
    layers = [ti.encoder_layer_weights(cfg, i, variant=True) for i in range(2)]
    cu, _ = enc.offsets(lens, cfg["max_seq"])
    xp = enc.remove_padding(x.astype(np.float64), lens)
    amaxes, h = [], xp
    for w in layers:
        amaxes.append(q8.calibrate(h, cu, w, heads, EPS))
        h = enc.encoder_layer(h, cu, w, heads, EPS)
    got = q8.encoder_stack_int8(xp, cu, layers, amaxes, heads, EPS)
    ref = enc.remove_padding(_brute_stack_int8(x, lens, layers, amaxes, heads), lens)
    assert np.abs(got - ref).max() <= 1e-9
    # the stored output of each layer is fp16: the result is on the fp16 grid
    assert np.array_equal(got, got.astype(np.float16).astype(np.float64))
    # the pin is sharp: the same two layers chained without the fp16 store in between (a
    # dropped rounding in the stack loop) move the result far beyond the 1e-9 above
    chained = xp
    for w, a in zip(layers, amaxes):
        chained = q8.encoder_layer_int8(chained, cu, w, heads, EPS, a)
    assert np.abs(chained - ref).max() > 1e-4


def test_int8_stack_of_one_is_the_rounded_layer():
    cfg, lens, x = _tiny_int8_case(seed=9)
    w = ti.encoder_layer_weights(cfg, 0, variant=True)
    cu, _ = enc.offsets(lens, cfg["max_seq"])
    xp = enc.remove_padding(x.astype(np.float64), lens)
    a = q8.calibrate(xp, cu, w, cfg["heads"], EPS)
    one = q8.encoder_stack_int8(xp, cu, [w], [a], cfg["heads"], EPS)
    ref = enc.remove_padding(brute.encoder_layer_int8_padded(x, lens, w, cfg["heads"], EPS, a), lens)
    assert np.array_equal(one, ref.astype(np.float16).astype(np.float64))


# ------------------------------------------------------------------ int8 attention
def _qkv_case(seed, lens, H=32, heads=2):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    qkv = (rng.standard_normal((T, 3 * H)) * 0.7).astype(np.float16)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    amax = [float(np.abs(qkv[:, i * H:(i + 1) * H].astype(np.float64)).max()) for i in range(3)]
    return qkv, cu, amax


def test_attention_int8_matches_padded_brute_force():
    lens = [5, 1, 0, 9]
    qkv, cu, amax = _qkv_case(11, lens)
    got = q8.attention_int8(qkv, cu, 2, amax)
    S = max(lens)
    pad = np.zeros((len(lens), S, qkv.shape[1]), np.float16)
    for b in range(len(lens)):
        pad[b, :lens[b]] = qkv[cu[b]:cu[b + 1]]
        pad[b, lens[b]:] = 9.0                                    # pads must not matter
    ref = brute.attention_int8_padded(pad, lens, 2, amax)
    assert np.abs(enc.remove_padding(ref, lens) - got).max() <= 1e-12


def test_attention_int8_special_cases():
    H, heads = 32, 2
    rng = np.random.default_rng(12)
    # identical keys: every probability is 1 (code 127), the output is the mean of V's codes
    L = 6
    qkv = (rng.standard_normal((L, 3 * H)) * 0.7).astype(np.float16)
    qkv[:, H:2 * H] = qkv[0, H:2 * H]
    amax = [float(np.abs(qkv[:, i * H:(i + 1) * H].astype(np.float64)).max()) for i in range(3)]
    cu = np.array([0, L])
    got = q8.attention_int8(qkv, cu, heads, amax)
    s_v, inv_v = q8.act_scale(amax[2])
    vq = q8.quantize_act(qkv[:, 2 * H:], inv_v).astype(np.float64)
    assert np.abs(got - float(s_v) * vq.mean(axis=0)).max() <= 1e-12
    # a single token attends to itself: its own V codes times s_v
    one = q8.attention_int8(qkv[:1], np.array([0, 1]), heads, amax)
    assert np.abs(one[0] - float(s_v) * vq[0]).max() <= 1e-12
    # V codes all equal c: the output is c * s_v whatever the probabilities
    qkv2 = qkv.copy()
    qkv2[:, 2 * H:] = np.float16(0.5)
    qkv2[:, H:2 * H] = (rng.standard_normal((L, H)) * 0.7).astype(np.float16)
    amax2 = [amax[0], float(np.abs(qkv2[:, H:2 * H].astype(np.float64)).max()), 1.0]
    got2 = q8.attention_int8(qkv2, cu, heads, amax2)
    assert np.abs(got2 - float(q8.act_scale(1.0)[0]) * 64).max() <= 1e-12   # rne(0.5 * 127) = 64


def test_attention_int8_sequences_are_isolated_and_close_to_float():
    lens = [7, 30, 12]
    qkv, cu, amax = _qkv_case(13, lens, H=64, heads=4)
    got = q8.attention_int8(qkv, cu, 4, amax)
    qkv2 = qkv.copy()
    qkv2[cu[1]:cu[2]] = (np.random.default_rng(1).standard_normal((30, 192)) * 0.7).astype(np.float16)
    got2 = q8.attention_int8(qkv2, cu, 4, amax)
    for b in (0, 2):
        assert np.array_equal(got[cu[b]:cu[b + 1]], got2[cu[b]:cu[b + 1]])
    ref = enc.attention(qkv.astype(np.float64), cu, 4)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 0.03


def test_int8_layer_with_int8_attention_matches_brute_force():
    cfg = ti.custom_encoder_config(2, 6, [6, 4], 32, 2, 64, dtype="f16", seed=14)
    lens, x = ti.encoder_input(cfg)
    w = ti.encoder_layer_weights(cfg, 0, variant=True)
    cu, _ = enc.offsets(lens, 6)
    xp = enc.remove_padding(x.astype(np.float64), lens)
    amax = q8.calibrate(xp, cu, w, 2, EPS)
    aa = q8.calibrate_attention(xp, cu, w, 2, EPS)
    y = q8.encoder_layer_int8(xp, cu, w, 2, EPS, amax, attn_amax=aa)
    ref = brute.encoder_layer_int8_padded(x, lens, w, 2, EPS, amax, attn_amax=aa)
    assert np.abs(enc.remove_padding(ref, lens) - y).max() <= 1e-9
    # and the float-attention int8 layer differs from it (the option is not a no-op)
    y_f = q8.encoder_layer_int8(xp, cu, w, 2, EPS, amax)
    assert np.abs(y_f - y).max() > 1e-6


def test_calibrate_attention_matches_brute_force_projection():
    cfg, lens, x = _tiny_int8_case(seed=15)
    w = ti.encoder_layer_weights(cfg, 0, variant=True)
    H = cfg["hidden"]
    cu, _ = enc.offsets(lens, cfg["max_seq"])
    xp = enc.remove_padding(x.astype(np.float64), lens)
    got = q8.calibrate_attention(xp, cu, w, cfg["heads"], EPS)
    Wq = np.asarray(w["w_qkv"], np.float64)
    bq = np.asarray(w["b_qkv"], np.float64)
    want = [0.0, 0.0, 0.0]
    for row in xp:
        for n in range(3 * H):
            v = abs(sum(Wq[n, k] * row[k] for k in range(H)) + bq[n])
            want[n // H] = max(want[n // H], v)
    assert np.abs(np.array(got) - np.array(want)).max() <= 1e-12


# ------------------------------------------------------------------ dynamic activation scales
def test_dynamic_int8_layer_matches_brute_force():
    cfg = ti.custom_encoder_config(3, 6, [6, 2, 5], 32, 2, 64, dtype="f16", seed=17)
    lens, x = ti.encoder_input(cfg)
    w = ti.encoder_layer_weights(cfg, 0, variant=True)
    cu, _ = enc.offsets(lens, 6)
    xp = enc.remove_padding(x.astype(np.float64), lens)
    y = q8.encoder_layer_int8(xp, cu, w, 2, EPS, None, dynamic=True)
    ref = brute.encoder_layer_int8_dynamic_padded(x, lens, w, 2, EPS)
    assert np.abs(enc.remove_padding(ref, lens) - y).max() <= 1e-9


def test_dynamic_scales_follow_the_batch():
    """The dynamic layer depends on the batch it runs: the same sequence run alone or beside
    a sequence of much larger activations gets other codes (its scales grow), while a static
    layer gives that sequence the same output either way; and the dynamic layer on the
    loud batch matches the stage-wise brute force."""
    cfg = ti.custom_encoder_config(2, 6, [6, 6], 32, 2, 64, dtype="f16", seed=18)
    lens, x = ti.encoder_input(cfg)
    w = ti.encoder_layer_weights(cfg, 0, variant=True)
    x = x.astype(np.float64)
    x[1] *= 8.0                                                   # a loud second sequence
    x = x.astype(np.float16).astype(np.float64)
    cu2, _ = enc.offsets(lens, 6)
    both = q8.encoder_layer_int8(enc.remove_padding(x, lens), cu2, w, 2, EPS, None, dynamic=True)
    alone = q8.encoder_layer_int8(x[0], np.array([0, 6]), w, 2, EPS, None, dynamic=True)
    assert np.abs(both[:6] - alone).max() > 1e-4
    a_static = [8.0, 1.0, 4.0, 0.5]
    s_both = q8.encoder_layer_int8(enc.remove_padding(x, lens), cu2, w, 2, EPS, a_static)
    s_alone = q8.encoder_layer_int8(x[0], np.array([0, 6]), w, 2, EPS, a_static)
    assert np.array_equal(s_both[:6], s_alone)
    dyn_ref = brute.encoder_layer_int8_dynamic_padded(x, lens, w, 2, EPS)
    assert np.abs(enc.remove_padding(dyn_ref, lens) - both).max() <= 1e-9
