"""GPU parity of the int8 GEMM variant: quantisation codes and int32 accumulators bit-exact
against the oracle; the int8 encoder layer against the Q-oracle (same codes rule, same
calibration scales) at the fp16 tolerance."""
import numpy as np
import pytest
import torch

import tel_inputs as ti
from oracle import encoder as enc
from oracle import int8 as q8
from tests.gpu_helpers import assert_close, dev, errors, gpu_encoder_forward, host, prepare_layers

pytestmark = pytest.mark.gpu

tel = pytest.importorskip("transformer_encoder_remove_amd")
EPS = ti.LN_EPS


@pytest.mark.parametrize("n", [1, 7, 8, 4096 + 5, 2557 * 768])
def test_quantize_act_bit_exact(n):
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * 2).astype(np.float16)
    x[: min(n, 8)] = np.array([2.5, -2.5, 0.5, 3.5, 300, -300, 0, -0.0], np.float16)[: min(n, 8)]
    for inv in (np.float32(1.0), np.float32(127.0) / np.float32(np.abs(x.astype(np.float32)).max())):
        q = torch.empty(n, dtype=torch.int8, device="cuda")
        tel.tel_quantize_i8(torch.from_numpy(x).cuda(), q, float(inv))
        torch.cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), q8.quantize_act(x, inv))


@pytest.mark.parametrize("N,K", [(9, 33), (2304, 768), (768, 3072)])
def test_quantize_weight_bit_exact(N, K):
    rng = np.random.default_rng(N)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    w[min(3, N - 1)] = 0
    q = torch.empty((N, K), dtype=torch.int8, device="cuda")
    s = torch.empty(N, dtype=torch.float32, device="cuda")
    tel.tel_quantize_weight_i8(torch.from_numpy(w).cuda(), q, s)
    torch.cuda.synchronize()
    ref_q, ref_s = q8.quantize_weight(w)
    assert np.array_equal(s.cpu().numpy(), ref_s)
    assert np.array_equal(q.cpu().numpy(), ref_q)


@pytest.mark.parametrize("M,N,K", [(1, 4, 16), (77, 100, 48), (2557, 2304, 768), (300, 768, 3072),
                                   (129, 3072, 768), (2557, 768, 768)])
def test_gemm_i8_i32_bit_exact(M, N, K):
    a, b = ti.int8_operands(M, N, K, seed=M + N)
    a[0, :] = -127                                      # extreme accumulator values
    b[0, :] = -127
    C = torch.empty((M, N), dtype=torch.int32, device="cuda")
    tel.tel_gemm_i8_i32(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), C)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy().astype(np.int64), q8.int8_matmul(a, b))


def _calibrated(cfg, lens, x, ws):
    """Per-layer calibration max-abs from a float64 oracle run of the float stack."""
    cu, _ = enc.offsets(lens, x.shape[1])
    xp = enc.remove_padding(x.astype(np.float64), lens)
    amaxes = []
    for w in ws:
        amaxes.append(q8.calibrate(xp, cu, w, cfg["heads"], EPS))
        xp = enc.encoder_layer(xp, cu, w, cfg["heads"], EPS)
    return amaxes


def _gpu_int8(cfg, lens, x, ws, amaxes):
    return gpu_encoder_forward(tel, cfg, lens, x, ws, int8=True, act_amax=amaxes)


@pytest.mark.parametrize("shape", [
    dict(B=2, S=8, lens=[5, 8], H=64, heads=4, F=256),
    dict(B=3, S=40, lens=[40, 1, 17], H=128, heads=2, F=256),
    # 128 tokens at BERT-base width: FFN2 runs split over k (int32 partial sums)
    dict(B=2, S=96, lens=[96, 32], H=768, heads=12, F=3072),
])
def test_int8_layer_small(shape):
    cfg = ti.custom_encoder_config(shape["B"], shape["S"], shape["lens"], shape["H"],
                                   shape["heads"], shape["F"], dtype="f16", seed=21)
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, 0, variant=True)]
    amaxes = _calibrated(cfg, lens, x, ws)
    y = _gpu_int8(cfg, lens, x, ws, amaxes)
    cu, _ = enc.offsets(lens, shape["S"])
    ref = q8.encoder_layer_int8(enc.remove_padding(x.astype(np.float64), lens), cu, ws[0],
                                shape["heads"], EPS, amaxes[0])
    assert_close(enc.remove_padding(y, lens), ref, "f16", f"int8 layer {shape}")


@pytest.mark.parametrize("variant", [False, True])
def test_int8_bert_base_layer_full_batch(variant):
    cfg = ti.ENCODER_CONFIGS["bert_base_int8"]
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, 0, variant)]
    amaxes = _calibrated(cfg, lens, x, ws)
    y = _gpu_int8(cfg, lens, x, ws, amaxes)
    cu, _ = enc.offsets(lens, cfg["max_seq"])
    xp = enc.remove_padding(x.astype(np.float64), lens)
    ref = q8.encoder_layer_int8(xp, cu, ws[0], cfg["heads"], EPS, amaxes[0])
    got = enc.remove_padding(y, lens)
    d = np.abs(got - ref)
    print(f"int8 layer vs Q-oracle: max_abs={d.max():.3e} rel_frob="
          f"{np.linalg.norm(got - ref) / np.linalg.norm(ref):.3e} n>2e-2: {(d > 2e-2).sum()} of {d.size}")
    assert_close(got, ref, "f16", "int8 bert_base L1 vs Q-oracle")
    ma, rel = errors(got, enc.encoder_layer(xp, cu, ws[0], cfg["heads"], EPS))
    print(f"int8 layer vs float oracle (reported, not gated): max_abs={ma:.3e} rel={rel:.3e}")


def test_int8_bert_base_12_layers_sampled():
    """12 int8 layers on the full batch: reported, not gated (the int8 workload is one
    layer). Code flips at quantisation boundaries compound over layers, so two correct
    implementations drift apart; the check is only that the stack stays finite and
    close to the float stack's scale."""
    cfg = ti.ENCODER_CONFIGS["bert_base_int8"]
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, i) for i in range(cfg["layers"])]
    amaxes = _calibrated(cfg, lens, x, ws)
    y = _gpu_int8(cfg, lens, x, ws, amaxes)
    pick = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 3, 17})
    cu, _ = enc.offsets(lens[pick], cfg["max_seq"])
    xp = enc.remove_padding(x[pick].astype(np.float64), lens[pick])
    ref = q8.encoder_stack_int8(xp, cu, ws, amaxes, cfg["heads"], EPS)
    got = enc.remove_padding(y[pick], lens[pick])
    ma, rel = errors(got, ref)
    print(f"int8 12 layers vs Q-oracle (reported): max_abs={ma:.3e} rel_frob={rel:.3e}")
    assert rel < 0.1


def test_calibrate_matches_oracle():
    """tel_encoder_calibrate's max-abs of the four GEMM inputs vs the oracle's calibration
    (fp16 intermediates on the GPU, float64 in the oracle: equal to ~fp16 precision)."""
    cfg = ti.ENCODER_CONFIGS["bert_base"]
    lens, x = ti.encoder_input(cfg)
    w = ti.encoder_layer_weights(cfg, 0, variant=True)
    desc = tel.make_encoder_desc(cfg["hidden"], cfg["heads"], cfg["ffn"], torch.float16, EPS)
    packed = tel.alloc_bytes(tel.tel_encoder_packed_size(desc))
    tel.tel_encoder_prepare(desc, {k: dev(v, "f16") for k, v in w.items()}, packed)
    xp = enc.remove_padding(x.astype(np.float64), lens)
    T = xp.shape[0]
    cu, _ = enc.offsets(lens, cfg["max_seq"])
    xd = dev(xp, "f16")
    yd = torch.empty_like(xd)
    amax = torch.zeros(7, dtype=torch.float32, device="cuda")
    ws = tel.alloc_bytes(tel.tel_encoder_workspace_size(desc, T))
    tel.tel_encoder_calibrate(desc, packed, xd, yd, torch.tensor(cu.astype(np.int32), device="cuda"),
                              T, int(lens.max()), amax, ws)
    torch.cuda.synchronize()
    ref = np.array(q8.calibrate(xp, cu, w, cfg["heads"], EPS) +
                   q8.calibrate_attention(xp, cu, w, cfg["heads"], EPS))
    got = amax.cpu().numpy().astype(np.float64)
    assert got[0] == ref[0]                               # the input itself: exact
    assert np.all(np.abs(got - ref) <= 5e-3 * ref), (got, ref)


def test_int8_small_stack_vs_q_oracle():
    """Three int8 layers through tel_encoder_forward, where each LN2 hands the next layer its
    input codes, against the Q-oracle stack."""
    cfg = ti.custom_encoder_config(3, 40, [40, 1, 17], 128, 2, 256, dtype="f16", seed=23,
                                   layers=3)
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, i, variant=True) for i in range(3)]
    amaxes = _calibrated(cfg, lens, x, ws)
    y = _gpu_int8(cfg, lens, x, ws, amaxes)
    cu, _ = enc.offsets(lens, cfg["max_seq"])
    ref = q8.encoder_stack_int8(enc.remove_padding(x.astype(np.float64), lens), cu, ws, amaxes,
                                cfg["heads"], EPS)
    assert_close(enc.remove_padding(y, lens), ref, "f16", "int8 3-layer stack")


def test_int8_stack_codes_equal_layer_by_layer():
    """The stack's chained codes (LN2 quantising for the next layer) are exactly the codes the
    per-layer entry point makes with its own quantise kernel: both runs agree bitwise."""
    cfg = dict(ti.ENCODER_CONFIGS["bert_base_int8"], layers=3)
    lens, x = ti.encoder_input(cfg)
    lens, x = lens[:8], x[:8]
    ws = [ti.encoder_layer_weights(cfg, i, variant=True) for i in range(3)]
    amaxes = [[3.0, 2.5, 4.0, 1.5], [3.5, 2.0, 4.5, 1.0], [2.5, 3.0, 3.5, 2.0]]
    y_stack = _gpu_int8(dict(cfg, batch=8), lens, x, ws, amaxes)
    desc = tel.make_encoder_desc(cfg["hidden"], cfg["heads"], cfg["ffn"], torch.float16,
                                 ti.LN_EPS, int8_gemm=True)
    packed = prepare_layers(tel, desc, ws, "f16", amaxes)
    cu_h, _ = enc.offsets(lens, cfg["max_seq"])
    T, max_len = int(np.sum(lens)), int(np.max(lens))
    cur = dev(enc.remove_padding(x.astype(np.float64), lens), "f16")
    cu = torch.from_numpy(np.asarray(cu_h, np.int32)).cuda()
    lws = tel.alloc_bytes(tel.tel_encoder_workspace_size(desc, T))
    for p in packed:
        nxt = torch.empty_like(cur)
        tel.tel_encoder_layer_forward(desc, p, cur, nxt, cu, T, max_len, lws)
        cur = nxt
    torch.cuda.synchronize()
    assert np.array_equal(enc.remove_padding(y_stack, lens), host(cur))


@pytest.mark.parametrize("epi", ["bias", "gelu", "resid", "qkv", "gelu_codes"])
@pytest.mark.parametrize("M,N,K", [(300, 768, 768), (77, 2304, 768), (2900, 3072, 768)])
def test_gemm_i8_epilogues(epi, M, N, K):
    """One int8-layer GEMM with each epilogue: exact int32 products, dequantise with the
    column scales, bias (+ GELU, + residual, head split) against the Q-oracle's steps."""
    if epi == "qkv" and N != 2304:
        pytest.skip("head split needs N = 3 * heads * head_dim")
    rng = np.random.default_rng(M + N)
    qa = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    s_w = (np.abs(rng.standard_normal(N)) * 2e-4 + 1e-5).astype(np.float32)
    s_a, _ = q8.act_scale(3.0)
    dq = (np.float32(s_a) * s_w).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    r = ti.to_storage(rng.standard_normal((M, N)), "f16")
    v = q8.dequantize(q8.int8_matmul(qa, qw), s_a, s_w, b)
    A, W = torch.from_numpy(qa).cuda(), torch.from_numpy(qw).cuda()
    dq_d, b_d = torch.from_numpy(dq).cuda(), torch.from_numpy(b).cuda()
    heads = 12
    code = {"bias": tel.TEL_EPI_BIAS, "gelu": tel.TEL_EPI_BIAS_GELU, "resid": tel.TEL_EPI_BIAS_RESID,
            "qkv": tel.TEL_EPI_QKV_SPLIT, "gelu_codes": tel.TEL_EPI_BIAS_GELU}[epi]
    if epi == "gelu_codes":
        _, inv = q8.act_scale(4.0)
        qinv = torch.tensor([inv], dtype=torch.float32, device="cuda")
        C = torch.zeros((M, N), dtype=torch.int8, device="cuda")
        tel.tel_gemm_i8(code, A, W, dq_d, b_d, C, qinv=qinv, out_int8=True)
        torch.cuda.synchronize()
        ref = q8.quantize_act(ti.to_storage(enc.gelu(v), "f16"), inv)
        d = np.abs(C.cpu().numpy().astype(np.int32) - ref.astype(np.int32))
        # against the oracle a code can differ by one where the kernel's fp16 GELU value
        # itself differs from the oracle's by a rounding step
        assert d.max() <= 1 and (d > 0).mean() < 5e-3, (d.max(), (d > 0).mean())
        return
    C = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    tel.tel_gemm_i8(code, A, W, dq_d, b_d, C, resid=dev(r, "f16") if epi == "resid" else None,
                    heads=heads)
    torch.cuda.synchronize()
    got = host(C)
    if epi == "bias":
        ref = v
    elif epi == "gelu":
        ref = enc.gelu(v)
    elif epi == "resid":
        ref = v + r.astype(np.float64)
    else:
        d_h = N // 3 // heads
        ref = v.reshape(M, 3, heads, d_h).transpose(1, 2, 0, 3)
        got = got.reshape(-1)[: 3 * heads * M * d_h].reshape(3, heads, M, d_h)
    assert_close(got, ref, "f16", f"int8 GEMM {epi} {M}x{N}x{K}")
