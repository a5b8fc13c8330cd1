"""GPU parity of int8 attention (both products on int8 codes) against the Q-oracle
(oracle/int8.py attention_int8): the kernel alone on codes the host makes, its int8-code
output, the QKV GEMM's head-split int8 codes, and whole int8 layers and a stack with
int8 attention (tel_encoder_desc.int8_gemm = 2)."""
import math

import numpy as np
import pytest
import torch

import tel_inputs as ti
from oracle import encoder as enc
from oracle import int8 as q8
from tests.gpu_helpers import assert_close, dev, errors, gpu_encoder_forward, host

pytestmark = pytest.mark.gpu

tel = pytest.importorskip("transformer_encoder_remove_amd")
EPS = ti.LN_EPS


def _scales(amax, head_dim, s_o_inv=10.0):
    """The kernel's constants exactly as tel_encoder_prepare forms them (float32)."""
    f32 = np.float32
    s = [f32(f32(a) / f32(127.0)) for a in amax]
    a2 = f32(f32(f32(s[0] * s[1]) / f32(math.sqrt(head_dim))) * f32(1.4426950408889634))
    return np.array([a2, s[2], s_o_inv], np.float32)


def _case(lens, heads, d, seed):
    rng = np.random.default_rng(seed)
    H = heads * d
    T = int(sum(lens))
    qkv = (rng.standard_normal((T, 3 * H)) * 0.8).astype(np.float16)
    amax = [float(np.abs(qkv[:, i * H:(i + 1) * H].astype(np.float64)).max()) for i in range(3)]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    # the codes as the QKV epilogue writes them: head-split [3][heads][T][d]
    codes = np.stack([q8.quantize_act(qkv[:, i * H:(i + 1) * H], q8.act_scale(amax[i])[1])
                      for i in range(3)])                                  # [3][T][H]
    split = codes.reshape(3, T, heads, d).transpose(0, 2, 1, 3).copy()
    return qkv, amax, cu, split


@pytest.mark.parametrize("lens,heads,d", [
    ([1], 2, 64), ([17, 64, 65, 0, 128], 12, 64), ([300, 5], 4, 64), ([33, 100], 2, 32),
    ([40, 7], 4, 16), ([70, 129], 2, 128), ([1000], 1, 64)])
def test_attention_int8_kernel_vs_oracle(lens, heads, d):
    qkv, amax, cu, split = _case(lens, heads, d, sum(lens) + d)
    T, H = qkv.shape[0], heads * d
    print(f"int8 attention lens {lens} heads {heads} d {d}", flush=True)
    out = torch.full((T, H), float("nan"), dtype=torch.float16, device="cuda")
    sc = torch.from_numpy(_scales(amax, d)).cuda()
    cu_d = torch.from_numpy(cu.astype(np.int32)).cuda()
    tel.tel_attention_int8(torch.from_numpy(split.reshape(-1)).cuda(), out, sc, cu_d, T, max(lens),
                           heads, d)
    torch.cuda.synchronize()
    ref = q8.attention_int8(qkv, cu, heads, amax)
    ma, rel = assert_close(host(out), ref, "f16", f"int8 attention {lens}")
    print(f"  max_abs={ma:.3e} rel_frob={rel:.3e}")
    # the context codes for the O projection: those of the kernel's own fp16 value
    codes = torch.zeros((T, H), dtype=torch.int8, device="cuda")
    tel.tel_attention_int8(torch.from_numpy(split.reshape(-1)).cuda(), codes, sc, cu_d, T,
                           max(lens), heads, d)
    torch.cuda.synchronize()
    own = q8.quantize_act(out.cpu().numpy(), np.float32(10.0))
    assert np.array_equal(codes.cpu().numpy(), own)


def test_qkv_gemm_int8_head_split_codes():
    M, H, heads = 300, 768, 12
    rng = np.random.default_rng(5)
    qa = rng.integers(-127, 128, size=(M, H)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(3 * H, H)).astype(np.int8)
    s_w = (np.abs(rng.standard_normal(3 * H)) * 2e-4 + 1e-5).astype(np.float32)
    s_a, _ = q8.act_scale(3.0)
    dq = (np.float32(s_a) * s_w).astype(np.float32)
    b = (rng.standard_normal(3 * H) * 0.1).astype(np.float32)
    v = q8.dequantize(q8.int8_matmul(qa, qw), s_a, s_w, b)
    inv = np.array([q8.act_scale(a)[1] for a in (2.0, 2.5, 3.0)], np.float32)
    C = torch.zeros(3 * M * H, dtype=torch.int8, device="cuda")
    tel.tel_gemm_i8(tel.TEL_EPI_QKV_SPLIT, torch.from_numpy(qa).cuda(), torch.from_numpy(qw).cuda(),
                    torch.from_numpy(dq).cuda(), torch.from_numpy(b).cuda(), C,
                    qinv=torch.from_numpy(inv).cuda(), out_int8=True, heads=heads)
    torch.cuda.synchronize()
    vh = ti.to_storage(v, "f16")
    ref = np.stack([q8.quantize_act(vh[:, i * H:(i + 1) * H], inv[i]) for i in range(3)])
    ref = ref.reshape(3, M, heads, H // heads).transpose(0, 2, 1, 3).reshape(-1)
    diff = np.abs(C.cpu().numpy().astype(np.int32) - ref.astype(np.int32))
    assert diff.max() <= 1 and (diff > 0).mean() < 5e-3, (diff.max(), (diff > 0).mean())


def _calibrated(cfg, lens, x, ws):
    cu, _ = enc.offsets(lens, x.shape[1])
    xp = enc.remove_padding(x.astype(np.float64), lens)
    amaxes, attn = [], []
    for w in ws:
        amaxes.append(q8.calibrate(xp, cu, w, cfg["heads"], EPS))
        attn.append(q8.calibrate_attention(xp, cu, w, cfg["heads"], EPS))
        xp = enc.encoder_layer(xp, cu, w, cfg["heads"], EPS)
    return amaxes, attn


@pytest.mark.parametrize("variant", [False, True])
def test_int8_attention_bert_base_layer_full_batch(variant):
    cfg = ti.ENCODER_CONFIGS["bert_base_int8_attn"]
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, 0, variant)]
    amaxes, attn = _calibrated(cfg, lens, x, ws)
    y = gpu_encoder_forward(tel, cfg, lens, x, ws, int8=2, act_amax=amaxes, attn_amax=attn)
    cu, _ = enc.offsets(lens, cfg["max_seq"])
    xp = enc.remove_padding(x.astype(np.float64), lens)
    ref = q8.encoder_layer_int8(xp, cu, ws[0], cfg["heads"], EPS, amaxes[0], attn_amax=attn[0])
    got = enc.remove_padding(y, lens)
    ma, rel = assert_close(got, ref, "f16", "int8-attention layer vs Q-oracle")
    print(f"int8-attention layer vs Q-oracle: max_abs={ma:.3e} rel_frob={rel:.3e}")
    ma, rel = errors(got, enc.encoder_layer(xp, cu, ws[0], cfg["heads"], EPS))
    print(f"int8-attention layer vs float oracle (reported): max_abs={ma:.3e} rel={rel:.3e}")


def test_int8_attention_small_stack_vs_q_oracle():
    cfg = ti.custom_encoder_config(4, 80, [80, 1, 33, 64], 256, 4, 512, dtype="f16", seed=27,
                                   layers=3)
    lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, i, variant=True) for i in range(3)]
    amaxes, attn = _calibrated(cfg, lens, x, ws)
    y = gpu_encoder_forward(tel, cfg, lens, x, ws, int8=2, act_amax=amaxes, attn_amax=attn)
    cu, _ = enc.offsets(lens, cfg["max_seq"])
    ref = q8.encoder_stack_int8(enc.remove_padding(x.astype(np.float64), lens), cu, ws, amaxes,
                                cfg["heads"], EPS, attn_amaxes=attn)
    assert_close(enc.remove_padding(y, lens), ref, "f16", "int8-attention 3-layer stack")
