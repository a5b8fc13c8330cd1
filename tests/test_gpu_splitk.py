"""GPU parity of the split-k partial GEMM (tel_gemm_partial) and the LayerNorm that finishes
its sum with bias and residual (tel_layernorm_reduce), against oracle/encoder.py and
oracle/int8.py: every tile configuration and several split counts on ragged shapes, exact
int32 sums for int8 codes, and the plans the encoder layer uses at BERT-base shape."""
import numpy as np
import pytest
import torch

import tel_inputs as ti
from oracle import encoder as enc
from oracle import int8 as q8
from tests.gpu_helpers import TORCH_DT, assert_close, dev, dev_f32, host

pytestmark = pytest.mark.gpu

tel = pytest.importorskip("transformer_encoder_remove_amd")
EPS = ti.LN_EPS
ES = {"f16": 2, "bf16": 2, "f32": 4}


def _fp_operands(M, N, K, dtype, seed):
    rng = np.random.default_rng(seed)
    a = ti.to_storage(rng.standard_normal((M, K)), dtype)
    w = ti.to_storage(rng.standard_normal((N, K)) * 0.05, dtype)
    return a, w


def _partials(A, W, cfg, sp, M, N, dtype=torch.float32):
    fill = float("nan") if dtype.is_floating_point else -(2 ** 31)
    out = torch.full((sp, M, N), fill, dtype=dtype, device="cuda")
    tel.tel_gemm_partial(cfg, sp, A, W, out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("M,N,K", [(300, 400, 512), (17, 1028, 1024)])
def test_partial_gemm_every_config_and_split(dtype, M, N, K):
    a, w = _fp_operands(M, N, K, dtype, seed=M + K)
    A, W = dev(a, dtype), dev(w, dtype)
    ref = enc.linear(a, w, np.zeros(N))
    nk = K * ES[dtype] // 128
    for cfg in range(-1, tel.tel_gemm_tile_configs()):
        for sp in (1, 2, 4):
            if sp > 1 and (cfg < 0 or nk % sp):
                continue
            P = _partials(A, W, cfg, sp, M, N)
            parts = host(P)
            assert np.isfinite(parts).all(), (cfg, sp)
            # the sum of the partials is the product (float32 accumulation)
            assert_close(parts.sum(axis=0), ref, "f32", f"partial sum cfg {cfg} splits {sp}")
            if sp > 1:   # each split covers its own k range
                kr = K // sp
                s1 = enc.linear(a[:, kr:2 * kr], w[:, kr:2 * kr], np.zeros(N))
                assert_close(parts[1], s1, "f32", f"split 1 of {sp}, cfg {cfg}")


@pytest.mark.parametrize("M,N,K", [(300, 400, 512), (2557, 768, 3072)])
def test_partial_gemm_int8_exact(M, N, K):
    rng = np.random.default_rng(M)
    qa = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    A, W = torch.from_numpy(qa).cuda(), torch.from_numpy(qw).cuda()
    ref = q8.int8_matmul(qa, qw)
    nk = K // 128
    cfgs = [tel.tel_gemm_partial_plan(tel.TEL_I8, M, N, K)[:2]] + \
        [(c, s) for c in range(5) for s in (1, 2, 4) if nk % s == 0]
    for cfg, sp in cfgs:
        P = _partials(A, W, cfg, sp, M, N, dtype=torch.int32)
        got = P.cpu().numpy().astype(np.int64).sum(axis=0)
        assert np.array_equal(got, ref), (cfg, sp)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("K", [768, 3072])
def test_partial_gemm_bert_base_plan(dtype, K):
    """The output projection (K 768) and FFN2 (K 3072) at 2557 tokens, in the configuration
    the encoder layer takes."""
    M, N = 2557, 768
    a, w = _fp_operands(M, N, K, dtype, seed=K)
    cfg, sp, pb = tel.tel_gemm_partial_plan(tel.DTYPE_CODE[TORCH_DT[dtype]], M, N, K)
    P = _partials(dev(a, dtype), dev(w, dtype), cfg, sp, M, N,
                  dtype=torch.float16 if pb == 2 else torch.float32)
    parts = host(P).astype(np.float64)
    # fp16 partial sums: each split is its k range's product rounded once to fp16
    tol = "f16" if pb == 2 else "f32"
    assert_close(parts.sum(axis=0), enc.linear(a, w, np.zeros(N)), tol, f"plan ({cfg}, {sp})")
    kr = K // sp
    for i in range(sp):
        ref_i = enc.linear(a[:, i * kr:(i + 1) * kr], w[:, i * kr:(i + 1) * kr], np.zeros(N))
        assert_close(parts[i], ref_i, tol, f"split {i} of plan ({cfg}, {sp})")


@pytest.mark.parametrize("M,N,K", [(300, 400, 512), (17, 1028, 1024), (2557, 768, 3072)])
def test_partial_gemm_fp16_partials(M, N, K):
    """16-bit partial sums (fp16 operands): every pipelined tile configuration and split
    count; each split's sums are its k range's product rounded to fp16."""
    a, w = _fp_operands(M, N, K, "f16", seed=3 * M + K)
    A, W = dev(a, "f16"), dev(w, "f16")
    nk = K * 2 // 128
    refs = {}
    for sp in (1, 2, 4):
        kr = K // sp
        for i in {0, sp - 1}:
            refs[sp, i] = enc.linear(a[:, i * kr:(i + 1) * kr], w[:, i * kr:(i + 1) * kr],
                                     np.zeros(N))
    for cfg in range(tel.tel_gemm_tile_configs()):
        for sp in (1, 2, 4):
            if nk % sp:
                continue
            parts = host(_partials(A, W, cfg, sp, M, N, dtype=torch.float16)).astype(np.float64)
            assert np.isfinite(parts).all(), (cfg, sp)
            for i in {0, sp - 1}:
                assert_close(parts[i], refs[sp, i], "f16", f"fp16 split {i}/{sp} cfg {cfg}")


@pytest.mark.parametrize("width", [768, 1024])
@pytest.mark.parametrize("sp", [1, 2, 3])
def test_layernorm_reduce_fp16_partials(width, sp):
    rows = 301
    parts, bias, gamma, beta, resid = _ln_case(rows, width, sp, seed=5 * width + sp)
    p16 = parts.astype(np.float16)
    r = ti.to_storage(resid, "f16")
    ref = enc.layer_norm(p16.astype(np.float64).sum(axis=0) + bias + r.astype(np.float64),
                         gamma, beta, EPS)
    y = torch.full((rows, width), float("nan"), dtype=torch.float16, device="cuda")
    tel.tel_layernorm_reduce(torch.from_numpy(p16).cuda(), sp, dev_f32(bias), dev(r, "f16"), y,
                             dev_f32(gamma), dev_f32(beta), EPS)
    torch.cuda.synchronize()
    assert_close(host(y), ref, "f16", f"reduce LN, fp16 partials, width {width} splits {sp}")


def _ln_case(rows, width, sp, seed):
    rng = np.random.default_rng(seed)
    parts = rng.standard_normal((sp, rows, width)).astype(np.float32)
    bias = (rng.standard_normal(width) * 0.1).astype(np.float32)
    gamma = (1 + rng.standard_normal(width) * 0.1).astype(np.float32)
    beta = (rng.standard_normal(width) * 0.1).astype(np.float32)
    resid = rng.standard_normal((rows, width)) * 2
    return parts, bias, gamma, beta, resid


@pytest.mark.parametrize("rdt,odt", [("f16", "f16"), ("bf16", "bf16"), ("f32", "bf16"),
                                     ("f32", "f32")])
@pytest.mark.parametrize("width", [64, 768, 1024])
@pytest.mark.parametrize("sp", [1, 2, 3])
def test_layernorm_reduce(rdt, odt, width, sp):
    rows = 301
    parts, bias, gamma, beta, resid = _ln_case(rows, width, sp, seed=width + sp)
    r = ti.to_storage(resid, rdt)
    ref = enc.layer_norm(parts.astype(np.float64).sum(axis=0) + bias + r.astype(np.float64),
                         gamma, beta, EPS)
    y = torch.full((rows, width), float("nan"), dtype=TORCH_DT[odt], device="cuda")
    y32 = torch.full((rows, width), float("nan"), device="cuda")
    tel.tel_layernorm_reduce(torch.from_numpy(parts).cuda(), sp, dev_f32(bias), dev(r, rdt), y,
                             dev_f32(gamma), dev_f32(beta), EPS, y32=y32)
    torch.cuda.synchronize()
    assert_close(host(y), ref, odt, f"reduce LN {rdt}->{odt} width {width} splits {sp}")
    assert_close(host(y32), ref, "f32", "float32 copy")


def test_layernorm_reduce_int8_codes():
    """int32 partials dequantised by dq, fp16 rounding of the sum, LayerNorm, and the int8
    codes of the fp16 output."""
    rows, width, sp = 257, 768, 2
    rng = np.random.default_rng(3)
    acc = rng.integers(-40000, 40000, size=(sp, rows, width)).astype(np.int32)
    s_w = (np.abs(rng.standard_normal(width)) * 1e-3 + 1e-4).astype(np.float32)
    s_a, inv_a = q8.act_scale(3.0)
    dq = (np.float32(s_a) * s_w).astype(np.float32)
    bias = (rng.standard_normal(width) * 0.1).astype(np.float32)
    gamma = (1 + rng.standard_normal(width) * 0.1).astype(np.float32)
    beta = (rng.standard_normal(width) * 0.1).astype(np.float32)
    resid = ti.to_storage(rng.standard_normal((rows, width)), "f16")
    pre = q8.dequantize(acc.astype(np.int64).sum(axis=0), s_a, s_w, bias) + resid
    ref = enc.layer_norm(ti.to_storage(pre, "f16"), gamma, beta, EPS)
    _, inv_out = q8.act_scale(4.0)
    ref_q = q8.quantize_act(ti.to_storage(ref, "f16"), inv_out)
    y = torch.full((rows, width), float("nan"), dtype=torch.float16, device="cuda")
    yq = torch.zeros((rows, width), dtype=torch.int8, device="cuda")
    qinv = torch.tensor([inv_out], dtype=torch.float32, device="cuda")
    tel.tel_layernorm_reduce(torch.from_numpy(acc).cuda(), sp, dev_f32(bias), dev(resid, "f16"),
                             y, dev_f32(gamma), dev_f32(beta), EPS, dq=dev_f32(dq), yq=yq,
                             qinv=qinv, round_pre=True)
    torch.cuda.synchronize()
    assert_close(host(y), ref, "f16", "int8 reduce LN")
    d = np.abs(yq.cpu().numpy().astype(np.int32) - ref_q.astype(np.int32))
    # a code can differ only where the fp16 output itself differs by one rounding step
    assert d.max() <= 1 and (d > 0).mean() < 5e-3, (d.max(), (d > 0).mean())
    # bit-exact: the codes are those of the kernel's own stored fp16 output
    assert np.array_equal(yq.cpu().numpy(), q8.quantize_act(y.cpu().numpy(), inv_out))
