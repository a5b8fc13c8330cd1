"""GPU parity of the layer's kernels, each against the oracle step it implements:
GEMM epilogues, variable-length attention and LayerNorm. Shapes span several tiles and
ragged tails; tolerances as stated in gpu_helpers (fp16/bf16: 2e-2 / 5e-3)."""
import numpy as np
import pytest
import torch

import tel_inputs as ti
from oracle import encoder as enc
from tests.gpu_helpers import assert_close, dev, dev_f32, host

pytestmark = pytest.mark.gpu

tel = pytest.importorskip("transformer_encoder_remove_amd")
EPS = ti.LN_EPS


def _operands(M, N, K, dtype, seed):
    rng = np.random.default_rng(seed)
    a = ti.to_storage(rng.standard_normal((M, K)), dtype)
    w = ti.to_storage(rng.standard_normal((N, K)) * 0.02, dtype)
    b = ti.to_storage(rng.standard_normal(N) * 0.02, dtype)
    r = ti.to_storage(rng.standard_normal((M, N)), dtype)
    return a, w, b, r


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (77, 192, 64), (300, 768, 768), (2560, 2304, 768),
                                   (513, 3072, 768), (129, 768, 3072), (64, 96, 8)])
def test_gemm_bias_gelu_resid(dtype, M, N, K):
    a, w, b, r = _operands(M, N, K, dtype, seed=M + N + K)
    A, W, R = dev(a, dtype), dev(w, dtype), dev(r, dtype)
    bias = dev_f32(b)
    lin = enc.linear(a, w, b)
    for epi, ref in ((tel.TEL_EPI_BIAS, lin), (tel.TEL_EPI_BIAS_GELU, enc.gelu(lin)),
                     (tel.TEL_EPI_BIAS_RESID, lin + r.astype(np.float64))):
        C = torch.full((M, N), float("nan"), dtype=A.dtype, device="cuda")
        tel.tel_gemm(epi, A, W, bias, C, resid=R if epi == tel.TEL_EPI_BIAS_RESID else None)
        torch.cuda.synchronize()
        assert_close(host(C), ref, dtype, f"epi {epi} {dtype} {M}x{N}x{K}")


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("M,H,heads", [(13, 64, 4), (2560, 768, 12), (333, 1024, 16), (50, 256, 2)])
def test_gemm_qkv_head_split(dtype, M, H, heads):
    a, w, b, _ = _operands(M, 3 * H, H, dtype, seed=M + H)
    C = torch.full((3 * M * H,), float("nan"), dtype=dev(a[:1], dtype).dtype, device="cuda")
    tel.tel_gemm(tel.TEL_EPI_QKV_SPLIT, dev(a, dtype), dev(w, dtype), dev_f32(b), C, heads=heads)
    torch.cuda.synchronize()
    d = H // heads
    ref = enc.linear(a, w, b).reshape(M, 3, heads, d).transpose(1, 2, 0, 3)   # [3][heads][M][d]
    assert_close(host(C).reshape(3, heads, M, d), ref, dtype, "qkv split")


def _attention_case(lens, heads, d, dtype, seed):
    rng = np.random.default_rng(seed)
    T, H = int(sum(lens)), heads * d
    qkv = ti.to_storage(rng.standard_normal((T, 3 * H)), dtype)
    cu, _ = enc.offsets(lens, max(max(lens), 1))
    ref = enc.attention(qkv, cu, heads)
    split = qkv.astype(np.float32).reshape(T, 3, heads, d).transpose(1, 2, 0, 3).copy()
    ctx = torch.full((T, H), float("nan"), dtype=dev(split[:1], dtype).dtype, device="cuda")
    cu_d = torch.tensor(cu.astype(np.int32), device="cuda")
    tel.tel_attention_varlen(dev(split, dtype), ctx, cu_d, T, int(max(lens)), heads, d)
    torch.cuda.synchronize()
    return host(ctx), ref


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_attention_head_dims(dtype, d):
    lens = [1, 64, 65, 130, 7]
    out, ref = _attention_case(lens, 2, d, dtype, seed=d)
    assert_close(out, ref, dtype, f"attention d={d}")


@pytest.mark.parametrize("lens", [[128] * 32, list(np.random.default_rng(1).integers(32, 129, 32)),
                                  [0, 5, 0, 1], [384, 64, 200], [1000, 3]])
def test_attention_lengths(lens):
    out, ref = _attention_case(lens, 12, 64, "f16", seed=len(lens))
    assert_close(out, ref, "f16", f"attention lens={lens[:4]}")


def test_attention_normalisation_with_ones():
    """V = 1 everywhere: every output is exactly the softmax normaliser ratio, i.e. 1."""
    lens, heads, d = [3, 70, 129], 4, 64
    T, H = sum(lens), heads * d
    rng = np.random.default_rng(2)
    qkv = rng.standard_normal((3, heads, T, d)).astype(np.float32) * 3
    qkv[2] = 1.0
    cu, _ = enc.offsets(lens, 129)
    ctx = torch.empty((T, H), dtype=torch.float16, device="cuda")
    tel.tel_attention_varlen(dev(qkv, "f16"), ctx, torch.tensor(cu.astype(np.int32), device="cuda"),
                             T, 129, heads, d)
    torch.cuda.synchronize()
    assert np.abs(host(ctx) - 1.0).max() <= 1e-3


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("rows,width", [(1, 64), (2560, 768), (333, 1024), (1000, 96), (7, 384)])
def test_layernorm(dtype, rows, width):
    rng = np.random.default_rng(rows + width)
    x = ti.to_storage(rng.standard_normal((rows, width)) * 2 + 0.5, dtype)
    g = 1 + rng.standard_normal(width) * 0.1
    b = rng.standard_normal(width) * 0.1
    y = torch.full((rows, width), float("nan"), dtype=dev(x[:1], dtype).dtype, device="cuda")
    tel.tel_layernorm(dev(x, dtype), y, dev_f32(g), dev_f32(b), EPS)
    torch.cuda.synchronize()
    assert_close(host(y), enc.layer_norm(x, g.astype(np.float32), b.astype(np.float32), EPS),
                 dtype, "layernorm")


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("M,N,K", [(300, 400, 320), (2557, 768, 768), (17, 1028, 64)])
def test_gemm_every_tile_config(dtype, M, N, K):
    """Each entry of the tile table (and the register-staged kernel) on ragged M and N."""
    a, w, b, r = _operands(M, N, K, dtype, seed=7 + M)
    A, W, R, bias = dev(a, dtype), dev(w, dtype), dev(r, dtype), dev_f32(b)
    ref = enc.linear(a, w, b) + r.astype(np.float64)
    for cfg in range(-1, tel.tel_gemm_tile_configs()):
        C = torch.full((M, N), float("nan"), dtype=A.dtype, device="cuda")
        tel.tel_gemm_ex(tel.TEL_EPI_BIAS_RESID, cfg, A, W, bias, C, resid=R)
        torch.cuda.synchronize()
        assert_close(host(C), ref, dtype, f"tile config {cfg} {dtype} {M}x{N}x{K}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("N,K", [(288, 96), (96, 96), (384, 96), (96, 384), (192, 192),
                                 (576, 192), (768, 192)])
def test_skinny_gemm_shapes(dtype, N, K):
    """The narrow projections of the shifted-window block (weights held in LDS, 8-column
    stores after a lane exchange), every plain epilogue, a ragged token count; at K 192
    (stage 2) the wider outputs run as 192-column slices side by side."""
    M = 1000
    a, w, b, r = _operands(M, N, K, dtype, seed=N + K)
    A, W, R = dev(a, dtype), dev(w, dtype), dev(r, dtype)
    bias = dev_f32(b)
    lin = enc.linear(a, w, b)
    for epi, ref in ((tel.TEL_EPI_BIAS, lin), (tel.TEL_EPI_BIAS_GELU, enc.gelu(lin)),
                     (tel.TEL_EPI_BIAS_RESID, lin + r.astype(np.float64))):
        C = torch.full((M, N), float("nan"), dtype=A.dtype, device="cuda")
        tel.tel_gemm(epi, A, W, bias, C, resid=R if epi == tel.TEL_EPI_BIAS_RESID else None)
        torch.cuda.synchronize()
        assert_close(host(C), ref, dtype, f"skinny epi {epi} {dtype} {M}x{N}x{K}")


@pytest.mark.parametrize("H,heads", [(96, 3), (96, 24), (192, 6)])
def test_skinny_qkv_split(H, heads):
    """QKV head split at the shifted-window block's widths (N 288, K 96; N 576, K 192 in
    three column slices): head_dim 32 runs on the skinny kernel, head_dim 4 (fewer than 8
    columns per head) on the tiled one."""
    M = 777
    a, w, b, _ = _operands(M, 3 * H, H, "f16", seed=heads)
    C = torch.full((3 * M * H,), float("nan"), dtype=torch.float16, device="cuda")
    tel.tel_gemm(tel.TEL_EPI_QKV_SPLIT, dev(a, "f16"), dev(w, "f16"), dev_f32(b), C, heads=heads)
    torch.cuda.synchronize()
    d = H // heads
    ref = enc.linear(a, w, b).reshape(M, 3, heads, d).transpose(1, 2, 0, 3)
    assert_close(host(C).reshape(3, heads, M, d), ref, "f16", f"qkv split heads {heads}")
