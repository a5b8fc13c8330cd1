"""GPU parity of the 2:4 structured-sparse path against oracle/sparse.py: the pruning
kernel bit for bit (kept values and index words), and the sparse-MFMA GEMM
(tel_gemm_2of4) with every epilogue and tile configuration on ragged shapes, against the
dense product with the oracle's pruned weights."""
import numpy as np
import pytest
import torch

import tel_inputs as ti
from oracle import encoder as enc
from oracle import sparse as sp
from tests.gpu_helpers import TORCH_DT, assert_close, dev, dev_f32, host

pytestmark = pytest.mark.gpu

tel = pytest.importorskip("transformer_encoder_remove_amd")


def _prune_gpu(w_np, dtype):
    N, K = w_np.shape
    W = dev(w_np, dtype)
    values = torch.full((N, K // 2), float("nan"), dtype=TORCH_DT[dtype], device="cuda")
    index = torch.full((N, K // 16), -1, dtype=torch.int16, device="cuda")
    tel.tel_prune_2of4(W, values, index)
    torch.cuda.synchronize()
    return values, index


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prune_bit_exact(dtype):
    rng = np.random.default_rng(0)
    # small integers (many ties and zeros) and continuous values
    w = np.concatenate([rng.integers(-3, 4, size=(37, 96)) * 0.25,
                        ti.to_storage(rng.standard_normal((37, 96)), dtype)])
    values, index = _prune_gpu(w, dtype)
    rv, ri = sp.compress_2of4(w)
    assert np.array_equal(host(values), rv)
    got_idx = index.cpu().numpy().view(np.uint16)
    assert np.array_equal(got_idx, ri)


def _sparse_case(M, N, K, dtype, seed):
    rng = np.random.default_rng(seed)
    a = ti.to_storage(rng.standard_normal((M, K)), dtype)
    w = ti.to_storage(rng.standard_normal((N, K)) / np.sqrt(K / 2), dtype)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    return a, w, b


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_sparse_gemm_every_config(dtype):
    """Ragged M and N (not multiples of any tile) under every tile configuration."""
    M, N, K = 300, 392, 384
    a, w, b = _sparse_case(M, N, K, dtype, seed=1)
    values, index = _prune_gpu(w, dtype)
    ref = enc.linear(a, sp.prune_2of4(w), b)
    A = dev(a, dtype)
    for cfg in range(tel.tel_gemm_2of4_tile_configs()):
        C = torch.full((M, N), float("nan"), dtype=TORCH_DT[dtype], device="cuda")
        tel.tel_gemm_2of4(tel.TEL_EPI_BIAS, A, values, index, dev_f32(b), C, tile_config=cfg)
        torch.cuda.synchronize()
        assert_close(host(C), ref, dtype, f"sparse GEMM {dtype} cfg {cfg}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_sparse_gemm_epilogues(dtype):
    M, H, heads = 259, 256, 4
    rng = np.random.default_rng(2)
    a, w, b = _sparse_case(M, 3 * H, H, dtype, seed=2)
    values, index = _prune_gpu(w, dtype)
    A = dev(a, dtype)
    lin = enc.linear(a, sp.prune_2of4(w), b)
    # bias + GELU
    C = torch.empty((M, 3 * H), dtype=TORCH_DT[dtype], device="cuda")
    tel.tel_gemm_2of4(tel.TEL_EPI_BIAS_GELU, A, values, index, dev_f32(b), C)
    torch.cuda.synchronize()
    assert_close(host(C), enc.gelu(lin), dtype, "bias + GELU")
    # QKV split [3][heads][M][d]
    tel.tel_gemm_2of4(tel.TEL_EPI_QKV_SPLIT, A, values, index, dev_f32(b), C, heads=heads)
    torch.cuda.synchronize()
    d = H // heads
    ref = lin.reshape(M, 3, heads, d).transpose(1, 2, 0, 3).reshape(-1)
    assert_close(host(C).reshape(-1), ref, dtype, "QKV split")
    # bias + residual
    r = ti.to_storage(rng.standard_normal((M, 3 * H)), dtype)
    tel.tel_gemm_2of4(tel.TEL_EPI_BIAS_RESID, A, values, index, dev_f32(b), C, resid=dev(r, dtype))
    torch.cuda.synchronize()
    assert_close(host(C), lin + r, dtype, "bias + residual")


@pytest.mark.parametrize("M,N,K", [(2557, 768, 3072), (2557, 3072, 768), (1, 128, 128),
                                   (64, 768, 768)])
def test_sparse_gemm_shapes_auto(M, N, K):
    """BERT-base FFN2 and FFN1 at 2557 tokens, a single row, one tile row."""
    a, w, b = _sparse_case(M, N, K, "f16", seed=M + K)
    values, index = _prune_gpu(w, "f16")
    C = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    tel.tel_gemm_2of4(tel.TEL_EPI_BIAS, dev(a, "f16"), values, index, dev_f32(b), C)
    torch.cuda.synchronize()
    assert_close(host(C), enc.linear(a, sp.prune_2of4(w), b), "f16", f"{M}x{N}x{K}")


def _sparse_stack(cfg, layers, lens=None, x=None):
    from tests.gpu_helpers import prepare_layers
    dt = cfg["dtype"]
    if lens is None:
        lens, x = ti.encoder_input(cfg)
    ws = [ti.encoder_layer_weights(cfg, i, variant=True) for i in range(layers)]
    desc = tel.make_encoder_desc(cfg["hidden"], cfg["heads"], cfg["ffn"], TORCH_DT[dt], ti.LN_EPS,
                                 sparse_2of4=True)
    packed = prepare_layers(tel, desc, ws, dt)
    B, S, H = x.shape
    X = dev(x, dt)
    Y = torch.full_like(X, float("nan"))
    lens_d = torch.from_numpy(np.asarray(lens, np.int32)).to("cuda")
    wsb = tel.alloc_bytes(tel.tel_encoder_forward_workspace_size(desc, B, S))
    tel.tel_encoder_forward(desc, packed, X, Y, lens_d, int(np.sum(lens)), int(np.max(lens)), wsb)
    torch.cuda.synchronize()
    pruned = [sp.prune_layer_weights(w) for w in ws]
    return lens, x, host(Y), pruned


@pytest.mark.parametrize("dtype,layers", [("f16", 2), ("bf16", 1)])
def test_sparse_encoder_stack(dtype, layers):
    """The whole path with 2:4 layers against the oracle's encoder on pruned weights; ragged
    lengths, an empty sequence and one single-token sequence."""
    cfg = ti.custom_encoder_config(4, 70, [70, 1, 0, 45], 256, 4, 1024, dtype=dtype, seed=11,
                                   layers=layers)
    lens, x, y, pruned = _sparse_stack(cfg, layers)
    ref = enc.encoder_forward(x, lens, pruned, cfg["heads"], ti.LN_EPS)
    assert_close(y, ref, dtype, f"sparse stack {dtype}")


def test_sparse_bert_base_one_layer_full_batch():
    """One BERT-base layer with 2:4 weights on the full seeded batch (what the benchmark's
    sparse line runs, one layer of it)."""
    cfg = dict(ti.ENCODER_CONFIGS["bert_base"])
    lens, x, y, pruned = _sparse_stack(cfg, 1)
    ref = enc.encoder_forward(x, lens, pruned, cfg["heads"], ti.LN_EPS)
    assert_close(enc.remove_padding(y, lens), enc.remove_padding(ref, lens), "f16",
                 "sparse bert_base layer")
