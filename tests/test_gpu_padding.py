"""GPU parity, bit-exact: offsets, padding removal and rebuild against the oracle."""
import numpy as np
import pytest
import torch

from oracle import encoder as enc

pytestmark = pytest.mark.gpu

tel = pytest.importorskip("transformer_encoder_remove_amd")


def run_offsets(lens, S):
    lens_d = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    B = len(lens)
    cu = torch.full((B + 1,), -7, dtype=torch.int32, device="cuda")
    po = torch.full((max(1, B * S),), -7, dtype=torch.int32, device="cuda")
    tel.tel_build_offsets(lens_d, S, cu, po)
    torch.cuda.synchronize()
    T = int(np.sum(lens))
    return cu.cpu().numpy(), po.cpu().numpy()[:T], po.cpu().numpy()[T:]


@pytest.mark.parametrize("lens,S", [
    ([5, 8], 8), ([0, 3, 0, 7], 7), ([1], 1), ([128] * 4, 128), ([0], 4),
])
def test_offsets_bit_exact(lens, S):
    cu, po, tail = run_offsets(lens, S)
    ref_cu, ref_po = enc.offsets(lens, S)
    assert np.array_equal(cu, ref_cu) and np.array_equal(po, ref_po)
    assert (tail == -7).all()                      # nothing written past T


@pytest.mark.parametrize("B", [4095, 4096, 4097, 16384, 16385, 20000])
def test_offsets_tile_boundaries(B):
    """Batch sizes around the scan's 4096-length tiles and its 4-tile look-ahead groups."""
    rng = np.random.default_rng(B)
    lens = rng.integers(0, 65, size=B)
    cu, po, tail = run_offsets(lens, 64)
    ref_cu, ref_po = enc.offsets(lens, 64)
    assert np.array_equal(cu, ref_cu) and np.array_equal(po, ref_po)
    assert (tail == -7).all()


def test_offsets_large_batch():
    """B = 65,536 sequences of U{0..512} tokens (T near 2^24): the one-workgroup scan's
    chunked path and the per-sequence fill."""
    import tel_inputs as ti
    lens = ti.offsets_stress_lengths()
    S = ti.OFFSETS_STRESS["max_seq"]
    cu, po, _ = run_offsets(lens, S)
    ref_cu, ref_po = enc.offsets(lens, S)
    assert np.array_equal(cu, ref_cu) and np.array_equal(po, ref_po)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16, torch.float32, torch.int8])
@pytest.mark.parametrize("lens,S,W", [([5, 8], 8, 64), ([0, 3, 1, 9], 9, 768), ([37] * 3, 40, 96)])
def test_remove_rebuild_bit_exact(dtype, lens, S, W):
    rng = np.random.default_rng(5)
    B = len(lens)
    if dtype == torch.int8:
        x_np = rng.integers(-128, 128, size=(B, S, W)).astype(np.int8)
        x = torch.from_numpy(x_np).cuda()
    else:
        x_np = rng.standard_normal((B, S, W)).astype(np.float32)
        x = torch.from_numpy(x_np).cuda().to(dtype)
        x_np = x.float().cpu().numpy()
    lens_d = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    cu = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    po = torch.empty(B * S, dtype=torch.int32, device="cuda")
    tel.tel_build_offsets(lens_d, S, cu, po)
    T = int(sum(lens))
    packed = torch.empty((max(T, 1), W), dtype=dtype, device="cuda")
    tel.tel_remove_padding(x, packed, po, T)
    back = torch.full_like(x, 3)
    tel.tel_rebuild_padding(packed, back, cu)
    torch.cuda.synchronize()
    ref_packed = enc.remove_padding(x_np, lens)
    ref_back = enc.rebuild_padding(ref_packed, lens, S)
    got_p = packed[:T].cpu().numpy() if dtype == torch.int8 else packed[:T].float().cpu().numpy()
    got_b = back.cpu().numpy() if dtype == torch.int8 else back.float().cpu().numpy()
    assert np.array_equal(got_p, ref_packed)
    assert np.array_equal(got_b, ref_back)         # pads are exactly zero
