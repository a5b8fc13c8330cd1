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


# ------------------------------------------------------------------ offset mask with holes
def run_offsets_mask(mask):
    m = torch.from_numpy(np.asarray(mask, np.uint8)).cuda()
    B, S = m.shape
    cu = torch.full((B + 1,), -7, dtype=torch.int32, device="cuda")
    po = torch.full((B * S,), -7, dtype=torch.int32, device="cuda")
    tel.tel_build_offsets_mask(m, cu, po)
    torch.cuda.synchronize()
    T = int(np.asarray(mask).astype(bool).sum())
    return m, cu, po, T


def _masks():
    rng = np.random.default_rng(21)
    out = [np.array([[1, 0, 1, 1], [0, 0, 0, 0], [0, 1, 0, 1]]),   # hand-worked fixture
           np.zeros((3, 5), np.uint8), np.ones((2, 300), np.uint8)]
    for B, S, p in ((5, 7, 0.5), (8, 256, 0.3), (3, 700, 0.8), (20000, 9, 0.5), (4097, 16, 0.9)):
        out.append((rng.random((B, S)) < p).astype(np.uint8) * rng.integers(1, 256, (B, S)).astype(np.uint8))
    return out


@pytest.mark.parametrize("idx", range(8))
def test_offsets_mask_bit_exact(idx):
    """Holes anywhere, empty and full sequences, more positions than one workgroup pass
    (S 300, 700), batch sizes across the scan's tiles; mask bytes other than 0/1 count as
    valid."""
    mask = _masks()[idx]
    _, cu, po, T = run_offsets_mask(mask)
    ref_cu, ref_po = enc.offsets_from_mask(mask)
    assert np.array_equal(cu.cpu().numpy(), ref_cu)
    assert np.array_equal(po.cpu().numpy()[:T], ref_po)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32, torch.int8])
def test_remove_rebuild_mask_bit_exact(dtype):
    rng = np.random.default_rng(22)
    B, S, W = 6, 37, 96
    mask = (rng.random((B, S)) < 0.55).astype(np.uint8)
    mask[2] = 0                                            # an empty sequence
    x = rng.standard_normal((B, S, W)) * 3
    xt = torch.from_numpy(x).to(dtype).cuda() if dtype != torch.int8 else \
        torch.from_numpy(np.clip(np.rint(x * 20), -127, 127).astype(np.int8)).cuda()
    m, cu, po, T = run_offsets_mask(mask)
    packed = torch.zeros((T, W), dtype=dtype, device="cuda")
    tel.tel_remove_padding(xt, packed, po, T)
    back = torch.full_like(xt, 7)
    tel.tel_rebuild_padding_mask(packed, back, m, po, T)
    torch.cuda.synchronize()
    xh = xt.cpu().numpy()
    assert np.array_equal(packed.cpu().numpy(), enc.remove_padding_mask(xh, mask))
    assert np.array_equal(back.cpu().numpy(), enc.rebuild_padding_mask(packed.cpu().numpy(), mask))


def test_layer_on_a_batch_with_holes():
    """Offsets from a mask with holes, removal, one fp16 encoder layer on the packed tokens,
    rebuild by the mask: the oracle's layer on the same packed tokens, holes zero."""
    import tel_inputs as ti
    from tests.gpu_helpers import assert_close
    rng = np.random.default_rng(23)
    B, S, H, nh, F = 6, 80, 256, 4, 512
    mask = (rng.random((B, S)) < 0.7).astype(np.uint8)
    mask[:, 0] = 1
    cfg = ti.custom_encoder_config(B, S, [S] * B, H, nh, F, dtype="f16", seed=24)
    _, x = ti.encoder_input(cfg)
    w = ti.encoder_layer_weights(cfg, 0, variant=True)
    m, cu, po, T = run_offsets_mask(mask)
    desc = tel.make_encoder_desc(H, nh, F, torch.float16, ti.LN_EPS)
    packed_w = tel.alloc_bytes(tel.tel_encoder_packed_size(desc))
    tel.tel_encoder_prepare(desc, {k: torch.from_numpy(np.asarray(v, np.float32)).cuda().half()
                                   for k, v in w.items()}, packed_w)
    xd = torch.from_numpy(x).cuda()
    xp = torch.empty((T, H), dtype=torch.float16, device="cuda")
    yp = torch.empty_like(xp)
    tel.tel_remove_padding(xd, xp, po, T)
    ws = tel.alloc_bytes(tel.tel_encoder_workspace_size(desc, T))
    tel.tel_encoder_layer_forward(desc, packed_w, xp, yp, cu, T, int(mask.sum(axis=1).max()), ws)
    y = torch.full_like(xd, float("nan"))
    tel.tel_rebuild_padding_mask(yp, y, m, po, T)
    torch.cuda.synchronize()
    ref_cu, _ = enc.offsets_from_mask(mask)
    ref = enc.rebuild_padding_mask(
        enc.encoder_layer(enc.remove_padding_mask(x.astype(np.float64), mask), ref_cu, w, nh,
                          ti.LN_EPS), mask)
    yh = y.float().cpu().numpy().astype(np.float64)
    assert not yh[mask == 0].any()
    assert_close(yh[mask == 1], ref[mask == 1], "f16", "layer with holes")
