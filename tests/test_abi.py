"""The C-ABI library loads, exports every symbol include/tel.h declares, and validates
arguments on the host before touching the GPU. CPU only: no call here reaches a kernel."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tel.h")

tel = pytest.importorskip("transformer_encoder_remove_amd",
                          reason="libtel.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tel_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(tel.EXPORTS)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(tel.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    assert "gfx950" in tel.tel_version()
    assert tel.tel_status_str(0) == "TEL_OK"
    assert "TEL_EINVAL" in tel.tel_status_str(1)
    assert "unknown" in tel.tel_status_str(99)


L = tel.lib
FAKE = ctypes.c_void_p(1 << 20)          # never dereferenced: validation fails first
FAKE_ODD = ctypes.c_void_p((1 << 20) + 2)


def test_offsets_validation():
    assert L.tel_build_offsets(None, 2, 8, FAKE, FAKE, None) == tel.TEL_EINVAL
    assert L.tel_build_offsets(FAKE, 0, 8, FAKE, FAKE, None) == tel.TEL_EINVAL
    assert L.tel_build_offsets(FAKE, 2, 0, FAKE, FAKE, None) == tel.TEL_EINVAL
    assert L.tel_build_offsets(FAKE, 1 << 20, 1 << 12, FAKE, FAKE, None) == tel.TEL_EUNSUPPORTED


def test_padding_validation():
    f16 = tel.TEL_F16
    assert L.tel_remove_padding(FAKE, FAKE, FAKE, -1, 64, f16, None) == tel.TEL_EINVAL
    assert L.tel_remove_padding(FAKE, FAKE, FAKE, 0, 64, f16, None) == tel.TEL_OK   # no-op
    assert L.tel_remove_padding(None, FAKE, FAKE, 3, 64, f16, None) == tel.TEL_EINVAL
    assert L.tel_remove_padding(FAKE_ODD, FAKE, FAKE, 3, 64, f16, None) == tel.TEL_EINVAL
    assert L.tel_remove_padding(FAKE, FAKE, FAKE, 3, 12, f16, None) == tel.TEL_EUNSUPPORTED
    assert L.tel_remove_padding(FAKE, FAKE, FAKE, 3, 64, 9, None) == tel.TEL_EINVAL
    assert L.tel_rebuild_padding(FAKE, FAKE, FAKE, 0, 8, 64, f16, None) == tel.TEL_EINVAL
    assert L.tel_rebuild_padding(FAKE, FAKE, None, 2, 8, 64, f16, None) == tel.TEL_EINVAL
    assert L.tel_rebuild_padding(FAKE, FAKE, FAKE, 2, 8, 4, f16, None) == tel.TEL_EUNSUPPORTED


def desc(**kw):
    d = dict(hidden=768, heads=12, ffn=3072, dtype=tel.TEL_F16, int8_gemm=0, ln_eps=1e-5)
    d.update(kw)
    return tel.tel_encoder_desc(**d)


def test_encoder_desc_validation_and_sizes():
    good = desc()
    assert tel.tel_encoder_packed_size(good) > 2 * (12 * 768 * 768)
    assert tel.tel_encoder_packed_size(desc(heads=7)) == 0            # 768 % 7
    assert tel.tel_encoder_packed_size(desc(hidden=96, heads=2)) == 0  # head_dim 48
    assert tel.tel_encoder_workspace_size(good, 2560) >= 2 * 2560 * (6 * 768 + 3072)
    assert tel.tel_encoder_workspace_size(good, 0) == 0
    assert tel.tel_encoder_forward_workspace_size(good, 32, 128) > \
        tel.tel_encoder_workspace_size(good, 32 * 128)


def test_layer_forward_validation():
    d = desc()
    ws_need = tel.tel_encoder_workspace_size(d, 100)
    args = lambda **kw: dict(dict(packed=FAKE, x=FAKE, y=ctypes.c_void_p(2 << 20), cu=FAKE,
                                  batch=2, T=100, max_len=64, ws=FAKE, wsb=ws_need), **kw)

    def call(**kw):
        a = args(**kw)
        return L.tel_encoder_layer_forward(ctypes.byref(kw.get("d", d)), a["packed"], a["x"],
                                           a["y"], a["cu"], a["batch"], a["T"], a["max_len"],
                                           a["ws"], a["wsb"], None)
    assert call(T=0) == tel.TEL_OK
    assert call(batch=0) == tel.TEL_EINVAL
    assert call(T=-1) == tel.TEL_EINVAL
    assert call(max_len=0) == tel.TEL_EINVAL
    assert call(x=None) == tel.TEL_EINVAL
    assert call(y=FAKE) == tel.TEL_EINVAL                               # aliasing
    assert call(ws=FAKE_ODD) == tel.TEL_EINVAL                          # misaligned
    assert call(wsb=ws_need - 1) == tel.TEL_EWORKSPACE
    assert call(d=desc(dtype=tel.TEL_I8)) == tel.TEL_EUNSUPPORTED
    assert call(d=desc(hidden=0)) == tel.TEL_EINVAL


def test_kernel_entry_validation():
    f16 = tel.TEL_F16
    assert L.tel_gemm(0, f16, FAKE, FAKE, FAKE, None, FAKE, 16, 64, 12, 1, None) == \
        tel.TEL_EUNSUPPORTED                                            # K % 8
    assert L.tel_gemm(2, f16, FAKE, FAKE, FAKE, None, FAKE, 16, 64, 64, 1, None) == tel.TEL_EINVAL
    assert L.tel_gemm(9, f16, FAKE, FAKE, FAKE, None, FAKE, 16, 64, 64, 1, None) == tel.TEL_EINVAL
    assert L.tel_gemm(3, f16, FAKE, FAKE, FAKE, None, FAKE, 16, 96, 64, 5, None) == \
        tel.TEL_EUNSUPPORTED
    assert L.tel_gemm(0, f16, FAKE, FAKE, FAKE, None, FAKE, 0, 64, 64, 1, None) == tel.TEL_OK
    assert L.tel_attention_varlen(FAKE, FAKE, FAKE, 2, 10, 8, 2, 48, f16, None) == \
        tel.TEL_EUNSUPPORTED
    assert L.tel_attention_varlen(FAKE, FAKE, FAKE, 2, 10, 0, 2, 64, f16, None) == tel.TEL_EINVAL
    assert L.tel_layernorm(FAKE, FAKE, FAKE, FAKE, 4, 20, 1e-5, f16, None) == tel.TEL_EUNSUPPORTED
    assert L.tel_layernorm(FAKE, FAKE, FAKE, FAKE, 4, 64, -1.0, f16, None) == tel.TEL_EINVAL


def test_partial_plan_invariants():
    """The k-split plan of the output projection / FFN2 GEMMs (host logic): 32-bit partial
    sums only when the unsplit tile grid is under 100 workgroups, a power of two up to 8,
    whole 128-byte slices with at least 8 per split, the smallest split reaching 100
    workgroups and then as many doublings as one round of 256 holds; fp16
    partials only for fp16 operands, K >= 2048, a 64-row unsplit tile filling one round of
    256 workgroups, and then two splits of the 128 x 128 tile that still fill one round."""
    # (BM, BN) of the pipelined tile table, in its order (gemm.hip PIPE_CFGS)
    cfgs = [(128, 256), (128, 192), (128, 128), (64, 128), (64, 64), (128, 256), (256, 128),
            (128, 128), (64, 128), (192, 192), (96, 128), (32, 64)]
    assert len(cfgs) == tel.tel_gemm_tile_configs()
    for dt, es in ((tel.TEL_F16, 2), (tel.TEL_BF16, 2), (tel.TEL_F32, 4), (tel.TEL_I8, 1)):
        for M in (1, 17, 128, 640, 2557, 14336, 24576):
            for N, K in ((768, 768), (768, 3072), (1024, 1024), (1024, 4096), (64, 256)):
                cfg, sp, pb = tel.tel_gemm_partial_plan(dt, M, N, K)
                nk = K * es // 128
                assert 0 <= cfg < tel.tel_gemm_tile_configs() and sp in (1, 2, 4, 8), \
                    (dt, M, N, K, cfg, sp)
                assert pb in (2, 4) and (pb == 4 or dt == tel.TEL_F16)
                bm, bn = cfgs[cfg]
                tiles = -(-M // bm) * -(-N // bn)
                if pb == 2:
                    assert (cfg, sp) == (2, 2) and K >= 2048 and 2 * tiles <= 256
                    assert nk % 2 == 0 and nk // 2 >= 8
                elif sp > 1:
                    assert tiles < 100 and nk % sp == 0 and nk // sp >= 8
                    # the smallest split that reaches 100 workgroups, then doublings that
                    # keep the grid within one round of 256
                    assert tiles * sp // 2 < 100 or tiles * sp <= 256
                    # and no further doubling was possible
                    assert (sp == 8 or tiles * sp * 2 > 256 or nk % (2 * sp) or
                            nk // (2 * sp) < 8)
                else:
                    assert tiles >= 100 or nk % 2 or nk // 2 < 8
    # a 128-token batch at BERT-large shape: 32 x 64 tiles (64 of them), the output
    # projection split in 2 (8 k-slices each), FFN2 in 4 (one round of 256 workgroups)
    assert tel.tel_gemm_partial_plan(tel.TEL_F16, 128, 1024, 1024) == (11, 2, 4)
    assert tel.tel_gemm_partial_plan(tel.TEL_F16, 128, 1024, 4096) == (11, 4, 4)
    # 2557 tokens at BERT-base shape: output projection and FFN2 (K 3072, one round of
    # 240 tiles of 64 x 128) unsplit, in every type
    assert tel.tel_gemm_partial_plan(tel.TEL_F16, 2557, 768, 768)[1] == 1
    assert tel.tel_gemm_partial_plan(tel.TEL_F16, 2557, 768, 3072)[1:] == (1, 4)
    assert tel.tel_gemm_partial_plan(tel.TEL_BF16, 2557, 768, 3072)[1:] == (1, 4)
    assert tel.tel_gemm_partial_plan(tel.TEL_I8, 2900, 768, 3072)[1:] == (1, 4)
    # BERT-large throughput batch: many rounds of 128 x 256 tiles, no split
    assert tel.tel_gemm_partial_plan(tel.TEL_F16, 13537, 1024, 4096)[1] == 1
    # K not a whole number of 128-byte slices: register-staged kernel, no split
    assert tel.tel_gemm_partial_plan(tel.TEL_F16, 100, 64, 72) == (-1, 1, 4)


def test_workspace_non_decreasing_in_tokens():
    """A workspace sized for T tokens serves every smaller batch, although fewer tokens
    can mean more k-splits (more partial-sum rows per token)."""
    for kw in (dict(), dict(int8_gemm=1), dict(dtype=tel.TEL_BF16),
               dict(hidden=1024, heads=16, ffn=4096)):
        d = desc(**kw)
        sizes = [tel.tel_encoder_workspace_size(d, t) for t in range(1, 3000, 37)]
        assert all(a <= b for a, b in zip(sizes, sizes[1:])), kw


def test_partial_gemm_and_reduce_validation():
    f16, bf16, f32 = tel.TEL_F16, tel.TEL_BF16, tel.TEL_F32
    P = L.tel_gemm_partial
    assert P(f16, 0, 1, FAKE, FAKE, FAKE, 4, 0, 64, 64, None) == tel.TEL_OK          # empty
    assert P(f16, 0, 0, FAKE, FAKE, FAKE, 4, 16, 64, 64, None) == tel.TEL_EINVAL     # splits
    assert P(f16, -2, 1, FAKE, FAKE, FAKE, 4, 16, 64, 64, None) == tel.TEL_EINVAL    # no auto
    assert P(f16, -1, 2, FAKE, FAKE, FAKE, 4, 16, 64, 128, None) == tel.TEL_EUNSUPPORTED
    assert P(f16, 0, 3, FAKE, FAKE, FAKE, 4, 16, 64, 256, None) == tel.TEL_EUNSUPPORTED
    assert P(f16, 0, 1, FAKE, FAKE, FAKE, 4, 16, 64, 72, None) == tel.TEL_EUNSUPPORTED   # 144 B
    assert P(tel.TEL_I8, -1, 1, FAKE, FAKE, FAKE, 4, 16, 64, 24, None) == tel.TEL_EUNSUPPORTED
    assert P(f16, 0, 1, FAKE_ODD, FAKE, FAKE, 4, 16, 64, 64, None) == tel.TEL_EINVAL
    assert P(f16, 0, 1, FAKE, FAKE, FAKE, 3, 16, 64, 64, None) == tel.TEL_EINVAL     # width
    assert P(bf16, 0, 1, FAKE, FAKE, FAKE, 2, 16, 64, 64, None) == tel.TEL_EUNSUPPORTED
    assert P(tel.TEL_I8, 0, 1, FAKE, FAKE, FAKE, 2, 16, 64, 128, None) == tel.TEL_EUNSUPPORTED
    R = L.tel_layernorm_reduce
    ok = [FAKE, 1, 4, None, FAKE, FAKE, f16, FAKE, f16, None, None, None, FAKE, FAKE, 4, 64,
          1e-5, 0, None]

    def call(**kw):
        a = list(ok)
        names = ["part", "splits", "pbytes", "dq", "bias", "resid", "rdt", "y", "odt", "y32",
                 "yq", "qinv", "g", "b", "rows", "width", "eps", "round", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return R(*a)
    assert call(rows=0) == tel.TEL_OK
    assert call(splits=0) == tel.TEL_EINVAL
    assert call(splits=9) == tel.TEL_EINVAL
    assert call(rdt=f16, odt=bf16) == tel.TEL_EUNSUPPORTED
    assert call(rdt=bf16, odt=f32) == tel.TEL_EUNSUPPORTED
    assert call(width=20) == tel.TEL_EUNSUPPORTED
    assert call(bias=None) == tel.TEL_EINVAL
    assert call(yq=FAKE) == tel.TEL_EINVAL                                     # no qinv
    assert call(resid=FAKE_ODD) == tel.TEL_EINVAL
    assert call(eps=float("nan")) == tel.TEL_EINVAL
    assert call(pbytes=8) == tel.TEL_EINVAL
    assert call(pbytes=2, rdt=bf16, odt=bf16) == tel.TEL_EUNSUPPORTED          # fp16 only
    assert call(pbytes=2, dq=FAKE) == tel.TEL_EUNSUPPORTED                     # not int32


def test_sparse_2of4_validation():
    f16 = tel.TEL_F16
    Pr = L.tel_prune_2of4
    assert Pr(FAKE, FAKE, FAKE, 0, 64, f16, None) == tel.TEL_OK                 # empty
    assert Pr(FAKE, FAKE, FAKE, 4, 24, f16, None) == tel.TEL_EUNSUPPORTED       # K % 16
    assert Pr(FAKE, FAKE, FAKE, 4, 64, tel.TEL_F32, None) == tel.TEL_EUNSUPPORTED
    assert Pr(FAKE_ODD, FAKE, FAKE, 4, 64, f16, None) == tel.TEL_EINVAL
    assert Pr(FAKE, FAKE, ctypes.c_void_p((1 << 20) + 1), 4, 64, f16, None) == tel.TEL_EINVAL
    assert Pr(None, FAKE, FAKE, 4, 64, f16, None) == tel.TEL_EINVAL
    G = L.tel_gemm_2of4
    n = tel.tel_gemm_2of4_tile_configs()
    assert n >= 1
    args = [tel.TEL_EPI_BIAS, f16, -2, FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, 64, 128, 1, None]
    assert G(*args) == tel.TEL_OK                                              # empty
    bad = list(args); bad[11] = 64                                             # K % 128
    assert G(*bad) == tel.TEL_EUNSUPPORTED
    bad = list(args); bad[2] = n                                               # tile config
    assert G(*bad) == tel.TEL_EINVAL
    bad = list(args); bad[2] = -1                                              # no staged kernel
    assert G(*bad) == tel.TEL_EINVAL
    bad = list(args); bad[1] = tel.TEL_I8
    assert G(*bad) == tel.TEL_EUNSUPPORTED
    bad = list(args); bad[0] = tel.TEL_EPI_BIAS_RESID; bad[9] = 4              # no residual
    assert G(*bad) == tel.TEL_EINVAL
    bad = list(args); bad[9] = 4; bad[3] = FAKE_ODD
    assert G(*bad) == tel.TEL_EINVAL


def test_sparse_encoder_desc():
    dense = tel.tel_encoder_packed_size(desc())
    sparse = tel.tel_encoder_packed_size(desc(sparse_2of4=1))
    # weights: half the values plus one 16-bit word per 16 weights (9/16 of the dense bytes)
    w = 12 * 768 * 768 * 2
    assert sparse < dense and abs((dense - sparse) - (w - w * 9 // 16)) < 64 * 1024
    assert tel.tel_encoder_packed_size(desc(sparse_2of4=1, dtype=tel.TEL_BF16)) == sparse
    for bad in (dict(int8_gemm=1), dict(dtype=tel.TEL_F32), dict(hidden=640, heads=10),
                dict(ffn=3000)):
        assert tel.tel_encoder_packed_size(desc(sparse_2of4=1, **bad)) == 0, bad


def test_swin_flag_validation():
    import torch
    d = tel.make_swin_desc(2, 56, 56, 96, 3, 7, 3, 384, torch.float16)
    wsb = tel.tel_swin_workspace_size(d)
    assert wsb > 0
    y = ctypes.c_void_p(2 << 20)

    def call(flags):
        return L.tel_window_attention_forward(ctypes.byref(d), FAKE, FAKE, y, flags, FAKE, wsb,
                                              None)
    assert call(2) == tel.TEL_EINVAL                                           # unknown bit
    assert call(tel.TEL_SWIN_ONE_STAGE(5)) == tel.TEL_EINVAL                   # no stage 5
    assert call(tel.TEL_SWIN_ONE_STAGE(14)) == tel.TEL_EINVAL
    assert call(1 << 12) == tel.TEL_EINVAL
    assert call(tel.TEL_SWIN_ONE_STAGE(0) | tel.TEL_SWIN_ATTN_ONLY) == tel.TEL_EINVAL
    assert L.tel_window_attention_forward(ctypes.byref(d), FAKE, FAKE, y, 0, FAKE, wsb - 1,
                                          None) == tel.TEL_EWORKSPACE


def test_offsets_mask_validation():
    f16 = tel.TEL_F16
    assert L.tel_build_offsets_mask(None, 2, 8, FAKE, FAKE, None) == tel.TEL_EINVAL
    assert L.tel_build_offsets_mask(FAKE, 0, 8, FAKE, FAKE, None) == tel.TEL_EINVAL
    assert L.tel_build_offsets_mask(FAKE, 2, 0, FAKE, FAKE, None) == tel.TEL_EINVAL
    assert L.tel_build_offsets_mask(FAKE, 1 << 20, 1 << 12, FAKE, FAKE, None) == \
        tel.TEL_EUNSUPPORTED
    R = L.tel_rebuild_padding_mask
    assert R(FAKE, FAKE, FAKE, FAKE, -1, 2, 8, 64, f16, None) == tel.TEL_EINVAL
    assert R(FAKE, FAKE, FAKE, FAKE, 17, 2, 8, 64, f16, None) == tel.TEL_EINVAL    # T > B*S
    assert R(FAKE, FAKE, None, FAKE, 3, 2, 8, 64, f16, None) == tel.TEL_EINVAL     # no mask
    assert R(FAKE, FAKE, FAKE, None, 3, 2, 8, 64, f16, None) == tel.TEL_EINVAL
    assert R(FAKE, FAKE_ODD, FAKE, FAKE, 3, 2, 8, 64, f16, None) == tel.TEL_EINVAL
    assert R(FAKE, FAKE, FAKE, FAKE, 3, 2, 8, 12, f16, None) == tel.TEL_EUNSUPPORTED
    assert R(FAKE, FAKE, FAKE, FAKE, 3, 2, 8, 64, 9, None) == tel.TEL_EINVAL


def test_noalloc_layer_validation():
    """tel_encoder_layer_forward_noalloc checks its arguments and the scratch limit on the
    host before looking up the scratch or enqueueing anything."""
    desc = tel.make_encoder_desc(768, 12, 3072, __import__("torch").float16, 1e-5)
    pd = ctypes.byref(desc)
    F = tel.lib.tel_encoder_layer_forward_noalloc
    A256 = ctypes.c_void_p(1 << 20)
    ok_T = 2557
    assert tel.tel_encoder_workspace_size(desc, ok_T) <= tel.TEL_NOALLOC_SCRATCH_BYTES
    big_T = 5000
    assert tel.tel_encoder_workspace_size(desc, big_T) > tel.TEL_NOALLOC_SCRATCH_BYTES
    # the limit the header states for this layer is exact
    limit = 4241
    assert "up to 4,241 tokens" in open(HEADER).read()
    assert tel.tel_encoder_workspace_size(desc, limit) <= tel.TEL_NOALLOC_SCRATCH_BYTES
    assert tel.tel_encoder_workspace_size(desc, limit + 1) > tel.TEL_NOALLOC_SCRATCH_BYTES
    assert F(pd, A256, A256, ctypes.c_void_p((1 << 20) + 4096), A256, 2, big_T, 128, None) == \
        tel.TEL_EWORKSPACE
    assert F(pd, A256, A256, A256, A256, 2, 100, 64, None) == tel.TEL_EINVAL        # x == y
    assert F(pd, None, A256, ctypes.c_void_p(2 << 20), A256, 2, 100, 64, None) == tel.TEL_EINVAL
    assert F(pd, A256, A256, ctypes.c_void_p(2 << 20), A256, 0, 100, 64, None) == tel.TEL_EINVAL
    assert F(pd, A256, A256, ctypes.c_void_p(2 << 20), A256, 2, 0, 0, None) == tel.TEL_OK
    assert tel.TEL_NOALLOC_SCRATCH_BYTES == 64 << 20
    text = open(HEADER).read()
    assert "#define TEL_NOALLOC_SCRATCH_BYTES (64u << 20)" in text


def test_binding_refuses_non_int32_lengths_and_wrong_activation_type():
    import torch
    with pytest.raises(TypeError):
        tel.tel_build_offsets(torch.zeros(4, dtype=torch.int64), 8, torch.zeros(5, dtype=torch.int32),
                              torch.zeros(32, dtype=torch.int32))
    desc = tel.make_encoder_desc(64, 4, 256, torch.float16, 1e-5)
    with pytest.raises(TypeError):
        tel.tel_encoder_layer_forward(desc, None, torch.zeros((3, 64), dtype=torch.float32),
                                      torch.zeros((3, 64), dtype=torch.float32),
                                      torch.tensor([0, 3], dtype=torch.int32), 3, 3, None)
    with pytest.raises(TypeError):
        tel.tel_encoder_layer_forward(desc, None, torch.zeros((3, 64), dtype=torch.float16),
                                      torch.zeros((3, 64), dtype=torch.float16),
                                      torch.tensor([0, 3], dtype=torch.int64), 3, 3, None)


def test_dynamic_scales_descriptor_validation():
    import torch
    ok = tel.make_encoder_desc(768, 12, 3072, torch.float16, 1e-5, int8_gemm=1, dynamic_scales=True)
    assert tel.tel_encoder_packed_size(ok) > 0
    assert tel.tel_encoder_workspace_size(ok, 2557) > 0
    for bad in (tel.make_encoder_desc(768, 12, 3072, torch.float16, 1e-5, dynamic_scales=True),
                tel.make_encoder_desc(768, 12, 3072, torch.float16, 1e-5, int8_gemm=2,
                                      dynamic_scales=True)):
        assert tel.tel_encoder_packed_size(bad) == 0
        assert tel.lib.tel_encoder_prepare(ctypes.byref(bad), None, None, 0, None) == \
            tel.TEL_EUNSUPPORTED
