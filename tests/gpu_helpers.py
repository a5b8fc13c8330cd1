"""Helpers for the GPU parity tests: run the library through its C ABI on seeded inputs
and compare with the oracle at the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import tel_inputs as ti

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# fp16/bf16 outputs vs the float64 oracle: max-abs 2e-2 and relative Frobenius 5e-3.
# fp32 outputs (float32 storage, float32 MFMA accumulation): 1e-4 and 1e-5.
TOL = {"f16": (2e-2, 5e-3), "bf16": (2e-2, 5e-3), "f32": (1e-4, 1e-5)}


def errors(out: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    assert np.isfinite(out).all(), "non-finite output"
    diff = out - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / den) if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_close(out, ref, dtype: str, what: str = ""):
    max_abs, rel = errors(out, ref)
    tmax, trel = TOL[dtype]
    assert max_abs <= tmax and rel <= trel, \
        f"{what}: max_abs={max_abs:.3e} (tol {tmax:.0e}) rel_frob={rel:.3e} (tol {trel:.0e})"
    return max_abs, rel


def dev(a: np.ndarray, dtype: str | torch.dtype) -> torch.Tensor:
    """Host array -> device tensor of the storage type (exact: values already rounded)."""
    dt = TORCH_DT[dtype] if isinstance(dtype, str) else dtype
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32))).to("cuda").to(dt)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32))).to("cuda")


def prepare_layers(tel, desc, layer_weights: list, dtype: str, act_amax=None,
                   attn_amax=None) -> list:
    packed = []
    n = tel.tel_encoder_packed_size(desc)
    assert n > 0
    for i, w in enumerate(layer_weights):
        dw = {k: dev(v, dtype) for k, v in w.items()}
        p = tel.alloc_bytes(n)
        if act_amax is None:
            tel.tel_encoder_prepare(desc, dw, p)
        elif attn_amax is None:
            tel.tel_encoder_prepare(desc, dw, p, act_amax=tuple(float(a) for a in act_amax[i]))
        else:
            tel.tel_encoder_prepare(desc, dw, p, act_amax=tuple(float(a) for a in act_amax[i]),
                                    attn_amax=tuple(float(a) for a in attn_amax[i]))
        packed.append(p)
    torch.cuda.synchronize()
    return packed


def gpu_encoder_forward(tel, cfg: dict, lens, x_pad, layer_weights: list, int8=False,
                        act_amax=None, attn_amax=None) -> np.ndarray:
    """Whole stack (offsets, remove, layers, rebuild) on the GPU; returns y_pad (float64).
    int8: the projection GEMMs in int8 with per-layer calibration max-abs act_amax[layer];
    int8 = 2: attention on int8 codes too, with the Q/K/V max-abs attn_amax[layer]."""
    dt = cfg["dtype"]
    desc = tel.make_encoder_desc(cfg["hidden"], cfg["heads"], cfg["ffn"], TORCH_DT[dt], ti.LN_EPS,
                                 int8_gemm=int8)
    packed = prepare_layers(tel, desc, layer_weights, dt, act_amax if int8 else None,
                            attn_amax if int8 == 2 else None)
    B, S, H = x_pad.shape
    x = dev(x_pad, dt)
    y = torch.full_like(x, float("nan"))
    lens_d = torch.from_numpy(np.asarray(lens, np.int32)).to("cuda")
    ws = tel.alloc_bytes(tel.tel_encoder_forward_workspace_size(desc, B, S))
    T, max_len = int(np.sum(lens)), int(np.max(lens))
    tel.tel_encoder_forward(desc, packed, x, y, lens_d, T, max_len, ws)
    torch.cuda.synchronize()
    return host(y)


def swin_block_gpu(tel, cfg: dict, w: dict):
    """(desc, packed, workspace) of one shifted-window block of config cfg."""
    dt = cfg["dtype"]
    desc = tel.make_swin_desc(cfg["batch"], cfg["height"], cfg["width"], cfg["channels"],
                              cfg["heads"], cfg["window"], cfg["shift"], cfg["mlp"], TORCH_DT[dt],
                              ti.LN_EPS)
    packed = tel.alloc_bytes(tel.tel_swin_packed_size(desc))
    tel.tel_swin_prepare(desc, {k: dev(v, dt) for k, v in w.items()}, packed)
    ws = tel.alloc_bytes(tel.tel_swin_workspace_size(desc))
    return desc, packed, ws


def swin_two_stages_gpu(tel, cfg: dict, x: np.ndarray, stage1: list, merge: dict, stage2: list,
                        keep_intermediates: bool = True):
    """Swin stage 1 (blocks alternating shift 0 / 3), patch merging, stage 2 on the GPU,
    through the C ABI. Returns the output and, with keep_intermediates, the input of every
    piece (host float64 copies), in order."""
    from oracle import swin as _sw   # only for the block shift pattern (stage_shifts)
    dt = cfg["dtype"]
    H, W, M = cfg["height"], cfg["width"], cfg["window"]
    cur = dev(x, dt)
    ins = []
    for stage, blocks in ((0, stage1), (1, stage2)):
        f = 2 ** stage
        for w, s in zip(blocks, _sw.stage_shifts(len(blocks), H // f, W // f, M)):
            bc = ti.swin_stage_block_config(cfg, stage, s)
            desc, packed, ws = swin_block_gpu(tel, bc, w)
            out = torch.empty_like(cur)
            if keep_intermediates:
                ins.append(host(cur))
            tel.tel_window_attention_forward(desc, packed, cur, out, ws)
            cur = out
        if stage == 0:
            C = cfg["channels"]
            out = torch.empty((cfg["batch"], (H // 2) * (W // 2), 2 * C), dtype=TORCH_DT[dt],
                              device="cuda")
            if keep_intermediates:
                ins.append(host(cur))
            tel.tel_patch_merging(cur, out, dev_f32(merge["norm_g"]), dev_f32(merge["norm_b"]),
                                  dev(merge["w_red"], dt), H, W, ti.LN_EPS)
            cur = out
    torch.cuda.synchronize()
    return host(cur), ins
