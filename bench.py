"""Benchmark: valid tokens/s per encoder layer (BERT-base-shaped stack, fp16) on one MI355X.

One step = one pass of the whole path over one seeded synthetic batch: offsets, padding
removal, the 12 encoder layers, padding rebuild (tel_encoder_forward). Inputs and
prepared weights are resident in HBM before the timed region. Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload bert_base] [--no-cpu]

Other workloads (same line format, measured the same way): bert_large_tput,
bert_large_latency (24 fp16 layers), bert_base_int8 (int8 GEMMs; static activation
scales from tel_encoder_calibrate on the same batch, i.e. post-training calibration,
outside the timed region), bert_base_sparse (the bert_base layers with their projection
matrices pruned 2:4 when prepared, on the sparse MFMA), swin_t_stage1 (one shifted-window
block, tokens/s per block), swin_t_stage12 (Swin-T stages 1 and 2, two blocks each, with the
patch merging between them; stage-1 tokens/s).

Also measured here, each with HIP events on the stream its kernel is launched on:
the average duration of every kernel of one layer (same shapes, launched through the
kernel-level entry points) and the roofline fraction of the dominant one; and the CPU
oracle timed on a bounded sample of the same workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_INT8_TOPS = 5000.0         # dense int8 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="bert_base")
    ap.add_argument("--dtype", default=None, help="override storage type (f16, bf16)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--tile-sweep", action="store_true",
                    help="time every GEMM tile configuration on the encoder's projection "
                         "shapes (back to back, fp16) and print a table")
    ap.add_argument("--graphs", action="store_true",
                    help="run the timed steps through the forward's HIP-graph cache")
    ap.add_argument("--streams", type=int, default=1,
                    help="split the batch into this many parts balanced by valid tokens, each "
                         "part's forward on its own stream (default priority), joined per step")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--no-hbm", action="store_true",
                    help="skip the memory-bound kernels' flushed-cache timings")
    ap.add_argument("--summarise-traffic", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "TABLE"),
                    help="no GPU work: turn the rocprofv3 FETCH_SIZE and WRITE_SIZE runs of "
                         "`bench.py --calib-copy` (output directories) and the kernel table "
                         "that run wrote (--kernel-table) into profiles/hbm_traffic.json")
    ap.add_argument("--kernel-table", default="kernel_table.json",
                    help="with --calib-copy: where to write the order of the per-kernel "
                         "launches, for --summarise-traffic")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (the scale of HBM counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_cpu() -> str:
    """The host processor's model name (Linux /proc/cpuinfo), for the CPU baseline."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.summarise_traffic:
        return summarise_traffic(*args.summarise_traffic)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the encoder "
              "forward shards by sequence with no collectives, and this benchmark measures one "
              "GPU's share.", file=sys.stderr)
        sys.exit(2)

    import torch

    import tel_inputs as ti
    import transformer_encoder_remove_amd as tel

    if args.tile_sweep:
        return tile_sweep(args)
    if args.workload in ti.SWIN_CONFIGS:
        return bench_swin(args)
    if args.workload in ti.SWIN_STAGES:
        return bench_swin_stages(args)
    cfg = dict(ti.ENCODER_CONFIGS[args.workload])
    if args.dtype:
        cfg["dtype"] = args.dtype
    int8 = bool(cfg.get("int8"))
    int8_mode = int(cfg.get("int8", 0))   # 1: int8 GEMMs, 2: and int8 attention
    sparse = bool(cfg.get("sparse"))
    dt = cfg["dtype"]
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dt]
    B, S, H, nh, F, NL = (cfg["batch"], cfg["max_seq"], cfg["hidden"], cfg["heads"], cfg["ffn"],
                          cfg["layers"])
    torch.cuda.set_device(0)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32))).cuda().to(tdt)

    lens, x_pad = ti.encoder_input(cfg)
    T, max_len = int(lens.sum()), int(lens.max())
    log(f"[bench] workload {args.workload}: B={B} S={S} T={T} H={H} heads={nh} F={F} layers={NL} "
        f"{dt}{' int8 GEMMs' if int8 else ''}{' 2:4-sparse weights' if sparse else ''}")
    desc = tel.make_encoder_desc(H, nh, F, tdt, ti.LN_EPS, sparse_2of4=sparse)
    psize = tel.tel_encoder_packed_size(desc)
    packed, layer_w, dws = [], [], []
    for i in range(NL):
        w = ti.encoder_layer_weights(cfg, i)
        dw = {k: dev(v) for k, v in w.items()}
        p = tel.alloc_bytes(psize)
        tel.tel_encoder_prepare(desc, dw, p)
        packed.append(p)
        dws.append(dw)
        if i == 0:
            layer_w = dw
    x = dev(x_pad)
    y = torch.empty_like(x)
    lens_d = torch.from_numpy(lens).cuda()
    cu_d = torch.from_numpy(np.r_[0, np.cumsum(lens)].astype(np.int32)).cuda()
    if int8 and cfg.get("dynamic"):
        # dynamic activation scales: no calibration, the weights quantised once
        desc = tel.make_encoder_desc(H, nh, F, tdt, ti.LN_EPS, int8_gemm=1, dynamic_scales=True)
        psize = tel.tel_encoder_packed_size(desc)
        packed = []
        for i in range(NL):
            p = tel.alloc_bytes(psize)
            tel.tel_encoder_prepare(desc, dws[i], p)
            packed.append(p)
    elif int8:
        # post-training calibration on this batch (the float stack, layer by layer), then
        # the int8 layers prepared with those static scales
        from_pad = torch.empty((T, H), dtype=tdt, device="cuda")
        po = torch.empty(B * S, dtype=torch.int32, device="cuda")
        tel.tel_build_offsets(lens_d, S, cu_d, po)
        tel.tel_remove_padding(x, from_pad, po, T)
        amax = torch.zeros((NL, 7), dtype=torch.float32, device="cuda")
        lws = tel.alloc_bytes(tel.tel_encoder_workspace_size(desc, T))
        cur, nxt = from_pad, torch.empty_like(from_pad)
        for i in range(NL):
            tel.tel_encoder_calibrate(desc, packed[i], cur, nxt, cu_d, T, max_len, amax[i], lws)
            cur, nxt = nxt, cur
        amax_h = amax.cpu().numpy()
        desc = tel.make_encoder_desc(H, nh, F, tdt, ti.LN_EPS, int8_gemm=int8_mode)
        psize = tel.tel_encoder_packed_size(desc)
        packed = []
        for i in range(NL):
            p = tel.alloc_bytes(psize)
            tel.tel_encoder_prepare(desc, dws[i], p, act_amax=tuple(float(a) for a in amax_h[i][:4]),
                                    attn_amax=tuple(float(a) for a in amax_h[i][4:7]))
            packed.append(p)
        log(f"[bench] calibrated act_amax layer 0: {amax_h[0]}")
    del dws
    ws = tel.alloc_bytes(tel.tel_encoder_forward_workspace_size(desc, B, S))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    if args.graphs:
        tel.tel_graph_cache(1)

    def step():
        tel.tel_encoder_forward(desc, packed, x, y, lens_d, T, max_len, ws, stream=stream)

    if args.streams > 1:
        # the batch cut into contiguous runs of sequences with about equal valid tokens, each
        # run's whole forward on its own stream; the main stream waits for all of them
        cum = np.cumsum(lens)
        cuts = [0] + [int(np.searchsorted(cum, T * k / args.streams)) + 1
                      for k in range(1, args.streams)] + [B]
        parts = []
        for k in range(args.streams):
            b0, b1 = cuts[k], cuts[k + 1]
            if b1 <= b0:
                continue
            pl = lens[b0:b1]
            parts.append(dict(x=x[b0:b1], y=y[b0:b1], lens=lens_d[b0:b1], T=int(pl.sum()),
                              max_len=int(pl.max()), st=torch.cuda.Stream(),
                              ws=tel.alloc_bytes(tel.tel_encoder_forward_workspace_size(
                                  desc, b1 - b0, S))))
        log(f"[bench] {len(parts)} streams: valid tokens per part "
            f"{[p['T'] for p in parts]}")

        def step():
            start = torch.cuda.Event()
            start.record(stream)
            for p in parts:
                p["st"].wait_event(start)
                tel.tel_encoder_forward(desc, packed, p["x"], p["y"], p["lens"], p["T"],
                                        p["max_len"], p["ws"], stream=p["st"])
                done = torch.cuda.Event()
                done.record(p["st"])
                stream.wait_event(done)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")
    # one event before every step and one after the last: the K steps run back to back,
    # the first-to-last span gives ms_per_step, the gaps give per-step statistics
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i].record(stream)
        step()
    evs[-1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = evs[0].elapsed_time(evs[-1])
    ms_per_step = gpu_ms / args.steps
    step_ms = step_stats([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    value = T * NL / (ms_per_step / 1e3)
    log(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step (wall {wall * 1e3 / args.steps:.4f}),"
        f" {value / 1e6:.2f} M valid tokens/s per layer")

    # ---------------------------------------------------------------- per-kernel timing
    # Each kernel of one layer, same shapes and launch configuration as inside the stack,
    # timed with HIP events on the stream it is launched on.
    qkv = torch.randn(3 * T * H, device="cuda").to(tdt)
    hid = torch.randn(T, H, device="cuda").to(tdt)
    ctx = torch.empty(T, H, device="cuda", dtype=tdt)
    pre = torch.empty(T, H, device="cuda", dtype=tdt)
    ffn = torch.randn(T, F, device="cuda").to(tdt)
    ffo = torch.empty(T, F, device="cuda", dtype=tdt)
    qkv_o = torch.empty(3 * T * H, device="cuda", dtype=tdt)
    bias = {n: torch.zeros(n, device="cuda", dtype=torch.float32) for n in (H, 3 * H, F)}
    b32 = lambda n: bias[n]
    g32 = torch.ones(H, device="cuda", dtype=torch.float32)
    cu = torch.from_numpy(np.r_[0, np.cumsum(lens)].astype(np.int32)).cuda()
    Lbar = float((lens.astype(np.float64) ** 2).sum() / lens.sum())

    reduce_ln = {}

    def resid_gemm(a, w, K, N, name):
        """The output projection / FFN2 GEMM as the layer launches it: bias + residual in
        the epilogue (then the LayerNorm kernel), or split over k into partial sums when the
        layer's plan splits it (then the reduce-LayerNorm kernel, timed as `name`)."""
        cfg_, sp_, pb_ = tel.tel_gemm_partial_plan(tel.DTYPE_CODE[tdt], T, N, K)
        if sp_ > 1 and not (int8 or sparse):   # those layers' own GEMMs replace these below
            part = torch.empty((sp_, T, N), device="cuda",
                               dtype=torch.float16 if pb_ == 2 else torch.float32)
            reduce_ln[name] = (lambda: tel.tel_layernorm_reduce(
                part, sp_, b32(N), hid, pre, g32, b32(N), ti.LN_EPS, stream=stream),
                part.numel() * part.element_size() + 2.0 * T * N * x.element_size())
            return lambda: tel.tel_gemm_partial(cfg_, sp_, a, w, part, stream=stream)
        return lambda: tel.tel_gemm(tel.TEL_EPI_BIAS_RESID, a, w, b32(N), pre, resid=hid,
                                    stream=stream)

    kernels = {
        "gemm_qkv": (lambda: tel.tel_gemm(tel.TEL_EPI_QKV_SPLIT, hid, layer_w["w_qkv"], b32(3 * H),
                                          qkv_o, heads=nh, stream=stream),
                     2.0 * T * H * 3 * H, 2.0 * (T * H + 3 * H * H + 3 * T * H)),
        "attention": (lambda: tel.tel_attention_varlen(qkv, ctx, cu, T, max_len, nh, H // nh,
                                                       stream=stream),
                      4.0 * T * H * Lbar, 2.0 * 4 * T * H),
        "gemm_o_resid": (resid_gemm(ctx, layer_w["w_o"], H, H, "ln1_reduce"),
                         2.0 * T * H * H, 2.0 * (3 * T * H + H * H)),
        "layernorm": (lambda: tel.tel_layernorm(pre, hid, g32, b32(H), ti.LN_EPS, stream=stream),
                      0.0, 2.0 * 2 * T * H),
        "gemm_ffn1_gelu": (lambda: tel.tel_gemm(tel.TEL_EPI_BIAS_GELU, hid, layer_w["w_1"], b32(F),
                                                ffo, stream=stream),
                           2.0 * T * H * F, 2.0 * (T * H + F * H + T * F)),
        "gemm_ffn2_resid": (resid_gemm(ffn, layer_w["w_2"], F, H, "ln2_reduce"),
                            2.0 * T * H * F, 2.0 * (T * F + F * H + 2 * T * H)),
    }
    # the reduce-LayerNorm kernel of a split GEMM: partials read, residual read, y written
    for name, (fn, nbytes) in reduce_ln.items():
        kernels[name] = (fn, 0.0, nbytes)
    if int8:
        # the int8 layer's GEMMs one by one (int8 codes in, epilogues as in the layer: head
        # split, dequantise + residual, GELU written as int8 codes); random codes and scales
        rnd = lambda *shape: torch.randint(-127, 128, shape, device="cuda", dtype=torch.int8)
        xq, cq, hq, fq = rnd(T, H), rnd(T, H), rnd(T, H), rnd(T, F)
        wq = {"qkv": rnd(3 * H, H), "o": rnd(H, H), "1": rnd(F, H), "2": rnd(H, F)}
        dqs = {n: torch.full((n,), 1e-4, device="cuda") for n in (H, 3 * H, F)}
        qinv = torch.full((1,), 10.0, device="cuda")
        f_codes = torch.empty(T, F, dtype=torch.int8, device="cuda")
        kernels.update({
            "gemm_qkv": (lambda: tel.tel_gemm_i8(tel.TEL_EPI_QKV_SPLIT, xq, wq["qkv"], dqs[3 * H],
                                                 b32(3 * H), qkv_o, heads=nh, stream=stream),
                         2.0 * T * H * 3 * H, T * H + 3 * H * H + 2.0 * 3 * T * H),
            "gemm_o_resid": (lambda: tel.tel_gemm_i8(tel.TEL_EPI_BIAS_RESID, cq, wq["o"], dqs[H],
                                                     b32(H), pre, resid=hid, stream=stream),
                             2.0 * T * H * H, T * H + H * H + 2.0 * 2 * T * H),
            "gemm_ffn1_gelu": (lambda: tel.tel_gemm_i8(tel.TEL_EPI_BIAS_GELU, hq, wq["1"], dqs[F],
                                                       b32(F), f_codes, qinv=qinv, out_int8=True,
                                                       stream=stream),
                               2.0 * T * H * F, T * H + F * H + 1.0 * T * F),
            "gemm_ffn2_resid": (lambda: tel.tel_gemm_i8(tel.TEL_EPI_BIAS_RESID, fq, wq["2"], dqs[H],
                                                        b32(H), pre, resid=hid, stream=stream),
                                2.0 * T * H * F, T * F + F * H + 2.0 * 2 * T * H),
        })
    if int8_mode == 2:
        # int8 attention: the QKV GEMM writes the codes of Q, K, V; attention reads codes and
        # writes the codes of its output (1 byte per value in and out)
        qkv8 = torch.empty(3 * T * H, dtype=torch.int8, device="cuda")
        qinv3 = torch.full((3,), 40.0, device="cuda")
        codes = rnd(3 * T * H)
        scl = torch.tensor([1e-3, 1e-2, 40.0], dtype=torch.float32, device="cuda")
        ctx8 = torch.empty(T, H, dtype=torch.int8, device="cuda")
        kernels.update({
            "gemm_qkv": (lambda: tel.tel_gemm_i8(tel.TEL_EPI_QKV_SPLIT, xq, wq["qkv"], dqs[3 * H],
                                                 b32(3 * H), qkv8, qinv=qinv3, out_int8=True,
                                                 heads=nh, stream=stream),
                         2.0 * T * H * 3 * H, T * H + 3 * H * H + 1.0 * 3 * T * H),
            "attention": (lambda: tel.tel_attention_int8(codes, ctx8, scl, cu, T, max_len, nh,
                                                         H // nh, stream=stream),
                          4.0 * T * H * Lbar, 1.0 * 4 * T * H),
        })
    if sparse:
        # the 2:4 layer's GEMMs (compressed weights of layer 0's matrices, as prepared);
        # flops count the kept weights only (half the dense product), bytes the compressed
        # weights (values + 16-bit index words: 9/16 of the dense weight bytes)
        comp = {}
        for k, (n_, k_) in {"w_qkv": (3 * H, H), "w_o": (H, H), "w_1": (F, H),
                            "w_2": (H, F)}.items():
            v_ = torch.empty((n_, k_ // 2), dtype=tdt, device="cuda")
            i_ = torch.empty((n_, k_ // 16), dtype=torch.int16, device="cuda")
            tel.tel_prune_2of4(layer_w[k], v_, i_)
            comp[k] = (v_, i_)
        wb = lambda n_, k_: 2.0 * n_ * k_ * 9 / 16
        kernels.update({
            "gemm_qkv": (lambda: tel.tel_gemm_2of4(tel.TEL_EPI_QKV_SPLIT, hid, *comp["w_qkv"],
                                                   b32(3 * H), qkv_o, heads=nh, stream=stream),
                         T * H * 3 * H, 2.0 * (T * H + 3 * T * H) + wb(3 * H, H)),
            "gemm_o_resid": (lambda: tel.tel_gemm_2of4(tel.TEL_EPI_BIAS_RESID, ctx, *comp["w_o"],
                                                       b32(H), pre, resid=hid, stream=stream),
                             T * H * H, 2.0 * 3 * T * H + wb(H, H)),
            "gemm_ffn1_gelu": (lambda: tel.tel_gemm_2of4(tel.TEL_EPI_BIAS_GELU, hid, *comp["w_1"],
                                                         b32(F), ffo, stream=stream),
                               T * H * F, 2.0 * (T * H + T * F) + wb(F, H)),
            "gemm_ffn2_resid": (lambda: tel.tel_gemm_2of4(tel.TEL_EPI_BIAS_RESID, ffn, *comp["w_2"],
                                                          b32(H), pre, resid=hid, stream=stream),
                                T * H * F, 2.0 * (T * F + 2 * T * H) + wb(H, F)),
        })
    per_kernel = {}
    for name, (fn, flops, nbytes) in kernels.items():
        us = back_to_back_us(fn, stream, args.kernel_reps)
        per_kernel[name] = dict(us=us, tflops=flops / us / 1e6, gbs=nbytes / us / 1e3,
                                flops=flops, bytes=nbytes)
        log(f"[bench] kernel {name:16s} {us:9.2f} us  {flops / us / 1e6:8.1f} TFLOP/s"
            f"  {nbytes / us / 1e3:8.1f} GB/s")
    gemms = {k: v for k, v in per_kernel.items() if k.startswith("gemm")}
    dom = max(gemms, key=lambda k: gemms[k]["us"])
    d = per_kernel[dom]
    peak = PEAK_INT8_TOPS if int8 else PEAK_FP32_TFLOPS if dt == "f32" else PEAK_FP16_TFLOPS
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(d["tflops"], 2), "peak": peak,
                "unit": "TOP/s" if int8 else "TFLOP/s", "frac": round(d["tflops"] / peak, 4),
                "traffic": measured_traffic(args.workload, "i8" if int8 else dt, dom),
                "avg_us": round(d["us"], 3), "flops_per_launch": d["flops"]}
    if args.calib_copy:
        write_kernel_table(args, "i8" if int8 else dt, per_kernel)
        calibration_copy(stream)
    # one layer launches every kernel above once, and the LayerNorm kernel once more for each
    # residual GEMM that is not split (a split one is finished by its reduce kernel)
    n_ln = 2 - len(reduce_ln)
    layer_sum_us = sum(v["us"] for v in per_kernel.values()) + \
        (n_ln - 1) * per_kernel["layernorm"]["us"]

    # ---------------------------------------------------------------- HBM-bound kernels
    # achieved bytes/s of the memory-bound kernels against 8 TB/s: back to back (operands
    # may sit in the 256 MB last-level cache) and with that cache flushed before every
    # launch (a 1 GiB buffer written in between)
    hbm = {}
    if not args.no_hbm:
        pad_o = torch.empty(B * S, dtype=torch.int32, device="cuda")
        tel.tel_build_offsets(lens_d, S, cu_d, pad_o)
        xp_o = torch.empty((T, H), dtype=tdt, device="cuda")
        xr_o = torch.empty_like(x)
        el = x.element_size()
        stress = ti.offsets_stress_lengths()
        Bs, Ss = ti.OFFSETS_STRESS["batch"], ti.OFFSETS_STRESS["max_seq"]
        Ts = int(stress.sum())
        lens_s = torch.from_numpy(stress).cuda()
        cu_s = torch.empty(Bs + 1, dtype=torch.int32, device="cuda")
        po_s = torch.empty(Bs * Ss, dtype=torch.int32, device="cuda")
        # the mask form at the same stress shape: random holes, about half the positions valid
        mask_s = torch.from_numpy(
            (np.random.default_rng(ti.OFFSETS_STRESS["seed"]).random((Bs, Ss)) < 0.5)
            .astype(np.uint8)).cuda()
        Tm = int(mask_s.sum().item())
        cu_m = torch.empty(Bs + 1, dtype=torch.int32, device="cuda")
        hbm_kernels = {
            f"offsets_mask_stress_B{Bs}_T{Tm}": (
                lambda: tel.tel_build_offsets_mask(mask_s, cu_m, po_s, stream=stream),
                1.0 * Bs * Ss + 4.0 * ((Bs + 1) + Tm)),
            "attention": (kernels["attention"][0], per_kernel["attention"]["bytes"]),
            "layernorm": (kernels["layernorm"][0], per_kernel["layernorm"]["bytes"]),
            "remove_padding": (lambda: tel.tel_remove_padding(x, xp_o, pad_o, T, stream=stream),
                               2.0 * T * H * el),
            "rebuild_padding": (lambda: tel.tel_rebuild_padding(xp_o, xr_o, cu_d, stream=stream),
                                (T + B * S) * H * el),
            # lengths read, cu_seqlens and T padding offsets written (4-byte integers)
            f"offsets_stress_B{Bs}_T{Ts}": (
                lambda: tel.tel_build_offsets(lens_s, Ss, cu_s, po_s, stream=stream),
                4.0 * (Bs + (Bs + 1) + Ts)),
        }
        # the same kernels at a bandwidth-bound size (~0.4 GB of packed rows)
        Bp, Sp, Hp = (ti.PADDING_STRESS[k] for k in ("batch", "max_seq", "hidden"))
        lens_p = ti.padding_stress_lengths()
        Tp = int(lens_p.sum())
        lens_pd = torch.from_numpy(lens_p).cuda()
        cu_p = torch.empty(Bp + 1, dtype=torch.int32, device="cuda")
        po_p = torch.empty(Bp * Sp, dtype=torch.int32, device="cuda")
        tel.tel_build_offsets(lens_pd, Sp, cu_p, po_p)
        xpad_p = torch.randn(Bp, Sp, Hp, device="cuda").to(tdt)
        xpk_p = torch.empty((Tp, Hp), dtype=tdt, device="cuda")
        ln_p = torch.empty_like(xpk_p)
        g_p = torch.ones(Hp, device="cuda")
        b_p = torch.zeros(Hp, device="cuda")
        hbm_kernels.update({
            f"remove_padding_stress_T{Tp}": (
                lambda: tel.tel_remove_padding(xpad_p, xpk_p, po_p, Tp, stream=stream),
                2.0 * Tp * Hp * el),
            f"layernorm_stress_T{Tp}": (
                lambda: tel.tel_layernorm(xpk_p, ln_p, g_p, b_p, ti.LN_EPS, stream=stream),
                2.0 * Tp * Hp * el),
            f"rebuild_padding_stress_T{Tp}": (
                lambda: tel.tel_rebuild_padding(xpk_p, xpad_p, cu_p, stream=stream),
                (Tp + Bp * Sp) * Hp * el),
        })
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        for name, (fn, nbytes) in hbm_kernels.items():
            b2b = per_kernel[name]["us"] if name in per_kernel else back_to_back_us(
                fn, stream, args.kernel_reps)
            fl = flushed_us(fn, stream, flush)
            hbm[name] = {"bytes": nbytes, "us": round(b2b, 3), "us_flushed": round(fl, 3),
                         "gbs": round(nbytes / b2b / 1e3, 1),
                         "gbs_flushed": round(nbytes / fl / 1e3, 1),
                         "frac_flushed": round(nbytes / fl / 1e3 / PEAK_HBM_GBS, 4)}
            log(f"[bench] hbm {name:28s} {b2b:8.2f} us ({nbytes / b2b / 1e3:7.1f} GB/s) "
                f"flushed {fl:8.2f} us ({nbytes / fl / 1e3:7.1f} GB/s)")
        del flush, xpad_p, xpk_p, ln_p, po_s, po_p, mask_s

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, lens, x_pad, args.cpu_seconds)

    return emit(args, cfg, value, ms_per_step, T, max_len, roofline, per_kernel, cpu,
                layer_sum_us, step_ms=step_ms, hbm=hbm)


# every kernel source: counters taken on other sources than the ones built now are stale
# The source files each measured kernel is compiled from: its own .hip file and the shared
# headers. A counter record stays valid while these are unchanged.
_HEADERS = ("device.h", "launch.h", "rows.h")
_KERNEL_FILE = {"attention": "attention.hip", "layernorm": "layernorm.hip",
                "ln1_reduce": "layernorm.hip", "ln2_reduce": "layernorm.hip",
                "window_attention": "swin.hip", "attention_half": "swin_fused.hip",
                "ln2_mlp_resid": "swin_fused.hip"}


def kernel_sources(kernel: str) -> tuple:
    """Files (relative to the repository) whose text fixes the named kernel: the GEMM-based
    ones (every gemm_* kernel and the shifted-window block's skinny projections) come from
    gemm.hip."""
    own = _KERNEL_FILE.get(kernel, "gemm.hip")
    return tuple(os.path.join("transformer_encoder_remove_amd", "csrc", f)
                 for f in (own,) + _HEADERS)


def kernel_sources_digest(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in kernel_sources(kernel):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, dtype: str, kernel: str):
    """HBM bytes per launch of the dominant kernel from the rocprofv3 FETCH_SIZE and
    WRITE_SIZE passes summarised in profiles/hbm_traffic.json, scaled by what the same
    counters read for a plain device copy of known size; null when the counters were taken
    on other kernel sources than the ones built now, or for another kernel/workload."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    for r in rec.get("kernels", []):
        if r.get("workload") == workload and r.get("dtype") == dtype and \
                r.get("kernel") == kernel and r.get("sources_sha256") == kernel_sources_digest(kernel):
            return r.get("bytes_per_launch")
    return None


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def write_kernel_table(args, dtype: str, per_kernel: dict):
    """What the counter runs need to attribute dispatches: the per-kernel timing launches
    each kernel 1 + kernel_reps times, in this order, after the timed steps; then the
    calibration copies follow. Library kernels only (torch's spin and fill kernels are
    filtered out by name when the counters are summarised)."""
    path = os.path.abspath(args.kernel_table)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    rec = {"workload": args.workload, "dtype": dtype, "reps": args.kernel_reps,
           "kernels": [{"name": k, "bytes": v["bytes"]} for k, v in per_kernel.items()]}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)


def _counter_rows(d: str, counter: str):
    """(kernel name, value) per dispatch, in dispatch order, from a rocprofv3 --pmc CSV."""
    import csv
    import glob
    paths = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not paths:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    per = {}
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return [(name, v) for (_, name), v in sorted(per.items())]


def summarise_traffic(fetch_dir: str, write_dir: str, table_path: str):
    """profiles/hbm_traffic.json from two `rocprofv3 --pmc` runs (FETCH_SIZE, WRITE_SIZE)
    of `bench.py --calib-copy --steps 1 --warmup 1 --no-cpu --no-hbm`: each kernel's counters
    averaged over its kernel_reps timed launches, scaled by what the same counters read for
    the calibration copies (256 MiB read and 256 MiB written each); entries of other
    workloads or dtypes already in the file are kept."""
    with open(table_path) as f:
        table = json.load(f)
    reps, names = table["reps"], [k["name"] for k in table["kernels"]]
    out = {"kernels": []}
    if os.path.exists(TRAFFIC_JSON):
        with open(TRAFFIC_JSON) as f:
            old = json.load(f)
        out["kernels"] = [k for k in old.get("kernels", [])
                          if (k.get("workload"), k.get("dtype")) != (table["workload"],
                                                                    table["dtype"])]
    calib, per_kernel = {}, {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d, counter)
        copies = [v for n, v in rows if "copyBuffer" in n]
        if len(copies) < 3:
            raise SystemExit(f"{counter}: calibration copies not found in {d}")
        calib[counter] = sum(copies[-3:]) / 3
        lib = [(n, v) for n, v in rows if n.startswith("_ZN3tel") or n.startswith("tel::")]
        block = lib[-(1 + reps) * len(names):]
        for i, name in enumerate(names):
            launches = block[i * (1 + reps) + 1:(i + 1) * (1 + reps)]
            per_kernel.setdefault(name, {})[counter] = sum(v for _, v in launches) / reps
            per_kernel[name]["symbol"] = launches[0][0]
    true_kib = 256 * 1024
    ff, wf = true_kib / calib["FETCH_SIZE"], true_kib / calib["WRITE_SIZE"]
    for k in table["kernels"]:
        c = per_kernel[k["name"]]
        total = (c["FETCH_SIZE"] * ff + c["WRITE_SIZE"] * wf) * 1024
        out["kernels"].append({
            "workload": table["workload"], "dtype": table["dtype"], "kernel": k["name"],
            "symbol": c["symbol"], "fetch_size_kib": round(c["FETCH_SIZE"], 2),
            "write_size_kib": round(c["WRITE_SIZE"], 2), "bytes_per_launch": int(total),
            "algorithmic_bytes": int(k["bytes"]), "ratio": round(total / k["bytes"], 2),
            "sources_sha256": kernel_sources_digest(k["name"])})
    out["description"] = (
        "HBM traffic per launch of the layer / block kernels, launched one by one as bench.py's "
        "per-kernel timing does; counters per dispatch, averaged over the timed launches. "
        "bytes_per_launch = FETCH_SIZE * fetch_factor + WRITE_SIZE * write_factor (KiB), the "
        "factors being what a plain 256 MiB device copy reads on the same counters. "
        "sources_sha256: SHA-256 of the kernel's own source file and the shared headers "
        "device.h, launch.h and rows.h (bench.py kernel_sources) when the counters were taken; "
        "bench.py reports a figure only while it matches.")
    out["calibration"] = {"copy": "__amd_rocclr_copyBuffer, 256 MiB device to device",
                          "fetch_size_kib": round(calib["FETCH_SIZE"], 1),
                          "write_size_kib": round(calib["WRITE_SIZE"], 1),
                          "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)}
    out["commands"] = [
        "cd /tmp && export TMPDIR=/tmp && timeout -s KILL 180 rocprofv3 --pmc FETCH_SIZE "
        "--output-format csv -d $OUT/pmc_fetch -o bench -- python3 $REPO/bench.py "
        "--steps 1 --warmup 1 --no-cpu --no-hbm --kernel-reps 3 --calib-copy "
        "--kernel-table $OUT/kernel_table.json [--workload W]",
        "the same with --pmc WRITE_SIZE -d $OUT/pmc_write",
        "python3 bench.py --summarise-traffic $OUT/pmc_fetch $OUT/pmc_write "
        "$OUT/kernel_table.json ($REPO: the repository, $OUT: any output directory)"]
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(out, f, indent=1)
    for k in out["kernels"]:
        print(f"{k['workload']:16s} {k['dtype']:4s} {k['kernel']:28s} {k['bytes_per_launch'] / 1e6:9.2f} MB"
              f" (algorithmic {k['algorithmic_bytes'] / 1e6:9.2f} MB, x{k['ratio']})")


def calibration_copy(stream, mib: int = 256, reps: int = 3):
    """A plain device-to-device copy of known size, the scale for rocprofv3's FETCH_SIZE /
    WRITE_SIZE counters (each copy reads and writes exactly mib MiB)."""
    import torch
    src = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy: {reps} x {mib} MiB device-to-device")


def back_to_back_us(fn, stream, reps: int) -> float:
    """Average duration of one launch in a back-to-back stream: a spin kernel holds the GPU
    while the host enqueues `reps` launches between one pair of HIP events on the launch
    stream (what rocprofv3's kernel-trace durations add up to inside the stack), free of
    host launch latency."""
    import torch
    fn()
    torch.cuda.synchronize()
    e_s, e_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(50_000_000)
    e_s.record(stream)
    for _ in range(reps):
        fn()
    e_e.record(stream)
    torch.cuda.synchronize()
    return e_s.elapsed_time(e_e) * 1e3 / reps


def flushed_us(fn, stream, flush, reps: int = 10) -> float:
    """Median duration of one launch right after a 1 GiB buffer has been written (larger
    than the 256 MB last-level cache, so the kernel's operands come from HBM): one HIP event
    pair around each launch, on the launch stream, which the flush keeps busy while the
    host enqueues."""
    import torch
    times = []
    for r in range(reps):
        e_s, e_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        flush.fill_(float(r))
        e_s.record(stream)
        fn()
        e_e.record(stream)
        torch.cuda.synchronize()
        times.append(e_s.elapsed_time(e_e) * 1e3)
    return float(np.median(times))


def step_stats(ms: list) -> dict:
    a = np.asarray(ms, dtype=np.float64)
    return {"mean": round(float(a.mean()), 5), "median": round(float(np.median(a)), 5),
            "min": round(float(a.min()), 5), "p90": round(float(np.percentile(a, 90)), 5)}


def emit(args, cfg, value, ms_per_step, T, max_len, roofline, per_kernel, cpu, layer_sum_us=None,
         step_ms=None, hbm=None):
    NL = cfg["layers"]
    int8 = bool(cfg.get("int8"))
    out = {
        "metric": "valid tokens/sec per encoder layer (BERT-base fp16) + % of MFMA/HBM roofline",
        "value": round(value, 1), "unit": "valid tokens/s per layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8" if int8 else cfg["dtype"],
        "data": "synthetic (seeded N(0,1) inputs, N(0,0.02) weights)",
        "config": {"workload": f"{args.workload}: {NL}-layer post-LN encoder"
                               f"{' with int8 GEMMs' if int8 else ''}"
                               f"{' and int8 attention' if cfg.get('int8') == 2 else ''}"
                               f"{' (dynamic activation scales)' if cfg.get('dynamic') else ''}"
                               f"{' with 2:4-sparse projection weights' if cfg.get('sparse') else ''}"
                               f", offsets + padding removal "
                               f"+ layers + rebuild", "batch": cfg["batch"],
                   "max_seq": cfg["max_seq"], "valid_tokens": T, "max_len": max_len,
                   "hidden": cfg["hidden"], "heads": cfg["heads"], "ffn": cfg["ffn"],
                   "layers": NL, "parallelism": "single GPU",
                   **({"graph_replay": True} if args.graphs else {}),
                   **({"streams": args.streams} if args.streams > 1 else {})},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "step_ms": step_ms,
    }
    if hbm:
        out["hbm_kernels"] = hbm
    if per_kernel:
        out["kernels_us"] = {k: round(v["us"], 3) for k, v in per_kernel.items()}
        out["layer_kernel_sum_us"] = round(layer_sum_us, 3)
    print(json.dumps(out), flush=True)


def bench_swin(args):
    """One shifted-window block (Swin-T stage-1 shape) per step; tokens/s per block."""
    import torch

    import tel_inputs as ti
    import transformer_encoder_remove_amd as tel
    cfg = ti.SWIN_CONFIGS[args.workload]
    torch.cuda.set_device(0)
    tdt = torch.float16
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32))).cuda().to(tdt)
    x_np = ti.swin_input(cfg)
    w = ti.swin_block_weights(cfg)
    desc = tel.make_swin_desc(cfg["batch"], cfg["height"], cfg["width"], cfg["channels"],
                              cfg["heads"], cfg["window"], cfg["shift"], cfg["mlp"], tdt, ti.LN_EPS)
    packed = tel.alloc_bytes(tel.tel_swin_packed_size(desc))
    tel.tel_swin_prepare(desc, {k: dev(v) for k, v in w.items()}, packed)
    x = dev(x_np)
    y = torch.empty_like(x)
    ws = tel.alloc_bytes(tel.tel_swin_workspace_size(desc))
    T = cfg["batch"] * cfg["height"] * cfg["width"]
    log(f"[bench] workload {args.workload}: {cfg} tokens={T}")
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        tel.tel_window_attention_forward(desc, packed, x, y, ws, stream=stream)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for i in range(args.steps):
        evs[i].record(stream)
        tel.tel_window_attention_forward(desc, packed, x, y, ws, stream=stream)
    evs[-1].record(stream)
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    step_ms = step_stats([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    value = T / (ms / 1e3)
    log(f"[bench] {args.steps} steps: {ms:.4f} ms/step, {value / 1e9:.3f} G tokens/s per block")

    # each kernel of the block as launched inside it (TEL_SWIN_ONE_STAGE on the workspace
    # the block leaves behind); algorithmic bytes: inputs read once, outputs written once
    C, F, el = cfg["channels"], cfg["mlp"], 2
    stages = {   # name: (stage, bytes per token, flops per token)
        "ln1_shift_partition_qkv": (0, el * (C + 3 * C), 2 * C * 3 * C),
        "window_attention": (1, el * (3 * C + C), 4 * cfg["window"] ** 2 * C),
        "proj_reverse_unshift_resid": (2, el * (C + C + C), 2 * C * C),
        "ln2_fc1_gelu": (3, el * (C + F), 2 * C * F),
        "fc2_resid": (4, el * (F + C + C), 2 * F * C),
    }
    fused = tel.tel_swin_fused_stages(desc)
    mlp_fused = bool(fused & tel.TEL_SWIN_FUSED_MLP)
    if fused & tel.TEL_SWIN_FUSED_ATTN:   # stage 0 is the whole attention half: x read, x1 written
        for k in ("ln1_shift_partition_qkv", "window_attention", "proj_reverse_unshift_resid"):
            del stages[k]
        stages = {"attention_half": (0, el * (C + C), 2 * C * 3 * C + 4 * cfg["window"] ** 2 * C
                                     + 2 * C * C), **stages}
    if mlp_fused:   # stage 3 is the whole MLP half (x1 read once, y written), stage 4 empty
        del stages["ln2_fc1_gelu"], stages["fc2_resid"]
        stages["ln2_mlp_resid"] = (3, el * (C + C), 4 * C * F)
    per_kernel = {}
    for name, (k, bpt, fpt) in stages.items():
        fn = lambda k=k: tel.tel_window_attention_forward(desc, packed, x, y, ws,
                                                          flags=tel.TEL_SWIN_ONE_STAGE(k),
                                                          stream=stream)
        us = back_to_back_us(fn, stream, args.kernel_reps)
        per_kernel[name] = dict(us=us, bytes=bpt * T, flops=fpt * T)
        log(f"[bench] kernel {name:28s} {us:9.2f} us  {bpt * T / us / 1e3:8.1f} GB/s"
            f"  {fpt * T / us / 1e6:7.1f} TFLOP/s")
    if args.calib_copy:
        write_kernel_table(args, "f16", per_kernel)
        calibration_copy(stream)
    dom = max(per_kernel, key=lambda k: per_kernel[k]["us"])
    d = per_kernel[dom]
    if dom in ("ln2_mlp_resid", "attention_half"):
        # a fused half moves 2 x 96 x 2 bytes per token against tens of kflops: far past the
        # ridge point, so it is priced against the fp16 MFMA peak
        roofline = {"kernel": dom, "bound": "mfma",
                    "achieved": round(d["flops"] / d["us"] / 1e6, 2), "peak": PEAK_FP16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(d["flops"] / d["us"] / 1e6 / PEAK_FP16_TFLOPS, 4),
                    "traffic": measured_traffic(args.workload, "f16", dom),
                    "avg_us": round(d["us"], 3), "flops_per_launch": d["flops"]}
    else:
        roofline = {"kernel": dom, "bound": "hbm",
                    "achieved": round(d["bytes"] / d["us"] / 1e3, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(d["bytes"] / d["us"] / 1e3 / PEAK_HBM_GBS, 4),
                    "traffic": measured_traffic(args.workload, "f16", dom),
                    "avg_us": round(d["us"], 3), "bytes_per_launch": d["bytes"]}
    cpu = None
    if not args.no_cpu:
        from oracle import swin
        n_img, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds and n_img < cfg["batch"]:
            t0 = time.perf_counter()
            swin.swin_block(x_np[n_img:n_img + 1], w, cfg["height"], cfg["width"], cfg["heads"],
                            cfg["window"], cfg["shift"], ti.LN_EPS)
            t_cpu += time.perf_counter() - t0
            n_img += 1
        tok = n_img * cfg["height"] * cfg["width"]
        cpu = {"value": round(tok / t_cpu, 1), "unit": "tokens/s per block",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "host_cpu": host_cpu(),
               "sample": f"{n_img} image(s) of the same block, float64 NumPy, {t_cpu:.1f} s"}
    out = {
        "metric": "tokens/sec per shifted-window block (Swin-T stage-1 fp16)",
        "value": round(value, 1), "unit": "tokens/s per block", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded N(0,1) inputs, N(0,0.02) weights and bias table)",
        "config": {"workload": f"{args.workload}: shifted-window block, LN1 + shift + partition, "
                               "QKV, window attention (bias + mask), proj + unshift + residual, "
                               "LN2, MLP" + (f" (fused stages {fused})" if fused else ""),
                   **{k: v for k, v in cfg.items() if k != "dtype"}},
        "roofline": roofline, "cpu_baseline": cpu, "step_ms": step_ms,
        "kernels_us": {k: round(v["us"], 3) for k, v in per_kernel.items()},
        "block_kernel_sum_us": round(sum(v["us"] for v in per_kernel.values()), 3),
    }
    print(json.dumps(out), flush=True)


def tile_sweep(args):
    """Back-to-back time of every tile configuration of the pipelined GEMM (and of the
    register-staged kernel, -1, and the automatic choice, -2) on the projection shapes of
    BERT-base (2557 tokens), the BERT-large latency batch (128 tokens) and BERT-large FFN1
    (13537 tokens), fp16, each with the epilogue the layer uses."""
    import torch

    import transformer_encoder_remove_amd as tel
    torch.manual_seed(0)
    st = torch.cuda.current_stream()
    E = {"bias": tel.TEL_EPI_BIAS, "gelu": tel.TEL_EPI_BIAS_GELU, "resid": tel.TEL_EPI_BIAS_RESID,
         "qkv": tel.TEL_EPI_QKV_SPLIT}
    shapes = [("base_qkv", 2557, 2304, 768, "qkv", 12), ("base_o", 2557, 768, 768, "resid", 12),
              ("base_ffn1", 2557, 3072, 768, "gelu", 12), ("base_ffn2", 2557, 768, 3072, "resid", 12),
              ("lat_qkv", 128, 3072, 1024, "qkv", 16), ("lat_ffn1", 128, 4096, 1024, "gelu", 16),
              ("lat_o", 128, 1024, 1024, "resid", 16), ("lat_ffn2", 128, 1024, 4096, "resid", 16),
              ("large_ffn1", 13537, 4096, 1024, "gelu", 16)]
    cfgs = [-2, -1] + list(range(tel.tel_gemm_tile_configs()))
    print("shape " + " ".join(f"{c:>7d}" for c in cfgs), flush=True)
    for name, M, N, K, epi, heads in shapes:
        A = torch.randn(M, K, device="cuda").half()
        W = (torch.randn(N, K, device="cuda") * 0.02).half()
        b = torch.zeros(N, device="cuda")
        R = torch.randn(M, N, device="cuda").half() if epi == "resid" else None
        C = torch.empty(M * N, device="cuda", dtype=torch.half)
        row = []
        for cfg in cfgs:
            fn = lambda cfg=cfg: tel.tel_gemm_ex(E[epi], cfg, A, W, b, C, resid=R, heads=heads,
                                                 stream=st)
            row.append(back_to_back_us(fn, st, args.kernel_reps))
        print(f"{name} " + " ".join(f"{t:7.2f}" for t in row), flush=True)


def bench_swin_stages(args):
    """Swin-T stage 1 (two blocks), patch merging, stage 2 (two blocks) per step; stage-1
    input tokens/s of the whole pipeline, and the patch-merging kernel against HBM."""
    import torch

    import tel_inputs as ti
    import transformer_encoder_remove_amd as tel
    from oracle import swin as sw_shifts   # block shift pattern only (stage_shifts)
    cfg = ti.SWIN_STAGES[args.workload]
    torch.cuda.set_device(0)
    tdt = torch.float16
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32))).cuda().to(tdt)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32))).cuda()
    B, H, W, C, M = cfg["batch"], cfg["height"], cfg["width"], cfg["channels"], cfg["window"]
    x_np = ti.swin_input(cfg)
    s1, mw, s2 = ti.swin_stage_weights(cfg)
    blocks = []   # (stage, desc, packed, workspace, input buffer, output buffer)
    x = dev(x_np)
    bufs = [torch.empty_like(x), torch.empty_like(x)]
    half = [torch.empty((B, (H // 2) * (W // 2), 2 * C), dtype=tdt, device="cuda")
            for _ in range(3)]
    for stage, ws_list in ((0, s1), (1, s2)):
        f = 2 ** stage
        for i, (w, s) in enumerate(zip(ws_list, sw_shifts.stage_shifts(len(ws_list), H // f,
                                                                       W // f, M))):
            bc = ti.swin_stage_block_config(cfg, stage, s)
            desc = tel.make_swin_desc(bc["batch"], bc["height"], bc["width"], bc["channels"],
                                      bc["heads"], bc["window"], bc["shift"], bc["mlp"], tdt,
                                      ti.LN_EPS)
            packed = tel.alloc_bytes(tel.tel_swin_packed_size(desc))
            tel.tel_swin_prepare(desc, {k: dev(v) for k, v in w.items()}, packed)
            ws = tel.alloc_bytes(tel.tel_swin_workspace_size(desc))
            src = (x if i == 0 else bufs[0]) if stage == 0 else half[i]
            dst = bufs[i] if stage == 0 else half[i + 1]
            blocks.append((stage, desc, packed, ws, src, dst))
    mg, mb, mwr = f32(mw["norm_g"]), f32(mw["norm_b"]), dev(mw["w_red"])
    T = B * H * W
    stream = torch.cuda.current_stream()
    log(f"[bench] workload {args.workload}: {cfg} stage-1 tokens={T}")

    def merge():
        tel.tel_patch_merging(bufs[1], half[0], mg, mb, mwr, H, W, ti.LN_EPS, stream=stream)

    def step():
        for stage, desc, packed, ws, src, dst in blocks:
            if stage == 1 and src is half[0]:
                merge()
            tel.tel_window_attention_forward(desc, packed, src, dst, ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for i in range(args.steps):
        evs[i].record(stream)
        step()
    evs[-1].record(stream)
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    step_ms = step_stats([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    value = T / (ms / 1e3)
    log(f"[bench] {args.steps} steps: {ms:.4f} ms/step, {value / 1e9:.3f} G stage-1 tokens/s, "
        f"{B / (ms / 1e3):.0f} images/s")
    per_piece = {}
    for n, (stage, desc, packed, ws, src, dst) in enumerate(blocks):
        fn = lambda d=desc, p=packed, w=ws, a=src, b=dst: tel.tel_window_attention_forward(
            d, p, a, b, w, stream=stream)
        per_piece[f"stage{stage + 1}_block{n % 2}_shift{desc.shift}"] = back_to_back_us(
            fn, stream, args.kernel_reps)
    mus = back_to_back_us(merge, stream, args.kernel_reps)
    per_piece["patch_merging"] = mus
    for k, v in per_piece.items():
        log(f"[bench] piece {k:28s} {v:9.2f} us")
    m_bytes = 2 * (T * C + (T // 4) * 2 * C + 2 * C * 4 * C)   # read x and W_red, write y
    roofline = {"kernel": "patch_merging (2x2 gather + LN 4C + 4C->2C)", "bound": "hbm",
                "achieved": round(m_bytes / mus / 1e3, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(m_bytes / mus / 1e3 / PEAK_HBM_GBS, 4), "traffic": None,
                "avg_us": round(mus, 3), "bytes_per_launch": m_bytes}
    cpu = None
    if not args.no_cpu:
        from oracle import swin
        t0 = time.perf_counter()
        swin.swin_two_stages(x_np[:1], s1, mw, s2, H, W, cfg["heads"][0], cfg["heads"][1], M,
                             ti.LN_EPS)
        t_cpu = time.perf_counter() - t0
        cpu = {"value": round(H * W / t_cpu, 1), "unit": "stage-1 tokens/s",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "host_cpu": host_cpu(),
               "sample": f"1 image through both stages and the merge, float64 NumPy, {t_cpu:.1f} s"}
    out = {
        "metric": "stage-1 tokens/sec through Swin-T stages 1 and 2 with patch merging (fp16)",
        "value": round(value, 1), "unit": "stage-1 tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded N(0,1) inputs, N(0,0.02) weights and bias tables)",
        "config": {"workload": f"{args.workload}: two shifted-window stages with the downsampling "
                               "between them", **{k: v for k, v in cfg.items() if k != "dtype"}},
        "images_per_s": round(B / (ms / 1e3), 1),
        "roofline": roofline, "cpu_baseline": cpu, "step_ms": step_ms,
        "pieces_us": {k: round(v, 3) for k, v in per_piece.items()},
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(cfg, lens, x_pad, seconds):
    """The oracle as it stands (float64 NumPy), on the host cores: layers of the same
    workload on the full batch, run one after another until `seconds` have passed."""
    import tel_inputs as ti
    from oracle import encoder as enc
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    S = cfg["max_seq"]
    cu, _ = enc.offsets(lens, S)
    xp = enc.remove_padding(x_pad.astype(np.float64), lens)
    T = int(lens.sum())
    weights = [ti.encoder_layer_weights(cfg, i) for i in range(cfg["layers"])]
    if cfg.get("sparse"):
        from oracle import sparse as sp
        weights = [sp.prune_layer_weights(w) for w in weights]
    int8 = bool(cfg.get("int8"))
    if int8:
        from oracle import int8 as q8
    elapsed, done = 0.0, 0
    while elapsed < seconds:
        w = weights[done % len(weights)]
        dyn = bool(cfg.get("dynamic"))
        amax = q8.calibrate(xp, cu, w, cfg["heads"], ti.LN_EPS) if int8 and not dyn else None
        aa = (q8.calibrate_attention(xp, cu, w, cfg["heads"], ti.LN_EPS)
              if cfg.get("int8") == 2 else None)
        t0 = time.perf_counter()
        if int8:
            xp = q8.encoder_layer_int8(xp, cu, w, cfg["heads"], ti.LN_EPS, amax, attn_amax=aa,
                                       dynamic=dyn)
        else:
            xp = enc.encoder_layer(xp, cu, w, cfg["heads"], ti.LN_EPS)
        elapsed += time.perf_counter() - t0
        done += 1
    cores = blas_threads or len(os.sched_getaffinity(0))
    log(f"[bench] cpu oracle: {done} layers x {T} tokens in {elapsed:.1f} s on {cores} threads")
    out = {"value": round(T * done / elapsed, 1), "unit": "valid tokens/s per layer",
           "cores": cores, "kind": "oracle", "host_cpu": host_cpu(),
           "sample": f"{done} layer(s) of the same workload on the full batch ({T} valid "
                     f"tokens), float64 NumPy, {elapsed:.1f} s"}
    # the same oracle on one thread: layer 0 on the leading sequences up to ~768 tokens
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        return out
    nb = max(1, int(np.searchsorted(np.cumsum(lens), 768, side="right")))
    sub_lens = lens[:nb]
    cu1, _ = enc.offsets(sub_lens, S)
    x1 = enc.remove_padding(x_pad[:nb].astype(np.float64), sub_lens)
    w = weights[0]
    with threadpool_limits(limits=1):
        dyn = bool(cfg.get("dynamic"))
        amax = q8.calibrate(x1, cu1, w, cfg["heads"], ti.LN_EPS) if int8 and not dyn else None
        aa = (q8.calibrate_attention(x1, cu1, w, cfg["heads"], ti.LN_EPS)
              if cfg.get("int8") == 2 else None)
        t0 = time.perf_counter()
        if int8:
            q8.encoder_layer_int8(x1, cu1, w, cfg["heads"], ti.LN_EPS, amax, attn_amax=aa,
                                  dynamic=dyn)
        else:
            enc.encoder_layer(x1, cu1, w, cfg["heads"], ti.LN_EPS)
        t1 = time.perf_counter() - t0
    t_sub = int(sub_lens.sum())
    out["value_1thread"] = round(t_sub / t1, 1)
    out["sample_1thread"] = (f"layer 0 on the first {nb} sequences ({t_sub} valid tokens), one "
                             f"BLAS thread, {t1:.2f} s")
    log(f"[bench] cpu oracle, 1 thread: {t_sub} tokens in {t1:.2f} s")
    return out


if __name__ == "__main__":
    main()
