"""Brute-force references used to pin the oracle on tiny inputs.

Written independently of oracle/: pure-Python loops over the PADDED batch with an
explicit key mask (the formulation that padding removal must reproduce), and a
shifted-window block computed directly in image coordinates (no roll, partition
or reverse). Only the tests use this module.
"""
from __future__ import annotations

import math

import numpy as np


def _dot(a, b):
    s = 0.0
    for i in range(len(a)):
        s += a[i] * b[i]
    return s


def _matvec(W, bias, v):
    """out[j] = bias[j] + sum_k W[j][k] * v[k] (W as nested lists, [out][in])."""
    return [bias[j] + _dot(W[j], v) for j in range(len(W))]


def _ln(v, g, b, eps):
    n = len(v)
    mu = sum(v) / n
    var = sum((x - mu) ** 2 for x in v) / n
    r = 1.0 / math.sqrt(var + eps)
    return [(v[i] - mu) * r * g[i] + b[i] for i in range(n)]


def _gelu(z):
    return 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0)))


def _softmax_masked(scores, valid):
    m = max(s for s, ok in zip(scores, valid) if ok)
    e = [math.exp(s - m) if ok else 0.0 for s, ok in zip(scores, valid)]
    tot = sum(e)
    return [x / tot for x in e]


def _lists(w):
    return {k: np.asarray(v, np.float64).tolist() for k, v in w.items()}


def encoder_layer_padded(x_pad, lens, w, heads, eps, mask=None, trace=None):
    """Post-LN encoder layer on the padded batch [B, S, H]: every position is projected,
    keys at positions >= lens[b] are masked out (or, with mask [B, S], keys where the mask
    is zero). Returns [B, S, H] (pad rows computed too, but only valid rows are
    meaningful). With ``trace`` (a dict), the layer's intermediate rows are appended to
    trace["x"], ["ctx"], ["h1"] and ["f"] for the valid positions only (the inputs of the
    four projection GEMMs: the layer input, the attention output, the first LayerNorm's
    output and the GELU output)."""
    x_pad = np.asarray(x_pad, np.float64)
    B, S, H = x_pad.shape
    d = H // heads
    W = _lists(w)
    out = np.zeros((B, S, H))
    if trace is not None:
        for key in ("x", "ctx", "h1", "f"):
            trace.setdefault(key, [])
    for b in range(B):
        L = int(lens[b])
        rows = [x_pad[b, i].tolist() for i in range(S)]
        qkv = [_matvec(W["w_qkv"], W["b_qkv"], r) for r in rows]
        for i in range(S):
            ctx = [0.0] * H
            for h in range(heads):
                q = qkv[i][h * d:(h + 1) * d]
                scores = [_dot(q, qkv[j][H + h * d:H + (h + 1) * d]) / math.sqrt(d)
                          for j in range(S)]
                valid = [bool(mask[b][j]) if mask is not None else j < L for j in range(S)]
                if not any(valid):
                    continue
                p = _softmax_masked(scores, valid)
                for c in range(d):
                    ctx[h * d + c] = sum(p[j] * qkv[j][2 * H + h * d + c] for j in range(S))
            a = _matvec(W["w_o"], W["b_o"], ctx)
            h1 = _ln([a[c] + rows[i][c] for c in range(H)], W["ln1_g"], W["ln1_b"], eps)
            f = [_gelu(z) for z in _matvec(W["w_1"], W["b_1"], h1)]
            o = _matvec(W["w_2"], W["b_2"], f)
            out[b, i] = _ln([o[c] + h1[c] for c in range(H)], W["ln2_g"], W["ln2_b"], eps)
            valid_row = bool(mask[b][i]) if mask is not None else i < L
            if trace is not None and valid_row:
                trace["x"].append(rows[i])
                trace["ctx"].append(ctx)
                trace["h1"].append(h1)
                trace["f"].append(f)
    return out


def _q8(v32):
    r = float(np.rint(np.float32(v32)))
    return int(max(-127, min(127, r)))


def attention_int8_padded(qkv_pad, lens, heads, attn_amax):
    """Int8 attention on the padded batch by loops: codes of the fp16 Q, K, V values at
    scales amax / 127; integer score sums over the valid keys only; base-2 scores and the
    probabilities in float32 scalars; probability codes rne(127 p); the context as s_v times
    the ratio of two integer sums. qkv_pad [B, S, 3H] fp16 values; returns [B, S, H] (rows
    past each length stay 0)."""
    f32 = np.float32
    qkv_pad = np.asarray(qkv_pad)
    B, S, H3 = qkv_pad.shape
    H = H3 // 3
    d = H // heads
    s_ = [f32(f32(a) / f32(127.0)) for a in attn_amax]
    inv = [f32(f32(127.0) / f32(a)) for a in attn_amax]
    a2 = f32(f32(f32(s_[0] * s_[1]) / f32(math.sqrt(d))) * f32(1.4426950408889634))
    code = lambda v, g: _q8(f32(f32(np.float16(v)) * inv[g]))
    out = np.zeros((B, S, H))
    for b in range(B):
        L = int(lens[b])
        qc = [[code(qkv_pad[b, i, c], 0) for c in range(H)] for i in range(L)]
        kc = [[code(qkv_pad[b, j, H + c], 1) for c in range(H)] for j in range(L)]
        vc = [[code(qkv_pad[b, j, 2 * H + c], 2) for c in range(H)] for j in range(L)]
        for h in range(heads):
            for i in range(L):
                t = []
                for j in range(L):
                    acc = 0
                    for c in range(h * d, (h + 1) * d):
                        acc += qc[i][c] * kc[j][c]
                    t.append(f32(f32(acc) * a2))
                m = max(t)
                r = [int(max(0, min(127, np.rint(f32(f32(np.exp2(f32(tj - m))) * f32(127.0))))))
                     for tj in t]
                den = sum(r)
                for c in range(h * d, (h + 1) * d):
                    num = 0
                    for j in range(L):
                        num += r[j] * vc[j][c]
                    out[b, i, c] = float(s_[2]) * num / den
    return out


def encoder_layer_int8_padded(x_pad, lens, w, heads, eps, amax, attn_amax=None):
    """Int8-GEMM layer, padded formulation, loops. Weights: per-row scale
    max|W|/127 (float32), codes rne(W/s) clamped; activations: fp16 storage, then
    one float32 multiply by 127/amax, rne, clamp; int accumulate; y = acc*(s_a*s_w)+b.
    Activations between the steps are fp16 values (the dequantised QKV, the attention
    output, the pre-LN sums, h1 and the GELU output)."""
    f32 = np.float32
    h = lambda v: float(np.float16(v))
    x_pad = np.asarray(x_pad, np.float64)
    B, S, H = x_pad.shape
    d = H // heads
    W = {k: np.asarray(v) for k, v in w.items()}

    def qweights(Wm):
        Wm = np.asarray(Wm, np.float32)
        codes, scales = [], []
        for row in Wm:
            mx = max(abs(f32(v)) for v in row)
            s = f32(mx / f32(127.0)) if mx > 0 else f32(1.0)
            scales.append(s)
            codes.append([_q8(f32(f32(v) / s)) for v in row])
        return codes, scales

    qW = {n: qweights(W[n]) for n in ("w_qkv", "w_o", "w_1", "w_2")}
    sa = [(f32(f32(a) / f32(127.0)), f32(f32(127.0) / f32(a))) for a in amax]

    def qlin(v, wn, bn, g):
        codes, scales = qW[wn]
        s, inv = sa[g]
        qa = [_q8(f32(f32(np.float16(x)) * inv)) for x in v]
        bias = np.asarray(W[bn], np.float64)
        out = []
        for n in range(len(codes)):
            acc = 0
            for k in range(len(qa)):
                acc += qa[k] * codes[n][k]
            out.append(acc * float(f32(s * scales[n])) + float(bias[n]))
        return out

    L64 = lambda n: np.asarray(W[n], np.float64).tolist()
    out = np.zeros((B, S, H))
    for b in range(B):
        L = int(lens[b])
        rows = [x_pad[b, i].tolist() for i in range(S)]
        qkv = [[h(v) for v in qlin(r, "w_qkv", "b_qkv", 0)] for r in rows]
        if attn_amax is not None:
            ctx8 = attention_int8_padded(np.asarray(qkv)[None], [L], heads, attn_amax)[0]
        for i in range(L):
            ctx = [0.0] * H
            if attn_amax is not None:
                ctx = [h(v) for v in ctx8[i]]
            for hh in range(heads if attn_amax is None else 0):
                q = qkv[i][hh * d:(hh + 1) * d]
                sc = [_dot(q, qkv[j][H + hh * d:H + (hh + 1) * d]) / math.sqrt(d) for j in range(S)]
                p = _softmax_masked(sc, [j < L for j in range(S)])
                for c in range(d):
                    ctx[hh * d + c] = h(sum(p[j] * qkv[j][2 * H + hh * d + c] for j in range(S)))
            a = qlin(ctx, "w_o", "b_o", 1)
            h1 = [h(v) for v in _ln([h(a[c] + rows[i][c]) for c in range(H)], L64("ln1_g"),
                                    L64("ln1_b"), eps)]
            f = [h(_gelu(z)) for z in qlin(h1, "w_1", "b_1", 2)]
            o = qlin(f, "w_2", "b_2", 3)
            out[b, i] = _ln([h(o[c] + h1[c]) for c in range(H)], L64("ln2_g"), L64("ln2_b"), eps)
    return out


def swin_block_direct(x, w, Hs, Ws, heads, M, s, eps):
    """Shifted-window block computed per image position: the token at (y, x) sits at
    shifted-frame position (Y, X) = ((y - s) mod Hs, (x - s) mod Ws); it attends to
    the tokens whose shifted positions share its window and its shift region; the
    bias is indexed by the in-window offsets. x is [B, Hs*Ws, C]."""
    x = np.asarray(x, np.float64)
    B, L, C = x.shape
    d = C // heads
    W = _lists(w)
    table = np.asarray(w["rpb_table"], np.float64)

    def region(c, n):
        if s == 0:
            return 0
        return 0 if c < n - M else (1 if c < n - s else 2)

    out = np.zeros_like(x)
    for b in range(B):
        z = [_ln(x[b, t].tolist(), W["ln1_g"], W["ln1_b"], eps) for t in range(L)]
        qkv = [_matvec(W["w_qkv"], W["b_qkv"], z[t]) for t in range(L)]
        pos = []
        for t in range(L):
            y, xx = divmod(t, Ws)
            Y, X = (y - s) % Hs, (xx - s) % Ws
            pos.append((Y // M, X // M, Y % M, X % M, region(Y, Hs), region(X, Ws)))
        for t in range(L):
            wy, wx, py, px, ry, rx = pos[t]
            keys = [u for u in range(L)
                    if pos[u][0] == wy and pos[u][1] == wx and pos[u][4] == ry and pos[u][5] == rx]
            o = [0.0] * C
            for h in range(heads):
                q = qkv[t][h * d:(h + 1) * d]
                sc = []
                for u in keys:
                    ky, kx = pos[u][2], pos[u][3]
                    bias = table[(py - ky + M - 1) * (2 * M - 1) + (px - kx + M - 1), h]
                    sc.append(_dot(q, qkv[u][C + h * d:C + (h + 1) * d]) / math.sqrt(d) + bias)
                p = _softmax_masked(sc, [True] * len(sc))
                for c in range(d):
                    o[h * d + c] = sum(p[j] * qkv[u][2 * C + h * d + c] for j, u in enumerate(keys))
            a = _matvec(W["w_proj"], W["b_proj"], o)
            x1 = [x[b, t, c] + a[c] for c in range(C)]
            hdn = [_gelu(v) for v in _matvec(W["w_1"], W["b_1"],
                                            _ln(x1, W["ln2_g"], W["ln2_b"], eps))]
            f = _matvec(W["w_2"], W["b_2"], hdn)
            out[b, t] = [x1[c] + f[c] for c in range(C)]
    return out


def patch_merging_direct(x, w, Hs, Ws, eps):
    """Patch merging by loops over output positions: part k of output token (i, j) is the
    image token at row 2i + (k % 2), column 2j + (k // 2); the 4C values are normalised
    together, then multiplied by W_red [2C][4C] (no bias). x is [B, Hs*Ws, C]."""
    x = np.asarray(x, np.float64)
    B, L, C = x.shape
    W = np.asarray(w["w_red"], np.float64).tolist()
    g = np.asarray(w["norm_g"], np.float64).tolist()
    be = np.asarray(w["norm_b"], np.float64).tolist()
    out = np.zeros((B, (Hs // 2) * (Ws // 2), len(W)))
    for b in range(B):
        for i in range(Hs // 2):
            for j in range(Ws // 2):
                v = []
                for k in range(4):
                    y, xx = 2 * i + k % 2, 2 * j + k // 2
                    v.extend(x[b, y * Ws + xx].tolist())
                out[b, i * (Ws // 2) + j] = _matvec(W, [0.0] * len(W), _ln(v, g, be, eps))
    return out


def encoder_layer_int8_dynamic_padded(x_pad, lens, w, heads, eps):
    """Int8-GEMM layer with dynamic activation scales, stage by stage over every valid
    position of the padded batch: each GEMM's input is stored as fp16, its scale is the
    max-abs of those stored values over all valid positions (divided by 127), then codes,
    integer sums and the dequantised result as in encoder_layer_int8_padded."""
    f32 = np.float32
    h = lambda v: float(np.float16(v))
    x_pad = np.asarray(x_pad, np.float64)
    B, S, H = x_pad.shape
    d = H // heads
    W = {k: np.asarray(v) for k, v in w.items()}
    L64 = lambda n: np.asarray(W[n], np.float64).tolist()
    pos = [(b, i) for b in range(B) for i in range(int(lens[b]))]

    def qweights(Wm):
        Wm = np.asarray(Wm, np.float32)
        codes, scales = [], []
        for row in Wm:
            mx = max(abs(f32(v)) for v in row)
            s = f32(mx / f32(127.0)) if mx > 0 else f32(1.0)
            scales.append(s)
            codes.append([_q8(f32(f32(v) / s)) for v in row])
        return codes, scales

    def qlin_all(rows, wn, bn):
        """rows: fp16 values of every valid position; the scale from their max-abs."""
        mx = max(abs(v) for r in rows for v in r)
        s, inv = (f32(f32(mx) / f32(127.0)), f32(f32(127.0) / f32(mx))) if mx > 0 else \
            (f32(1.0), f32(1.0))
        codes, scales = qweights(W[wn])
        bias = np.asarray(W[bn], np.float64)
        out = []
        for r in rows:
            qa = [_q8(f32(f32(v) * inv)) for v in r]
            out.append([sum(qa[k] * codes[n][k] for k in range(len(qa))) * float(f32(s * scales[n]))
                        + float(bias[n]) for n in range(len(codes))])
        return out

    xs = [[h(v) for v in x_pad[b, i]] for b, i in pos]
    qkv = [[h(v) for v in r] for r in qlin_all(xs, "w_qkv", "b_qkv")]
    row_of = {p: n for n, p in enumerate(pos)}
    ctx = []
    for b, i in pos:
        c = [0.0] * H
        keys = [row_of[(b, j)] for j in range(int(lens[b]))]
        for hh in range(heads):
            q = qkv[row_of[(b, i)]][hh * d:(hh + 1) * d]
            sc = [_dot(q, qkv[k][H + hh * d:H + (hh + 1) * d]) / math.sqrt(d) for k in keys]
            p = _softmax_masked(sc, [True] * len(keys))
            for cc in range(d):
                c[hh * d + cc] = h(sum(p[j] * qkv[k][2 * H + hh * d + cc] for j, k in enumerate(keys)))
        ctx.append(c)
    a = qlin_all(ctx, "w_o", "b_o")
    h1 = [[h(v) for v in _ln([h(a[n][c] + x_pad[b, i, c]) for c in range(H)], L64("ln1_g"),
                             L64("ln1_b"), eps)] for n, (b, i) in enumerate(pos)]
    f = [[h(_gelu(z)) for z in r] for r in qlin_all(h1, "w_1", "b_1")]
    o = qlin_all(f, "w_2", "b_2")
    out = np.zeros((B, S, H))
    for n, (b, i) in enumerate(pos):
        out[b, i] = _ln([h(o[n][c] + h1[n][c]) for c in range(H)], L64("ln2_g"), L64("ln2_b"), eps)
    return out
