"""A brute-force encoder in pure Python loops, for tiny inputs only.

Written independently of the vectorised oracle (scalar loops over explicit
indices, the math module only) so that an indexing, transposition or
dropped-term mistake in either one shows up as a mismatch.  Used by the
oracle's pin tests; never by the HIP path.
"""
from __future__ import annotations

import cmath
import math


def _embed(dims, w, frames):
    B, T, H, W, _ = frames.shape
    kt, p, D = dims["tubelet"], dims["patch"], dims["dim"]
    Tt, Hp, Wp = T // kt, H // p, W // p
    Wpe, bpe, pos = w["enc.patch_embed.weight"], w["enc.patch_embed.bias"], w.get("enc.pos_embed")
    out = []
    for b in range(B):
        toks = []
        if dims["has_cls"]:
            toks.append([float(w["enc.cls_token"][d]) for d in range(D)])
        for tt in range(Tt):
            for i in range(Hp):
                for j in range(Wp):
                    v = []
                    for dt in range(kt):
                        for dy in range(p):
                            for dx in range(p):
                                for c in range(3):
                                    u = int(frames[b, tt * kt + dt, i * p + dy, j * p + dx, c])
                                    v.append((u / 255.0 - dims["mean"][c]) / dims["std"][c])
                    toks.append([float(bpe[d]) + sum(float(Wpe[d, k]) * v[k] for k in range(len(v)))
                                 for d in range(D)])
        out.append([[toks[n][d] + (float(pos[n, d]) if pos is not None else 0.0) for d in range(D)]
                    for n in range(len(toks))])
    return out


def _ln(row, g, bta, eps):
    D = len(row)
    mu = sum(row) / D
    var = sum((r - mu) ** 2 for r in row) / D
    return [(row[d] - mu) / math.sqrt(var + eps) * float(g[d]) + float(bta[d]) for d in range(D)]


def _lin(row, W, bias):
    return [float(bias[o]) + sum(float(W[o, i]) * row[i] for i in range(len(row)))
            for o in range(W.shape[0])]


def _may_attend(dims, i, j):
    if dims["mask"] == "bidir":
        return True
    per_slot = (dims["img_h"] // dims["patch"]) * (dims["img_w"] // dims["patch"])
    c = int(dims["has_cls"])
    if c and i == 0:
        return True            # CLS sees every token
    if c and j == 0:
        return False           # no patch token sees CLS
    return (j - c) // per_slot <= (i - c) // per_slot


def _rotary(dims, vec):
    """3-D rotary position of q or k: vec[N][dh] of one head -> rotated copy.

    Each dimension pair is read as one complex number and multiplied by the
    unit complex number of angle position * frequency; the head is split into
    a t, an h and a w segment of 2*floor(dh/6) dimensions each, the rest is
    left alone, and a CLS token (no position) is not rotated."""
    dh = len(vec[0])
    seg = 2 * (dh // 6)
    c = int(dims["has_cls"])
    Hp, Wp = dims["img_h"] // dims["patch"], dims["img_w"] // dims["patch"]
    pos = [None] * c
    for tt in range(dims["frames"] // dims["tubelet"]):
        for i in range(Hp):
            for j in range(Wp):
                pos.append((tt, i, j))
    out = []
    for n, row in enumerate(vec):
        r = list(row)
        if pos[n] is not None:
            for axis in range(3):
                for k in range(seg // 2):
                    d = axis * seg + 2 * k
                    z = complex(row[d], row[d + 1]) * cmath.exp(1j * pos[n][axis] / 10000.0 ** (2.0 * k / seg))
                    r[d], r[d + 1] = z.real, z.imag
        out.append(r)
    return out


def _block(dims, w, p, x, rotary, may_attend):
    """One pre-LN block (tensors under prefix p) on one item's rows x [N][D]."""
    D, H = dims["dim"], dims["heads"]
    dh = D // H
    eps = dims["ln_eps"]
    N = len(x)
    qkv = [_lin(_ln(x[n], w[p + "ln1.weight"], w[p + "ln1.bias"], eps),
                w[p + "attn_qkv.weight"], w[p + "attn_qkv.bias"]) for n in range(N)]
    o = [[0.0] * D for _ in range(N)]
    for a in range(H):
        qa = [qkv[n][a * dh:(a + 1) * dh] for n in range(N)]
        ka = [qkv[n][D + a * dh:D + (a + 1) * dh] for n in range(N)]
        if rotary:
            qa, ka = _rotary(dims, qa), _rotary(dims, ka)
        for i in range(N):
            js = [j for j in range(N) if may_attend(i, j)]
            s = [sum(qa[i][t] * ka[j][t] for t in range(dh)) / math.sqrt(dh) for j in js]
            m = max(s)
            e = [math.exp(v - m) for v in s]
            z = sum(e)
            for t in range(dh):
                o[i][a * dh + t] = sum(e[q] / z * qkv[js[q]][2 * D + a * dh + t] for q in range(len(js)))
    att = [_lin(o[n], w[p + "attn_out.weight"], w[p + "attn_out.bias"]) for n in range(N)]
    x = [[x[n][d] + att[n][d] for d in range(D)] for n in range(N)]
    mlp = []
    for n in range(N):
        h = _lin(_ln(x[n], w[p + "ln2.weight"], w[p + "ln2.bias"], eps), w[p + "ffn_up.weight"], w[p + "ffn_up.bias"])
        h = [0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0))) for z in h]
        mlp.append(_lin(h, w[p + "ffn_down.weight"], w[p + "ffn_down.bias"]))
    return [[x[n][d] + mlp[n][d] for d in range(D)] for n in range(N)]


def encode(dims, w, frames):
    """frames uint8 [B, T, H, W, 3] -> list [B][N][D] of floats."""
    X = _embed(dims, w, frames)
    for li in range(dims["depth"]):
        for b in range(len(X)):
            X[b] = _block(dims, w, f"enc.blk.{li}.", X[b], dims.get("rope"),
                          lambda i, j: _may_attend(dims, i, j))
    eps = dims["ln_eps"]
    return [[_ln(r, w["enc.norm.weight"], w["enc.norm.bias"], eps) for r in xb] for xb in X]


def classify(dims, w, y):
    """Attentive-pool head on a token map y [B][N][D] -> class scores [B][C]:
    the head's blocks, then one learned query attending (per head) over the
    layer-normalised tokens, its out-projection added to the query, an MLP
    with residual, and the classifier."""
    D, H = dims["dim"], dims["heads"]
    dh = D // H
    eps = dims["ln_eps"]
    p = "head.xattn."
    q0 = [float(t) for t in w["head.query_token"]]
    q = _lin(q0, w[p + "attn_q.weight"], w[p + "attn_q.bias"])
    out = []
    for xb in y:
        x = [list(r) for r in xb]
        for i in range(dims["head_blocks"]):
            x = _block(dims, w, f"head.blk.{i}.", x, False, lambda i_, j_: True)
        hs = [_ln(r, w[p + "ln1.weight"], w[p + "ln1.bias"], eps) for r in x]
        ks = [_lin(h, w[p + "attn_k.weight"], w[p + "attn_k.bias"]) for h in hs]
        vs = [_lin(h, w[p + "attn_v.weight"], w[p + "attn_v.bias"]) for h in hs]
        o = [0.0] * D
        for a in range(H):
            s = [sum(q[a * dh + t] * k[a * dh + t] for t in range(dh)) / math.sqrt(dh) for k in ks]
            m = max(s)
            e = [math.exp(v - m) for v in s]
            z = sum(e)
            for t in range(dh):
                o[a * dh + t] = sum(e[n] / z * vs[n][a * dh + t] for n in range(len(vs)))
        att = _lin(o, w[p + "attn_out.weight"], w[p + "attn_out.bias"])
        xq = [q0[d] + att[d] for d in range(D)]
        u = _lin(_ln(xq, w[p + "ln2.weight"], w[p + "ln2.bias"], eps), w[p + "ffn_up.weight"], w[p + "ffn_up.bias"])
        u = [0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0))) for z in u]
        mlp = _lin(u, w[p + "ffn_down.weight"], w[p + "ffn_down.bias"])
        xq = [xq[d] + mlp[d] for d in range(D)]
        out.append(_lin(xq, w["head.classifier.weight"], w["head.classifier.bias"]))
    return out


def _f32(v: float) -> float:
    """v rounded to the nearest f32 (ties to even), as a Python float."""
    import struct
    return struct.unpack("<f", struct.pack("<f", v))[0]


def quantize_act_q8(row):
    """One row (a multiple of 32 long) -> (codes, scales), scalar loops.

    The f32 quotient of two f32 values is the f64 quotient rounded to f32 (the
    double rounding is harmless for division: 53 >= 2*24 + 2)."""
    codes, scales = [], []
    for b0 in range(0, len(row), 32):
        blk = [_f32(float(v)) for v in row[b0:b0 + 32]]
        amax = 0.0
        for v in blk:
            amax = max(amax, abs(v))
        d = _f32(amax / 127.0)
        scales.append(d)
        for v in blk:
            if d == 0.0:
                codes.append(0)
                continue
            t = _f32(v / d)
            q = math.floor(abs(t) + 0.5)
            q = min(q, 127)
            codes.append(int(q) if t >= 0 else -int(q))
    return codes, scales
