"""Block quantisation formats q8_0, q4_0, q4_K and q6_K, and exact widening.  Test infrastructure.

The jepa.cpp Quantization page ("File sizes") gives q8_0 as 8.5 bits per
weight and q4_0 as 4.5: one f16 scale per block of 32 weights along a row,
then 32 int8 codes (34 bytes) or 32 four-bit codes (18 bytes).  The page
names the formats by their ggml names; the workloads define them as:

  q8_0: d = max|x| / 127, code q = round(x / d), weight w = d * q.
  q4_0: d = m / -8 where m is the element of largest magnitude (sign kept),
        code q in 0..15, weight w = d * (q - 8).

Readings taken where the pages are silent (all follow the published ggml
block definitions, so that files stay interchangeable):
  * The scale is computed in f32, stored as f16 (round to nearest even); the
    codes are computed from the f32 scale and its f32 reciprocal.
  * q8_0 rounds half away from zero.
  * q4_0 takes the first element of largest magnitude on ties, computes
    floor(x / d + 8.5) in f32 and clamps it to 15; byte j of a block holds
    element j in its low nibble and element j + 16 in its high nibble.
  * An all-zero block has d = 0 and codes 0 (q8_0) or 8 (q4_0).
  * Dequantisation widens d to f32 and multiplies by the integer code; the
    product is exact in f32 (11-bit by at most 8-bit significands).
"""
from __future__ import annotations

import numpy as np

QK = 32                      # weights per block
Q8_0_BLOCK_BYTES = 2 + QK    # f16 scale + 32 int8
Q4_0_BLOCK_BYTES = 2 + QK // 2  # f16 scale + 16 bytes of nibbles


def block_bytes(dtype: str) -> int:
    return {"q8_0": Q8_0_BLOCK_BYTES, "q4_0": Q4_0_BLOCK_BYTES}[dtype]


def _blocks(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % QK:
        raise ValueError("rows must be a multiple of 32 long")
    return x.reshape(x.shape[0], x.shape[1] // QK, QK)


def _pack(d32: np.ndarray, payload: np.ndarray) -> np.ndarray:
    """[rows, nb] f32 scales + [rows, nb, n] uint8 payload -> [rows, nb*(2+n)] bytes."""
    d16 = d32.astype(np.float16).view(np.uint8).reshape(*d32.shape, 2)
    blk = np.concatenate([d16, payload], axis=2)
    return np.ascontiguousarray(blk.reshape(blk.shape[0], -1))


def quantize_q8_0(x: np.ndarray) -> np.ndarray:
    """f32 [rows, K] -> uint8 [rows, K/32*34]."""
    b = _blocks(x)
    amax = np.max(np.abs(b), axis=2)
    d = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(d != 0, np.float32(1.0) / d, np.float32(0.0)).astype(np.float32)
    v = (b * inv[:, :, None]).astype(np.float32).astype(np.float64)
    # round half away from zero; |v| + 0.5 is exact in float64 for an f32 v
    q = (np.sign(v) * np.floor(np.abs(v) + 0.5)).astype(np.int8)
    return _pack(d, q.view(np.uint8))


def quantize_q4_0(x: np.ndarray) -> np.ndarray:
    """f32 [rows, K] -> uint8 [rows, K/32*18]."""
    b = _blocks(x)
    idx = np.argmax(np.abs(b), axis=2)          # first index of the largest |x|
    m = np.take_along_axis(b, idx[:, :, None], axis=2)[:, :, 0]
    d = (m / np.float32(-8.0)).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(d != 0, np.float32(1.0) / d, np.float32(0.0)).astype(np.float32)
    v = (b * inv[:, :, None]).astype(np.float32) + np.float32(8.5)
    q = np.minimum(np.floor(v), 15).astype(np.uint8)
    nib = (q[:, :, :16] | (q[:, :, 16:] << 4)).astype(np.uint8)
    return _pack(d, nib)


def quantize(dtype: str, x: np.ndarray) -> np.ndarray:
    return {"q8_0": quantize_q8_0, "q4_0": quantize_q4_0, "q4_k": quantize_q4_k,
            "q6_k": quantize_q6_k}[dtype](x)


def _unpack(raw: np.ndarray, rows: int, cols: int, bb: int):
    raw = np.ascontiguousarray(raw, dtype=np.uint8).reshape(rows, cols // QK, bb)
    d = raw[:, :, :2].copy().view(np.float16)[:, :, 0].astype(np.float32)
    return d, raw[:, :, 2:]


def dequantize_q8_0(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """uint8 blocks -> exact f32 weights [rows, cols]."""
    d, qs = _unpack(raw, rows, cols, Q8_0_BLOCK_BYTES)
    q = qs.view(np.int8).astype(np.float32)
    return (d[:, :, None] * q).reshape(rows, cols).astype(np.float32)


def dequantize_q4_0(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """uint8 blocks -> exact f32 weights [rows, cols]."""
    d, qs = _unpack(raw, rows, cols, Q4_0_BLOCK_BYTES)
    lo = (qs & 0x0F).astype(np.int32) - 8
    hi = (qs >> 4).astype(np.int32) - 8
    q = np.concatenate([lo, hi], axis=2).astype(np.float32)
    return (d[:, :, None] * q).reshape(rows, cols).astype(np.float32)


# ---------------------------------------------------------------------------
# Activation blocks for integer matrix products (the int8 path of block
# matrices).  The Benchmarks page ("Effect of the weight dtype on a GPU
# (encoder)") times q8_0 and K-quant encoders whose products run on int8
# arithmetic, and the Quantization page says the q8_0 CPU path quantises the
# activations of every product; neither prints the activation format.  The
# reading taken (R17): each row of a product's input is cut into blocks of 32
# along K, like the weight blocks, and quantised the way q8_0 weights are
# (symmetric, d = max|x| / 127, code round(x / d) half away from zero), with
# the scale kept in f32, not rounded to f16.  x / d is one correctly rounded
# f32 division: the codes are integer decisions taken in f32, the precision
# the GPU kernel takes them in.  An all-zero block has d = 0 and codes 0.
#
# The product of such a row with a q8_0 / q4_0 weight row is
#   sum_b d_a[b] d_w[b] sum_{k in b} q_a[k] q_w[k] = sum_k (d_a q_a)[k] w[k],
# exactly, with w the exactly dequantised weights: so the plain product of
# the dequantised activations (act_q8_values) with the stored weights is the
# int8 path's result, with nothing about the integer arithmetic left out.
# ---------------------------------------------------------------------------

def quantize_act_q8(x: np.ndarray):
    """[..., K] -> (int8 codes [..., K], f32 scales [..., K/32])  (R17)."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    K = x32.shape[-1]
    if K % QK:
        raise ValueError("rows must be a multiple of 32 long")
    b = x32.reshape(*x32.shape[:-1], K // QK, QK)
    amax = np.max(np.abs(b), axis=-1)
    d = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(d[..., None] != 0, b / d[..., None], np.float32(0.0)).astype(np.float32)
    v = v.astype(np.float64)
    # round half away from zero; |v| + 0.5 is exact in float64 for an f32 v
    q = np.clip(np.sign(v) * np.floor(np.abs(v) + 0.5), -127, 127).astype(np.int8)
    return q.reshape(x32.shape), d


def act_q8_values(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Codes and scales of quantize_act_q8 -> the float64 values d * q."""
    K = q.shape[-1]
    v = q.reshape(*q.shape[:-1], K // QK, QK).astype(np.float64) * np.asarray(d, np.float64)[..., None]
    return v.reshape(q.shape)


# ---------------------------------------------------------------------------
# K-quants: super-blocks of 256 weights along a row (Quantization page, "The
# rule": "block 256"; "File sizes": q4_k has q4_0's 4.5 bits per weight).  The
# pages name the formats by their ggml names (q4_K, q6_K); their layouts are
# the published ggml ones, restated here:
#   q4_K (144 bytes): f16 d, f16 dmin, 12 bytes of 6-bit sub-block scales and
#        mins, 128 bytes of 4-bit codes.  Sub-block j (32 weights) has scale
#        sc_j and min m_j: for j < 4, sc_j = s[j] & 63 and m_j = s[j+4] & 63;
#        for j >= 4, sc_j = (s[j+4] & 15) | (s[j-4] >> 6) << 4 and
#        m_j = (s[j+4] >> 4) | (s[j] >> 6) << 4.  Bytes 32p .. 32p+31 of the
#        codes hold sub-block 2p in their low nibbles and 2p+1 in their high
#        ones.  w = d sc_j q - dmin m_j.
#   q6_K (210 bytes): 128 bytes of low code bits, 64 bytes of high code
#        bits, 16 int8 sub-block scales, f16 d.  Weight k of a half
#        h = k // 128 (r = k % 128 = 32 t + l, l < 32) has the 6-bit code
#        whose low 4 bits are the low (t < 2) or high (t >= 2) nibble of low
#        byte 64 h + l + 32 (t % 2) and whose high 2 bits are bits 2t, 2t+1
#        of high byte 32 h + l; its scale is scales[k // 16].
#        w = d scales[k // 16] (code - 32).
# Dequantised values are the exact results rounded once to f32.  (Every
# product above has at most 24 significant bits -- an f16 significand of 11
# bits times 6- to 8-bit integers -- so only q4_K's subtraction rounds.)
# ---------------------------------------------------------------------------
QK_K = 256
Q4_K_BLOCK_BYTES = 144
Q6_K_BLOCK_BYTES = 210


def _superblocks(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % QK_K:
        raise ValueError("rows must be a multiple of 256 long")
    return x.reshape(x.shape[0], x.shape[1] // QK_K, QK_K)


def _f16(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float32).astype(np.float16)


def q4_k_scale_min(scales: np.ndarray):
    """The 12 packed bytes of q4_K -> (sc, m), each [..., 8] of 6-bit integers."""
    s = scales.astype(np.int64)
    sc = np.empty(s.shape[:-1] + (8,), np.int64)
    m = np.empty_like(sc)
    for j in range(4):
        sc[..., j] = s[..., j] & 63
        m[..., j] = s[..., j + 4] & 63
    for j in range(4, 8):
        sc[..., j] = (s[..., j + 4] & 15) | ((s[..., j - 4] >> 6) << 4)
        m[..., j] = (s[..., j + 4] >> 4) | ((s[..., j] >> 6) << 4)
    return sc, m


def dequantize_q4_k(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """uint8 q4_K super-blocks -> f32 weights [rows, cols] (exact, rounded once)."""
    b = np.ascontiguousarray(raw, dtype=np.uint8).reshape(rows, cols // QK_K, Q4_K_BLOCK_BYTES)
    d = b[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    dmin = b[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    sc, m = q4_k_scale_min(b[..., 4:16])
    qs = b[..., 16:144].astype(np.int64)
    w = np.empty((rows, cols // QK_K, QK_K), np.float64)
    for p in range(4):
        byte = qs[..., 32 * p:32 * p + 32]
        for half, code in ((0, byte & 15), (1, byte >> 4)):
            j = 2 * p + half
            w[..., 64 * p + 32 * half:64 * p + 32 * half + 32] = (
                (d * sc[..., j])[..., None] * code - (dmin * m[..., j])[..., None])
    return w.reshape(rows, cols).astype(np.float32)


def q6_k_codes(ql: np.ndarray, qh: np.ndarray) -> np.ndarray:
    """low [..., 128] and high [..., 64] code bytes -> the 256 6-bit codes."""
    ql = ql.astype(np.int64)
    qh = qh.astype(np.int64)
    c = np.empty(ql.shape[:-1] + (QK_K,), np.int64)
    for h in range(2):
        for t in range(4):
            lo = ql[..., 64 * h + 32 * (t % 2):64 * h + 32 * (t % 2) + 32]
            lo = lo & 15 if t < 2 else lo >> 4
            hi = (qh[..., 32 * h:32 * h + 32] >> (2 * t)) & 3
            c[..., 128 * h + 32 * t:128 * h + 32 * t + 32] = lo | (hi << 4)
    return c


def dequantize_q6_k(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """uint8 q6_K super-blocks -> f32 weights [rows, cols] (exact, rounded once)."""
    b = np.ascontiguousarray(raw, dtype=np.uint8).reshape(rows, cols // QK_K, Q6_K_BLOCK_BYTES)
    code = q6_k_codes(b[..., 0:128], b[..., 128:192])
    sc = b[..., 192:208].view(np.int8).astype(np.float64)
    d = b[..., 208:210].copy().view(np.float16)[..., 0].astype(np.float64)
    w = d[..., None] * np.repeat(sc, 16, axis=-1) * (code - 32)
    return w.reshape(rows, cols).astype(np.float32)


def quantize_q6_k(x: np.ndarray) -> np.ndarray:
    """f32 [rows, K] -> q6_K blocks [rows, K/256*210].

    A plain encoder (any encoder that writes the format is valid; this one is
    not ggml's search): sub-block scale s = max|x| / 31 over 16 weights,
    d = max(s) / 127 stored as f16, scales[i] = round(s_i / d16) clamped to
    127, codes round(x / (d16 scales[i])) + 32 clamped to 0 .. 63."""
    b = _superblocks(x).astype(np.float64)
    R, NB, _ = b.shape
    sub = b.reshape(R, NB, 16, 16)
    s = np.max(np.abs(sub), axis=-1) / 31.0
    d16 = _f16(np.max(s, axis=-1) / 127.0).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d16[..., None] > 0, np.round(s / d16[..., None]), 0)
        sc = np.clip(sc, 0, 127)
        step = d16[..., None] * sc
        q = np.where(step[..., None] > 0, np.round(sub / step[..., None]), 0)
    code = (np.clip(q, -32, 31) + 32).astype(np.int64).reshape(R, NB, QK_K)
    ql = np.zeros((R, NB, 128), np.int64)
    qh = np.zeros((R, NB, 64), np.int64)
    for h in range(2):
        for t in range(4):
            c = code[..., 128 * h + 32 * t:128 * h + 32 * t + 32]
            lo = slice(64 * h + 32 * (t % 2), 64 * h + 32 * (t % 2) + 32)
            ql[..., lo] |= (c & 15) << (0 if t < 2 else 4)
            qh[..., 32 * h:32 * h + 32] |= (c >> 4) << (2 * t)
    out = np.concatenate([ql.astype(np.uint8), qh.astype(np.uint8), sc.astype(np.int8).view(np.uint8),
                          d16.astype(np.float16).view(np.uint8).reshape(R, NB, 2)], axis=-1)
    return np.ascontiguousarray(out.reshape(R, NB * Q6_K_BLOCK_BYTES))


def quantize_q4_k(x: np.ndarray) -> np.ndarray:
    """f32 [rows, K] -> q4_K blocks [rows, K/256*144].

    A plain encoder: over each 32 weights, the min mn = min(x, 0) and the
    scale (max x - mn) / 15; d = max(scale) / 63 and dmin = max(-mn) / 63
    stored as f16; sc = round(scale / d16), m = round(-mn / dmin16), both
    clamped to 0 .. 63; codes round((x + dmin16 m) / (d16 sc)) clamped to
    0 .. 15."""
    b = _superblocks(x).astype(np.float64)
    R, NB, _ = b.shape
    sub = b.reshape(R, NB, 8, 32)
    mn = np.minimum(np.min(sub, axis=-1), 0.0)
    scale = (np.max(sub, axis=-1) - mn) / 15.0
    d16 = _f16(np.max(scale, axis=-1) / 63.0).astype(np.float64)
    dm16 = _f16(np.max(-mn, axis=-1) / 63.0).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.clip(np.where(d16[..., None] > 0, np.round(scale / d16[..., None]), 0), 0, 63)
        m = np.clip(np.where(dm16[..., None] > 0, np.round(-mn / dm16[..., None]), 0), 0, 63)
        step = d16[..., None] * sc
        q = np.where(step[..., None] > 0, np.round((sub + (dm16[..., None] * m)[..., None]) / step[..., None]), 0)
    q = np.clip(q, 0, 15).astype(np.int64)
    sc = sc.astype(np.int64)
    m = m.astype(np.int64)
    s = np.zeros((R, NB, 12), np.int64)
    for j in range(4):
        s[..., j] = sc[..., j] | ((sc[..., j + 4] >> 4) << 6)
        s[..., j + 4] = m[..., j] | ((m[..., j + 4] >> 4) << 6)
        s[..., j + 8] = (sc[..., j + 4] & 15) | ((m[..., j + 4] & 15) << 4)
    qs = np.zeros((R, NB, 128), np.int64)
    for p in range(4):
        qs[..., 32 * p:32 * p + 32] = q[..., 2 * p, :] | (q[..., 2 * p + 1, :] << 4)
    out = np.concatenate([d16.astype(np.float16).view(np.uint8).reshape(R, NB, 2),
                          dm16.astype(np.float16).view(np.uint8).reshape(R, NB, 2),
                          s.astype(np.uint8), qs.astype(np.uint8)], axis=-1)
    return np.ascontiguousarray(out.reshape(R, NB * Q4_K_BLOCK_BYTES))


# The re-typing tool's fallback (Quantization page, "The rule"): a matrix
# whose row length ne0 is not a multiple of a K-quant's 256 keeps to the
# legacy type of the same width.
K_QUANT_FALLBACK = {"q4_k": "q4_0", "q5_k": "q5_0", "q6_k": "q8_0"}


def type_for(target: str, ne0: int) -> str:
    """The type a block matrix of row length ne0 gets when `target` is asked for."""
    if target in K_QUANT_FALLBACK and ne0 % QK_K:
        return K_QUANT_FALLBACK[target]
    return target


def block_bytes_of(dtype: str) -> tuple[int, int]:
    """(weights per block, bytes per block) of a block format."""
    return {"q8_0": (32, Q8_0_BLOCK_BYTES), "q4_0": (32, Q4_0_BLOCK_BYTES),
            "q4_k": (QK_K, Q4_K_BLOCK_BYTES), "q6_k": (QK_K, Q6_K_BLOCK_BYTES)}[dtype]


def widen_half(bits: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(bits).view(np.float16).astype(np.float64)


def widen_bfloat16(bits: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def stored_to_f64(t: dict) -> np.ndarray:
    """A stored tensor (name, dtype, ne0, ne1, data) -> exact float64 values.

    Matrices come back as [ne1, ne0] (rows = out-features), vectors as [ne0].
    """
    dt, ne0, ne1, data = t["dtype"], t["ne0"], t["ne1"], t["data"]
    if dt == "f32":
        v = np.asarray(data, dtype=np.float32).astype(np.float64)
    elif dt == "f16":
        v = widen_half(data)
    elif dt == "bf16":
        v = widen_bfloat16(data)
    elif dt == "q8_0":
        v = dequantize_q8_0(data, ne1, ne0).astype(np.float64)
    elif dt == "q4_0":
        v = dequantize_q4_0(data, ne1, ne0).astype(np.float64)
    elif dt == "q4_k":
        v = dequantize_q4_k(data, ne1, ne0).astype(np.float64)
    elif dt == "q6_k":
        v = dequantize_q6_k(data, ne1, ne0).astype(np.float64)
    else:
        raise ValueError(dt)
    return v.reshape(ne1, ne0) if ne1 > 1 else v.reshape(ne0)
