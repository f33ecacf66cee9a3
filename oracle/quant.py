"""Block quantisation formats q8_0 and q4_0, and exact widening.  Test infrastructure.

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
    return {"q8_0": quantize_q8_0, "q4_0": quantize_q4_0}[dtype](x)


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
    else:
        raise ValueError(dt)
    return v.reshape(ne1, ne0) if ne1 > 1 else v.reshape(ne0)
