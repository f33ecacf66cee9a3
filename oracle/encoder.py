"""The JEPA ViT encoder forward pass, written as its plain definition in float64.

TEST INFRASTRUCTURE (see the package docstring).  Every step below is the
textbook operation; numpy's matmul is the only library primitive used, for
the dense products.  Nothing is blocked, fused or reordered.

Where the pages are silent the readings are:
  R1  CLS is token 0 of each item; the pos table has N rows and row 0 belongs
      to CLS; pos is added after patch-embed (and to the CLS token).
  R2  A patch vector lists its elements in (dt, dy, dx, c) order with c
      fastest; tokens are slot-major, then raster order inside a slot.
  R3  qkv output columns are [q | k | v], each D wide; head a owns columns
      a*64 .. a*64+63 of each third.
  R4  Scores are scaled by 1/sqrt(head_dim); softmax subtracts the row max;
      masked pairs are excluded (probability exactly 0).
  R5  Block-causal (LeVJEPA card, opening paragraph): a patch token of
      temporal slot t attends to patch tokens of slots <= t and never to
      CLS; CLS attends to every token including itself.
  R6  LayerNorm uses the biased variance over D and eps inside the square
      root; GELU is the erf form 0.5 z (1 + erf(z / sqrt 2)).
  R7  Pixels are normalised as (u / 255 - mean_c) / std_c.
  R8  Mean pooling averages the final-LayerNorm rows of the patch tokens
      only (CLS excluded).
  R12 3-D rotary position (V-JEPA 2 encoders; the pages name "3-D RoPE" and
      give no formula).  The plainest reading of the published technique
      (RoFormer rotary embedding, one axis per third of the head): each
      head's dimensions are cut into three segments of ds = 2*floor(dh/6)
      (20 of 64), for the tubelet's temporal index t, patch row h and patch
      column w; the dh - 3*ds left over are not rotated.  Pair (2i, 2i+1) of
      a segment is rotated by pos_axis * 10000^(-2i/ds).  q and k are rotated
      before the scores; v is not.  A CLS token has no position (angle 0),
      and with rotary position the model has no additive table.
  R17 The int8 path of block matrices (see quant.quantize_act_q8): the input
      of each of a block's four products is quantised per 32-block and
      dequantised exactly before the product; nothing else changes.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from scipy.special import erf

from . import quant


# ---------------------------------------------------------------------------
# input
# ---------------------------------------------------------------------------

def normalize(frames: np.ndarray, mean, std) -> np.ndarray:
    """uint8 [B, T, H, W, 3] -> float64, (u / 255 - mean_c) / std_c  (R7)."""
    u = np.asarray(frames, dtype=np.float64)
    m = np.asarray(mean, dtype=np.float64)
    s = np.asarray(std, dtype=np.float64)
    return (u / 255.0 - m) / s


def patchify(x: np.ndarray, tubelet: int, patch: int) -> np.ndarray:
    """[B, T, H, W, 3] -> [B, Np, tubelet*patch*patch*3]  (R2).

    Token (tt, i, j) takes frames tt*tubelet .. tt*tubelet+tubelet-1, rows
    i*patch .. , columns j*patch .. ; the V-JEPA 2 card's tubelet 2 groups two
    consecutive frames into one token.
    """
    B, T, H, W, C = x.shape
    kt, p = tubelet, patch
    Tt, Hp, Wp = T // kt, H // p, W // p
    y = x.reshape(B, Tt, kt, Hp, p, Wp, p, C)
    y = y.transpose(0, 1, 3, 5, 2, 4, 6, 7)      # B, tt, i, j, dt, dy, dx, c
    return y.reshape(B, Tt * Hp * Wp, kt * p * p * C)


# ---------------------------------------------------------------------------
# per-token operations
# ---------------------------------------------------------------------------

def linear_act_q8(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """x w^T + b with x first quantised per 32-block as the int8 path does (R17)."""
    return linear(quant.act_q8_values(*quant.quantize_act_q8(x)), w, b)


def linear(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """x [..., in] times w [out, in] transposed, plus b [out]."""
    return x @ w.T + b


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) * g + b over the last axis  (R6)."""
    mu = np.mean(x, axis=-1, keepdims=True)
    var = np.mean((x - mu) ** 2, axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def gelu(z: np.ndarray) -> np.ndarray:
    """0.5 z (1 + erf(z / sqrt(2)))  (R6)."""
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def token_slots(n_slots: int, tokens_per_slot: int, has_cls: bool) -> np.ndarray:
    """Temporal slot of every token of one item; -1 marks CLS (token 0, R1)."""
    s = np.repeat(np.arange(n_slots), tokens_per_slot)
    return np.concatenate([[-1], s]) if has_cls else s


def block_causal_allowed(n_slots: int, tokens_per_slot: int, has_cls: bool) -> np.ndarray:
    """allowed[i, j]: may query token i attend to key token j  (R5)."""
    s = token_slots(n_slots, tokens_per_slot, has_cls)
    is_cls = s < 0
    patch_pair = (~is_cls[:, None]) & (~is_cls[None, :]) & (s[None, :] <= s[:, None])
    cls_row = is_cls[:, None] & np.ones_like(patch_pair)
    return patch_pair | cls_row


def softmax_masked(s: np.ndarray, allowed) -> np.ndarray:
    """Row softmax of s over the allowed entries; excluded entries get 0  (R4)."""
    if allowed is not None:
        s = np.where(allowed, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_head(q, k, v, allowed):
    """One head: softmax(q k^T / sqrt(dh) over allowed) v."""
    s = (q @ k.T) / math.sqrt(q.shape[-1])
    return softmax_masked(s, allowed) @ v


def rope_angles(dims: dict) -> np.ndarray:
    """[N, dh/2] rotation angle of every token and dimension pair (R12)."""
    dh = dims["dim"] // dims["heads"]
    ds = 2 * (dh // 6)
    Tt = dims["frames"] // dims["tubelet"]
    Hp, Wp = dims["img_h"] // dims["patch"], dims["img_w"] // dims["patch"]
    pn = np.arange(Tt * Hp * Wp)
    axes = [pn // (Hp * Wp), (pn // Wp) % Hp, pn % Wp]        # t, h, w of each patch token
    ang = np.zeros((pn.size, dh // 2))
    for a, pos in enumerate(axes):
        for i in range(ds // 2):
            ang[:, a * ds // 2 + i] = pos * 10000.0 ** (-2.0 * i / ds)
    if dims["has_cls"]:
        ang = np.concatenate([np.zeros((1, dh // 2)), ang])  # CLS: no position
    return ang


def rope(x: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """x [N, dh] of one head: pair (2p, 2p+1) of token n rotated by ang[n, p] (R12)."""
    c, s = np.cos(ang), np.sin(ang)
    y = np.empty_like(x)
    y[:, 0::2] = x[:, 0::2] * c - x[:, 1::2] * s
    y[:, 1::2] = x[:, 0::2] * s + x[:, 1::2] * c
    return y


def attention(qkv: np.ndarray, heads: int, allowed, threads: int = 8, ang=None) -> np.ndarray:
    """Multi-head attention of one item.

    qkv [N, 3D] with columns [q | k | v] (R3) -> concat of head outputs [N, D].
    With ang (rope_angles), q and k are rotated per head first (R12).  Heads are
    independent, so they are evaluated on a thread pool; each is the plain
    definition.
    """
    N, threeD = qkv.shape
    D = threeD // 3
    dh = D // heads
    q, k, v = qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:]
    out = np.empty((N, D))

    def one(a):
        sl = slice(a * dh, (a + 1) * dh)
        qa, ka = q[:, sl], k[:, sl]
        if ang is not None:
            qa, ka = rope(qa, ang), rope(ka, ang)
        out[:, sl] = attention_head(qa, ka, v[:, sl], allowed)

    with ThreadPoolExecutor(max_workers=max(1, min(threads, heads))) as ex:
        list(ex.map(one, range(heads)))
    return out


# ---------------------------------------------------------------------------
# the encoder
# ---------------------------------------------------------------------------

def weights_f64(stored: list) -> dict:
    """Stored tensors -> name -> exact float64 values."""
    return {t["name"]: quant.stored_to_f64(t) for t in stored}


def allowed_for(dims: dict):
    """The attention mask of the dims, or None for bidirectional."""
    if dims["mask"] == "bidir":
        return None
    n_slots = dims["frames"] // dims["tubelet"]
    per_slot = (dims["img_h"] // dims["patch"]) * (dims["img_w"] // dims["patch"])
    return block_causal_allowed(n_slots, per_slot, bool(dims["has_cls"]))


def embed(dims: dict, w: dict, frames: np.ndarray) -> np.ndarray:
    """Normalise, patchify, patch-embed, prepend CLS, add pos -> X0 [B, N, D]  (R1)."""
    x = normalize(frames, dims["mean"], dims["std"])
    e = linear(patchify(x, dims["tubelet"], dims["patch"]),
               w["enc.patch_embed.weight"], w["enc.patch_embed.bias"])
    if dims["has_cls"]:
        cls = np.broadcast_to(w["enc.cls_token"], (e.shape[0], 1, e.shape[2]))
        e = np.concatenate([cls, e], axis=1)
    return e + w["enc.pos_embed"] if "enc.pos_embed" in w else e     # none with rotary position (R12)


def block(dims: dict, w: dict, i: int, x: np.ndarray, allowed, prefix: str = "enc.blk.",
          rotary: bool | None = None, act_q8: bool = False) -> np.ndarray:
    """One pre-LN block on X [B, N, D]:  x += Attn(LN1 x);  x += MLP(LN2 x).

    prefix names the block's tensors ("enc.blk." or, for the classifier
    head, "head.blk."); rotary defaults to the model's setting (R12);
    act_q8 runs the four products on quantised inputs (R17)."""
    p = f"{prefix}{i}."
    linear = linear_act_q8 if act_q8 else globals()["linear"]
    eps = dims["ln_eps"]
    h = layer_norm(x, w[p + "ln1.weight"], w[p + "ln1.bias"], eps)
    qkv = linear(h, w[p + "attn_qkv.weight"], w[p + "attn_qkv.bias"])
    if rotary is None:
        rotary = bool(dims.get("rope"))
    ang = rope_angles(dims) if rotary else None
    o = np.stack([attention(qkv[b], dims["heads"], allowed, ang=ang) for b in range(x.shape[0])])
    x = x + linear(o, w[p + "attn_out.weight"], w[p + "attn_out.bias"])
    h = layer_norm(x, w[p + "ln2.weight"], w[p + "ln2.bias"], eps)
    u = gelu(linear(h, w[p + "ffn_up.weight"], w[p + "ffn_up.bias"]))
    return x + linear(u, w[p + "ffn_down.weight"], w[p + "ffn_down.bias"])


def encode(dims: dict, w: dict, frames: np.ndarray, depth: int | None = None,
           return_pre_norm: bool = False, act_q8: bool = False):
    """frames uint8 [B, T, H, W, 3] -> final-LN token map [B, N, D] (float64).

    `depth` evaluates only the first blocks (used to time a bounded sample).
    With return_pre_norm, also returns the residual stream before the final
    LayerNorm.  act_q8: the int8 path of block matrices (R17).
    """
    allowed = allowed_for(dims)
    x = embed(dims, w, frames)
    for i in range(dims["depth"] if depth is None else depth):
        x = block(dims, w, i, x, allowed, act_q8=act_q8)
    y = layer_norm(x, w["enc.norm.weight"], w["enc.norm.bias"], dims["ln_eps"])
    return (y, x) if return_pre_norm else y


def pool(y: np.ndarray, mode: str, has_cls: bool) -> np.ndarray:
    """cls -> y[:, 0]; mean -> mean of the patch rows (R8); none -> y."""
    if mode == "cls":
        if not has_cls:
            raise ValueError("no CLS token")
        return y[:, 0]
    if mode == "mean":
        return np.mean(y[:, 1:] if has_cls else y, axis=1)
    if mode == "none":
        return y
    raise ValueError(mode)
