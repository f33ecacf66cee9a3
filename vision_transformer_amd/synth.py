"""Seeded synthetic workloads shaped like the jepa.cpp pages' encoders.

This module only draws random numbers and names tensors.  It holds none of
the encoder's arithmetic.  The HIP path and the CPU oracle both take their
inputs from here, as plain numpy arrays.

The jepa.cpp "measured benchmarks" page ("Box and build" section) feeds its
encoder timings with seeded random bytes as pixels, normalised by the
model's own recipe, rather than real clips.  The workloads below do the same
at the model shapes the pages describe:
  * ViT-Ti/14 image encoder, 224x224 (LeWorldModel Push-T card, "Files");
  * ViT-L/16 224x224 image encoder;
  * LeVJEPA ViT-L/16, 16 frames, tubelet 1, block-causal (LeVJEPA card,
    opening paragraph);
  * V-JEPA 2 ViT-L/16, tubelet 2, 256x256, 16 and 64 frames (V-JEPA 2 SSv2
    card, opening paragraph; benchmarks page, "Encoder" table).
Real checkpoints and fixture clips are not used: weights are i.i.d.
N(0, 0.02) and pixels are i.i.d. uniform bytes.
"""
from __future__ import annotations

import copy

import numpy as np

# Storage dtypes a tensor may have (jepa.cpp Quantization page, "The rule":
# only the four 2-D block matrices may be re-typed to a block format).
DTYPES = ("f32", "f16", "bf16", "q8_0", "q4_0", "q4_k", "q6_k")
# The same rule: a K-quant target applies only to rows that are a multiple
# of 256 long; other rows take these formats instead.
K_QUANT_ROW = 256
K_QUANT_FALLBACK = {"q4_k": "q4_0", "q6_k": "q8_0"}
BLOCK_MATRICES = ("attn_qkv", "attn_q", "attn_k", "attn_v", "attn_out", "ffn_up", "ffn_down")


def _dims(**kw):
    d = dict(dim=192, depth=12, heads=3, mlp_dim=768, patch=14, tubelet=1,
             img_h=224, img_w=224, frames=1, has_cls=1, mask="bidir",
             ln_eps=1e-6, mean=(0.5, 0.5, 0.5), std=(0.5, 0.5, 0.5),
             act_dtype="f32", mat_dtype="f32", rest_dtype="f32", rope=0,
             head_blocks=0, head_classes=0)
    d.update(kw)
    return d


_VITL = dict(dim=1024, depth=24, heads=16, mlp_dim=4096, patch=16)

# The full-size workloads.  Each entry: dims, batch, frame seed, weight
# seed, which pooled outputs the workload reports.
WORKLOADS = {
    "vit_ti14_image_f32": dict(
        dims=_dims(), batch=1, frame_seed=1000, weight_seed=2000,
        outputs=("tokens", "cls", "mean")),
    "vit_l16_image_bf16_b32": dict(
        dims=_dims(**_VITL, act_dtype="bf16", mat_dtype="bf16", rest_dtype="bf16"),
        batch=32, frame_seed=1001, weight_seed=2001, outputs=("cls",)),
    "levjepa_vit_l16_16f_bf16_b4": dict(
        dims=_dims(**_VITL, frames=16, mask="block_causal", act_dtype="bf16",
                   mat_dtype="bf16", rest_dtype="bf16"),
        batch=4, frame_seed=1002, weight_seed=2002, outputs=("cls",)),
    "vjepa2_vit_l16_16f256_q8_0_b4": dict(
        dims=_dims(**_VITL, frames=16, tubelet=2, img_h=256, img_w=256, has_cls=0,
                   act_dtype="f16", mat_dtype="q8_0", rest_dtype="f16"),
        batch=4, frame_seed=1003, weight_seed=2003, outputs=("mean",)),
    "vjepa2_vit_l16_64f256_f16": dict(
        dims=_dims(**_VITL, frames=64, tubelet=2, img_h=256, img_w=256, has_cls=0,
                   act_dtype="f16", mat_dtype="f16", rest_dtype="f16"),
        batch=1, frame_seed=1004, weight_seed=2004, outputs=("tokens", "mean")),
    "vjepa2_vit_l16_64f256_q4_0": dict(
        dims=_dims(**_VITL, frames=64, tubelet=2, img_h=256, img_w=256, has_cls=0,
                   act_dtype="f16", mat_dtype="q4_0", rest_dtype="f16"),
        batch=1, frame_seed=1004, weight_seed=2004, outputs=("tokens", "mean")),
    # the V-JEPA 2 encoder with its 3-D rotary position instead of an
    # additive table (V-JEPA 2 card, opening paragraph)
    "vjepa2_rope_vit_l16_16f256_f16_b4": dict(
        dims=_dims(**_VITL, frames=16, tubelet=2, img_h=256, img_w=256, has_cls=0,
                   act_dtype="f16", mat_dtype="f16", rest_dtype="f16", rope=1),
        batch=4, frame_seed=1005, weight_seed=2005, outputs=("mean",)),
    # blocks of the V-JEPA 2 predictor's width (12 layers, 384-d, heads of
    # 32) at its worst case on the benchmarks page ("Masked predictor"
    # table: context = target = every token of a 16-frame 256x256 clip, 4096
    # tokens), with 3-D rotary position; the tokens come from 32 frames
    "vjepa2_predictor_width_384d_dh32_4096tok_bf16_b4": dict(
        dims=_dims(dim=384, depth=12, heads=12, mlp_dim=1536, patch=16, frames=32, tubelet=2,
                   img_h=256, img_w=256, has_cls=0, act_dtype="bf16", mat_dtype="bf16",
                   rest_dtype="bf16", rope=1),
        batch=4, frame_seed=1006, weight_seed=2006, outputs=("mean",)),
    # the V-JEPA 2 ViT-L/16 SSv2 classifier (V-JEPA 2 SSv2 card, opening
    # paragraph): the encoder with 3-D rotary position and the attentive-pool
    # head, 3 self-attention blocks and 174 classes
    "vjepa2_ssv2_classifier_vit_l16_16f256_f16_b4": dict(
        dims=_dims(**_VITL, frames=16, tubelet=2, img_h=256, img_w=256, has_cls=0,
                   act_dtype="f16", mat_dtype="f16", rest_dtype="f16", rope=1,
                   head_blocks=3, head_classes=174),
        batch=4, frame_seed=1007, weight_seed=2007, outputs=("logits", "mean")),
}

# Small workloads the oracle finishes in seconds.  They keep the structure of
# the big ones (CLS or not, block-causal frames, tubelet 2, block formats) and
# are sized to span several kernel tiles with ragged tails.
SMALL_WORKLOADS = {
    "small_blockcausal_bf16": dict(
        dims=_dims(dim=128, depth=2, heads=2, mlp_dim=512, patch=16, img_h=96,
                   img_w=96, frames=8, mask="block_causal", act_dtype="bf16",
                   mat_dtype="bf16", rest_dtype="bf16"),
        batch=3, frame_seed=11, weight_seed=21),
    "small_bidir_cls_bf16": dict(
        dims=_dims(dim=192, depth=2, heads=3, mlp_dim=768, patch=16, img_h=80,
                   img_w=112, frames=3, act_dtype="bf16", mat_dtype="bf16",
                   rest_dtype="bf16"),
        batch=2, frame_seed=12, weight_seed=22),
    "small_bidir_f32": dict(
        dims=_dims(dim=128, depth=2, heads=2, mlp_dim=256, patch=14, img_h=84,
                   img_w=98, frames=2, act_dtype="f32", mat_dtype="f32",
                   rest_dtype="f32"),
        batch=2, frame_seed=13, weight_seed=23),
    "small_tubelet2_q8_0": dict(
        dims=_dims(dim=128, depth=2, heads=2, mlp_dim=512, patch=16, tubelet=2,
                   img_h=96, img_w=112, frames=6, has_cls=0, act_dtype="f16",
                   mat_dtype="q8_0", rest_dtype="f16"),
        batch=2, frame_seed=14, weight_seed=24),
    "small_tubelet2_q4_0": dict(
        dims=_dims(dim=128, depth=2, heads=2, mlp_dim=512, patch=16, tubelet=2,
                   img_h=96, img_w=112, frames=6, has_cls=0, act_dtype="f16",
                   mat_dtype="q4_0", rest_dtype="f16"),
        batch=2, frame_seed=14, weight_seed=24),
    "small_tubelet2_f16_blockcausal": dict(
        dims=_dims(dim=128, depth=2, heads=2, mlp_dim=512, patch=16, tubelet=2,
                   img_h=64, img_w=96, frames=8, has_cls=0, mask="block_causal",
                   act_dtype="f16", mat_dtype="f16", rest_dtype="f16"),
        batch=2, frame_seed=15, weight_seed=25),
    # 3-D rotary position instead of the additive table (V-JEPA 2 card: the
    # encoder's "3-D RoPE"); with and without a CLS token
    "small_rope_tubelet2_f16": dict(
        dims=_dims(dim=128, depth=2, heads=2, mlp_dim=512, patch=16, tubelet=2,
                   img_h=96, img_w=112, frames=6, has_cls=0, act_dtype="f16",
                   mat_dtype="f16", rest_dtype="f16", rope=1),
        batch=2, frame_seed=16, weight_seed=26),
    "small_rope_cls_blockcausal_bf16": dict(
        dims=_dims(dim=192, depth=2, heads=3, mlp_dim=768, patch=16, img_h=64,
                   img_w=80, frames=5, mask="block_causal", act_dtype="bf16",
                   mat_dtype="bf16", rest_dtype="bf16", rope=1),
        batch=2, frame_seed=17, weight_seed=27),
    "small_rope_f32": dict(
        dims=_dims(dim=128, depth=2, heads=2, mlp_dim=256, patch=14, img_h=84,
                   img_w=98, frames=2, act_dtype="f32", mat_dtype="f32",
                   rest_dtype="f32", rope=1),
        batch=2, frame_seed=18, weight_seed=28),
    # heads of 32 (the V-JEPA 2 predictor's head width)
    "small_dh32_cls_bf16": dict(
        dims=_dims(dim=192, depth=2, heads=6, mlp_dim=768, patch=16, img_h=80,
                   img_w=112, frames=3, act_dtype="bf16", mat_dtype="bf16",
                   rest_dtype="bf16"),
        batch=2, frame_seed=20, weight_seed=30),
    "small_dh32_rope_blockcausal_f16": dict(
        dims=_dims(dim=128, depth=2, heads=4, mlp_dim=512, patch=16, tubelet=2,
                   img_h=64, img_w=96, frames=8, has_cls=0, mask="block_causal",
                   act_dtype="f16", mat_dtype="f16", rest_dtype="f16", rope=1),
        batch=2, frame_seed=21, weight_seed=31),
    "small_dh32_f32": dict(
        dims=_dims(dim=128, depth=2, heads=4, mlp_dim=256, patch=14, img_h=84,
                   img_w=98, frames=2, act_dtype="f32", mat_dtype="f32",
                   rest_dtype="f32", rope=1),
        batch=2, frame_seed=22, weight_seed=32),
    # f32, block-causal with CLS (small f32 models split keys and K over
    # workgroups; queries early in a frame see no key in the later splits)
    "small_blockcausal_f32": dict(
        dims=_dims(dim=128, depth=2, heads=2, mlp_dim=512, patch=16, img_h=64,
                   img_w=96, frames=6, mask="block_causal", act_dtype="f32",
                   mat_dtype="f32", rest_dtype="f32"),
        batch=2, frame_seed=26, weight_seed=36),
    # with the attentive-pool classifier head
    "small_head_bf16": dict(
        dims=_dims(dim=128, depth=2, heads=2, mlp_dim=512, patch=16, tubelet=2,
                   img_h=64, img_w=96, frames=4, has_cls=0, act_dtype="bf16",
                   mat_dtype="bf16", rest_dtype="bf16", rope=1, head_blocks=3,
                   head_classes=10),
        batch=3, frame_seed=23, weight_seed=33),
    "small_head_cls_q8_0": dict(
        dims=_dims(dim=192, depth=2, heads=3, mlp_dim=768, patch=16, img_h=80,
                   img_w=112, frames=3, act_dtype="f16", mat_dtype="q8_0",
                   rest_dtype="f16", head_blocks=1, head_classes=70),
        batch=2, frame_seed=24, weight_seed=34),
    "small_head_dh32_f32": dict(
        dims=_dims(dim=128, depth=2, heads=4, mlp_dim=256, patch=14, img_h=84,
                   img_w=98, frames=2, act_dtype="f32", mat_dtype="f32",
                   rest_dtype="f32", head_blocks=2, head_classes=5),
        batch=2, frame_seed=25, weight_seed=35),
    "small_rope_q4_0": dict(
        dims=_dims(dim=128, depth=2, heads=2, mlp_dim=512, patch=16, tubelet=2,
                   img_h=96, img_w=112, frames=6, has_cls=0, act_dtype="f16",
                   mat_dtype="q4_0", rest_dtype="f16", rope=1),
        batch=2, frame_seed=19, weight_seed=29),
    # K-quant targets (super-blocks of 256 weights): D = 192 rows fall back
    # to q4_0, the 768-long ffn_down rows (and the head's) stay q4_K
    "small_q4_k_fallback_head_bf16": dict(
        dims=_dims(dim=192, depth=2, heads=3, mlp_dim=768, patch=16, img_h=80,
                   img_w=112, frames=3, act_dtype="bf16", mat_dtype="q4_k",
                   rest_dtype="bf16", head_blocks=1, head_classes=12),
        batch=2, frame_seed=61, weight_seed=71),
    "small_q6_k_rope_blockcausal_f16": dict(
        dims=_dims(dim=256, depth=2, heads=4, mlp_dim=1024, patch=16, tubelet=2,
                   img_h=64, img_w=96, frames=4, has_cls=0, mask="block_causal",
                   act_dtype="f16", mat_dtype="q6_k", rest_dtype="f16", rope=1),
        batch=2, frame_seed=62, weight_seed=72),
    "small_q4_k_dh32_cls_bf16": dict(
        dims=_dims(dim=256, depth=2, heads=8, mlp_dim=512, patch=16, img_h=96,
                   img_w=80, frames=2, act_dtype="bf16", mat_dtype="q4_k",
                   rest_dtype="bf16"),
        batch=3, frame_seed=63, weight_seed=73),
}


# ViT-L/16 widths (D 1024, 16 heads, MLP 4096) at two blocks and about a
# thousand rows per batch: every GEMM shape of the full-size encoders (qkv,
# out-proj, fc1, fc2) on the 256-row tiles, small enough for the oracle to
# check every token.
MID_WORKLOADS = {
    "mid_vitl_blockcausal_bf16": dict(
        dims=_dims(**dict(_VITL, depth=2), frames=4, mask="block_causal", act_dtype="bf16",
                   mat_dtype="bf16", rest_dtype="bf16"),
        batch=2, frame_seed=41, weight_seed=51),
    "mid_vitl_tubelet2_q8_0": dict(
        dims=_dims(**dict(_VITL, depth=2), frames=4, tubelet=2, img_h=256, img_w=256, has_cls=0,
                   act_dtype="f16", mat_dtype="q8_0", rest_dtype="f16"),
        batch=2, frame_seed=42, weight_seed=52),
    "mid_vitl_rope_q4_0": dict(
        dims=_dims(**dict(_VITL, depth=2), frames=4, tubelet=2, img_h=256, img_w=256, has_cls=0,
                   act_dtype="f16", mat_dtype="q4_0", rest_dtype="f16", rope=1),
        batch=2, frame_seed=43, weight_seed=53),
    "mid_vitl_q4_k": dict(
        dims=_dims(**dict(_VITL, depth=2), frames=4, tubelet=2, img_h=256, img_w=256, has_cls=0,
                   act_dtype="f16", mat_dtype="q4_k", rest_dtype="f16"),
        batch=2, frame_seed=44, weight_seed=54),
}


def workload(name: str) -> dict:
    """A deep copy of a named workload (full-size, mid-size or small)."""
    for table in (WORKLOADS, MID_WORKLOADS, SMALL_WORKLOADS):
        if name in table:
            return copy.deepcopy(table[name])
    raise KeyError(name)


# ----------------------------------------------------------------------------
# shapes
# ----------------------------------------------------------------------------

def grid(dims: dict) -> tuple[int, int, int]:
    """(temporal slots, patch rows, patch columns)."""
    return (dims["frames"] // dims["tubelet"], dims["img_h"] // dims["patch"],
            dims["img_w"] // dims["patch"])


def n_patches(dims: dict) -> int:
    t, h, w = grid(dims)
    return t * h * w


def n_tokens(dims: dict) -> int:
    return n_patches(dims) + int(dims["has_cls"])


def patch_dim(dims: dict) -> int:
    return dims["tubelet"] * dims["patch"] * dims["patch"] * 3


def tensor_specs(dims: dict) -> list[tuple[str, int, int]]:
    """(name, ne0, ne1) for every tensor, in the fixed draw order.

    ne0 is the row length (in-features for a matrix), ne1 the row count
    (out-features); vectors have ne1 = 1.  Names follow the tensor schema
    on the jepa.cpp Quantization page ("The rule" table and the CLI listing).
    """
    D, F, P, N = dims["dim"], dims["mlp_dim"], patch_dim(dims), n_tokens(dims)
    s = [("enc.patch_embed.weight", P, D), ("enc.patch_embed.bias", D, 1)]
    if dims["has_cls"]:
        s.append(("enc.cls_token", D, 1))
    if not dims.get("rope"):
        s.append(("enc.pos_embed", D, N))
    for i in range(dims["depth"]):
        p = f"enc.blk.{i}."
        s += [(p + "ln1.weight", D, 1), (p + "ln1.bias", D, 1),
              (p + "attn_qkv.weight", D, 3 * D), (p + "attn_qkv.bias", 3 * D, 1),
              (p + "attn_out.weight", D, D), (p + "attn_out.bias", D, 1),
              (p + "ln2.weight", D, 1), (p + "ln2.bias", D, 1),
              (p + "ffn_up.weight", D, F), (p + "ffn_up.bias", F, 1),
              (p + "ffn_down.weight", F, D), (p + "ffn_down.bias", D, 1)]
    s += [("enc.norm.weight", D, 1), ("enc.norm.bias", D, 1)]
    if dims.get("head_classes"):
        # the attentive-pool classifier head (V-JEPA 2 SSv2 card): its
        # self-attention blocks, the cross-attention query block, the classifier
        for i in range(dims["head_blocks"]):
            p = f"head.blk.{i}."
            s += [(p + "ln1.weight", D, 1), (p + "ln1.bias", D, 1),
                  (p + "attn_qkv.weight", D, 3 * D), (p + "attn_qkv.bias", 3 * D, 1),
                  (p + "attn_out.weight", D, D), (p + "attn_out.bias", D, 1),
                  (p + "ln2.weight", D, 1), (p + "ln2.bias", D, 1),
                  (p + "ffn_up.weight", D, F), (p + "ffn_up.bias", F, 1),
                  (p + "ffn_down.weight", F, D), (p + "ffn_down.bias", D, 1)]
        p = "head.xattn."
        s += [("head.query_token", D, 1),
              (p + "ln1.weight", D, 1), (p + "ln1.bias", D, 1),
              (p + "attn_q.weight", D, D), (p + "attn_q.bias", D, 1),
              (p + "attn_k.weight", D, D), (p + "attn_k.bias", D, 1),
              (p + "attn_v.weight", D, D), (p + "attn_v.bias", D, 1),
              (p + "attn_out.weight", D, D), (p + "attn_out.bias", D, 1),
              (p + "ln2.weight", D, 1), (p + "ln2.bias", D, 1),
              (p + "ffn_up.weight", D, F), (p + "ffn_up.bias", F, 1),
              (p + "ffn_down.weight", F, D), (p + "ffn_down.bias", D, 1),
              ("head.classifier.weight", D, dims["head_classes"]),
              ("head.classifier.bias", dims["head_classes"], 1)]
    return s


def is_block_matrix(name: str) -> bool:
    return name.endswith(".weight") and any(f".{m}." in name for m in BLOCK_MATRICES)


def is_layernorm(name: str) -> bool:
    return name.startswith("enc.norm.") or ".ln1." in name or ".ln2." in name


def storage_dtype(dims: dict, name: str, ne0: int | None = None) -> str:
    """The stored dtype of a tensor under the re-typing rule (ne0, its row
    length, decides the K-quant fallback)."""
    if not is_block_matrix(name):
        return dims["rest_dtype"]
    dt = dims["mat_dtype"]
    if dt in K_QUANT_FALLBACK and ne0 is not None and ne0 % K_QUANT_ROW:
        return K_QUANT_FALLBACK[dt]
    return dt


# ----------------------------------------------------------------------------
# random draws
# ----------------------------------------------------------------------------

def make_frames(dims: dict, batch: int, seed: int) -> np.ndarray:
    """uint8 frames [B, T, H, W, 3], HWC, i.i.d. uniform over 0..255."""
    rng = np.random.default_rng(seed)
    shape = (batch, dims["frames"], dims["img_h"], dims["img_w"], 3)
    return rng.integers(0, 256, size=shape, dtype=np.uint8)


def make_f32_weights(dims: dict, seed: int, ln_affine: bool = False) -> dict:
    """f32 weights drawn i.i.d. N(0, 0.02) in tensor_specs order.

    LayerNorm gains are 1 and shifts 0, unless ln_affine is set, in which case
    gains are 1 + N(0, 0.02) and shifts N(0, 0.02) (drawn in order too).
    """
    rng = np.random.default_rng(seed)
    out = {}
    for name, ne0, ne1 in tensor_specs(dims):
        shape = (ne1, ne0) if ne1 > 1 else (ne0,)
        if is_layernorm(name):
            if ln_affine:
                w = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
                if name.endswith(".weight"):
                    w = w + np.float32(1.0)
            else:
                w = np.ones(shape, np.float32) if name.endswith(".weight") \
                    else np.zeros(shape, np.float32)
        else:
            w = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
        out[name] = w.astype(np.float32)
    return out


def to_half_bits(w: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (round to nearest even) as uint16."""
    return np.ascontiguousarray(w, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bfloat16_bits(w: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (round to nearest even, via torch) as uint16."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def stored_weights(dims: dict, w32: dict, quantize=None) -> list[dict]:
    """The weight set as stored tensors, in tensor_specs order.

    Each entry: name, dtype, ne0, ne1 and data (a contiguous numpy array of
    the raw storage: float32, uint16 half/bfloat16 bits, or uint8 blocks).
    Block formats need `quantize(dtype, f32_matrix) -> uint8 array`, which
    the caller supplies; this module does no quantisation itself.
    """
    out = []
    for name, ne0, ne1 in tensor_specs(dims):
        dt = storage_dtype(dims, name, ne0)
        w = w32[name]
        if dt == "f32":
            data = np.ascontiguousarray(w, dtype=np.float32)
        elif dt == "f16":
            data = to_half_bits(w)
        elif dt == "bf16":
            data = to_bfloat16_bits(w)
        else:
            if quantize is None:
                raise ValueError(f"{name}: {dt} storage needs a quantizer")
            data = np.ascontiguousarray(quantize(dt, w.reshape(ne1, ne0)), dtype=np.uint8)
        out.append(dict(name=name, dtype=dt, ne0=ne0, ne1=ne1, data=data))
    return out
