"""Pins of the CPU oracle to things other than itself (CPU only).

Each test fixes part of the oracle against a closed form, an invariant,
a printed value of the pages, or a brute-force evaluation on a tiny input,
chosen so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import encoder as E
from oracle import metrics as M
from oracle import quant as Q
from tests import brute
from vision_transformer_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# normalisation and patchify
# ---------------------------------------------------------------------------

def test_normalize_closed_form():
    u = np.array([0, 255, 51, 204], dtype=np.uint8).reshape(1, 1, 1, 4, 1).repeat(3, axis=4)
    x = E.normalize(u, (0.5, 0.5, 0.5), (0.5, 0.5, 0.5))
    np.testing.assert_allclose(x[0, 0, 0, :, 0], [-1.0, 1.0, -0.6, 0.6], rtol=0, atol=1e-15)
    # per-channel constants land on their own channel
    y = E.normalize(u, (0.1, 0.2, 0.3), (1.0, 2.0, 4.0))
    assert y[0, 0, 0, 1, 0] == pytest.approx((1 - 0.1) / 1.0)
    assert y[0, 0, 0, 1, 1] == pytest.approx((1 - 0.2) / 2.0)
    assert y[0, 0, 0, 1, 2] == pytest.approx((1 - 0.3) / 4.0)


def test_patchify_brute_force():
    rng = np.random.default_rng(0)
    B, T, H, W, kt, p = 2, 4, 6, 9, 2, 3
    x = rng.standard_normal((B, T, H, W, 3))
    P = E.patchify(x, kt, p)
    Tt, Hp, Wp = T // kt, H // p, W // p
    assert P.shape == (B, Tt * Hp * Wp, kt * p * p * 3)
    for b in range(B):
        for tt in range(Tt):
            for i in range(Hp):
                for j in range(Wp):
                    n = (tt * Hp + i) * Wp + j
                    k = 0
                    for dt in range(kt):
                        for dy in range(p):
                            for dx in range(p):
                                for c in range(3):
                                    assert P[b, n, k] == x[b, tt * kt + dt, i * p + dy, j * p + dx, c]
                                    k += 1


def test_identity_patch_embed_selects_patch_elements():
    """W_pe rows = unit vectors, bias = pos = 0: token n's feature k is patch element k."""
    dims = synth.workload("small_tubelet2_q8_0")["dims"]
    dims.update(img_h=32, img_w=48, frames=4)
    P, D = synth.patch_dim(dims), dims["dim"]
    frames = np.random.default_rng(1).integers(0, 256, (1, 4, 32, 48, 3), dtype=np.uint8)
    x = E.normalize(frames, dims["mean"], dims["std"])
    for off in range(0, P, D):            # two offset runs cover P > D
        W = np.zeros((D, P))
        for k in range(min(D, P - off)):
            W[k, off + k] = 1.0
        w = {"enc.patch_embed.weight": W, "enc.patch_embed.bias": np.zeros(D),
             "enc.pos_embed": np.zeros((synth.n_tokens(dims), D))}
        e = E.embed(dims, w, frames)
        Tt, Hp, Wp = synth.grid(dims)
        for n in (0, 5, Tt * Hp * Wp - 1):
            tt, r = divmod(n, Hp * Wp)
            i, j = divmod(r, Wp)
            for k in range(min(D, P - off)):
                kk = off + k
                dt, rem = divmod(kk, 16 * 16 * 3)
                dy, rem = divmod(rem, 16 * 3)
                dx, c = divmod(rem, 3)
                assert e[0, n, k] == x[0, 2 * tt + dt, 16 * i + dy, 16 * j + dx, c]


# ---------------------------------------------------------------------------
# linear, LayerNorm, GELU
# ---------------------------------------------------------------------------

def test_linear_orientation_one_hot():
    """W [out, in] with a single 1 at (o, i): output column o is input column i plus b[o]."""
    x = np.arange(15, dtype=np.float64).reshape(3, 5)
    W = np.zeros((4, 5))
    W[2, 3] = 1.0
    b = np.array([0.5, -1.0, 2.0, 3.0])
    y = E.linear(x, W, b)
    assert y.shape == (3, 4)
    np.testing.assert_array_equal(y[:, 2], x[:, 3] + 2.0)
    np.testing.assert_array_equal(y[:, 0], np.full(3, 0.5))


def test_layer_norm_closed_forms():
    rng = np.random.default_rng(2)
    D, eps = 96, 1e-6
    x = rng.standard_normal((7, D)) * 3 + 1.5
    y = E.layer_norm(x, np.ones(D), np.zeros(D), eps)
    var = np.var(x, axis=1)
    np.testing.assert_allclose(y.sum(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose((y ** 2).sum(axis=1), D * var / (var + eps), rtol=1e-12)
    # a constant row normalises to the shift
    beta = rng.standard_normal(D)
    c = E.layer_norm(np.full((1, D), 4.25), np.ones(D) * 3, beta, eps)
    np.testing.assert_allclose(c[0], beta, atol=1e-12)
    # gain and shift apply per feature after normalising
    g = rng.standard_normal(D)
    z = E.layer_norm(x, g, beta, eps)
    np.testing.assert_allclose(z, y * g + beta, rtol=1e-12, atol=1e-12)


def test_gelu_closed_forms():
    # Phi(1) and Phi(2) from the standard normal table
    assert E.gelu(np.array(1.0)) == pytest.approx(0.8413447460685429, rel=1e-14)
    assert E.gelu(np.array(2.0)) == pytest.approx(2 * 0.9772498680518208, rel=1e-14)
    assert E.gelu(np.array(0.0)) == 0.0
    z = np.linspace(-6, 6, 101)
    np.testing.assert_allclose(E.gelu(z) - E.gelu(-z), z, atol=1e-14)   # erf is odd
    np.testing.assert_allclose(E.gelu(np.array([30.0])), [30.0])


# ---------------------------------------------------------------------------
# softmax and attention
# ---------------------------------------------------------------------------

def test_masked_softmax_rows_sum_to_one_and_masked_are_zero():
    rng = np.random.default_rng(3)
    allowed = E.block_causal_allowed(4, 5, True)
    s = rng.standard_normal((21, 21)) * 4
    p = E.softmax_masked(s, allowed)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(p[~allowed] == 0.0)
    assert np.all(p[allowed] > 0.0)


def test_block_causal_mask_brute_force():
    """3 frames of 2x2 patches plus CLS, and without CLS, against the rule stated pairwise."""
    for has_cls in (True, False):
        a = E.block_causal_allowed(3, 4, has_cls)
        c = int(has_cls)
        N = 12 + c
        assert a.shape == (N, N)
        for i in range(N):
            for j in range(N):
                if has_cls and i == 0:
                    want = True                      # CLS reads every token
                elif has_cls and j == 0:
                    want = False                     # nobody reads CLS
                else:
                    want = (j - c) // 4 <= (i - c) // 4
                assert a[i, j] == want, (has_cls, i, j)


def test_attention_closed_forms():
    rng = np.random.default_rng(4)
    dh = 64
    # one token: the output is its own value
    q, k, v = rng.standard_normal((3, 1, dh))
    np.testing.assert_allclose(E.attention_head(q, k, v, None), v, rtol=1e-14)
    # identical keys: every query gets the mean of the values it may read
    N = 9
    q = rng.standard_normal((N, dh))
    k = np.tile(rng.standard_normal((1, dh)), (N, 1))
    v = rng.standard_normal((N, dh))
    allowed = E.block_causal_allowed(2, 4, True)
    o = E.attention_head(q, k, v, allowed)
    for i in range(N):
        np.testing.assert_allclose(o[i], v[allowed[i]].mean(axis=0), rtol=1e-12, atol=1e-14)
    # zero query: same
    o0 = E.attention_head(np.zeros((N, dh)), rng.standard_normal((N, dh)), v, allowed)
    for i in range(N):
        np.testing.assert_allclose(o0[i], v[allowed[i]].mean(axis=0), rtol=1e-12, atol=1e-14)
    # two keys, one query: softmax of two scores by hand
    q = np.zeros((1, dh)); q[0, 0] = 8.0
    k = np.zeros((2, dh)); k[0, 0] = 1.0; k[1, 0] = -1.0
    v = np.array([[1.0] + [0.0] * (dh - 1), [0.0] * dh])
    o = E.attention_head(q, k, v, None)
    assert o[0, 0] == pytest.approx(math.exp(1) / (math.exp(1) + math.exp(-1)), rel=1e-14)


def test_all_allowed_mask_equals_unmasked():
    """CLS with a fully bidirectional mask equals the unmasked result."""
    rng = np.random.default_rng(5)
    qkv = rng.standard_normal((13, 3 * 128))
    a = E.attention(qkv, 2, None)
    b = E.attention(qkv, 2, np.ones((13, 13), dtype=bool))
    np.testing.assert_array_equal(a, b)


def test_attention_heads_use_their_own_columns():
    """Zeroing head 1's q/k/v columns changes only head 1's output columns."""
    rng = np.random.default_rng(6)
    D, H = 128, 2
    qkv = rng.standard_normal((10, 3 * D))
    base = E.attention(qkv, H, None)
    z = qkv.copy()
    for part in range(3):
        z[:, part * D + 64: part * D + 128] = 0.0
    out = E.attention(z, H, None)
    np.testing.assert_array_equal(out[:, :64], base[:, :64])
    np.testing.assert_allclose(out[:, 64:], 0.0, atol=0)


# ---------------------------------------------------------------------------
# the whole encoder
# ---------------------------------------------------------------------------

def _tiny_dims(**kw):
    d = dict(dim=8, depth=2, heads=2, mlp_dim=16, patch=2, tubelet=1, img_h=4, img_w=4,
             frames=3, has_cls=1, mask="block_causal", ln_eps=1e-6,
             mean=(0.5, 0.4, 0.3), std=(0.5, 0.25, 0.2),
             act_dtype="f32", mat_dtype="f32", rest_dtype="f32")
    d.update(kw)
    return d


def _tiny_weights(dims, seed):
    w32 = synth.make_f32_weights(dims, seed, ln_affine=True)
    return {k: v.astype(np.float64) for k, v in w32.items()}


@pytest.mark.parametrize("kw", [
    dict(),                                                  # block-causal, CLS
    dict(mask="bidir"),                                      # bidirectional, CLS
    dict(has_cls=0, tubelet=2, frames=4),                    # block-causal, tubelet 2
    dict(has_cls=0, mask="bidir", img_w=6),                  # bidirectional, no CLS
])
def test_encoder_matches_brute_force(kw):
    dims = _tiny_dims(**kw)
    w = _tiny_weights(dims, 7)
    frames = synth.make_frames(dims, 2, 8)
    y = E.encode(dims, w, frames)
    ref = np.array(brute.encode(dims, w, frames))
    assert y.shape == ref.shape == (2, synth.n_tokens(dims), dims["dim"])
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-11)


def test_encoder_zero_blocks_is_final_ln_of_embedding_plus_biases():
    """With every block weight zero, each block adds only b_out + b_down."""
    dims = _tiny_dims(mask="bidir")
    w = _tiny_weights(dims, 9)
    for i in range(dims["depth"]):
        for m in ("attn_qkv", "attn_out", "ffn_up", "ffn_down"):
            w[f"enc.blk.{i}.{m}.weight"] = np.zeros_like(w[f"enc.blk.{i}.{m}.weight"])
    frames = synth.make_frames(dims, 1, 10)
    x0 = np.array(brute._embed(dims, w, frames))
    shift = sum(w[f"enc.blk.{i}.attn_out.bias"] + w[f"enc.blk.{i}.ffn_down.bias"]
                for i in range(dims["depth"]))
    x = x0 + shift
    mu = x.mean(axis=-1, keepdims=True)
    sd = np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True) + dims["ln_eps"])
    want = (x - mu) / sd * w["enc.norm.weight"] + w["enc.norm.bias"]
    np.testing.assert_allclose(E.encode(dims, w, frames), want, rtol=1e-12, atol=1e-12)


def test_block_causal_causality_is_bit_exact():
    """Perturbing the pixels of slot t leaves every patch row of slots < t bit-identical."""
    dims = _tiny_dims(frames=4)
    w = _tiny_weights(dims, 11)
    f = synth.make_frames(dims, 1, 12)
    y = E.encode(dims, w, f)
    g = f.copy()
    g[:, 2] = 255 - g[:, 2]                   # slot 2
    z = E.encode(dims, w, g)
    per = 4
    np.testing.assert_array_equal(y[:, 1:1 + 2 * per], z[:, 1:1 + 2 * per])
    assert not np.array_equal(y[:, 1 + 2 * per:], z[:, 1 + 2 * per:])
    assert not np.array_equal(y[:, 0], z[:, 0])   # CLS reads slot 2


def test_block_causal_cls_is_read_only():
    """Changing the CLS token (and its pos row) leaves every patch row bit-identical."""
    dims = _tiny_dims()
    w = _tiny_weights(dims, 13)
    f = synth.make_frames(dims, 2, 14)
    y = E.encode(dims, w, f)
    w2 = dict(w)
    w2["enc.cls_token"] = w["enc.cls_token"] + 1.0
    pos = w["enc.pos_embed"].copy()
    pos[0] -= 3.0
    w2["enc.pos_embed"] = pos
    z = E.encode(dims, w2, f)
    np.testing.assert_array_equal(y[:, 1:], z[:, 1:])
    assert not np.array_equal(y[:, 0], z[:, 0])


def test_block_causal_single_frame_is_bidirectional_without_cls():
    dims = _tiny_dims(frames=1)
    w = _tiny_weights(dims, 15)
    f = synth.make_frames(dims, 2, 16)
    y = E.encode(dims, w, f)
    d2 = _tiny_dims(frames=1, has_cls=0, mask="bidir")
    w2 = {k: v for k, v in w.items() if k != "enc.cls_token"}
    w2["enc.pos_embed"] = w["enc.pos_embed"][1:]
    z = E.encode(d2, w2, f)
    np.testing.assert_allclose(y[:, 1:], z, rtol=1e-13, atol=1e-13)


def test_batch_items_are_independent():
    dims = _tiny_dims()
    w = _tiny_weights(dims, 17)
    f = synth.make_frames(dims, 3, 18)
    y = E.encode(dims, w, f)
    for b in range(3):
        np.testing.assert_array_equal(y[b:b + 1], E.encode(dims, w, f[b:b + 1]))


def test_pool_modes():
    y = np.arange(2 * 4 * 3, dtype=np.float64).reshape(2, 4, 3)
    np.testing.assert_array_equal(E.pool(y, "cls", True), y[:, 0])
    np.testing.assert_array_equal(E.pool(y, "mean", True), y[:, 1:].mean(axis=1))
    np.testing.assert_array_equal(E.pool(y, "mean", False), y.mean(axis=1))
    np.testing.assert_array_equal(E.pool(y, "none", True), y)
    with pytest.raises(ValueError):
        E.pool(y, "cls", False)


# ---------------------------------------------------------------------------
# 3-D rotary position (V-JEPA 2 card: the encoder's "3-D RoPE"; RoFormer's
# rotation, one third of each head per axis)
# ---------------------------------------------------------------------------

_VJ2_16F = dict(dim=1024, heads=16, patch=16, tubelet=2, img_h=256, img_w=256, frames=16,
                has_cls=0)


def test_rope_angles_hand_values():
    """dh 64: segments of 20 dims for t, h, w, dims 60-63 unrotated; the
    frequency of pair i of a segment is 10000^(-i/10)."""
    ang = E.rope_angles(_VJ2_16F)
    assert ang.shape == (8 * 16 * 16, 32)
    tok = lambda t, h, w: (t * 16 + h) * 16 + w
    f = 10000.0 ** (-np.arange(10) / 10.0)
    np.testing.assert_array_equal(ang[tok(0, 0, 0)], 0.0)
    np.testing.assert_allclose(ang[tok(3, 0, 0)], np.r_[3 * f, np.zeros(22)], rtol=1e-15)
    np.testing.assert_allclose(ang[tok(0, 5, 0)], np.r_[np.zeros(10), 5 * f, np.zeros(12)], rtol=1e-15)
    np.testing.assert_allclose(ang[tok(7, 15, 11)], np.r_[7 * f, 15 * f, 11 * f, 0, 0], rtol=1e-15)
    assert ang[tok(1, 0, 0), 1] == pytest.approx(10 ** -0.4, rel=1e-15)
    # heads of 32: segments of 10 dims, pair i of a segment at 10000^(-i/5),
    # the last pair unrotated
    a32 = E.rope_angles(dict(_VJ2_16F, dim=384, heads=12))
    f5 = 10000.0 ** (-np.arange(5) / 5.0)
    assert a32.shape == (8 * 16 * 16, 16)
    np.testing.assert_allclose(a32[tok(2, 3, 4)], np.r_[2 * f5, 3 * f5, 4 * f5, 0], rtol=1e-15)
    # a CLS token (no position) is token 0 and is never rotated
    ac = E.rope_angles(dict(_VJ2_16F, has_cls=1))
    np.testing.assert_array_equal(ac[0], 0.0)
    np.testing.assert_array_equal(ac[1:], ang)


def test_rope_rotates_pairs_by_hand():
    """e_0 at t = 1 -> (cos 1, sin 1) in dims 0, 1; e_41 at w = 1 -> (-sin 1,
    cos 1) in dims 40, 41; dims 60-63 pass through."""
    ang = E.rope_angles(_VJ2_16F)
    x = np.zeros((ang.shape[0], 64))
    t1, w1 = 16 * 16, 1
    x[t1, 0] = 1.0
    x[w1, 41] = 1.0
    x[:, 60:] = 2.5
    y = E.rope(x, ang)
    np.testing.assert_allclose(y[t1, :2], [math.cos(1), math.sin(1)], rtol=1e-15)
    np.testing.assert_allclose(y[w1, 40:42], [-math.sin(1), math.cos(1)], rtol=1e-15)
    np.testing.assert_array_equal(np.delete(y[t1], [0, 1]), np.delete(x[t1], [0, 1]))
    np.testing.assert_array_equal(y[:, 60:], 2.5)


def test_rope_is_a_rotation_and_relative():
    """Rotation keeps every pair's length; q.k after rotation depends only on
    the difference of the two tokens' (t, h, w) positions."""
    rng = np.random.default_rng(30)
    ang = E.rope_angles(_VJ2_16F)
    x = rng.standard_normal((ang.shape[0], 64))
    y = E.rope(x, ang)
    np.testing.assert_allclose((y ** 2).reshape(-1, 32, 2).sum(-1), (x ** 2).reshape(-1, 32, 2).sum(-1),
                               rtol=1e-13)
    q, k = rng.standard_normal((2, 1, 64))
    tok = lambda t, h, w: (t * 16 + h) * 16 + w
    dot = lambda a, b: float((E.rope(q, ang[[a]]) @ E.rope(k, ang[[b]]).T)[0, 0])
    for (p0, p1), s in [(((0, 0, 0), (2, 3, 5)), (4, 7, 1)), (((5, 9, 2), (1, 0, 14)), (2, 6, 1))]:
        moved = [tuple(a + b for a, b in zip(p, s)) for p in (p0, p1)]
        assert dot(tok(*moved[0]), tok(*moved[1])) == pytest.approx(dot(tok(*p0), tok(*p1)), rel=1e-12)
    # and it does depend on the difference: a shift of one token only changes it
    assert abs(dot(tok(0, 0, 0), tok(0, 0, 1)) - dot(tok(0, 0, 0), tok(0, 0, 0))) > 1e-3


@pytest.mark.parametrize("kw", [
    dict(mask="bidir"),                                      # CLS, not rotated
    dict(has_cls=0, tubelet=2, frames=4, mask="bidir"),      # V-JEPA 2 shape
    dict(),                                                  # block-causal, CLS
])
def test_rope_encoder_matches_brute_force(kw):
    """dh 14: segments of 4 dims per axis and 2 left over, on a 2x3 patch
    grid, against the scalar-loop encoder whose rotation is a complex
    multiplication."""
    dims = _tiny_dims(dim=28, heads=2, mlp_dim=32, img_h=4, img_w=6, rope=1, **kw)
    w = _tiny_weights(dims, 31)
    assert "enc.pos_embed" not in w
    frames = synth.make_frames(dims, 2, 32)
    y = E.encode(dims, w, frames)
    ref = np.array(brute.encode(dims, w, frames))
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-11)
    # and the rotation is not a no-op
    y0 = E.encode(dict(dims, rope=0), dict(w, **{"enc.pos_embed": np.zeros((synth.n_tokens(dims), 28))}),
                  frames)
    assert np.abs(y - y0).max() > 1e-4


# ---------------------------------------------------------------------------
# the attentive-pool classifier head (V-JEPA 2 SSv2 card; reading R13)
# ---------------------------------------------------------------------------

def _head_case(seed, N=5, **kw):
    from oracle import head as HD
    dims = _tiny_dims(dim=8, heads=2, mlp_dim=16, head_blocks=2, head_classes=3, **kw)
    w = _tiny_weights(dims, seed)
    y = np.random.default_rng(seed + 1).standard_normal((2, N, dims["dim"]))
    return HD, dims, w, y


def test_head_matches_brute_force():
    HD, dims, w, y = _head_case(40)
    got = HD.classify(dims, w, y)
    ref = np.array(brute.classify(dims, w, y.tolist()))
    assert got.shape == (2, 3)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_head_is_invariant_to_token_order():
    """No position enters the head: shuffling the tokens leaves the scores."""
    HD, dims, w, y = _head_case(41, N=7)
    perm = np.random.default_rng(3).permutation(7)
    np.testing.assert_allclose(HD.classify(dims, w, y[:, perm]), HD.classify(dims, w, y),
                               rtol=1e-12, atol=1e-13)


def test_head_repeated_token_equals_single_token():
    """Attention over copies of one token averages equal values: N copies
    score exactly like the token alone (catches a sum where a softmax-weighted
    mean belongs)."""
    HD, dims, w, y = _head_case(42, N=1)
    many = np.repeat(y, 6, axis=1)
    np.testing.assert_allclose(HD.classify(dims, w, many), HD.classify(dims, w, y), rtol=1e-12, atol=1e-13)
    # and the head is not blind to its input (a shift of every feature alike
    # is removed by the LayerNorms; a change of one feature is not)
    z = y.copy()
    z[..., 0] += 1.0
    assert np.abs(HD.classify(dims, w, z) - HD.classify(dims, w, y)).max() > 1e-4


# ---------------------------------------------------------------------------
# block formats
# ---------------------------------------------------------------------------

def test_q8_0_hand_worked_block():
    """amax 127 gives d = 1 exactly, so the codes are the rounded inputs."""
    x = np.zeros((1, 32), np.float32)
    x[0, :6] = [-127.0, 2.5, -2.5, 0.49, 100.5, 126.4]
    raw = Q.quantize_q8_0(x)
    assert raw.shape == (1, 34)
    assert list(raw[0, :2]) == [0x00, 0x3C]                  # f16 1.0, little endian
    codes = raw[0, 2:].view(np.int8)
    assert list(codes[:6]) == [-127, 3, -3, 0, 101, 126]     # half away from zero
    assert np.all(codes[6:] == 0)


def test_q4_0_hand_worked_block():
    """x_j = j - 16: m = -16 (first largest), d = 2, q_j = floor(x_j / 2 + 8.5) clamped to 15."""
    x = (np.arange(32, dtype=np.float32) - 16).reshape(1, 32)
    raw = Q.quantize_q4_0(x)
    assert raw.shape == (1, 18)
    assert list(raw[0, :2]) == [0x00, 0x40]                  # f16 2.0
    q = [0, 1, 1, 2, 2, 3, 3, 4, 4, 5, 5, 6, 6, 7, 7, 8,
         8, 9, 9, 10, 10, 11, 11, 12, 12, 13, 13, 14, 14, 15, 15, 15]
    want = [q[j] | (q[j + 16] << 4) for j in range(16)]
    assert list(raw[0, 2:]) == want
    w = Q.dequantize_q4_0(raw, 1, 32)[0]
    np.testing.assert_array_equal(w, [2.0 * (v - 8) for v in q])


def _ieee_value(code: int, exp_bits: int, man_bits: int) -> float:
    """The value an IEEE-754 style code denotes, from the format's definition:
    sign, biased exponent, fraction; exponent 0 is subnormal (no implicit 1),
    the all-ones exponent is inf (fraction 0) or NaN.  Exact: every value of
    binary16 and bfloat16 is a Python float."""
    bias = (1 << (exp_bits - 1)) - 1
    sign = -1.0 if code >> (exp_bits + man_bits) else 1.0
    e = (code >> man_bits) & ((1 << exp_bits) - 1)
    m = code & ((1 << man_bits) - 1)
    if e == (1 << exp_bits) - 1:
        return sign * math.inf if m == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(m, 1 - bias - man_bits)
    return sign * math.ldexp((1 << man_bits) + m, e - bias - man_bits)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_widening_matches_the_format_definition(fmt):
    """widen_half / widen_bfloat16 (and stored_to_f64's f16 / bf16 branches)
    against the value each of the 65536 codes denotes: binary16 has 5
    exponent and 10 fraction bits, bfloat16 8 and 7."""
    eb, mb = (5, 10) if fmt == "f16" else (8, 7)
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = Q.widen_half(codes) if fmt == "f16" else Q.widen_bfloat16(codes)
    want = np.array([_ieee_value(int(c), eb, mb) for c in range(1 << 16)])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))
    # the stored-tensor path takes the same branch, as a vector and as a matrix
    t = dict(name="x", dtype=fmt, ne0=256, ne1=256, data=codes)
    m = Q.stored_to_f64(t)
    assert m.shape == (256, 256)
    assert np.array_equal(np.isnan(m.ravel()), nan)
    assert np.array_equal(m.ravel()[~nan], want[~nan])


def test_widening_named_codes():
    """Codes whose values the formats fix by hand."""
    bf = {0x3F80: 1.0, 0xC040: -3.0, 0x0001: 2.0 ** -133, 0x7F80: math.inf,
          0x0080: 2.0 ** -126, 0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127, 0x8000: -0.0}
    h = {0x3C00: 1.0, 0x0001: 2.0 ** -24, 0xFBFF: -65504.0, 0x0400: 2.0 ** -14,
         0x3555: 0.333251953125, 0x7C00: math.inf, 0xC000: -2.0}
    got = Q.widen_bfloat16(np.array(list(bf), np.uint16))
    assert list(got) == list(bf.values())
    got = Q.widen_half(np.array(list(h), np.uint16))
    assert list(got) == list(h.values())


def _f32_scale_q8(x):
    return np.max(np.abs(x.reshape(-1, 32)), axis=1) / np.float32(127)


def test_q8_0_error_bound():
    """|x - d16 q| <= |d32|/2 + 127 |d32 - d16| per element (scale rounding included)."""
    rng = np.random.default_rng(19)
    x = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    raw = Q.quantize_q8_0(x)
    w = Q.dequantize_q8_0(raw, 64, 256).astype(np.float64)
    d32 = _f32_scale_q8(x).astype(np.float64)
    d16 = d32.astype(np.float32).astype(np.float16).astype(np.float64)
    bound = np.abs(d32) / 2 * (1 + 1e-6) + 127 * np.abs(d32 - d16)
    err = np.abs(x.astype(np.float64) - w).reshape(-1, 32)
    assert np.all(err <= bound[:, None])
    # the integer step alone keeps within half a step of the unrounded scale
    q = raw.reshape(-1, 34)[:, 2:].view(np.int8).astype(np.float64)
    assert np.all(np.abs(x.reshape(-1, 32) - d32[:, None] * q) <= d32[:, None] / 2 * (1 + 1e-6))


def test_q4_0_error_bound():
    """|x - d q| <= |d|/2 except clamped elements (x/d > 7.5), which stay within |d|."""
    rng = np.random.default_rng(20)
    x = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    raw = Q.quantize_q4_0(x)
    blk = raw.reshape(-1, 18)
    d16 = blk[:, :2].copy().view(np.float16)[:, 0].astype(np.float64)
    xb = x.reshape(-1, 32).astype(np.float64)
    m = xb[np.arange(len(xb)), np.argmax(np.abs(xb), axis=1)]
    d32 = (m.astype(np.float32) / np.float32(-8)).astype(np.float64)
    w = Q.dequantize_q4_0(raw, 64, 256).astype(np.float64).reshape(-1, 32)
    slack = np.broadcast_to(8 * np.abs(d32 - d16)[:, None], xb.shape)
    step = np.broadcast_to(np.abs(d32)[:, None], xb.shape)
    clamped = xb / d32[:, None] > 7.5
    err = np.abs(xb - w)
    assert np.all(err[~clamped] <= (step / 2 * (1 + 1e-6) + slack)[~clamped])
    assert np.all(err[clamped] <= (step * (1 + 1e-6) + slack)[clamped])
    assert clamped.any()


def test_zero_block_and_idempotence():
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((8, 128)) * 0.02).astype(np.float32)
    x[3, 32:64] = 0.0
    for dt, deq in (("q8_0", Q.dequantize_q8_0), ("q4_0", Q.dequantize_q4_0)):
        raw = Q.quantize(dt, x)
        w = deq(raw, 8, 128)
        assert np.all(w[3, 32:64] == 0.0)
        # quantising the dequantised weights reproduces the blocks byte for byte,
        # except the sign of an all-zero q4_0 block's scale (d = m / -8 with m = +-0)
        again = Q.quantize(dt, w).reshape(-1, Q.block_bytes(dt)).copy()
        want = raw.reshape(-1, Q.block_bytes(dt)).copy()
        zero = want[:, :2].copy().view(np.float16)[:, 0] == 0
        assert zero.sum() == 1
        assert np.all(again[zero, :2].view(np.float16) == 0)
        again[zero, :2] = want[zero, :2]
        np.testing.assert_array_equal(again, want)


def test_block_sizes_match_printed_bits_per_weight():
    g = json.load(open(os.path.join(GOLDEN, "page_file_sizes.json")))
    for dt in ("q8_0", "q4_0"):
        raw = Q.quantize(dt, np.ones((1, 32), np.float32))
        assert raw.nbytes == Q.block_bytes(dt)
        assert raw.nbytes * 8 / 32 == g["bits_per_weight"][dt]
    # ViT-S qkv [1152, 384] at q4_0
    raw = Q.quantize_q4_0(np.ones((1152, 384), np.float32))
    assert raw.nbytes / 1024 == g["vits_qkv_q4_0_kib"]


def test_levjepa_file_sizes_and_counts():
    """The LeVJEPA ViT-L/16 file (no pos table) at each type against the printed sizes."""
    g = json.load(open(os.path.join(GOLDEN, "page_file_sizes.json")))
    dims = synth.workload("levjepa_vit_l16_16f_bf16_b4")["dims"]
    specs = [s for s in synth.tensor_specs(dims) if s[0] != "enc.pos_embed"]
    mats = [s for s in specs if synth.is_block_matrix(s[0])]
    rest = [s for s in specs if not synth.is_block_matrix(s[0])]
    assert (len(rest), len(mats)) == (g["levjepa_tensor_counts"]["F32"], g["levjepa_tensor_counts"]["Q8_0"])
    n_mat = sum(a * b for _, a, b in mats)
    rest_bytes = sum(a * b for _, a, b in rest) * 4
    assert abs(rest_bytes / 2 ** 20 - g["levjepa_remainder_mib"]) < 0.05
    mib = g["levjepa_vitl16_mib"]
    tol = g["tolerance_mib"]
    for dt in ("q8_0", "q4_0"):
        total = n_mat // 32 * Q.block_bytes(dt) + rest_bytes
        assert abs(total / 2 ** 20 - mib[dt]) <= tol, dt
    assert abs((n_mat * 4 + rest_bytes) / 2 ** 20 - mib["f32"]) <= tol
    # f16 file: the 96 matrices and the patch-embed matrix in f16
    pe = [s for s in rest if s[0] == "enc.patch_embed.weight"][0]
    f16_total = (n_mat + pe[1] * pe[2]) * 2 + rest_bytes - pe[1] * pe[2] * 4
    assert len(mats) + 1 == g["levjepa_tensor_counts_f16"]["F16"]
    assert any(abs(f16_total / 2 ** 20 - v) <= tol for v in mib["f16"])


# ---------------------------------------------------------------------------
# K-quants (q4_K, q6_K)
# ---------------------------------------------------------------------------

def test_q6_k_hand_worked_block():
    """Every low byte 0x21 (low nibble 1, high 2), every high byte 0b11100100
    (bit pairs 0, 1, 2, 3 from the bottom), d = 1, all scales 1.  By the
    format, the four 32-weight runs t of each half take their low bits from
    the low nibble (t = 0, 1) or high nibble (t = 2, 3) and their high bits
    from bit pair t: codes 1, 1 + 16, 2 + 32, 2 + 48, i.e. weights -31, -15,
    2, 18.  Then scales 1..16 (weight k uses scale k // 16) and d = 0.5."""
    blk = np.zeros(210, np.uint8)
    blk[:128] = 0x21
    blk[128:192] = 0b11100100
    blk[192:208] = 1
    blk[208:210] = np.array([1.0], np.float16).view(np.uint8)
    run = np.repeat([-31.0, -15.0, 2.0, 18.0], 32)
    np.testing.assert_array_equal(Q.dequantize_q6_k(blk, 1, 256)[0], np.tile(run, 2))
    blk[192:208] = np.arange(1, 17).astype(np.int8).view(np.uint8)
    blk[208:210] = np.array([0.5], np.float16).view(np.uint8)
    want = 0.5 * np.repeat(np.arange(1, 17), 16) * np.tile(run, 2)
    np.testing.assert_array_equal(Q.dequantize_q6_k(blk, 1, 256)[0], want)
    blk[192] = np.int8(-3).view(np.uint8)                   # a negative scale
    assert Q.dequantize_q6_k(blk, 1, 256)[0][0] == 0.5 * -3 * -31


def test_q4_k_hand_worked_block():
    """Sub-block scales 1, 2, 3, 4, 17, 33, 49, 63 and mins 0, 1, 2, 3, 16,
    32, 48, 63 packed by hand into the 12 bytes (the j >= 4 values split into
    a low nibble in bytes 8-11 and two high bits in bytes 0-7), d = 1,
    dmin = 0.5, every code byte 0x25 (low nibble 5 for the even sub-blocks,
    high 2 for the odd ones): sub-block j weighs sc_j q - 0.5 m_j."""
    blk = np.zeros(144, np.uint8)
    blk[0:2] = np.array([1.0], np.float16).view(np.uint8)
    blk[2:4] = np.array([0.5], np.float16).view(np.uint8)
    blk[4:16] = [65, 130, 195, 196, 64, 129, 194, 195, 1, 1, 1, 255]
    blk[16:144] = 0x25
    sc, m = Q.q4_k_scale_min(blk[4:16])
    assert list(sc) == [1, 2, 3, 4, 17, 33, 49, 63]
    assert list(m) == [0, 1, 2, 3, 16, 32, 48, 63]
    want = np.repeat([5.0, 3.5, 14.0, 6.5, 77.0, 50.0, 221.0, 94.5], 32)
    np.testing.assert_array_equal(Q.dequantize_q4_k(blk, 1, 256)[0], want)


@pytest.mark.parametrize("dt", ["q4_k", "q6_k"])
def test_k_quant_round_trip_and_zero_block(dt):
    """The oracle's encoders: codes within the format's ranges reproduce a
    zero super-block exactly, and every other weight within one quantisation
    step of the sub-block (q4_K: plus half a min step)."""
    rng = np.random.default_rng(22)
    x = (rng.standard_normal((6, 512)) * 0.02).astype(np.float32)
    x[2, 256:] = 0.0
    raw = Q.quantize(dt, x)
    per, bb = Q.block_bytes_of(dt)
    assert raw.shape == (6, 512 // per * bb)
    w = Q.stored_to_f64(dict(dtype=dt, ne0=512, ne1=6, data=raw))
    assert np.all(w[2, 256:] == 0.0)
    blk = raw.reshape(-1, bb)
    if dt == "q6_k":
        d = blk[:, 208:210].copy().view(np.float16)[:, 0].astype(np.float64)
        sc = blk[:, 192:208].view(np.int8).astype(np.float64)
        step = np.repeat(d[:, None] * np.abs(sc), 16, axis=1)
        slack = 0.0
    else:
        d = blk[:, 0:2].copy().view(np.float16)[:, 0].astype(np.float64)
        dmin = blk[:, 2:4].copy().view(np.float16)[:, 0].astype(np.float64)
        sc, _ = Q.q4_k_scale_min(blk[:, 4:16])
        step = np.repeat(d[:, None] * sc, 32, axis=1)
        slack = np.repeat(dmin[:, None], 256, axis=1) / 2
    err = np.abs(w.reshape(-1, 256) - x.astype(np.float64).reshape(-1, 256))
    assert np.all(err <= step + slack + 1e-12)


def test_k_quant_block_bytes_match_printed_sizes():
    """q4_K: 144 bytes per 256 weights, the 4.5 bits per weight of q4_0; the
    CLI's ffn_down [384,1536] -> q4_K 324.0 KiB."""
    g = json.load(open(os.path.join(GOLDEN, "page_file_sizes.json")))
    assert Q.quantize_q4_k(np.ones((1, 256), np.float32)).nbytes * 8 / 256 == g["bits_per_weight"]["q4_k"]
    raw = Q.quantize_q4_k(np.ones((384, 1536), np.float32))
    assert raw.nbytes / 1024 == g["vits_ffn_down_q4_k_kib"]


def test_k_quant_fallback_rule():
    """Quantization page, "The rule": K-quants need row lengths that are a
    multiple of 256, else the legacy type of the same width; ViT-S's 384-wide
    matrices fall back, its ffn_down (1536) does not, ViT-L (1024 / 4096)
    never does."""
    assert Q.type_for("q4_k", 384) == "q4_0" and Q.type_for("q6_k", 384) == "q8_0"
    assert Q.type_for("q5_k", 384) == "q5_0"
    assert Q.type_for("q4_k", 1536) == "q4_k" and Q.type_for("q6_k", 1536) == "q6_k"
    assert all(Q.type_for(t, n) == t for t in ("q4_k", "q6_k") for n in (1024, 4096, 768, 3072, 1280, 5120))
    assert Q.type_for("q8_0", 384) == "q8_0"


def test_vits16_file_sizes_per_type():
    """The LeJEPA ViT-S/16 file (224^2, CLS, pos table) at each type, with the
    fallback rule: the f32 remainder and the q4_k tensor data to the byte, the
    type counts, and the 'File sizes' row within its 0.1 MiB rounding."""
    g = json.load(open(os.path.join(GOLDEN, "page_file_sizes.json")))
    v = g["vits16"]
    dims = synth._dims(**v["dims"])
    totals, counts = {}, {}
    for target in v["mib"]:
        tot, n = 0, {}
        for name, ne0, ne1 in synth.tensor_specs(dims):
            if synth.is_block_matrix(name) and target != "f32":
                t = Q.type_for(target, ne0)
                b = ne0 * ne1 * 2 if t == "f16" else ne0 * ne1 // Q.block_bytes_of(t)[0] * Q.block_bytes_of(t)[1]
            else:
                t, b = "f32", ne0 * ne1 * 4
            n[t.upper().replace("_K", "_K")] = n.get(t.upper(), 0) + 1
            tot += b
        totals[target], counts[target] = tot, n
    rest = sum(ne0 * ne1 * 4 for name, ne0, ne1 in synth.tensor_specs(dims) if not synth.is_block_matrix(name))
    assert rest == v["f32_remainder_bytes"]
    assert totals["q4_k"] == v["q4_k_tensor_data_bytes"]
    for t, mib in v["mib"].items():
        assert abs(totals[t] / 2 ** 20 - mib) <= g["tolerance_mib"], t
    for t, want in v["counts"].items():
        assert counts[t] == want, (t, counts[t])


# ---------------------------------------------------------------------------
# metrics
# ---------------------------------------------------------------------------

def test_metrics_closed_forms():
    b = np.array([[1.0, 0.0], [0.0, 2.0]])
    a = np.array([[1.0, 1.0], [0.0, 2.0]])
    c = M.token_cosines(a, b)
    np.testing.assert_allclose(c, [1 / math.sqrt(2), 1.0])
    assert M.rel_max(a, b) == pytest.approx(0.5)
    assert M.rel_fro(a, b) == pytest.approx(1 / math.sqrt(5))


# ---------------------------------------------------------------------------
# int8 path: activations quantised per 32-block (R17)
# ---------------------------------------------------------------------------

def test_act_q8_closed_form_integer_multiples():
    # a block of k * 2^e with k integers and max |k| = 127: d is exactly 2^e
    # and every code is its k
    rng = np.random.default_rng(5)
    k = rng.integers(-127, 128, size=(3, 64))
    k[:, 7] = 127
    k[:, 40] = -127
    for e in (-9, 0, 4):
        q, d = Q.quantize_act_q8(k * 2.0 ** e)
        assert d.dtype == np.float32 and q.dtype == np.int8
        assert np.all(d == np.float32(2.0 ** e))
        assert np.array_equal(q.astype(np.int64), k)


def test_act_q8_ties_round_half_away_from_zero():
    x = np.zeros(32)
    x[:9] = [127.0, 0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 126.5, 0.49999997]
    q, d = Q.quantize_act_q8(x[None])
    assert d[0, 0] == 1.0
    assert list(q[0, :9]) == [127, 1, -1, 2, -2, 3, -3, 127, 0]


def test_act_q8_zero_and_single_value_blocks():
    x = np.zeros((2, 64))
    x[1, 33] = -3.0e-5
    q, d = Q.quantize_act_q8(x)
    assert np.all(d[0] == 0) and np.all(q[0] == 0) and d[1, 0] == 0
    assert d[1, 1] == np.float32(np.float32(3.0e-5) / np.float32(127.0))
    assert q[1, 33] == -127 and np.count_nonzero(q[1]) == 1


def test_act_q8_error_bound_and_extremes():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-6, 6, (64, 1)))).astype(np.float32)
    q, d = Q.quantize_act_q8(x)
    b = x.reshape(64, 8, 32).astype(np.float64)
    amax = np.max(np.abs(b), axis=2)
    # the scale is amax / 127 rounded once to f32
    assert np.all(np.abs(d - amax / 127.0) <= 2.0 ** -24 * amax / 127.0)
    # every value is within half a step of d * q, and the largest maps to 127
    err = np.abs(Q.act_q8_values(q, d).reshape(64, 8, 32) - b)
    assert np.all(err <= 0.5 * d[..., None].astype(np.float64) * (1 + 2.0 ** -20))
    qa = np.abs(q.astype(np.int64)).reshape(64, 8, 32)
    assert np.all(qa <= 127) and np.all(np.max(qa, axis=2) == 127)


def test_act_q8_matches_scalar_brute_force():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((5, 96)) * 0.3).astype(np.float32)
    x[2, 32:64] = 0.0
    q, d = Q.quantize_act_q8(x)
    for r in range(5):
        bq, bd = brute.quantize_act_q8([float(v) for v in x[r]])
        assert list(q[r].astype(int)) == bq
        assert [float(v) for v in d[r]] == bd


def test_int8_product_is_the_block_sum_of_integer_dots():
    # the int8 path's sum over blocks of d_a d_w (q_a . q_w), in exact
    # rationals, against the oracle's product of the dequantised operands
    from fractions import Fraction
    rng = np.random.default_rng(8)
    K, N = 96, 3
    x = rng.standard_normal((2, K)).astype(np.float32)
    wt = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    bias = rng.standard_normal(N)
    for dt in ("q8_0", "q4_0"):
        raw = Q.quantize(dt, wt)
        wdq = (Q.dequantize_q8_0 if dt == "q8_0" else Q.dequantize_q4_0)(raw, N, K)
        bb = Q.block_bytes(dt)
        blocks = raw.reshape(N, K // 32, bb)
        dw = blocks[:, :, :2].copy().view(np.float16)[:, :, 0].astype(np.float64)
        if dt == "q8_0":
            qw = blocks[:, :, 2:].view(np.int8).astype(np.int64)
        else:
            nib = blocks[:, :, 2:].astype(np.int64)
            qw = np.concatenate([(nib & 15) - 8, (nib >> 4) - 8], axis=2)
        qa, da = Q.quantize_act_q8(x)
        got = E.linear_act_q8(x.astype(np.float64), wdq.astype(np.float64), bias)
        for m in range(2):
            for n in range(N):
                s = Fraction(float(bias[n]))
                for b in range(K // 32):
                    dot = sum(int(qa[m, 32 * b + k]) * int(qw[n, b, k]) for k in range(32))
                    s += Fraction(float(da[m, b])) * Fraction(float(dw[n, b])) * dot
                assert abs(got[m, n] - float(s)) <= 1e-12 * (1 + abs(float(s)))


def test_act_q8_encoder_stays_close_to_dense():
    # the int8 path changes each product's input by at most half a step per
    # 32-block, so on a tiny encoder its tokens stay close to the dense ones
    dims = _tiny_dims(dim=32, mlp_dim=64)
    w = _tiny_weights(dims, 3)
    frames = synth.make_frames(dims, 2, 3)
    y = E.encode(dims, w, frames)
    y8 = E.encode(dims, w, frames, act_q8=True)
    assert not np.array_equal(y, y8)
    cos = np.sum(y * y8, -1) / np.linalg.norm(y, axis=-1) / np.linalg.norm(y8, axis=-1)
    assert cos.min() > 0.999
