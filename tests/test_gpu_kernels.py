"""Each HIP kernel, through the C ABI, against the oracle's definition of its
step, on seeded inputs that span several tiles with ragged tails.

The operands are rounded to the activation dtype once, on the host, and the
oracle sees exactly those rounded values, so what is measured is the
kernel's own arithmetic: f32 accumulation order, and the roundings the kernel
makes (its output, the probabilities fed to the PV product, dequantised
weights)."""
import math

import numpy as np
import pytest

from oracle import encoder as E
from oracle import quant as Q
from tests.helpers import rounded, say, vt_pos

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    from vision_transformer_amd import _lib
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return _lib


# bound on |gpu - oracle| for one output rounded to act dtype from an f32 value
OUT_REL = {"f32": 1e-6, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}


@pytest.mark.parametrize("act", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", [(1, 2, 32, 48, 1, 16), (2, 4, 64, 80, 2, 16), (1, 1, 56, 42, 1, 14)])
def test_patchify(lib, act, shape):
    B, T, H, W, kt, p = shape
    say(f"patchify {act} {shape}")
    frames = np.random.default_rng(40).integers(0, 256, (B, T, H, W, 3), dtype=np.uint8)
    mean, std = (0.485, 0.456, 0.406), (0.229, 0.224, 0.225)
    P = kt * p * p * 3
    ld = -(-P // 64) * 64
    np_ = (T // kt) * (H // p) * (W // p)
    out = torch.full((B * np_, ld), 7.0, dtype=torch.float32, device="cuda").to(
        {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[act])
    lib.jepa_op_patchify(act, torch.from_numpy(frames).cuda(), kt, p, mean, std, out, ld)
    got = out.double().cpu().numpy()
    ref = E.patchify(E.normalize(frames, mean, std), kt, p).reshape(B * np_, P)
    assert np.all(got[:, P:] == 0)
    err = np.abs(got[:, :P] - ref)
    assert np.all(err <= OUT_REL[act] * np.abs(ref) + 1e-6), err.max()


# (act, B, T, H, W, tubelet, patch, n, has_cls, pos): ragged row tiles, the
# LeVJEPA front end (3136 patch rows, K 768) and the V-JEPA 2 one (K 1536)
PATCH_EMBED_CASES = [
    ("bf16", 3, 2, 96, 112, 1, 16, 192, True, True),
    ("f16", 2, 4, 64, 96, 2, 16, 128, False, True),
    ("bf16", 1, 16, 224, 224, 1, 16, 1024, True, True),
    ("f16", 1, 4, 256, 256, 2, 16, 256, False, False),
]


@pytest.mark.parametrize("case", PATCH_EMBED_CASES)
def test_patch_embed_from_frames_every_element(lib, case):
    """The patch-embed GEMM that gathers its A tile from the uint8 frames:
    every output element against the oracle's normalise + patchify + linear
    (+ pos), in float64 on the act-dtype-rounded patch values; CLS rows are
    left as they were.  Bound: 2e-3 of sum |x||w| (one rounding flip of a
    patch value where the f32 normalisation and the exact one straddle an
    act-dtype boundary, plus f32 accumulation); a wrong index in the gather
    moves an output by about sum |x||w| / sqrt(K)."""
    act, B, T, H, W, kt, p, n, has_cls, use_pos = case
    say(f"patch_embed {case}")
    rng = np.random.default_rng(44)
    frames = rng.integers(0, 256, (B, T, H, W, 3), dtype=np.uint8)
    mean, std = (0.485, 0.456, 0.406), (0.229, 0.224, 0.225)
    P = kt * p * p * 3
    kp = -(-P // 64) * 64
    np_ = (T // kt) * (H // p) * (W // p)
    ntok = np_ + int(has_cls)
    w = np.zeros((n, kp), np.float32)
    w[:, :P] = rng.standard_normal((n, P)) * 0.02
    w_dev, w64 = rounded(act, w)
    bias = (rng.standard_normal(n) * 0.1).astype(np.float32)
    pos = (rng.standard_normal((ntok, n)) * 0.1).astype(np.float32) if use_pos else None
    out = torch.full((B, ntok, n), 7.0, device="cuda")
    lib.jepa_op_patch_embed(act, torch.from_numpy(frames).cuda(), kt, p, mean, std, w_dev,
                            torch.from_numpy(bias).cuda(), None if pos is None else torch.from_numpy(pos).cuda(),
                            has_cls, out)
    got = out.double().cpu().numpy()
    x = E.patchify(E.normalize(frames, mean, std), kt, p).reshape(B * np_, P)
    _, x64 = rounded(act, x)
    ref = x64 @ w64[:, :P].T + bias.astype(np.float64)
    scale = np.abs(x64) @ np.abs(w64[:, :P]).T
    ref = ref.reshape(B, np_, n)
    if use_pos:
        ref = ref + pos[int(has_cls):].astype(np.float64)
    err = np.abs(got[:, int(has_cls):] - ref)
    bound = 2e-3 * scale.reshape(B, np_, n) + 1e-6
    assert np.all(err <= bound), (err / bound).max()
    if has_cls:
        assert np.all(got[:, 0] == 7.0)


@pytest.mark.parametrize("act", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("dim", [128, 192, 1024])
def test_layernorm(lib, act, dim):
    say(f"layernorm {act} {dim}")
    rng = np.random.default_rng(41)
    rows = 301
    x = (rng.standard_normal((rows, dim)) * 2 + 0.5).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(dim)).astype(np.float32)
    b = (0.1 * rng.standard_normal(dim)).astype(np.float32)
    y = torch.empty((rows, dim), dtype={"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[act],
                    device="cuda")
    lib.jepa_op_layernorm(torch.from_numpy(x).cuda(), torch.from_numpy(g).cuda(), torch.from_numpy(b).cuda(),
                          1e-6, y, act)
    got = y.double().cpu().numpy()
    ref = E.layer_norm(x.astype(np.float64), g.astype(np.float64), b.astype(np.float64), 1e-6)
    err = np.abs(got - ref)
    assert np.all(err <= OUT_REL[act] * np.abs(ref) + 2e-5), err.max()


def _gemm_case(lib, act, wfmt, epi, M, N, K, seed):
    rng = np.random.default_rng(seed)
    a_dev, a = rounded(act, rng.standard_normal((M, K)))
    w32 = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    bias = (rng.standard_normal(N) * 0.1).astype(np.float32)
    scale = None
    if wfmt in ("q8_0", "q4_0"):
        raw = Q.quantize(wfmt, w32)
        w = Q.stored_to_f64(dict(dtype=wfmt, ne0=K, ne1=N, data=raw))
        codes, scales = lib.jepa_pack_blocks(wfmt, raw, N, K)
        w_dev = torch.from_numpy(codes).cuda()
        scale = torch.from_numpy(scales.view(np.int16)).cuda()
    else:
        w_dev, w = rounded(act, w32)
    ref = E.linear(a, w, bias.astype(np.float64))
    b_dev = torch.from_numpy(bias).cuda()
    if epi == "resid":
        x0 = rng.standard_normal((M, N)).astype(np.float32)
        out = torch.from_numpy(x0.copy()).cuda()
        ref = ref + x0
    else:
        out = torch.empty((M, N), dtype={"f32": torch.float32, "bf16": torch.bfloat16,
                                         "f16": torch.float16}[act], device="cuda")
        if epi == "gelu":
            ref = E.gelu(ref)
    lib.jepa_op_gemm(act, a_dev, w_dev, wfmt if wfmt != "dense" else act, N, b_dev, epi, out,
                     w_scale=scale)
    got = out.double().cpu().numpy()
    return got, ref, a, w


@pytest.mark.parametrize("act", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("epi", ["store", "gelu", "resid"])
@pytest.mark.parametrize("mnk", [(300, 192, 256), (129, 320, 512), (1000, 3072, 1024), (2100, 1152, 384)])
def test_gemm_dense(lib, act, epi, mnk):
    M, N, K = mnk
    if act == "f32" and M * N * K > 1e9:
        pytest.skip("the f32 path only serves small models")
    say(f"gemm dense {act} {epi} {mnk}")
    got, ref, a, w = _gemm_case(lib, act, "dense", epi, M, N, K, 42)
    # accumulation error of an f32 dot product of length K, plus the output rounding
    acc = 4 * K * 2.0 ** -24 * (np.abs(a) @ np.abs(w).T)
    out_r = 0.0 if epi == "resid" else OUT_REL[act]
    err = np.abs(got - ref)
    assert np.all(err <= acc + out_r * np.abs(ref) + 1e-6), (err - acc - out_r * np.abs(ref)).max()


@pytest.mark.parametrize("variant,N", [("big128", 384), ("big256", 512)])
@pytest.mark.parametrize("K", [64, 128, 192, 320, 1024])
@pytest.mark.parametrize("epi", ["store", "gelu", "resid"])
def test_gemm_large_tile(lib, monkeypatch, variant, N, K, epi):
    """The 256-row tile kernel pinned by name: K steps of 64 from 1 (fewer
    than its LDS stages) to 16, M = 1300 ending in a ragged tile."""
    monkeypatch.setenv("JEPA_GEMM_VARIANT", variant)
    M = 1300
    say(f"gemm {variant} bf16 {epi} M={M} N={N} K={K}")
    got, ref, a, w = _gemm_case(lib, "bf16", "dense", epi, M, N, K, 44)
    acc = 4 * K * 2.0 ** -24 * (np.abs(a) @ np.abs(w).T)
    out_r = 0.0 if epi == "resid" else OUT_REL["bf16"]
    err = np.abs(got - ref)
    assert np.all(err <= acc + out_r * np.abs(ref) + 1e-6), (err - acc - out_r * np.abs(ref)).max()


@pytest.mark.parametrize("M", [1088, 1152, 1153, 1300])
@pytest.mark.parametrize("epi", ["store", "gelu", "resid"])
def test_gemm_large_tile_half_row_tile(lib, monkeypatch, M, epi):
    """The 256-row tile's last row tile when at most 128 of its rows exist:
    the four waves then share those 128 rows (64 each).  M = 1088 and 1152
    leave 64 and 128 rows (the half tile), 1153 leaves 129 (the full tile),
    1300 leaves 20; K = 1024, every element against the oracle."""
    monkeypatch.setenv("JEPA_GEMM_VARIANT", "big256")
    N, K = 512, 1024
    say(f"gemm big256 bf16 {epi} M={M} N={N} K={K} (last row tile {M - 1024} rows)")
    got, ref, a, w = _gemm_case(lib, "bf16", "dense", epi, M, N, K, 45)
    acc = 4 * K * 2.0 ** -24 * (np.abs(a) @ np.abs(w).T)
    out_r = 0.0 if epi == "resid" else OUT_REL["bf16"]
    err = np.abs(got - ref)
    assert np.all(err <= acc + out_r * np.abs(ref) + 1e-6), (err - acc - out_r * np.abs(ref)).max()


FFN_CASES = [
    # name, M, N, K, epilogue, variant ("" = the launcher's own choice)
    # LeVJEPA ViT-L/16, batch 4, in one part: the 256 x 256 tiles would leave
    # a 4th round 12 % full, so 12288 rows take them and 260 the 64-wide tiles
    ("fc1", 12548, 4096, 1024, "gelu", ""),
    # the qkv width with a plain store: 10752 rows on 256 x 256 tiles, 1796 on
    # 256 x 128 ones (a 3rd round 34 % full avoided)
    ("qkv", 12548, 3072, 1024, "store", ""),
    ("fc2", 12548, 1024, 4096, "resid", ""),       # 64 K steps, 256 x 256 tiles
    ("fc1", 1300, 4096, 1024, "gelu", "big256"),
    ("fc2", 1300, 1024, 4096, "resid", "big256"),
    ("fc1", 1300, 4096, 1024, "gelu", "big128"),
    ("fc2", 1300, 1024, 4096, "resid", "big128"),
    ("fc1", 3137, 4096, 1024, "gelu", ""),         # one clip, the batch-part shape
    ("fc2", 3137, 1024, 4096, "resid", ""),
]


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("case", FFN_CASES, ids=[f"{c[0]}-M{c[1]}-{c[5] or 'auto'}" for c in FFN_CASES])
def test_gemm_ffn_shapes_every_element(lib, monkeypatch, act, case):
    """The MLP GEMMs at the ViT-L/16 shapes (N 4096 / K 1024 with the GELU
    epilogue, N 1024 / K 4096 with the residual one) through the 256-row
    tiles, every output element against the oracle: full-batch M, one
    clip's M, and a ragged M = 1300 with each tile width pinned."""
    name, M, N, K, epi, variant = case
    if variant:
        monkeypatch.setenv("JEPA_GEMM_VARIANT", variant)
    else:
        monkeypatch.delenv("JEPA_GEMM_VARIANT", raising=False)
    say(f"gemm {name} {act} M={M} N={N} K={K} {epi} {variant or 'auto'}")
    got, ref, a, w = _gemm_case(lib, act, "dense", epi, M, N, K, 50)
    # the bound's product in f32 (its own rounding covered by the 1 % margin)
    acc = 1.01 * 4 * K * 2.0 ** -24 * (np.abs(a).astype(np.float32) @ np.abs(w).astype(np.float32).T)
    out_r = 0.0 if epi == "resid" else OUT_REL[act]
    err = np.abs(got - ref)
    assert np.all(err <= acc + out_r * np.abs(ref) + 1e-6), (err - acc - out_r * np.abs(ref)).max()


@pytest.mark.parametrize("wfmt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("epi", ["store", "resid"])
def test_gemm_block_formats(lib, wfmt, act, epi):
    M, N, K = 333, 256, 1024
    say(f"gemm {wfmt} {act} {epi}")
    got, ref, a, w = _gemm_case(lib, act, wfmt, epi, M, N, K, 43)
    # the kernel rounds each dequantised weight to act dtype (relative 2^-11 f16,
    # 2^-8 bf16), an error the oracle's exact weights do not have
    wr = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}[act]
    bound = (wr + 4 * K * 2.0 ** -24) * (np.abs(a) @ np.abs(w).T)
    out_r = 0.0 if epi == "resid" else OUT_REL[act]
    err = np.abs(got - ref)
    assert np.all(err <= bound + out_r * np.abs(ref) + 1e-6)


@pytest.mark.parametrize("dh", [64, 32], ids=["dh64", "dh32"])
@pytest.mark.parametrize("rope", [False, True], ids=["norope", "rope"])
@pytest.mark.parametrize("qscaled", [False, True], ids=["q", "qscaled"])
@pytest.mark.parametrize("act,wfmt,B,N,heads,K", [
    ("bf16", "dense", 7, 197, 4, 256),      # M = 1379: 256-row tiles, items straddling 32-row blocks
    ("bf16", "dense", 2, 289, 2, 128),      # M = 578: 128-row tiles
    ("f16", "q8_0", 3, 106, 2, 256),
    ("bf16", "q4_0", 2, 126, 2, 128),
    ("f32", "dense", 2, 85, 2, 64),
    ("bf16", "dense", 2, 3137, 16, 1024),   # the LeVJEPA ViT-L/16 qkv layer, two clips
    ("bf16", "dense", 9, 197, 4, 640),      # 256-row tiles, 256 wide, several items per wave tile
    ("f16", "dense", 5, 301, 6, 576),       # 256-row tiles, 128 wide (N = 1152)
    # items starting at multiples of 16 rows: V^T rows written straight from the accumulators
    ("bf16", "dense", 1, 3137, 16, 1024),   # one LeVJEPA clip (one batch part): the last run crosses M
    ("f16", "dense", 3, 512, 4, 640),       # 256 wide, items of 512 tokens
    ("bf16", "dense", 2, 1024, 6, 640),     # 128 wide (N = 1152), items of 1024 tokens
])
def test_gemm_qkv_writes_v_transposed(lib, act, wfmt, B, N, heads, K, qscaled, rope, dh):
    """q and k columns as a plain linear layer (rotated pairwise by a table of
    per-token angles, then q times q_scale, before their one rounding); v
    columns straight into V^T [B, D, npad] (the attention kernel's layout),
    padding untouched.  Heads of 64 and of 32 (the same widths).  The angles
    are seeded uniform in [-pi, pi] for every token and pair, so every table
    entry is exercised."""
    heads = heads * 64 // dh                     # the same width in heads of dh
    q_scale = lib.attn_q_scale(dh) if qscaled else 0.0
    say(f"gemm qkv {act} {wfmt} B={B} N={N} heads={heads}x{dh} K={K} q_scale={q_scale} rope={rope}")
    rng = np.random.default_rng(47)
    M, D = B * N, heads * dh
    a_dev, a = rounded(act, rng.standard_normal((M, K)))
    w32 = (rng.standard_normal((3 * D, K)) * 0.05).astype(np.float32)
    bias = (rng.standard_normal(3 * D) * 0.1).astype(np.float32)
    scale, wr = None, 0.0
    if wfmt in ("q8_0", "q4_0"):
        raw = Q.quantize(wfmt, w32)
        w = Q.stored_to_f64(dict(dtype=wfmt, ne0=K, ne1=3 * D, data=raw))
        codes, scales = lib.jepa_pack_blocks(wfmt, raw, 3 * D, K)
        w_dev = torch.from_numpy(codes).cuda()
        scale = torch.from_numpy(scales.view(np.int16)).cuda()
        wr = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}[act]
    else:
        w_dev, w = rounded(act, w32)
    ref = E.linear(a, w, bias.astype(np.float64))
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[act]
    npad = -(-N // 64) * 64
    qk = torch.zeros((M, 3 * D), dtype=tdt, device="cuda")
    vt = torch.full((B, D, npad), 7.0, dtype=tdt, device="cuda")
    table = None
    if rope:
        ang = np.random.default_rng(48).uniform(-math.pi, math.pi, (N, dh // 2))
        table = torch.from_numpy(np.stack([np.cos(ang), np.sin(ang)], -1).astype(np.float32)).cuda()
    lib.jepa_op_gemm_qkv(act, a_dev, w_dev, wfmt if wfmt != "dense" else act, heads,
                         torch.from_numpy(bias).cuda(), N, qk, vt, w_scale=scale, q_scale=q_scale,
                         rope=table, head_dim=dh)
    pre = (wr + 4 * K * 2.0 ** -24) * (np.abs(a) @ np.abs(w).T) + 1e-6
    if rope:
        # oracle rotation of every head's q and k; the f32 rotation adds at
        # most e0 + e1 of the pair's errors plus a few f32 roundings of
        # |z0| + |z1| (the table's cos / sin are rounded too)
        ref = ref.copy()
        ang_b = np.tile(ang, (B, 1))
        for c0 in range(0, 2 * D, dh):
            z = ref[:, c0:c0 + dh].copy()
            ref[:, c0:c0 + dh] = E.rope(z, ang_b)
            e = pre[:, c0:c0 + dh].reshape(M, dh // 2, 2).sum(-1)
            zz = np.abs(z).reshape(M, dh // 2, 2).sum(-1)
            pre[:, c0:c0 + dh] = np.repeat(e + 4 * 2.0 ** -24 * zz, 2, axis=1)
    bound = pre + OUT_REL[act] * np.abs(ref)
    if q_scale:
        ref = ref.copy()
        ref[:, :D] *= q_scale
        bound[:, :D] = bound[:, :D] * q_scale + OUT_REL[act] * np.abs(ref[:, :D])
    got_qk = qk.double().cpu().numpy()
    assert np.all(np.abs(got_qk[:, :2 * D] - ref[:, :2 * D]) <= bound[:, :2 * D])
    assert np.all(got_qk[:, 2 * D:] == 0)                       # v columns not written
    got_vt = vt.double().cpu().numpy()
    want = ref[:, 2 * D:].reshape(B, N, D).transpose(0, 2, 1)
    bnd = bound[:, 2 * D:].reshape(B, N, D).transpose(0, 2, 1)
    pos = vt_pos(np.arange(N))
    assert np.all(np.abs(got_vt[..., pos] - want) <= bnd)
    free = np.setdiff1d(np.arange(npad), pos)
    assert np.all(got_vt[..., free] == 7.0)                      # positions of no token untouched


@pytest.mark.parametrize("rope", [False, True], ids=["norope", "rope"])
def test_gemm_qkv_rows_split_over_two_tilings(lib, rope):
    """The LeVJEPA ViT-L/16 qkv layer on the whole batch of 4 clips in one
    launch (12548 rows): the rows of the full rounds of 256 x 256 tiles
    (10752) and the rest (1796, 256 x 128 tiles) go to two launches, both
    writing V^T from the accumulators; every q, k and V^T element checked."""
    test_gemm_qkv_writes_v_transposed(lib, "bf16", "dense", 4, 3137, 16, 1024, True, rope, 64)


def _vt_of(lib, act, qkv_dev, B, N, heads, dh=64):
    npad = -(-N // 64) * 64
    vt = torch.zeros((B, heads * dh, npad), dtype=qkv_dev.dtype, device="cuda")
    lib.jepa_op_transpose_v(act, qkv_dev, B, N, heads, vt, head_dim=dh)
    return vt


def _attend(lib, act, qkv_dev, B, N, heads, has_cls, mask, per_slot, prescaled=False, dh=64):
    vt = _vt_of(lib, act, qkv_dev, B, N, heads, dh)
    out = torch.empty((B * N, heads * dh), dtype=qkv_dev.dtype, device="cuda")
    lib.jepa_op_attention(act, qkv_dev, vt, B, N, heads, has_cls, mask, per_slot, out, q_prescaled=prescaled,
                          head_dim=dh)
    return out


def _attn_case(lib, act, B, N, heads, has_cls, mask, per_slot, seed, prescaled=False, mag=1.0, dh=64):
    """GPU attention vs the oracle on seeded q, k, v.  prescaled: the device q
    columns hold q * log2(e)/sqrt(dh) rounded to act (as the qkv layer writes
    them); the oracle gets the q those rounded values stand for."""
    rng = np.random.default_rng(seed)
    D = heads * dh
    x = rng.standard_normal((B * N, 3 * D)) * mag
    qs = lib.attn_q_scale(dh)
    if prescaled:
        x[:, :D] *= qs
    qkv_dev, qkv = rounded(act, x)
    if prescaled:
        qkv = qkv.copy()
        qkv[:, :D] /= qs
    out = _attend(lib, act, qkv_dev, B, N, heads, has_cls, mask, per_slot, prescaled, dh)
    got = out.double().cpu().numpy().reshape(B, N, D)
    if mask == "bidir":
        allowed = None
    else:
        allowed = E.block_causal_allowed((N - int(has_cls)) // per_slot, per_slot, has_cls)
    ref = np.stack([E.attention(qkv.reshape(B, N, 3 * D)[b], heads, allowed) for b in range(B)])
    return got, ref


ATTN_CASES = [
    # B, N, heads, has_cls, mask, per_slot
    (2, 289, 2, True, "block_causal", 36),     # 8 slots of 6x6 + CLS
    (1, 3137, 1, True, "block_causal", 196),   # the LeVJEPA shape, one head
    (2, 197, 3, True, "bidir", 1),
    (1, 300, 2, False, "bidir", 1),
    (2, 96, 2, False, "block_causal", 24),      # tubelet slots, no CLS
    (1, 1, 1, True, "bidir", 1),               # a single token
]


@pytest.mark.parametrize("dh", [64, 32], ids=["dh64", "dh32"])
@pytest.mark.parametrize("prescaled", [False, True], ids=["q", "qscaled"])
@pytest.mark.parametrize("act", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("case", ATTN_CASES, ids=[f"{c[1]}tok-{c[4]}-cls{int(c[3])}" for c in ATTN_CASES])
def test_attention(lib, act, case, prescaled, dh):
    B, N, heads, has_cls, mask, per = case
    heads = heads * 64 // dh                      # the same width in heads of dh
    say(f"attention {act} {case} heads={heads}x{dh} prescaled={prescaled}")
    got, ref = _attn_case(lib, act, B, N, heads, has_cls, mask, per, seed=44, prescaled=prescaled, dh=dh)
    D = heads * dh
    g = got.reshape(-1, D)
    r = ref.reshape(-1, D)
    if act == "f32":
        assert np.max(np.abs(g - r)) <= 2e-5 * np.max(np.abs(r)) + 1e-6
    else:
        # probabilities and output rounded to act dtype: per-row relative error
        # a small multiple of the dtype's half-ulp
        err = np.abs(g - r).max(axis=1) / np.abs(r).max(axis=1)
        assert err.max() <= {"bf16": 2e-2, "f16": 3e-3}[act], err.max()


@pytest.mark.parametrize("prescaled", [False, True], ids=["q", "qscaled"])
@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("mag", [0.05, 3.0])
def test_attention_score_range(lib, act, mag, prescaled):
    """Scores far from O(1): nearly flat (0.05) and very peaked (3.0: score
    spread of hundreds in the base-2 exponent), so the softmax reference is
    set low on the first key tile and raised several times later."""
    case = (2, 289, 2, True, "block_causal", 36)
    say(f"attention score range {act} mag={mag} prescaled={prescaled}")
    got, ref = _attn_case(lib, act, *case, seed=48, prescaled=prescaled, mag=mag)
    g = got.reshape(-1, 128)
    r = ref.reshape(-1, 128)
    err = np.abs(g - r).max(axis=1) / np.abs(r).max(axis=1)
    assert err.max() <= {"bf16": 2e-2, "f16": 3e-3}[act], err.max()


@pytest.mark.parametrize("prescaled", [False, True], ids=["q", "qscaled"])
@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("has_cls,mag", [(False, 1.0), (True, 1.0), (False, 3.0)], ids=["nocls", "cls", "peaked"])
def test_attention_long_bidirectional(lib, act, has_cls, mag, prescaled):
    """Bidirectional head-64 sequences from 4096 tokens take the layout with
    64 queries per wave (256 per workgroup); 4100 tokens leave a ragged last
    query tile of 4 and a ragged last key tile.  mag 3.0 makes the scores
    peaked, so each query block raises its softmax reference on its own."""
    case = (1, 4100, 2, has_cls, "bidir", 1)
    say(f"attention long bidir {act} cls={has_cls} mag={mag} prescaled={prescaled}")
    got, ref = _attn_case(lib, act, *case, seed=49, prescaled=prescaled, mag=mag)
    g = got.reshape(-1, 128)
    r = ref.reshape(-1, 128)
    err = np.abs(g - r).max(axis=1) / np.abs(r).max(axis=1)
    assert err.max() <= {"bf16": 2e-2, "f16": 3e-3}[act], err.max()


def test_attention_block_causal_rows_ignore_future_slots(lib):
    """Changing the keys and values of the last slot leaves every earlier
    patch row bit-identical (whole future tiles and masked elements alike)."""
    B, N, heads, per = 1, 1 + 6 * 100, 2, 100
    D = heads * 64
    rng = np.random.default_rng(45)
    qkv = rng.standard_normal((N, 3 * D)).astype(np.float32)
    a_dev, _ = rounded("bf16", qkv)
    qkv2 = qkv.copy()
    qkv2[1 + 5 * per:, D:] = rng.standard_normal((per, 2 * D))
    b_dev, _ = rounded("bf16", qkv2)
    outs = [_attend(lib, "bf16", x, B, N, heads, True, "block_causal", per).cpu() for x in (a_dev, b_dev)]
    assert torch.equal(outs[0][1:1 + 5 * per], outs[1][1:1 + 5 * per])
    assert not torch.equal(outs[0][0], outs[1][0])          # CLS reads the last slot


MASK_CASES = [
    # B, N, heads, per_slot: the LeVJEPA shape (16 slots of 196 + CLS) and
    # 8 slots of 36 + CLS (slot boundaries inside key tiles)
    (1, 3137, 2, 196),
    (2, 289, 2, 36),
]


@pytest.mark.parametrize("prescaled", [False, True], ids=["q", "qscaled"])
@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("case", MASK_CASES, ids=[f"{c[1]}tok" for c in MASK_CASES])
def test_attention_block_causal_mask_is_exact(lib, act, case, prescaled):
    """Each key on a mask boundary carries a marker value of 1000 in a
    dimension of its own: the first patch key of slot s in dimension s, the
    last patch key of slot s in dimension 32 + s, the CLS key in dimension 31
    (every other value is noise of 1e-3).  With q = 0 every allowed key gets
    probability 1 / (allowed keys), so a patch query of slot t must show
    1000 / (196 (t + 1)) (or / (36 (t + 1))) in dimensions s and 32 + s for
    s <= t and noise for s > t and for the CLS dimension; the CLS query sees
    every key.  One key admitted or dropped at a boundary moves a marker
    dimension by at least 1000 / 3136, against a bound of a few bf16 ulps."""
    B, N, heads, per = case
    T = (N - 1) // per
    D = heads * 64
    rng = np.random.default_rng(52)
    x = np.zeros((B * N, 3 * D))
    x[:, D:2 * D] = rng.standard_normal((B * N, D))            # keys: any values
    v = rng.standard_normal((B, N, D)) * 1e-3
    for h in range(heads):
        c0 = h * 64
        v[:, 0, c0 + 31] = 1000.0                               # CLS key
        for s_ in range(T):
            v[:, 1 + s_ * per, c0 + s_] = 1000.0                # first key of slot s
            v[:, (s_ + 1) * per, c0 + 32 + s_] = 1000.0         # last key of slot s
    x[:, 2 * D:] = v.reshape(B * N, D)
    qkv_dev, qkv = rounded(act, x)
    say(f"attention mask markers {act} N={N} slots={T} prescaled={prescaled}")
    out = _attend(lib, act, qkv_dev, B, N, heads, True, "block_causal", per, prescaled)
    got = out.double().cpu().numpy().reshape(B, N, heads, 64)
    vr = qkv[:, 2 * D:].reshape(B, N, heads, 64)
    slot = np.concatenate([[-1], np.repeat(np.arange(T), per)])
    # q = 0: a query's output is the mean of its allowed values; patch keys
    # of slots <= t are the first (t + 1) * per patch rows
    csum = np.cumsum(vr[:, 1:], axis=1)
    want = np.empty_like(got)
    want[:, 0] = vr.mean(axis=1)
    n_allowed = (slot[1:] + 1) * per
    want[:, 1:] = csum[:, n_allowed - 1] / n_allowed[None, :, None, None]
    # f32 accumulation and the probabilities' and output's roundings
    tol = OUT_REL[act] * 4 * np.abs(want) + 4e-3
    bad = np.argwhere(np.abs(got - want) > tol)
    assert bad.size == 0, (bad[:5], np.abs(got - want).max())
    # the markers separate the boundary cases by far more than the tolerance
    t = 3
    row = got[0, 1 + t * per + per // 2, 0]
    assert abs(row[31]) < 0.1                                    # CLS key excluded
    assert abs(row[t] - 1000 / (per * (t + 1))) < 0.1 and abs(row[t + 1]) < 0.1
    assert abs(row[32 + t] - 1000 / (per * (t + 1))) < 0.1 and abs(row[32 + t + 1]) < 0.1
    assert abs(got[0, 0, 0, 31] - 1000 / N) < 0.1                # the CLS query sees its own key


def test_kernels_reject_out_of_contract_shapes(lib):
    x = torch.zeros((64, 100), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, 100), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(64, device="cuda")
    out = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.JepaError, match="JEPA_E_SHAPE"):
        lib.jepa_op_gemm("bf16", x, w, "bf16", 64, b, "store", out)      # K % 64 != 0
    q = torch.zeros((10, 3 * 64), dtype=torch.bfloat16, device="cuda")
    vt = torch.zeros((1, 64, 64), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((10, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.JepaError, match="JEPA_E_SHAPE"):
        lib.jepa_op_attention("bf16", q, vt, 1, 10, 1, True, "block_causal", 4, o)   # 9 % 4 != 0
    vt_short = torch.zeros((1, 64, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.JepaError, match="JEPA_E_SHAPE"):
        lib.jepa_op_attention("bf16", q, vt_short, 1, 10, 1, True, "bidir", 1, o)   # npad < 64
    with pytest.raises(lib.JepaError, match="JEPA_E_UNSUPPORTED"):
        lib.jepa_op_attention("bf16", q, vt, 1, 10, 4, True, "bidir", 1, o, head_dim=16)


def test_size_limits_are_rejected_before_launch(lib):
    """The largest shapes each kernel's 32-bit offsets and grid limits allow
    end in a status, not a launch: calls that claim sizes past them (on small
    buffers the kernels would overrun) are refused during validation."""
    raw = lib._lib
    q = torch.zeros((64, 3 * 1024), dtype=torch.bfloat16, device="cuda")
    vt = torch.zeros((1, 1024, 64), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((64, 1024), dtype=torch.bfloat16, device="cuda")
    BF16, SHAPE = lib.DTYPE["bf16"], -2
    # attention: (N + 64) * ld_qk * 2 bytes must stay below 2^31
    N = 700000
    assert raw.jepa_op_attention(BF16, q.data_ptr(), 3 * 1024, vt.data_ptr(), -(-N // 64) * 64, 1, N, 16, 64,
                                 0, 0, 1, 1, o.data_ptr(), None) == SHAPE
    # GEMM: at most 65534 row tiles of 128
    w = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(64, device="cuda")
    assert raw.jepa_op_gemm(BF16, q.data_ptr(), 65535 * 128, 64, w.data_ptr(), BF16, None, 64, b.data_ptr(),
                            0, o.data_ptr(), 64, None) == SHAPE
    # attention with no items
    assert raw.jepa_op_attention(BF16, q.data_ptr(), 3 * 1024, vt.data_ptr(), 64, 0, 10, 16, 64,
                                 0, 0, 1, 1, o.data_ptr(), None) == SHAPE
    # the encoder: batch * tokens beyond its grid limit, refused before any copy
    from tests.helpers import workload_inputs
    wl, dims, frames, stored = workload_inputs("small_bidir_f32")
    ctx = lib.jepa_create(dims, stored)
    fr = torch.from_numpy(frames).cuda()
    assert raw.jepa_encode(ctx, fr.data_ptr(), 1_000_000, 1, None, None) == -7     # JEPA_E_UNSUPPORTED
    assert raw.jepa_encode(ctx, fr.data_ptr(), 0, 1, None, None) == -1             # JEPA_E_INVALID_ARG
    lib.jepa_free(ctx)


@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("B,N,heads,dh", [(2, 3137, 16, 64), (3, 289, 2, 64), (1, 1, 1, 64), (2, 197, 6, 32)])
def test_transpose_v(lib, act, B, N, heads, dh):
    if act == "f32" and B * N * heads > 10000:
        pytest.skip("the f32 path only serves small models")
    rng = np.random.default_rng(46)
    D = heads * dh
    qkv_dev, _ = rounded(act, rng.standard_normal((B * N, 3 * D)))
    vt = _vt_of(lib, act, qkv_dev, B, N, heads, dh)
    v = qkv_dev[:, 2 * D:].float().cpu().numpy().reshape(B, N, D)
    got = vt.float().cpu().numpy()
    pos = vt_pos(np.arange(N))
    assert np.array_equal(got[..., pos], v.transpose(0, 2, 1))
    assert np.all(got[..., np.setdiff1d(np.arange(got.shape[-1]), pos)] == 0)


def test_int8_mfma_and_its_per_block_rescale(lib):
    """The int8 matrix path's ceiling on this chip: the plain int8 MFMA rate
    and the rate left when each 32-wide K block's int32 result is rescaled
    into f32 (per-row and per-column block scales; one scale per row),
    beside the dense bf16 rate.  Prints the rates; checks the launches and
    their op counts."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.full((2 * cus * 256,), float("nan"), device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def rate(fn, *args):
        fn(*args)                                 # warm-up
        torch.cuda.synchronize()
        e0.record()
        ops = fn(*args)
        e1.record()
        torch.cuda.synchronize()
        assert torch.isfinite(out[:args[0] * 256]).all()
        return ops / (e0.elapsed_time(e1) * 1e-3) / 1e12

    bf16 = rate(lib.jepa_op_mfma_probe, cus, 20000, out)
    bf16r = rate(lib.jepa_op_mfma_probe, cus, 20000, out, 1)
    i8 = [rate(lib.jepa_op_mfma_i8_probe, 2 * cus, 10000, m, out) for m in (0, 1, 2)]
    say(f"  dense bf16 MFMA {bf16:.0f} TFLOP/s ({bf16r:.0f} with random operands); int8 MFMA "
        f"{i8[0]:.0f} TOP/s; with per-block row and column scales {i8[1]:.0f} TOP/s; with "
        f"per-block column scales {i8[2]:.0f} TOP/s")
    assert lib.jepa_op_mfma_i8_probe(1, 3, 1, out) == 1 * 4 * 3 * 4 * 65536
    with pytest.raises(lib.JepaError, match="JEPA_E_INVALID_ARG"):
        lib.jepa_op_mfma_i8_probe(1, 3, 3, out)


@pytest.mark.parametrize("operands", [0, 1])
def test_mfma_probe_runs_and_reports_its_flops(lib, operands):
    """The calibration kernel, constant or random operands: finite output
    from every thread, and the work it reports is workgroups x 4 waves x
    iters x 8 MFMAs of 32x32x16x2."""
    out = torch.full((8 * 256,), float("nan"), device="cuda")
    flops = lib.jepa_op_mfma_probe(8, 100, out, operands)
    torch.cuda.synchronize()
    assert flops == 8 * 4 * 100 * 8 * 32768
    assert torch.isfinite(out).all()
    with pytest.raises(lib.JepaError, match="JEPA_E_INVALID_ARG"):
        lib.jepa_op_mfma_probe(0, 100, out, operands)
    with pytest.raises(lib.JepaError, match="JEPA_E_INVALID_ARG"):
        lib.jepa_op_mfma_probe(8, 100, out, 2)
