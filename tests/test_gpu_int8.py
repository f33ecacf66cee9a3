"""The int8 path of q8_0 / q4_0 matrices, through the C ABI, against the
oracle (activations quantised per 32-block, reading R17 of the oracle).

The quantiser's codes and scales are integer decisions taken in f32 on both
sides, so they must match bit for bit.  The int8 product is then compared
element by element with the oracle's product of the dequantised activations
and weights, which is exactly the sum of the blocks' scaled integer dot
products; the bound is the f32 accumulation of one rounded scale product and
one FMA per block.  The encoder with the path on is compared with the
oracle encoder that quantises every product's input the same way."""
import numpy as np
import pytest

from oracle import encoder as E
from oracle import quant as Q
from tests import helpers as H
from tests.helpers import rounded, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    from vision_transformer_amd import _lib
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return _lib


OUT_REL = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def _act_rows(act, rng, M, K):
    """Rows of varied magnitude, with an all-zero block, a one-value block
    and exact half-step ties (a block of k + 1/2 times a power of two whose
    largest value is 127 times it)."""
    x = rng.standard_normal((M, K)) * np.exp(rng.uniform(-4, 4, (M, 1)))
    x[0, :32] = 0.0
    x[1, 32:64] = 0.0
    x[1, 40] = -3.0
    x[2, :32] = (rng.integers(-127, 127, 32) + 0.5) * 2.0 ** -6
    x[2, 5] = 127 * 2.0 ** -6
    return rounded(act, x)


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("M,K", [(777, 1024), (3, 4096), (12548, 1024)])
def test_quantize_act_bit_exact(lib, act, M, K):
    say(f"quantize_act {act} M={M} K={K}")
    rng = np.random.default_rng(11)
    x_dev, x = _act_rows(act, rng, M, K)
    q_dev = torch.empty((M, K), dtype=torch.int8, device="cuda")
    d_dev = torch.empty((M, K // 32), dtype=torch.float32, device="cuda")
    lib.jepa_op_quantize_act(act, x_dev, q_dev, d_dev)
    torch.cuda.synchronize()
    q, d = Q.quantize_act_q8(x)
    assert np.array_equal(d_dev.cpu().numpy().view(np.uint32), d.view(np.uint32))
    assert np.array_equal(q_dev.cpu().numpy(), q)


def _i8_case(lib, act, wfmt, epi, M, N, K, seed):
    rng = np.random.default_rng(seed)
    _, a = rounded(act, rng.standard_normal((M, K)))
    qa, da = Q.quantize_act_q8(a)
    xa = Q.act_q8_values(qa, da)
    w32 = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    bias = (rng.standard_normal(N) * 0.1).astype(np.float32)
    raw = Q.quantize(wfmt, w32)
    w = Q.stored_to_f64(dict(dtype=wfmt, ne0=K, ne1=N, data=raw))
    codes, scales = lib.jepa_pack_blocks(wfmt, raw, N, K)
    w_dev = torch.from_numpy(codes).cuda()
    ws_dev = torch.from_numpy(scales.view(np.int16)).cuda()
    qa_dev = torch.from_numpy(qa).cuda()
    da_dev = torch.from_numpy(da).cuda()
    ref = E.linear(xa, w, bias.astype(np.float64))
    b_dev = torch.from_numpy(bias).cuda()
    if epi == "resid":
        x0 = rng.standard_normal((M, N)).astype(np.float32)
        out = torch.from_numpy(x0.copy()).cuda()
        ref = ref + x0
    else:
        out = torch.empty((M, N), dtype=H.torch_dtype(act), device="cuda")
        if epi == "gelu":
            ref = E.gelu(ref)
    lib.jepa_op_gemm_i8(act, qa_dev, da_dev, w_dev, wfmt, N, b_dev, epi, out, ws_dev)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), ref, xa, w


@pytest.mark.parametrize("wfmt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("epi", ["store", "gelu", "resid"])
@pytest.mark.parametrize("mnk", [(333, 320, 1024), (129, 192, 4096), (1300, 1024, 256)])
def test_gemm_i8_every_element(lib, wfmt, act, epi, mnk):
    M, N, K = mnk
    say(f"gemm_i8 {wfmt} {act} {epi} M={M} N={N} K={K}")
    got, ref, xa, w = _i8_case(lib, act, wfmt, epi, M, N, K, 53)
    # per block: the scale product and the FMA round once each (2^-24
    # relative), over K / 32 blocks of f32 accumulation
    mag = np.abs(xa) @ np.abs(w).T
    bound = (4 * (K // 32) + 4) * 2.0 ** -24 * mag
    out_r = 0.0 if epi == "resid" else OUT_REL[act]
    err = np.abs(got - ref)
    assert np.all(err <= bound + out_r * np.abs(ref) + 1e-6), (err - bound - out_r * np.abs(ref)).max()
    # the bound is far below what losing one block of the sum would cost
    assert np.median(mag / (K // 32)) > 50 * np.median(bound)


def test_gemm_i8_rejects_out_of_contract_shapes(lib):
    M, N, K = 64, 128, 96      # K not a multiple of 128
    qa = torch.zeros((M, K), dtype=torch.int8, device="cuda")
    da = torch.zeros((M, K // 32), dtype=torch.float32, device="cuda")
    w = torch.zeros((N, K), dtype=torch.int8, device="cuda")
    ws = torch.zeros((N, K // 32), dtype=torch.int16, device="cuda")
    b = torch.zeros(N, dtype=torch.float32, device="cuda")
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    with pytest.raises(lib.JepaError):
        lib.jepa_op_gemm_i8("f16", qa, da, w, "q8_0", N, b, "store", out, ws)
    with pytest.raises(lib.JepaError):
        lib.jepa_op_gemm_i8("f32", qa, da, w, "q8_0", N, b, "store", out, ws)


@pytest.fixture(scope="module")
def Encoder():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vision_transformer_amd.encoder import Encoder
    return Encoder


def _encode(enc, frames):
    y = enc.encode(torch.from_numpy(frames).cuda())
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("name", ["small_tubelet2_q8_0", "small_tubelet2_q4_0", "small_rope_q4_0",
                                  "mid_vitl_tubelet2_q8_0"])
def test_int8_encoder_every_token(Encoder, name):
    """Every token and the mean pool with the int8 path on, against the oracle
    encoder that quantises each product's input (R17); the default path on
    the same context afterwards still matches the plain oracle."""
    say(f"encoder {name}, int8 products")
    wl, dims, frames, stored = H.workload_inputs(name, ln_affine=True)
    w = E.weights_f64(stored)
    ref8 = E.encode(dims, w, frames, act_q8=True)
    enc = Encoder(dims, stored)
    enc.set_int8_matmul(True)
    y8 = _encode(enc, frames).cpu().numpy()
    H.check_rows(dims["act_dtype"], y8, ref8, "tokens (int8 path vs int8 oracle)")
    mean = enc.pool("mean", wl["batch"]).cpu().numpy()
    H.check_rows(dims["act_dtype"], mean, E.pool(ref8, "mean", bool(dims["has_cls"])), "mean")
    ref = E.encode(dims, w, frames)
    r = H.M.report(y8, ref)
    say(f"  int8 path vs the dense oracle: cos worst {r['cos_worst']:.7f} mean {r['cos_mean']:.7f}")
    enc.set_int8_matmul(False)
    y = _encode(enc, frames).cpu().numpy()
    H.check_rows(dims["act_dtype"], y, ref, "tokens (default path)")
    enc.close()


def test_int8_full_size_whole_token_map(Encoder):
    """V-JEPA 2 ViT-L/16 16 frames 256x256, q8_0 matrices, batch 4 (8192
    tokens), in the benchmark's launch configuration, every token against
    the int8 oracle run here."""
    import time
    name = "vjepa2_vit_l16_16f256_q8_0_b4"
    say(f"encoder {name}, int8 products (full size, whole token map)")
    wl, dims, frames, stored = H.workload_inputs(name)
    enc = Encoder(dims, stored)
    enc.set_int8_matmul(True)
    y = _encode(enc, frames).cpu().numpy()
    mean = enc.pool("mean", wl["batch"]).cpu().numpy()
    enc.close()
    t0 = time.time()
    ref = E.encode(dims, E.weights_f64(stored), frames, act_q8=True)
    say(f"  oracle: {time.time() - t0:.1f} s")
    r = H.check_rows(dims["act_dtype"], y, ref, f"all {y.shape[0] * y.shape[1]} tokens")
    say(f"  per-token cosine: mean {r['cos_mean']:.7f} median {r['cos_median']:.7f} worst {r['cos_worst']:.7f}")
    H.check_rows(dims["act_dtype"], mean, E.pool(ref, "mean", False), "mean")


def test_int8_switch_errors(Encoder):
    from vision_transformer_amd import _lib
    for name in ("small_bidir_f32", "small_head_cls_q8_0", "small_q6_k_rope_blockcausal_f16"):
        wl, dims, frames, stored = H.workload_inputs(name)
        enc = Encoder(dims, stored)
        with pytest.raises(_lib.JepaError) as e:
            enc.set_int8_matmul(True)
        assert e.value.status == -7     # f32 model; dim 192; K-quants
        enc.close()


def test_int8_batch_parts_and_graph_replay_bit_exact(Encoder):
    """With the int8 path on, 1 to 4 concurrent batch parts give
    bit-identical tokens (batch 5), and encode + pool captured into one HIP
    graph replays to the eager result, with eager work in between."""
    from vision_transformer_amd import _lib
    wl, dims, _, stored = H.workload_inputs("small_tubelet2_q4_0")
    frames = H.synth.make_frames(dims, 5, 79)
    enc = Encoder(dims, stored)
    enc.set_int8_matmul(True)
    fr = torch.from_numpy(frames).cuda()
    ys = []
    for parts in (1, 2, 3, 4):
        say(f"int8 encoder batch 5 in {parts} parts")
        _lib.jepa_set_batch_parts(enc.ctx, parts)
        ys.append(_encode(enc, frames).cpu().clone())
    for y in ys[1:]:
        assert torch.equal(ys[0], y)
    B = 5
    tokens = torch.empty((B, enc.n_tokens, dims["dim"]), dtype=torch.float32, device="cuda")
    pooled = torch.empty((B, dims["dim"]), dtype=torch.float32, device="cuda")
    enc.encode(fr, tokens)
    enc.pool("mean", B, pooled)
    torch.cuda.synchronize()
    want_t, want_p = tokens.clone(), pooled.clone()
    assert torch.equal(want_t.cpu(), ys[-1])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        enc.encode(fr, tokens)
        enc.pool("mean", B, pooled)
    for r in range(3):
        say(f"int8 graph replay {r}")
        tokens.zero_()
        pooled.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(tokens, want_t) and torch.equal(pooled, want_p)
        enc.encode(fr, tokens)
        torch.cuda.synchronize()
        assert torch.equal(tokens, want_t)
    del graph
    enc.close()


def test_int8_noalloc_matches_encode(lib):
    """jepa_encode_noalloc with the int8 path on (its quantised inputs in the
    static array too) equals jepa_encode bit for bit, on two calls in a row,
    the second with a smaller batch."""
    wl, dims, _, stored = H.workload_inputs("small_tubelet2_q8_0")
    frames = H.synth.make_frames(dims, 3, 95)
    ctx = lib.jepa_create(dims, stored)
    lib.jepa_set_int8_matmul(ctx, True)
    lib.jepa_set_batch_parts(ctx, 1)
    N, D = H.synth.n_tokens(dims), dims["dim"]
    try:
        for B in (3, 1):
            say(f"int8 encode_noalloc batch {B}")
            fr = torch.from_numpy(np.ascontiguousarray(frames[:B])).cuda()
            want = torch.empty((B, N, D), device="cuda")
            got = torch.full((B, N, D), float("nan"), device="cuda")
            lib.jepa_encode(ctx, fr, B, want)
            torch.cuda.synchronize()
            lib.jepa_encode_noalloc(ctx, fr, B, got)
            torch.cuda.synchronize()
            assert torch.equal(got, want)
    finally:
        lib.jepa_free(ctx)


@pytest.mark.parametrize("mat", ["q8_0", "q4_0"])
def test_int8_encoder_bf16_activations_every_token(Encoder, mat):
    """The small tubelet-2 model with bf16 activations (LN, biases and the
    patch table bf16 too) and q8_0 / q4_0 matrices: every token with the int8
    path on against the int8 oracle."""
    from vision_transformer_amd import synth
    wl = synth.workload("small_tubelet2_q8_0")
    dims = dict(wl["dims"], act_dtype="bf16", rest_dtype="bf16", mat_dtype=mat)
    frames = synth.make_frames(dims, wl["batch"], 31)
    stored = synth.stored_weights(dims, synth.make_f32_weights(dims, 32, ln_affine=True), quantize=Q.quantize)
    say(f"int8 encoder, bf16 activations, {mat}")
    ref8 = E.encode(dims, E.weights_f64(stored), frames, act_q8=True)
    enc = Encoder(dims, stored)
    enc.set_int8_matmul(True)
    y8 = _encode(enc, frames).cpu().numpy()
    enc.close()
    H.check_rows("bf16", y8, ref8, "tokens (int8 path vs int8 oracle)")
