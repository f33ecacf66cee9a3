"""The whole encoder through the C ABI against the oracle.

* Small workloads (the oracle runs in seconds): every token of the token map,
  and the CLS / mean pools, against the oracle computed live.
* The ViT-Ti/14 f32 image workload at its full size, live.
* The ViT-L workloads at full size (additive or 3-D rotary position), in
  the launch configuration the benchmark times: sampled token rows and the
  pooled features against the oracle's stored outputs
  (tests/golden/make_golden.py).
* Invariants that must hold bit for bit: block-causal causality, the CLS
  token being read-only, batch items being independent.
* Dequantised weights bit-exact against the oracle.
"""
import os

import numpy as np
import pytest

from oracle import encoder as E
from oracle import quant as Q
from tests import gguf_file as G
from tests import helpers as H
from vision_transformer_amd import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def Encoder():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vision_transformer_amd.encoder import Encoder
    return Encoder


def _run(enc, frames):
    y = enc.encode(torch.from_numpy(frames).cuda())
    torch.cuda.synchronize()
    return y


def _check_pools(enc, dims, y_ref, B):
    act = dims["act_dtype"]
    if dims["has_cls"]:
        cls = enc.pool("cls", B).cpu().numpy()
        H.check_rows(act, cls, E.pool(y_ref, "cls", True), "cls")
    mean = enc.pool("mean", B).cpu().numpy()
    H.check_rows(act, mean, E.pool(y_ref, "mean", bool(dims["has_cls"])), "mean")


@pytest.mark.parametrize("name", list(synth.SMALL_WORKLOADS))
def test_small_workload_every_token(Encoder, name):
    H.say(f"encoder {name}")
    wl, dims, frames, stored = H.workload_inputs(name, ln_affine=True)
    enc = Encoder(dims, stored)
    y_dev = _run(enc, frames)        # kept alive: pool() reads the last encode's token map
    y = y_dev.cpu().numpy()
    ref = H.oracle_tokens(dims, stored, frames)
    H.check_rows(dims["act_dtype"], y, ref, "tokens")
    _check_pools(enc, dims, ref, wl["batch"])
    none = enc.pool("none", wl["batch"]).cpu().numpy()
    assert np.array_equal(none, y)
    enc.close()


def test_vit_ti14_image_f32_full(Encoder):
    H.say("encoder vit_ti14_image_f32")
    wl, dims, frames, stored = H.workload_inputs("vit_ti14_image_f32")
    enc = Encoder(dims, stored)
    y_dev = _run(enc, frames)        # kept alive: pool() reads the last encode's token map
    y = y_dev.cpu().numpy()
    ref = H.oracle_tokens(dims, stored, frames)
    r = H.check_rows("f32", y, ref, "tokens")
    assert r["cos_worst"] >= H.F32_COS
    _check_pools(enc, dims, ref, wl["batch"])
    assert enc.last_compute_ms() > 0
    enc.close()


@pytest.mark.parametrize("name", list(synth.MID_WORKLOADS))
def test_mid_vitl_every_token(Encoder, name, monkeypatch):
    """ViT-L/16 widths at two blocks: with the batch in one part every GEMM
    (qkv, out-proj, fc1 with GELU, fc2 at K 4096) runs on the 256-row tiles,
    the block matrices expanded to the act dtype; every token and the pools
    against the live oracle.  Then the default batch parts (smaller tiles,
    weights dequantised in the tile load) against the same oracle."""
    from vision_transformer_amd import _lib
    H.say(f"encoder {name}, one part")
    wl, dims, frames, stored = H.workload_inputs(name, ln_affine=True)
    ref = H.oracle_tokens(dims, stored, frames)
    enc = Encoder(dims, stored)
    _lib.jepa_set_batch_parts(enc.ctx, 1)
    if dims["mat_dtype"] in ("q8_0", "q4_0"):
        monkeypatch.setenv("JEPA_Q_EXPAND", "1")     # (K-quants always expand)
    y = _run(enc, frames)
    H.check_rows(dims["act_dtype"], y.cpu().numpy(), ref, "tokens")
    _check_pools(enc, dims, ref, wl["batch"])
    monkeypatch.delenv("JEPA_Q_EXPAND", raising=False)
    _lib.jepa_set_batch_parts(enc.ctx, 0)
    H.say(f"encoder {name}, default parts")
    y = _run(enc, frames)
    H.check_rows(dims["act_dtype"], y.cpu().numpy(), ref, "tokens")
    enc.close()


# the two workloads compared over their whole token maps against the oracle
# computed in the test (the block-causal headline and the attention-heavy
# 8192-token clip); about a minute of CPU each
LIVE_FULL = ["levjepa_vit_l16_16f_bf16_b4", "vjepa2_vit_l16_64f256_f16"]


@pytest.mark.parametrize("name", LIVE_FULL)
def test_full_workload_whole_token_map_live(Encoder, name):
    """Every token of a full-size token map, in the launch configuration the
    benchmark times, against the oracle run here on the same inputs: the
    worst-token cosine bar over all B x N tokens, with the mean and median
    reported as the LeVJEPA card's "Files" table does."""
    import time
    H.say(f"encoder {name} (full size, whole token map)")
    wl, dims, frames, stored = H.workload_inputs(name)
    enc = Encoder(dims, stored)
    y = _run(enc, frames).cpu().numpy()
    B = wl["batch"]
    pools = {}
    if dims["has_cls"]:
        pools["cls"] = enc.pool("cls", B).cpu().numpy()
    pools["mean"] = enc.pool("mean", B).cpu().numpy()
    enc.close()
    t0 = time.time()
    ref = H.oracle_tokens(dims, stored, frames)
    H.say(f"  oracle: {time.time() - t0:.1f} s for {B} x {ref.shape[1]} tokens")
    r = H.check_rows(dims["act_dtype"], y, ref, f"all {B * ref.shape[1]} tokens")
    H.say(f"  per-token cosine: mean {r['cos_mean']:.7f} median {r['cos_median']:.7f} "
          f"worst {r['cos_worst']:.7f}")
    for mode, got in pools.items():
        H.check_rows(dims["act_dtype"], got, E.pool(ref, mode, bool(dims["has_cls"])), mode)


FULL = ["vit_l16_image_bf16_b32", "levjepa_vit_l16_16f_bf16_b4",
        "vjepa2_vit_l16_16f256_q8_0_b4", "vjepa2_vit_l16_64f256_f16",
        "vjepa2_vit_l16_64f256_q4_0", "vjepa2_rope_vit_l16_16f256_f16_b4",
        "vjepa2_predictor_width_384d_dh32_4096tok_bf16_b4",
        "vjepa2_ssv2_classifier_vit_l16_16f256_f16_b4"]


@pytest.mark.parametrize("name", FULL)
def test_full_workload_against_stored_oracle(Encoder, name):
    path = os.path.join(H.GOLDEN, f"{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    g = np.load(path, allow_pickle=False)
    H.say(f"encoder {name} (full size)")
    wl, dims, frames, stored = H.workload_inputs(name)
    import hashlib
    assert hashlib.sha256(frames.tobytes()).hexdigest() == str(g["frames_sha256"])
    assert H.digest_weights(stored) == str(g["weights_sha256"])
    enc = Encoder(dims, stored)
    del stored
    y = _run(enc, frames)
    rows = g["rows"]
    got = y[torch.from_numpy(rows[:, 0]).cuda(), torch.from_numpy(rows[:, 1]).cuda()].cpu().numpy()
    act = dims["act_dtype"]
    H.check_rows(act, got, g["sampled"], f"{len(rows)} sampled tokens")
    B = wl["batch"]
    if dims["has_cls"]:
        H.check_rows(act, enc.pool("cls", B).cpu().numpy(), g["cls"], "cls")
    H.check_rows(act, enc.pool("mean", B).cpu().numpy(), g["mean"], "mean")
    if "logits" in g.files:
        H.check_rows(act, enc.classify(B).cpu().numpy(), g["logits"], "class scores")
    enc.close()


# ---------------------------------------------------------------------------
# invariants, bit for bit
# ---------------------------------------------------------------------------

def test_block_causal_causality_bit_exact(Encoder):
    wl, dims, frames, stored = H.workload_inputs("small_blockcausal_bf16")
    enc = Encoder(dims, stored)
    y0 = _run(enc, frames).cpu()
    f2 = frames.copy()
    t = 5
    f2[:, t] = 255 - f2[:, t]
    y1 = _run(enc, f2).cpu()
    per = synth.grid(dims)[1] * synth.grid(dims)[2]
    keep = 1 + t * per
    assert torch.equal(y0[:, 1:keep], y1[:, 1:keep])
    assert not torch.equal(y0[:, keep:], y1[:, keep:])
    enc.close()


def test_cls_token_is_read_only_bit_exact(Encoder):
    wl, dims, frames, stored = H.workload_inputs("small_blockcausal_bf16")
    enc = Encoder(dims, stored)
    y0 = _run(enc, frames).cpu()
    enc.close()
    s2 = [dict(t) for t in stored]
    for t in s2:
        if t["name"] == "enc.cls_token":
            t["data"] = synth.to_bfloat16_bits(np.full(dims["dim"], 0.5, np.float32))
    enc = Encoder(dims, s2)
    y1 = _run(enc, frames).cpu()
    assert torch.equal(y0[:, 1:], y1[:, 1:])
    assert not torch.equal(y0[:, 0], y1[:, 0])
    enc.close()


@pytest.mark.parametrize("name", ["small_blockcausal_bf16", "small_tubelet2_q8_0"])
def test_batch_items_independent_bit_exact(Encoder, name):
    wl, dims, frames, stored = H.workload_inputs(name)
    enc = Encoder(dims, stored)
    y = _run(enc, frames).cpu()
    for b in range(frames.shape[0]):
        yb = _run(enc, np.ascontiguousarray(frames[b:b + 1])).cpu()
        assert torch.equal(y[b:b + 1], yb)
    enc.close()


@pytest.mark.parametrize("name", ["small_blockcausal_bf16", "small_tubelet2_q4_0"])
def test_batch_parts_do_not_change_tokens(Encoder, name):
    """The batch runs as concurrent parts (one HIP stream each); items never
    interact, so 1 to 4 parts give bit-identical tokens (batch 5: ragged
    parts of 3+2, 2+2+1 and 2+1+1+1 items)."""
    from vision_transformer_amd import _lib
    wl, dims, _, stored = H.workload_inputs(name)
    frames = synth.make_frames(dims, 5, 77)
    enc = Encoder(dims, stored)
    ys = []
    for parts in (1, 2, 3, 4):
        H.say(f"encoder {name} batch 5 in {parts} parts")
        _lib.jepa_set_batch_parts(enc.ctx, parts)
        ys.append(_run(enc, frames).cpu().clone())
    for y in ys[1:]:
        assert torch.equal(ys[0], y)
    with pytest.raises(_lib.JepaError, match="JEPA_E_INVALID_ARG"):
        _lib.jepa_set_batch_parts(enc.ctx, 5)
    enc.close()


@pytest.mark.parametrize("parts", [1, 3])
def test_graph_replay_matches_eager(Encoder, parts):
    """encode + pool captured into one HIP graph (with the batch in concurrent
    parts: the fork / join events become graph edges).  Every replay, with
    eager work and synchronisations in between, equals the eager result bit
    for bit."""
    from vision_transformer_amd import _lib
    wl, dims, frames, stored = H.workload_inputs("small_blockcausal_bf16")
    enc = Encoder(dims, stored)
    _lib.jepa_set_batch_parts(enc.ctx, parts)
    fr = torch.from_numpy(frames).cuda()
    B = frames.shape[0]
    tokens = torch.empty((B, enc.n_tokens, dims["dim"]), dtype=torch.float32, device="cuda")
    pooled = torch.empty((B, dims["dim"]), dtype=torch.float32, device="cuda")
    enc.encode(fr, tokens)
    enc.pool("cls", B, pooled)
    torch.cuda.synchronize()
    want_t, want_p = tokens.clone(), pooled.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        enc.encode(fr, tokens)
        enc.pool("cls", B, pooled)
    for r in range(3):
        H.say(f"graph replay {r}, parts {parts}")
        tokens.zero_()
        pooled.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(tokens, want_t) and torch.equal(pooled, want_p)
        enc.encode(fr, tokens)              # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(tokens, want_t)
    del graph
    enc.close()


@pytest.mark.parametrize("name", ["small_tubelet2_q8_0", "small_tubelet2_q4_0", "small_rope_q4_0"])
def test_expanded_block_matrices_every_token(Encoder, name, monkeypatch):
    """JEPA_Q_EXPAND=1: the q8_0 / q4_0 matrices are expanded to the act dtype
    before the first layer and the GEMMs run dense; every token and the mean
    pool against the oracle.  The workspace size counts the copy."""
    from vision_transformer_amd import _lib
    wl, dims, frames, stored = H.workload_inputs(name, ln_affine=True)
    enc = Encoder(dims, stored)
    plain = _lib.jepa_workspace_bytes(enc.ctx, wl["batch"])
    monkeypatch.setenv("JEPA_Q_EXPAND", "1")
    H.say(f"encoder {name}, block matrices expanded")
    assert _lib.jepa_workspace_bytes(enc.ctx, wl["batch"]) > plain
    y_dev = _run(enc, frames)
    ref = H.oracle_tokens(dims, stored, frames)
    H.check_rows(dims["act_dtype"], y_dev.cpu().numpy(), ref, "tokens")
    _check_pools(enc, dims, ref, wl["batch"])
    enc.close()


def test_expanded_copy_written_once_and_reused(Encoder, monkeypatch):
    """The act-dtype copy of the block matrices depends on the weights only:
    the first encode that takes the expanded path writes it, later ones (a
    different batch, an encode without it in between, another stream) reuse
    it.  Each token map matches the oracle's, a repeat is bit-identical, and
    the expansion kernel ran once."""
    from vision_transformer_amd import _lib
    monkeypatch.setenv("JEPA_Q_EXPAND", "1")
    wl, dims, frames, stored = H.workload_inputs("small_tubelet2_q8_0", ln_affine=True)
    enc = Encoder(dims, stored)
    _lib.jepa_set_profiling(enc.ctx, 0xFFFFFFFF)
    H.say("encoder small_tubelet2_q8_0: three expanded encodes, one plain between")
    y1 = _run(enc, frames).clone()
    H.check_rows(dims["act_dtype"], y1.cpu().numpy(), H.oracle_tokens(dims, stored, frames), "first")
    monkeypatch.setenv("JEPA_Q_EXPAND", "0")
    fr2 = synth.make_frames(dims, 3, 79)
    y2 = _run(enc, fr2).clone()
    monkeypatch.setenv("JEPA_Q_EXPAND", "1")
    ref2 = H.oracle_tokens(dims, stored, fr2)
    H.check_rows(dims["act_dtype"], y2.cpu().numpy(), ref2, "plain path")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        y3 = enc.encode(torch.from_numpy(fr2).cuda()).clone()
    torch.cuda.synchronize()
    H.check_rows(dims["act_dtype"], y3.cpu().numpy(), ref2, "expanded, other stream")
    y4 = _run(enc, frames)
    assert torch.equal(y4, y1)
    stats = _lib.jepa_kernel_stats(enc.ctx)
    assert stats["expand_weights"]["launches"] == 1, stats["expand_weights"]
    enc.close()


def test_expansion_chosen_by_rows_per_part(Encoder, monkeypatch):
    """Without the override, 9 items of 126 tokens in one part (1134 rows)
    take the expanded path and match the oracle; in 4 parts (at most 378
    rows each) they do not expand."""
    from vision_transformer_amd import _lib
    monkeypatch.delenv("JEPA_Q_EXPAND", raising=False)
    wl, dims, _, stored = H.workload_inputs("small_tubelet2_q8_0", ln_affine=True)
    frames = synth.make_frames(dims, 9, 78)
    enc = Encoder(dims, stored)
    _lib.jepa_set_batch_parts(enc.ctx, 4)
    small = _lib.jepa_workspace_bytes(enc.ctx, 9)
    _lib.jepa_set_batch_parts(enc.ctx, 1)
    assert _lib.jepa_workspace_bytes(enc.ctx, 9) > small
    H.say("encoder small_tubelet2_q8_0, batch 9 in one part")
    y_dev = _run(enc, frames)
    ref = H.oracle_tokens(dims, stored, frames)
    H.check_rows(dims["act_dtype"], y_dev.cpu().numpy(), ref, "tokens")
    enc.close()


@pytest.mark.parametrize("name", ["small_head_bf16", "small_head_cls_q8_0", "small_head_dh32_f32",
                                  "small_q4_k_fallback_head_bf16"])
def test_classifier_head_scores(Encoder, name):
    """The attentive-pool head on the encoder's token map: class scores of
    every item against the oracle (its blocks, cross-attention query, MLP and
    classifier; rotary or additive position, CLS, q8_0 matrices, heads of 32)."""
    from oracle import head as HD
    H.say(f"classifier head {name}")
    wl, dims, frames, stored = H.workload_inputs(name, ln_affine=True)
    enc = Encoder(dims, stored)
    y_dev = _run(enc, frames)
    logits = enc.classify(wl["batch"])
    torch.cuda.synchronize()
    ref_y = H.oracle_tokens(dims, stored, frames)
    H.check_rows(dims["act_dtype"], y_dev.cpu().numpy(), ref_y, "tokens")
    ref = HD.classify(dims, E.weights_f64(stored), ref_y)
    H.check_rows(dims["act_dtype"], logits.cpu().numpy(), ref, "class scores")
    enc.close()


def test_classify_state_errors(Encoder):
    from vision_transformer_amd import _lib
    wl, dims, frames, stored = H.workload_inputs("small_head_bf16")
    enc = Encoder(dims, stored)
    with pytest.raises(_lib.JepaError, match="JEPA_E_STATE"):
        enc.classify(1)
    enc.close()
    wl, dims, frames, stored = H.workload_inputs("small_bidir_f32")
    enc = Encoder(dims, stored)
    _run(enc, frames)
    with pytest.raises(_lib.JepaError, match="JEPA_E_UNSUPPORTED"):
        _lib.jepa_classify(enc.ctx, torch.empty((2, 1), device="cuda"))
    enc.close()


@pytest.mark.parametrize("name", ["small_blockcausal_f32", "small_head_bf16"])
def test_graph_replay_of_split_passes_and_head(Encoder, name):
    """Captured encode (+ classify): the f32 model's K and key splits with
    their ordered second passes, and the classifier head's fills and copies,
    replay bit for bit, with eager work between the replays."""
    wl, dims, frames, stored = H.workload_inputs(name)
    enc = Encoder(dims, stored)
    fr = torch.from_numpy(frames).cuda()
    B = frames.shape[0]
    head = bool(dims.get("head_classes"))
    tokens = torch.empty((B, enc.n_tokens, dims["dim"]), dtype=torch.float32, device="cuda")
    scores = torch.empty((B, dims["head_classes"]), dtype=torch.float32, device="cuda") if head else None

    def step():
        enc.encode(fr, tokens)
        if head:
            enc.classify(B, scores)

    step()
    torch.cuda.synchronize()
    want_t = tokens.clone()
    want_s = scores.clone() if head else None
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        H.say(f"graph replay {r}, {name}")
        tokens.zero_()
        if head:
            scores.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(tokens, want_t)
        if head:
            assert torch.equal(scores, want_s)
        step()                                   # eager work between replays
        torch.cuda.synchronize()
    del graph
    enc.close()


def test_workspace_grows_and_contexts_coexist(Encoder):
    """A larger batch after a smaller one reallocates the workspace; a second
    context alive at the same time keeps its own weights and results."""
    wl, dims, frames, stored = H.workload_inputs("small_bidir_f32")
    a = Encoder(dims, stored)
    wl2, dims2, frames2, stored2 = H.workload_inputs("small_blockcausal_bf16")
    b = Encoder(dims2, stored2)
    ya1 = _run(a, frames[:1]).cpu()
    yb = _run(b, frames2).cpu()
    big = synth.make_frames(dims, 5, 91)
    big[:1] = frames[:1]
    ya5 = _run(a, big).cpu()
    assert torch.equal(ya5[:1], ya1)
    assert torch.equal(_run(b, frames2).cpu(), yb)
    ya1b = _run(a, frames[:1]).cpu()                # smaller again
    assert torch.equal(ya1b, ya1)
    a.close()
    b.close()


def test_host_frames_match_device_frames(Encoder):
    wl, dims, frames, stored = H.workload_inputs("small_bidir_cls_bf16")
    enc = Encoder(dims, stored)
    y_dev = _run(enc, frames).cpu()
    y_host = enc.encode(frames)
    torch.cuda.synchronize()
    assert torch.equal(y_dev, y_host.cpu())
    enc.close()


# ---------------------------------------------------------------------------
# weights as the GEMMs see them
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["small_tubelet2_q8_0", "small_tubelet2_q4_0", "small_bidir_f32",
                                  "small_blockcausal_bf16", "small_q4_k_fallback_head_bf16",
                                  "small_q6_k_rope_blockcausal_f16", "small_q4_k_dh32_cls_bf16"])
def test_dequantised_weights_bit_exact(Encoder, name):
    wl, dims, frames, stored = H.workload_inputs(name)
    enc = Encoder(dims, stored)
    for t in stored:
        shape = (t["ne1"], t["ne0"]) if t["ne1"] > 1 else (t["ne0"],)
        got = enc.dequant(t["name"], shape).cpu().numpy()
        want = Q.stored_to_f64(t).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), t["name"]
    enc.close()


def test_model_bytes_of_a_levjepa_shaped_q8_0_set(Encoder):
    """jepa_model_n_bytes of the LeVJEPA ViT-L/16 shape at q8_0 with an f32
    remainder, minus the pos table the published file does not carry, is the
    LeVJEPA card's 310.3 MiB (within the 0.1 MiB the page rounds to)."""
    import json
    pages = json.load(open(os.path.join(H.GOLDEN, "page_file_sizes.json")))
    from vision_transformer_amd import _lib
    dims = dict(synth.workload("levjepa_vit_l16_16f_bf16_b4")["dims"], act_dtype="f16",
                mat_dtype="q8_0", rest_dtype="f32")
    stored = []
    for name, ne0, ne1 in synth.tensor_specs(dims):
        dt = synth.storage_dtype(dims, name)
        if dt == "q8_0":
            data = np.zeros((ne1, ne0 // 32 * 34), np.uint8)
        else:
            data = np.zeros(ne0 * ne1, np.float32)
        stored.append(dict(name=name, dtype=dt, ne0=ne0, ne1=ne1, data=data))
    enc = Encoder(dims, stored)
    pos = synth.n_tokens(dims) * dims["dim"] * 4
    mib = (_lib.jepa_model_n_bytes(enc.ctx) - pos) / 2 ** 20
    H.say(f"  LeVJEPA-shaped q8_0 model bytes without pos: {mib:.2f} MiB")
    assert abs(mib - pages["levjepa_vitl16_mib"]["q8_0"]) <= pages["tolerance_mib"]
    enc.close()


def test_model_bytes_of_a_vits16_q4_k_set(Encoder):
    """jepa_model_n_bytes of a ViT-S/16 weight set re-typed to q4_K (the
    rows of 384 fall back to q4_0, the 1536-long ffn_down rows stay q4_K)
    with an f32 remainder: the Quantization page's tensor counts per type
    and the tensor-data total they give with the block sizes."""
    import json
    pages = json.load(open(os.path.join(H.GOLDEN, "page_file_sizes.json")))
    v = pages["vits16"]
    from vision_transformer_amd import _lib
    dims = synth._dims(dim=384, depth=12, heads=6, mlp_dim=1536, patch=16, img_h=224,
                       img_w=224, act_dtype="f16", mat_dtype="q4_k", rest_dtype="f32")
    stored, kinds = [], {}
    for name, ne0, ne1 in synth.tensor_specs(dims):
        dt = synth.storage_dtype(dims, name, ne0)
        kinds[dt] = kinds.get(dt, 0) + 1
        data = np.zeros(Q.block_bytes_of(dt)[1] * (ne0 * ne1 // Q.block_bytes_of(dt)[0]), np.uint8) \
            if dt in ("q4_0", "q4_k") else np.zeros(ne0 * ne1, np.float32)
        stored.append(dict(name=name, dtype=dt, ne0=ne0, ne1=ne1, data=data))
    assert kinds["q4_k"] == 12 and kinds["q4_0"] == 36
    enc = Encoder(dims, stored)
    got = _lib.jepa_model_n_bytes(enc.ctx)    # (the page's f32 remainder includes the pos table)
    H.say(f"  ViT-S/16 q4_K set: {got} bytes")
    assert got == v["q4_k_tensor_data_bytes"]
    enc.close()


@pytest.mark.parametrize("name", ["small_q4_k_fallback_head_bf16", "small_q6_k_rope_blockcausal_f16",
                                  "small_tubelet2_q8_0", "small_bidir_f32"])
def test_gguf_file_runs_as_the_in_memory_set(Encoder, name, tmp_path):
    """A weight set written as a GGUF file and read back by
    jepa_create_from_gguf encodes (and classifies) bit for bit as the same
    set given to jepa_create; the model bytes agree with the file's."""
    from vision_transformer_amd import _lib
    H.say(f"gguf {name}")
    wl, dims, frames, stored = H.workload_inputs(name)
    path = str(tmp_path / f"{name}.gguf")
    G.write(path, dims, stored, file_type=G.file_type_codes().get(dims["mat_dtype"]), alignment=64)
    info = _lib.jepa_gguf_read_info(path)
    a = Encoder(dims, stored)
    b = Encoder.from_gguf(path, dims["act_dtype"])
    assert _lib.jepa_model_n_bytes(b.ctx) == _lib.jepa_model_n_bytes(a.ctx) == info["tensor_bytes"]
    ya = _run(a, frames)
    yb = _run(b, frames)
    assert torch.equal(ya, yb)
    if dims["head_classes"]:
        assert torch.equal(a.classify(), b.classify())
    a.close()
    b.close()


def test_k_quant_model_refused_by_noalloc(Encoder):
    from vision_transformer_amd import _lib
    wl, dims, frames, stored = H.workload_inputs("small_q4_k_dh32_cls_bf16")
    enc = Encoder(dims, stored)
    out = torch.empty((1, synth.n_tokens(dims), dims["dim"]), device="cuda")
    with pytest.raises(_lib.JepaError, match="JEPA_E_UNSUPPORTED"):
        _lib.jepa_encode_noalloc(enc.ctx, torch.from_numpy(frames[:1]).cuda(), 1, out)
    enc.close()


def test_failed_encode_forgets_the_previous_token_map(Encoder, monkeypatch):
    """An encode that fails (here: the workspace a larger batch needs is over
    JEPA_MAX_WORKSPACE) leaves no token map behind: pool and classify return
    JEPA_E_STATE instead of reading the previous encode's buffers, and the
    next successful encode works as before."""
    from vision_transformer_amd import _lib
    wl, dims, frames, stored = H.workload_inputs("small_head_bf16")
    enc = Encoder(dims, stored)
    y1 = _run(enc, frames[:1]).cpu()
    enc.pool("mean")
    enc.classify()
    torch.cuda.synchronize()
    big = synth.make_frames(dims, 5, 92)
    monkeypatch.setenv("JEPA_MAX_WORKSPACE", str(_lib.jepa_workspace_bytes(enc.ctx, 1) + 1))
    with pytest.raises(_lib.JepaError, match="JEPA_E_OOM"):
        enc.encode(torch.from_numpy(big).cuda())
    out = torch.empty((1, dims["dim"]), device="cuda")
    with pytest.raises(_lib.JepaError, match="JEPA_E_STATE"):
        _lib.jepa_pool(enc.ctx, "mean", out)
    with pytest.raises(_lib.JepaError, match="JEPA_E_STATE"):
        _lib.jepa_classify(enc.ctx, torch.empty((1, dims["head_classes"]), device="cuda"))
    assert _lib.jepa_last_compute_ms(enc.ctx) < 0
    monkeypatch.delenv("JEPA_MAX_WORKSPACE")
    big[:1] = frames[:1]
    y5 = _run(enc, big).cpu()
    assert torch.equal(y5[:1], y1)
    # outputs sized from a different batch are refused before the call
    with pytest.raises(ValueError):
        enc.pool("mean", 3)
    with pytest.raises(ValueError):
        enc.pool("mean", out=torch.empty((4, dims["dim"]), device="cuda"))
    with pytest.raises(ValueError):
        enc.encode(torch.from_numpy(big[:, :1]).cuda())               # wrong frame count
    enc.close()


def test_pool_before_encode_is_a_state_error(Encoder):
    from vision_transformer_amd import _lib
    wl, dims, frames, stored = H.workload_inputs("small_bidir_f32")
    enc = Encoder(dims, stored)
    with pytest.raises(_lib.JepaError, match="JEPA_E_STATE"):
        enc.pool("cls", 1)
    enc.close()
