"""The C-ABI library on the CPU: it loads, exports every declared entry point,
and its host-side logic (validation, the quantizer, block packing, the rotary
table) is right.
Nothing here launches a GPU kernel."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import encoder as E
from oracle import quant as Q
from vision_transformer_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"\b(jepa_\w+)\s*\(", src)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    from vision_transformer_amd import _lib
    return _lib


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 21
    so = ctypes.CDLL(lib.LIB_PATH)
    for n in names:
        assert hasattr(so, n), n


def test_binding_covers_every_entry_point(lib):
    for n in declared_functions():
        assert callable(getattr(lib, n)), n


@pytest.mark.parametrize("dt", ["q8_0", "q4_0"])
def test_host_quantizer_matches_oracle_bit_exact(lib, dt):
    rng = np.random.default_rng(30)
    x = (rng.standard_normal((257, 1024)) * 0.02).astype(np.float32)
    x[5, 64:96] = 0.0                                    # a zero block
    x[6, :32] = np.linspace(-1, 1, 32, dtype=np.float32)  # exact ties of magnitude
    x[7, :32] = np.float32(3.0)                          # a constant block
    x[8, 32:64] = (np.arange(32) - 16).astype(np.float32)
    np.testing.assert_array_equal(lib.jepa_quantize(dt, x), Q.quantize(dt, x))


@pytest.mark.parametrize("dt", ["q8_0", "q4_0"])
def test_pack_blocks_is_a_pure_split(lib, dt):
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((3, 128)) * 0.02).astype(np.float32)
    raw = Q.quantize(dt, x)
    codes, scales = lib.jepa_pack_blocks(dt, raw, 3, 128)
    bb = Q.block_bytes(dt)
    blk = raw.reshape(-1, bb)
    np.testing.assert_array_equal(scales.view(np.uint8).reshape(-1, 2), blk[:, :2])
    np.testing.assert_array_equal(codes.reshape(-1, bb - 2), blk[:, 2:])


def _small():
    wl = synth.workload("small_bidir_cls_bf16")
    dims = wl["dims"]
    w32 = synth.make_f32_weights(dims, 1)
    return dims, synth.stored_weights(dims, w32)


def _expect_error(lib, status_name, dims, stored):
    with pytest.raises(lib.JepaError) as e:
        lib.jepa_create(dims, stored)
    assert status_name in str(e.value), str(e.value)
    return str(e.value)


def test_create_rejects_a_missing_tensor(lib):
    dims, stored = _small()
    msg = _expect_error(lib, "JEPA_E_MISSING_TENSOR", dims,
                        [t for t in stored if t["name"] != "enc.blk.1.ffn_up.bias"])
    assert "enc.blk.1.ffn_up.bias" in msg


def test_create_rejects_wrong_shape_and_size(lib):
    dims, stored = _small()
    bad = [dict(t) for t in stored]
    bad[0]["ne1"] += 1
    _expect_error(lib, "JEPA_E_SHAPE", dims, bad)
    bad = [dict(t) for t in stored]
    bad[0]["data"] = bad[0]["data"][:-1]
    _expect_error(lib, "JEPA_E_SHAPE", dims, bad)


def test_create_rejects_block_format_outside_the_rule(lib):
    dims, stored = _small()
    bad = [dict(t) for t in stored]
    for t in bad:
        if t["name"] == "enc.blk.0.ln1.weight":
            t["dtype"] = "q8_0"
            t["data"] = Q.quantize("q8_0", np.ones((1, t["ne0"]), np.float32))
    _expect_error(lib, "JEPA_E_DTYPE", dims, bad)


def _retyped(dims, target):
    """The small weight set with every block matrix of row length ne0 stored
    as `target` regardless of the fallback (zero bytes of the right size)."""
    stored = []
    for name, ne0, ne1 in synth.tensor_specs(dims):
        if synth.is_block_matrix(name):
            per, nb = Q.block_bytes_of(target)
            data = np.zeros(ne0 * ne1 // per * nb, np.uint8)
            stored.append(dict(name=name, dtype=target, ne0=ne0, ne1=ne1, data=data))
        else:
            stored.append(dict(name=name, dtype="f32", ne0=ne0, ne1=ne1, data=np.zeros(ne0 * ne1, np.float32)))
    return stored


@pytest.mark.parametrize("dt", ["q4_k", "q6_k"])
def test_create_rejects_k_quant_rows_not_a_multiple_of_256(lib, dt):
    """Quantization page, "The rule": a K-quant needs rows of a multiple of
    256 (D = 192 here); such rows must be stored as q4_0 / q8_0."""
    dims, _ = _small()
    msg = _expect_error(lib, "JEPA_E_SHAPE", dict(dims, act_dtype="f16"), _retyped(dims, dt))
    assert "256" in msg


def test_create_rejects_k_quant_outside_the_rule_and_on_f32(lib):
    dims = synth.workload("small_q4_k_dh32_cls_bf16")["dims"]
    w32 = synth.make_f32_weights(dims, 3)
    stored = synth.stored_weights(dims, w32, quantize=Q.quantize)
    bad = [dict(t) for t in stored]
    for t in bad:
        if t["name"] == "enc.norm.weight":          # a vector
            t["dtype"] = "q4_k"
            t["data"] = Q.quantize("q4_k", np.ones((1, t["ne0"]), np.float32))
    _expect_error(lib, "JEPA_E_DTYPE", dims, bad)
    _expect_error(lib, "JEPA_E_UNSUPPORTED", dict(dims, act_dtype="f32"),
                  synth.stored_weights(dict(dims, rest_dtype="f32"), w32, quantize=Q.quantize))


@pytest.mark.parametrize("name", [n for n, w in synth.SMALL_WORKLOADS.items()
                                  if w["dims"]["mat_dtype"] in ("q4_k", "q6_k")]
                         + ["mid_vitl_q4_k"])
def test_synthetic_k_quant_sets_follow_the_fallback(name):
    """The stored types the workloads hand to both sides are the oracle's
    choice under the fallback rule, and the sizes its block formats give."""
    dims = synth.workload(name)["dims"]
    for tname, ne0, ne1 in synth.tensor_specs(dims):
        if synth.is_block_matrix(tname):
            assert synth.storage_dtype(dims, tname, ne0) == Q.type_for(dims["mat_dtype"], ne0), tname


def test_create_rejects_unknown_and_duplicate_names(lib):
    dims, stored = _small()
    _expect_error(lib, "JEPA_E_INVALID_ARG", dims, stored + [dict(stored[0], name="enc.bogus")])
    _expect_error(lib, "JEPA_E_INVALID_ARG", dims, stored + [stored[0]])


def test_create_rejects_bad_dims(lib):
    dims, stored = _small()
    for change, status in [(dict(heads=2), "JEPA_E_UNSUPPORTED"),      # head_dim 96
                           (dict(img_w=100), "JEPA_E_SHAPE"),          # not a multiple of patch
                           (dict(frames=3, tubelet=2), "JEPA_E_SHAPE"),
                           (dict(ln_eps=0.0), "JEPA_E_INVALID_ARG"),
                           (dict(act_dtype="q8_0"), "JEPA_E_DTYPE")]:
        d = dict(dims, **change)
        _expect_error(lib, status, d, stored)


def test_null_context_calls_fail_cleanly(lib):
    with pytest.raises(lib.JepaError, match="JEPA_E_INVALID_ARG"):
        lib.jepa_encode(None, np.zeros((1, 1, 16, 16, 3), np.uint8), 1)
    with pytest.raises(lib.JepaError, match="JEPA_E_INVALID_ARG"):
        lib.jepa_pool(None, "cls", np.zeros(4, np.float32))
    with pytest.raises(lib.JepaError, match="JEPA_E_INVALID_ARG"):
        lib.jepa_set_batch_parts(None, 2)
    with pytest.raises(lib.JepaError, match="JEPA_E_INVALID_ARG"):
        lib.jepa_set_int8_matmul(None, True)
    assert lib.jepa_last_compute_ms(None) < 0
    assert lib.jepa_model_n_bytes(None) == 0
    lib.jepa_free(None)


# ---------------------------------------------------------------------------
# 3-D rotary position: the host table and the schema
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["vjepa2_vit_l16_64f256_f16", "small_rope_cls_blockcausal_bf16",
                                  "vjepa2_predictor_width_384d_dh32_4096tok_bf16_b4"])
def test_rope_table_is_the_oracle_angles(lib, name):
    """jepa_rope_table's (cos, sin) are the oracle's angles' cos / sin rounded
    to f32 (to within the one ulp by which two libm's may differ)."""
    dims = dict(synth.workload(name)["dims"], rope=1)
    got = lib.jepa_rope_table(dims)
    ang = E.rope_angles(dims)
    dh = dims["dim"] // dims["heads"]
    assert got.shape == (synth.n_tokens(dims), dh // 2, 2)
    np.testing.assert_allclose(got[..., 0], np.cos(ang), rtol=0, atol=1.2e-7)
    np.testing.assert_allclose(got[..., 1], np.sin(ang), rtol=0, atol=1.2e-7)
    rest = 3 * (dh // 6)                       # pairs past the three segments
    assert np.array_equal(got[:, rest:], np.tile(np.float32([1, 0]), (got.shape[0], dh // 2 - rest, 1)))


def test_create_with_rope_has_no_pos_table(lib):
    wl = synth.workload("small_rope_tubelet2_f16")
    dims = wl["dims"]
    stored = synth.stored_weights(dims, synth.make_f32_weights(dims, 1))
    extra = dict(name="enc.pos_embed", dtype="f16", ne0=dims["dim"], ne1=synth.n_tokens(dims),
                 data=np.zeros(dims["dim"] * synth.n_tokens(dims), np.uint16))
    msg = _expect_error(lib, "JEPA_E_INVALID_ARG", dims, stored + [extra])
    assert "enc.pos_embed" in msg
    _expect_error(lib, "JEPA_E_INVALID_ARG", dict(dims, rope=2), stored)
    _expect_error(lib, "JEPA_E_MISSING_TENSOR", dict(dims, rope=0), stored)


def test_create_checks_the_classifier_head_schema(lib):
    wl = synth.workload("small_head_bf16")
    dims = wl["dims"]
    stored = synth.stored_weights(dims, synth.make_f32_weights(dims, 1))
    msg = _expect_error(lib, "JEPA_E_MISSING_TENSOR", dims,
                        [t for t in stored if t["name"] != "head.xattn.attn_v.bias"])
    assert "head.xattn.attn_v.bias" in msg
    _expect_error(lib, "JEPA_E_INVALID_ARG", dict(dims, head_classes=0), stored)   # unknown head tensors
    bad = [dict(t) for t in stored]
    for t in bad:
        if t["name"] == "head.classifier.weight":      # not a block matrix: stays dense
            t["dtype"] = "q8_0"
            t["data"] = Q.quantize("q8_0", np.zeros((t["ne1"], t["ne0"]), np.float32))
    _expect_error(lib, "JEPA_E_DTYPE", dims, bad)
    _expect_error(lib, "JEPA_E_INVALID_ARG", dict(dims, head_blocks=-1), stored)
