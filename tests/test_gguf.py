"""The GGUF reader on the CPU: header, keys and tensor records of written
files read back; general.file_type codes; malformed files refused with a
status, never a crash (every truncation of a file's metadata, corrupted
fields, random byte flips).  Nothing here touches a GPU: jepa_gguf_read_info
is host-only and jepa_create_from_gguf is only called where it must fail
before any device work."""
import os
import struct

import numpy as np
import pytest

from oracle import quant as Q
from tests import gguf_file as G
from vision_transformer_amd import synth


@pytest.fixture(scope="module")
def lib():
    from vision_transformer_amd import _lib
    return _lib


def _weights(name):
    wl = synth.workload(name)
    dims = wl["dims"]
    w32 = synth.make_f32_weights(dims, wl["weight_seed"])
    return dims, synth.stored_weights(dims, w32, quantize=Q.quantize)


def _status(lib, fn, *args):
    try:
        fn(*args)
    except lib.JepaError as e:
        return e.status
    return 0


def test_info_reads_back_what_was_written(lib, tmp_path):
    dims, stored = _weights("small_q4_k_fallback_head_bf16")
    path = str(tmp_path / "m.gguf")
    codes = G.file_type_codes()
    where = G.write(path, dims, stored, file_type=codes["q4_k"])
    info = lib.jepa_gguf_read_info(path)
    d = info["dims"]
    for k in ("dim", "depth", "heads", "mlp_dim", "patch", "tubelet", "img_h", "img_w", "frames",
              "has_cls", "rope", "head_blocks", "head_classes", "mask"):
        assert d[k] == dims[k], k
    assert d["ln_eps"] == np.float32(dims["ln_eps"])
    assert np.array_equal(np.float32(d["mean"]), np.float32(dims["mean"]))
    assert np.array_equal(np.float32(d["std"]), np.float32(dims["std"]))
    assert info["version"] == 3 and info["file_type"] == codes["q4_k"]
    assert info["n_tensors"] == len(stored) and info["n_kv"] == len(G.model_keys(dims, 0))
    assert info["alignment"] == 32 and info["data_offset"] == where["data"]
    assert info["tensor_bytes"] == sum(np.ascontiguousarray(t["data"]).nbytes for t in stored)
    assert lib.jepa_file_type_name(info["file_type"]) == "q4_k"


def test_file_type_codes_are_the_pages(lib):
    codes = G.file_type_codes()
    for name, code in codes.items():
        assert lib.jepa_file_type_name(code) == name
    for code in set(range(64)) - set(codes.values()):
        assert lib.jepa_file_type_name(code) is None


@pytest.mark.parametrize("alignment,version", [(64, 3), (32, 2), (4096, 3)])
def test_alignment_and_version_2(lib, tmp_path, alignment, version):
    dims, stored = _weights("small_tubelet2_q8_0")
    path = str(tmp_path / "m.gguf")
    G.write(path, dims, stored, alignment=alignment, version=version)
    info = lib.jepa_gguf_read_info(path)
    assert info["alignment"] == alignment and info["data_offset"] % alignment == 0
    assert info["version"] == version


def _tiny_blob():
    """A small, complete file (a few tensors, every key) for byte-level tests."""
    dims = synth.workload("small_bidir_cls_bf16")["dims"]
    stored = [dict(name="enc.norm.weight", dtype="f32", ne0=192, ne1=1, data=np.ones(192, np.float32)),
              dict(name="enc.blk.0.ffn_down.weight", dtype="q4_k", ne0=256, ne1=2,
                   data=Q.quantize("q4_k", np.ones((2, 256), np.float32) * 0.01)),
              dict(name="enc.blk.0.attn_out.weight", dtype="q8_0", ne0=64, ne1=3,
                   data=Q.quantize("q8_0", np.ones((3, 64), np.float32) * 0.02))]
    kv = G.model_keys(dims, 12) + [("general.name", G.STR, "tiny"),
                                   ("jepa.labels", G.ARR, (G.STR, ["a", "bb", "ccc"]))]
    blob, where = G.encode(kv, stored)
    return dims, stored, kv, blob, where


def _read_blob(lib, tmp_path, blob, name="x.gguf"):
    path = str(tmp_path / name)
    with open(path, "wb") as f:
        f.write(blob)
    return _status(lib, lib.jepa_gguf_read_info, path)


def test_every_truncation_is_refused(lib, tmp_path):
    _, _, _, blob, where = _tiny_blob()
    assert _read_blob(lib, tmp_path, blob) == 0
    for n in list(range(0, where["data"] + 1)) + [len(blob) - 1]:
        st = _read_blob(lib, tmp_path, blob[:n])
        assert st in (-9, -7, -1), (n, st)      # FORMAT (an empty file too), or its kin
        assert st != 0, n


def _patch(blob, at, fmt, value):
    b = bytearray(blob)
    struct.pack_into(fmt, b, at, value)
    return bytes(b)


def test_corrupted_fields_are_refused(lib, tmp_path):
    dims, stored, kv, blob, where = _tiny_blob()
    rec = where["records"]
    name_len = len(stored[0]["name"].encode())
    nd_at = rec[0] + 8 + name_len                         # record 0: n_dims
    type_at = nd_at + 4 + 8                               # (one dimension)
    off_at = type_at + 4
    cases = {
        "magic": (_patch(blob, 0, "<4s", b"GGUG"), -9),
        "version 1": (_patch(blob, 4, "<I", 1), -7),
        "tensor count": (_patch(blob, 8, "<Q", 1 << 40), -9),
        "n_dims 5": (_patch(blob, nd_at, "<I", 5), -9),
        "n_dims 0": (_patch(blob, nd_at, "<I", 0), -9),
        "dimension 0": (_patch(blob, nd_at + 4, "<Q", 0), -9),
        "unknown type": (_patch(blob, type_at, "<I", 99), -7),
        "misaligned offset": (_patch(blob, off_at, "<Q", 4), -9),
        "offset past the end": (_patch(blob, off_at, "<Q", 1 << 30), -9),
        "string length": (_patch(blob, 24, "<Q", 1 << 62), -9),
        "key value type": (_patch(blob, 24 + 8 + len(b"general.architecture"), "<I", 77), -9),
    }
    for what, (b, want) in cases.items():
        assert _read_blob(lib, tmp_path, b) == want, what


@pytest.mark.parametrize("change,want", [
    (lambda kv: [e for e in kv if e[0] != "jepa.dim"], -9),
    (lambda kv: [e for e in kv if e[0] != "general.architecture"], -9),
    (lambda kv: [("general.architecture", G.STR, "llama")] + kv[1:], -7),
    (lambda kv: [e if e[0] != "jepa.pre.mean" else (e[0], G.ARR, (G.F32, [0.5, 0.5])) for e in kv], -9),
    (lambda kv: [e if e[0] != "jepa.mask" else (e[0], G.STR, "causal") for e in kv], -9),
    (lambda kv: [e if e[0] != "jepa.dim" else (e[0], G.F32, 192.0) for e in kv], -9),
    (lambda kv: kv + [kv[1]], -9),                                  # a key twice
    (lambda kv: kv + [("general.alignment", G.U32, 12)], -9),
])
def test_bad_keys_are_refused(lib, tmp_path, change, want):
    dims, stored, kv, _, _ = _tiny_blob()
    blob, _ = G.encode(change(kv), stored)
    assert _read_blob(lib, tmp_path, blob) == want


def test_random_byte_flips_never_crash(lib, tmp_path):
    _, _, _, blob, where = _tiny_blob()
    rng = np.random.default_rng(5)
    for i in range(400):
        b = bytearray(blob)
        for _ in range(int(rng.integers(1, 4))):
            at = int(rng.integers(0, where["data"]))
            b[at] = int(rng.integers(0, 256))
        assert _read_blob(lib, tmp_path, bytes(b)) in (0, -1, -7, -9)


def test_missing_file_and_null_arguments(lib, tmp_path):
    assert _status(lib, lib.jepa_gguf_read_info, str(tmp_path / "none.gguf")) == -1
    assert _status(lib, lib.jepa_gguf_read_info, str(tmp_path)) == -1       # a directory
    assert _read_blob(lib, tmp_path, b"") == -9


def test_create_from_gguf_refuses_before_device_work(lib, tmp_path):
    """Failures the reader and the schema check find come back before any
    device allocation: a type the library does not run (named), and a
    missing tensor."""
    dims, stored = _weights("small_bidir_cls_bf16")
    path = str(tmp_path / "m.gguf")
    bad = [dict(t) for t in stored]
    i = next(k for k, t in enumerate(bad) if t["name"] == "enc.blk.0.attn_out.weight")
    bad[i] = dict(bad[i], dtype="q4_1", data=np.zeros(bad[i]["ne0"] * bad[i]["ne1"] // 32 * 20, np.uint8))
    G.write(path, dims, bad)
    with pytest.raises(lib.JepaError, match="JEPA_E_UNSUPPORTED.*q4_1"):
        lib.jepa_create_from_gguf(path)
    G.write(path, dims, [t for t in stored if t["name"] != "enc.norm.bias"])
    with pytest.raises(lib.JepaError, match="JEPA_E_MISSING_TENSOR.*enc.norm.bias"):
        lib.jepa_create_from_gguf(path)
