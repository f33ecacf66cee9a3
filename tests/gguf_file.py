"""A GGUF writer for the tests: a synthetic weight set as the file the
library's reader takes (container layout and keys as include/jepa_mi355x.h
states them), plus byte-level access for the malformed-file tests.

Tensor data are the stored bytes as they are (the block formats' bytes are
ggml's own layouts), so a file and the in-memory jepa_create call see the
same weights."""
from __future__ import annotations

import json
import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# ggml tensor type ids
GGML_TYPE = {"f32": 0, "f16": 1, "q4_0": 2, "q4_1": 3, "q5_0": 6, "q5_1": 7, "q8_0": 8,
             "q4_k": 12, "q5_k": 13, "q6_k": 14, "bf16": 30}
# GGUF value types
U8, I8, U16, I16, U32, I32, F32, BOOL, STR, ARR, U64, I64, F64 = range(13)


def file_type_codes() -> dict:
    """general.file_type per requested type, as the Quantization page prints them."""
    return json.load(open(os.path.join(GOLDEN, "page_file_sizes.json")))["file_type_codes"]


def _str(s: str) -> bytes:
    b = s.encode()
    return struct.pack("<Q", len(b)) + b


def _value(vtype: int, v) -> bytes:
    fmt = {U8: "<B", I8: "<b", U16: "<H", I16: "<h", U32: "<I", I32: "<i", F32: "<f",
           BOOL: "<B", U64: "<Q", I64: "<q", F64: "<d"}
    if vtype == STR:
        return _str(v)
    if vtype == ARR:
        etype, items = v
        out = struct.pack("<IQ", etype, len(items))
        for x in items:
            out += _value(etype, x)
        return out
    return struct.pack(fmt[vtype], v)


def model_keys(dims: dict, file_type: int | None = None) -> list:
    """(key, value type, value) for a model's dims."""
    kv = [("general.architecture", STR, "jepa")]
    if file_type is not None:
        kv.append(("general.file_type", U32, file_type))
    for k in ("dim", "depth", "heads", "mlp_dim", "patch", "tubelet", "img_h", "img_w", "frames"):
        kv.append((f"jepa.{k}", U32, int(dims[k])))
    kv.append(("jepa.has_cls", BOOL, int(dims["has_cls"])))
    kv.append(("jepa.mask", STR, "block_causal" if dims["mask"] == "block_causal" else "bidirectional"))
    kv.append(("jepa.ln_eps", F32, float(dims["ln_eps"])))
    kv.append(("jepa.rope", BOOL, int(dims.get("rope", 0))))
    kv.append(("jepa.head.blocks", U32, int(dims.get("head_blocks", 0))))
    kv.append(("jepa.head.classes", U32, int(dims.get("head_classes", 0))))
    kv.append(("jepa.pre.mean", ARR, (F32, [float(x) for x in dims["mean"]])))
    kv.append(("jepa.pre.std", ARR, (F32, [float(x) for x in dims["std"]])))
    return kv


def encode(kv: list, stored: list, alignment: int = 32, version: int = 3) -> tuple[bytes, dict]:
    """The file's bytes and where its parts start (header end, each tensor
    record, data section)."""
    head = b"GGUF" + struct.pack("<IQQ", version, len(stored), len(kv))
    for key, vtype, v in kv:
        head += _str(key) + struct.pack("<I", vtype) + _value(vtype, v)
    where = {"kv_end": len(head), "records": []}
    offsets, off = [], 0
    for t in stored:
        nb = np.ascontiguousarray(t["data"]).nbytes
        offsets.append(off)
        off = (off + nb + alignment - 1) // alignment * alignment
    for t, o in zip(stored, offsets):
        where["records"].append(len(head))
        dims = [t["ne0"]] if t["ne1"] == 1 else [t["ne0"], t["ne1"]]
        head += _str(t["name"]) + struct.pack("<I", len(dims))
        head += b"".join(struct.pack("<Q", d) for d in dims)
        head += struct.pack("<IQ", GGML_TYPE[t["dtype"]], o)
    data_start = (len(head) + alignment - 1) // alignment * alignment
    where["data"] = data_start
    body = bytearray(head + b"\0" * (data_start - len(head)))
    for t, o in zip(stored, offsets):
        raw = np.ascontiguousarray(t["data"]).tobytes()
        body += b"\0" * (data_start + o - len(body))
        body += raw
    return bytes(body), where


def write(path: str, dims: dict, stored: list, file_type: int | None = None, alignment: int = 32,
          extra_kv: list = (), version: int = 3) -> dict:
    kv = model_keys(dims, file_type)
    if alignment != 32:
        kv.append(("general.alignment", U32, alignment))
    kv += list(extra_kv)
    blob, where = encode(kv, stored, alignment, version)
    with open(path, "wb") as f:
        f.write(blob)
    return where
