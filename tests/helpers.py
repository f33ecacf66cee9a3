"""Shared test plumbing: build a workload's inputs, move arrays to the GPU,
and the acceptance checks.  Inputs come from the seeded generator; block
formats use the oracle's quantizer; expected values come from the oracle."""
from __future__ import annotations

import hashlib
import os
import sys

import numpy as np

from oracle import encoder as E
from oracle import metrics as M
from oracle import quant as Q
from vision_transformer_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# acceptance bars: f32 paths, every token; reduced-precision paths, the worst token
F32_COS, F32_REL_MAX, LOWP_COS = 0.99999, 1e-3, 0.9995


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def workload_inputs(name: str, ln_affine: bool = False):
    wl = synth.workload(name)
    dims = wl["dims"]
    frames = synth.make_frames(dims, wl["batch"], wl["frame_seed"])
    w32 = synth.make_f32_weights(dims, wl["weight_seed"], ln_affine=ln_affine)
    stored = synth.stored_weights(dims, w32, quantize=Q.quantize)
    return wl, dims, frames, stored


def digest_weights(stored) -> str:
    h = hashlib.sha256()
    for t in stored:
        h.update(t["name"].encode())
        h.update(np.ascontiguousarray(t["data"]).tobytes())
    return h.hexdigest()


def check_rows(act_dtype: str, got: np.ndarray, ref: np.ndarray, what: str) -> dict:
    """Per-row (token) cosine and rel_max against the oracle, with the bar
    that applies to the path's precision."""
    r = M.report(got, ref)
    say(f"  {what}: cos mean {r['cos_mean']:.7f} median {r['cos_median']:.7f} worst {r['cos_worst']:.7f} "
        f"rel_max {r['rel_max']:.3e} rel_fro {r['rel_fro']:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    if act_dtype == "f32":
        assert r["cos_worst"] >= F32_COS, (what, r)
        assert r["rel_max"] <= F32_REL_MAX, (what, r)
    else:
        assert r["cos_worst"] >= LOWP_COS, (what, r)
    return r


def torch_dtype(act: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[act]


def rounded(act: str, x: np.ndarray):
    """x (float) -> (CUDA tensor in act dtype, float64 numpy of the rounded values)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch_dtype(act))
    return t.cuda(), t.to(torch.float64).numpy()


def oracle_tokens(dims, stored, frames):
    return E.encode(dims, E.weights_f64(stored), frames)


def vt_pos(n):
    """Position of token n in a transposed-V row: bits 2 and 3 swapped (each
    aligned run of 16 tokens stored as 0-3, 8-11, 4-7, 12-15)."""
    n = np.asarray(n, dtype=np.int64)
    return (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1)
