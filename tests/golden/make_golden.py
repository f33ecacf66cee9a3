"""Write the oracle's expected outputs for the full-size workloads.

Runs the CPU oracle (float64) on the seeded synthetic inputs of each
full-size workload and stores, per workload, a small .npz:
  * the pooled features the workload reports (CLS rows and/or mean pools);
  * a deterministic sample of token rows of the final token map;
  * sha256 digests of the frames and of the stored weight bytes, so a test
    can confirm it regenerated the same inputs;
  * the spread of the per-token standard deviation before the final
    LayerNorm (the jepa.cpp Quantization page ties the worst tokens to the
    smallest such spread; reported, not compared).
Everything here comes from the oracle; nothing is read from the HIP path.

usage: python tests/golden/make_golden.py [workload ...]
"""
from __future__ import annotations

import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import encoder as E          # noqa: E402
from oracle import quant as Q            # noqa: E402
from vision_transformer_amd import synth  # noqa: E402

FULL = ["vit_l16_image_bf16_b32", "levjepa_vit_l16_16f_bf16_b4",
        "vjepa2_vit_l16_16f256_q8_0_b4", "vjepa2_vit_l16_64f256_f16",
        "vjepa2_vit_l16_64f256_q4_0", "vjepa2_rope_vit_l16_16f256_f16_b4",
        "vjepa2_predictor_width_384d_dh32_4096tok_bf16_b4", "vjepa2_ssv2_classifier_vit_l16_16f256_f16_b4"]
N_SAMPLE = 32


def digest_weights(stored) -> str:
    h = hashlib.sha256()
    for t in stored:
        h.update(t["name"].encode())
        h.update(np.ascontiguousarray(t["data"]).tobytes())
    return h.hexdigest()


def sample_rows(dims, batch, seed=777):
    """Deterministic (item, token) pairs covering every part of the token map
    that a kernel tile or a mask boundary could get wrong on its own:
      * the first and last token of the first and last item;
      * every item's CLS row (when the model has one);
      * one row drawn uniformly inside every 256-row block of the batch's
        flattened rows (b * N + n), the GEMMs' largest row tile;
      * one patch token drawn uniformly inside every (item, temporal slot);
      * uniform draws up to at least 32 rows."""
    N = synth.n_tokens(dims)
    has_cls = int(dims["has_cls"])
    per_slot = synth.grid(dims)[1] * synth.grid(dims)[2]
    n_slots = synth.grid(dims)[0]
    rng = np.random.default_rng(seed)
    pairs = {(0, 0), (0, N - 1), (batch - 1, 0), (batch - 1, N - 1)}
    if has_cls:
        pairs |= {(b, 0) for b in range(batch)}
    M = batch * N
    for r0 in range(0, M, 256):
        r = int(rng.integers(r0, min(M, r0 + 256)))
        pairs.add((r // N, r % N))
    for b in range(batch):
        for t in range(n_slots):
            pairs.add((b, has_cls + t * per_slot + int(rng.integers(per_slot))))
    while len(pairs) < N_SAMPLE:
        pairs.add((int(rng.integers(batch)), int(rng.integers(N))))
    return np.array(sorted(pairs), dtype=np.int64)


def inputs(name):
    wl = synth.workload(name)
    dims = wl["dims"]
    frames = synth.make_frames(dims, wl["batch"], wl["frame_seed"])
    w32 = synth.make_f32_weights(dims, wl["weight_seed"])
    stored = synth.stored_weights(dims, w32, quantize=Q.quantize)
    return wl, dims, frames, stored


def make(name):
    t0 = time.time()
    wl, dims, frames, stored = inputs(name)
    weights_sha = digest_weights(stored)
    w = E.weights_f64(stored)
    del stored
    y, x = E.encode(dims, w, frames, return_pre_norm=True)
    rows = sample_rows(dims, wl["batch"])
    out = dict(rows=rows, sampled=y[rows[:, 0], rows[:, 1]].astype(np.float32),
               frames_sha256=np.array(hashlib.sha256(frames.tobytes()).hexdigest()))
    out["weights_sha256"] = np.array(weights_sha)
    if dims["has_cls"]:
        out["cls"] = E.pool(y, "cls", True).astype(np.float32)
    out["mean"] = E.pool(y, "mean", bool(dims["has_cls"])).astype(np.float32)
    if dims.get("head_classes"):
        from oracle import head as HD
        out["logits"] = HD.classify(dims, w, y).astype(np.float32)
    sd = np.std(x, axis=-1)
    out["pre_norm_std_min_median_max"] = np.array([sd.min(), np.median(sd), sd.max()])
    path = os.path.join(HERE, f"{name}.npz")
    np.savez_compressed(path, **out)
    print(f"{name}: {time.time() - t0:.1f} s -> {os.path.relpath(path, ROOT)}", flush=True)


if __name__ == "__main__":
    for n in sys.argv[1:] or FULL:
        make(n)
