"""An owning wrapper around one jepa_ctx."""
from __future__ import annotations

import torch

from . import _lib
from . import synth


class Encoder:
    """Weights resident on the current GPU; encode() and pool() enqueue on a
    torch stream (the current one by default)."""

    def __init__(self, dims: dict, tensors: list[dict]):
        self.dims = dict(dims)
        self.n_tokens = synth.n_tokens(dims)
        self.ctx = _lib.jepa_create(dims, tensors)

    def close(self):
        if getattr(self, "ctx", None):
            _lib.jepa_free(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def encode(self, frames, tokens_out=None, stream=None):
        """frames: uint8 [B, T, H, W, 3] (CUDA tensor, or host numpy).  Returns
        tokens_out (allocated if None): f32 [B, N, D] on the GPU."""
        B = frames.shape[0]
        if tokens_out is None:
            tokens_out = torch.empty((B, self.n_tokens, self.dims["dim"]), dtype=torch.float32,
                                     device="cuda")
        _lib.jepa_encode(self.ctx, frames, B, tokens_out, stream)
        return tokens_out

    def pool(self, mode: str, batch: int, out=None, stream=None):
        if out is None:
            shape = (batch, self.n_tokens, self.dims["dim"]) if mode == "none" else (batch, self.dims["dim"])
            out = torch.empty(shape, dtype=torch.float32, device="cuda")
        _lib.jepa_pool(self.ctx, mode, out, stream)
        return out

    def classify(self, batch: int, out=None, stream=None):
        """Class scores f32 [batch, head_classes] of the last encode's tokens."""
        if out is None:
            out = torch.empty((batch, self.dims["head_classes"]), dtype=torch.float32, device="cuda")
        _lib.jepa_classify(self.ctx, out, stream)
        return out

    def dequant(self, name: str, shape, stream=None):
        out = torch.empty(shape, dtype=torch.float32, device="cuda")
        _lib.jepa_dequant_tensor(self.ctx, name, out, stream)
        return out

    def last_compute_ms(self) -> float:
        return _lib.jepa_last_compute_ms(self.ctx)

    def model_n_bytes(self) -> int:
        return _lib.jepa_model_n_bytes(self.ctx)
