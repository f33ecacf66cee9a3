"""An owning wrapper around one jepa_ctx."""
from __future__ import annotations

import numpy as np
import torch

from . import _lib
from . import synth


class Encoder:
    """Weights resident on the current GPU; encode() and pool() enqueue on a
    torch stream (the current one by default).

    The library's pool() and classify() read the token map where the last
    encode() wrote it, so the wrapper keeps that tensor alive until the next
    encode, and sizes their outputs from that encode's batch."""

    def __init__(self, dims: dict, tensors: list[dict]):
        self.dims = dict(dims)
        self.n_tokens = synth.n_tokens(dims)
        self.ctx = _lib.jepa_create(dims, tensors)
        self._last_tokens = None
        self.last_batch = 0

    @classmethod
    def from_gguf(cls, path: str, act_dtype: str | None = None) -> "Encoder":
        """A model read from a GGUF file (dims from its keys; act_dtype None
        lets the library choose from the stored types)."""
        info = _lib.jepa_gguf_read_info(path)
        self = cls.__new__(cls)
        self.dims = dict(info["dims"], act_dtype=act_dtype)
        self.n_tokens = synth.n_tokens(self.dims)
        self._last_tokens = None
        self.last_batch = 0
        self.ctx = _lib.jepa_create_from_gguf(path, act_dtype)
        return self

    def close(self):
        if getattr(self, "ctx", None):
            _lib.jepa_free(self.ctx)
            self.ctx = None
        self._last_tokens = None
        self.last_batch = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _frame_shape(self, batch: int) -> tuple:
        d = self.dims
        return (batch, d["frames"], d["img_h"], d["img_w"], 3)

    def encode(self, frames, tokens_out=None, stream=None):
        """frames: uint8 [B, T, H, W, 3] (CUDA tensor, or host numpy / CPU
        tensor).  Returns tokens_out (allocated if None): f32 [B, N, D] on the
        GPU.  The tensor stays referenced here until the next encode."""
        B = int(frames.shape[0])
        if tuple(frames.shape) != self._frame_shape(B):
            raise ValueError(f"frames shape {tuple(frames.shape)}, expected {self._frame_shape(B)}")
        is_uint8 = frames.dtype == torch.uint8 if isinstance(frames, torch.Tensor) else frames.dtype == np.uint8
        if not is_uint8:
            raise ValueError(f"frames dtype {frames.dtype}, expected uint8")
        want = (B, self.n_tokens, self.dims["dim"])
        if tokens_out is None:
            tokens_out = torch.empty(want, dtype=torch.float32, device="cuda")
        elif (tuple(tokens_out.shape) != want or tokens_out.dtype != torch.float32
              or not tokens_out.is_cuda):
            raise ValueError(f"tokens_out must be a CUDA f32 tensor of shape {want}")
        # the previous token map is forgotten as soon as the call starts
        self._last_tokens = None
        self.last_batch = 0
        _lib.jepa_encode(self.ctx, frames, B, tokens_out, stream)
        self._last_tokens = tokens_out
        self.last_batch = B
        return tokens_out

    def _check_batch(self, batch):
        if self.last_batch == 0:
            return 0          # the library reports JEPA_E_STATE
        if batch is not None and batch != self.last_batch:
            raise ValueError(f"batch {batch} differs from the last encode's {self.last_batch}")
        return self.last_batch

    @staticmethod
    def _check_out(out, shape):
        if tuple(out.shape) != shape or out.dtype != torch.float32 or not out.is_cuda:
            raise ValueError(f"out must be a CUDA f32 tensor of shape {shape}")

    def pool(self, mode: str, batch: int | None = None, out=None, stream=None):
        """Pool the last encode's token map: [B, D] (cls, mean) or [B, N, D]
        (none).  batch, if given, must equal the last encode's."""
        B = self._check_batch(batch)
        shape = (B, self.n_tokens, self.dims["dim"]) if mode == "none" else (B, self.dims["dim"])
        if out is None:
            out = torch.empty((max(B, 1),) + shape[1:], dtype=torch.float32, device="cuda")
        elif B:
            self._check_out(out, shape)
        _lib.jepa_pool(self.ctx, mode, out, stream)
        return out

    def classify(self, batch: int | None = None, out=None, stream=None):
        """Class scores f32 [B, head_classes] of the last encode's tokens."""
        B = self._check_batch(batch)
        shape = (B, self.dims["head_classes"])
        if out is None:
            out = torch.empty((max(B, 1), shape[1]), dtype=torch.float32, device="cuda")
        elif B:
            self._check_out(out, shape)
        _lib.jepa_classify(self.ctx, out, stream)
        return out

    def set_int8_matmul(self, enable: bool) -> None:
        """q8_0 / q4_0 products on int8 MFMA with inputs quantised per
        32-block (enable), or on dequantised weights (the default).  A change
        frees the library's workspace and with it the last encode's state."""
        enable = bool(enable)
        if enable != getattr(self, "int8_matmul", False):
            _lib.jepa_set_int8_matmul(self.ctx, enable)
            self._last_tokens = None
            self.last_batch = 0
        self.int8_matmul = enable

    def dequant(self, name: str, shape, stream=None):
        out = torch.empty(shape, dtype=torch.float32, device="cuda")
        _lib.jepa_dequant_tensor(self.ctx, name, out, stream)
        return out

    def last_compute_ms(self) -> float:
        return _lib.jepa_last_compute_ms(self.ctx)

    def model_n_bytes(self) -> int:
        return _lib.jepa_model_n_bytes(self.ctx)
