"""ctypes binding of libjepa_mi355x.so: one Python function per C entry point
of include/jepa_mi355x.h, with the same name.  Argument marshalling only:
every step of the encoder runs in the library's HIP kernels.  torch supplies
device memory and streams.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

import torch  # noqa: F401  (loads the HIP runtime the library binds to)

_PKG = os.path.dirname(os.path.abspath(__file__))
# JEPA_LIB_PATH selects another build of the library (e.g. the sanitized one)
LIB_PATH = os.environ.get("JEPA_LIB_PATH") or os.path.join(_PKG, "libjepa_mi355x.so")

F32, F16, BF16, Q8_0, Q4_0, Q4_K, Q6_K = 0, 1, 2, 3, 4, 5, 6
DTYPE = {"f32": F32, "f16": F16, "bf16": BF16, "q8_0": Q8_0, "q4_0": Q4_0, "q4_k": Q4_K, "q6_k": Q6_K}
MASK = {"bidir": 0, "block_causal": 1}
POOL = {"none": 0, "cls": 1, "mean": 2}
STATUS = {0: "JEPA_OK", -1: "JEPA_E_INVALID_ARG", -2: "JEPA_E_SHAPE", -3: "JEPA_E_DTYPE",
          -4: "JEPA_E_MISSING_TENSOR", -5: "JEPA_E_OOM", -6: "JEPA_E_HIP",
          -7: "JEPA_E_UNSUPPORTED", -8: "JEPA_E_STATE", -9: "JEPA_E_FORMAT"}


class JepaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class jepa_dims(C.Structure):
    _fields_ = [("dim", C.c_int32), ("depth", C.c_int32), ("heads", C.c_int32),
                ("mlp_dim", C.c_int32), ("patch", C.c_int32), ("tubelet", C.c_int32),
                ("img_h", C.c_int32), ("img_w", C.c_int32), ("frames", C.c_int32),
                ("has_cls", C.c_int32), ("mask", C.c_int32), ("act_dtype", C.c_int32),
                ("ln_eps", C.c_float), ("mean", C.c_float * 3), ("std", C.c_float * 3),
                ("rope", C.c_int32), ("head_blocks", C.c_int32), ("head_classes", C.c_int32)]


class jepa_tensor(C.Structure):
    _fields_ = [("name", C.c_char_p), ("dtype", C.c_int32), ("ne0", C.c_int64),
                ("ne1", C.c_int64), ("data", C.c_void_p), ("nbytes", C.c_size_t)]


class jepa_gguf_info(C.Structure):
    _fields_ = [("dims", jepa_dims), ("version", C.c_int32), ("file_type", C.c_int32),
                ("n_tensors", C.c_int64), ("n_kv", C.c_int64), ("alignment", C.c_int64),
                ("data_offset", C.c_int64), ("tensor_bytes", C.c_int64)]


class jepa_kernel_stat(C.Structure):
    _fields_ = [("name", C.c_char_p), ("launches", C.c_int64), ("total_ms", C.c_double)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m vision_transformer_amd.build` "
                          "(there is no CPU fallback)")
    lib = C.CDLL(LIB_PATH)
    P, I, I64, SZ = C.c_void_p, C.c_int, C.c_int64, C.c_size_t
    sig = {
        "jepa_create": (I, [C.POINTER(jepa_dims), C.POINTER(jepa_tensor), I, C.POINTER(P)]),
        "jepa_encode": (I, [P, P, I, I, P, P]),
        "jepa_encode_noalloc": (I, [P, P, I, P, P]),
        "jepa_pool": (I, [P, I, P, P]),
        "jepa_classify": (I, [P, P, P]),
        "jepa_free": (None, [P]),
        "jepa_last_error": (C.c_char_p, []),
        "jepa_last_compute_ms": (C.c_float, [P]),
        "jepa_model_n_bytes": (SZ, [P]),
        "jepa_device_weight_bytes": (SZ, [P]),
        "jepa_workspace_bytes": (SZ, [P, I]),
        "jepa_dequant_tensor": (I, [P, C.c_char_p, P, P]),
        "jepa_quantize": (I, [I, P, I64, I64, P]),
        "jepa_set_profiling": (I, [P, C.c_uint32]),
        "jepa_set_batch_parts": (I, [P, I]),
        "jepa_set_int8_matmul": (I, [P, I]),
        "jepa_kernel_stats": (I, [P, C.POINTER(jepa_kernel_stat), I]),
        "jepa_reset_kernel_stats": (None, [P]),
        "jepa_op_patchify": (I, [I, P, I, I, I, I, I, I, C.POINTER(C.c_float), C.POINTER(C.c_float), P, I64, P]),
        "jepa_op_layernorm": (I, [P, I64, I, P, P, C.c_float, P, I, P]),
        "jepa_op_gemm": (I, [I, P, I64, I64, P, I, P, I64, P, I, P, I64, P]),
        "jepa_op_quantize_act": (I, [I, P, I64, I64, P, P, P]),
        "jepa_op_gemm_i8": (I, [I, P, P, I64, I64, P, I, P, I64, P, I, P, I64, P]),
        "jepa_op_gemm_qkv": (I, [I, P, I64, I64, P, I, P, I, I, P, I, P, I64, P, I64, P, C.c_float, P]),
        "jepa_op_attention": (I, [I, P, I64, P, I64, I, I, I, I, I, I, I, I, P, P]),
        "jepa_op_transpose_v": (I, [I, P, I, I, I, I, P, I64, P]),
        "jepa_pack_blocks": (I, [I, P, I64, I64, P, P]),
        "jepa_rope_table": (I, [C.POINTER(jepa_dims), P]),
        "jepa_op_mfma_probe": (I, [I, I, I, P, P]),
        "jepa_op_mfma_i8_probe": (I, [I, I, I, P, P]),
        "jepa_op_patch_embed": (I, [I, P, I, I, I, I, I, I, C.POINTER(C.c_float), C.POINTER(C.c_float), P, I64,
                                    I64, P, P, I, P, P]),
        "jepa_gguf_read_info": (I, [C.c_char_p, C.POINTER(jepa_gguf_info)]),
        "jepa_create_from_gguf": (I, [C.c_char_p, I, C.POINTER(P)]),
        "jepa_file_type_name": (C.c_char_p, [I]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def _check(status: int):
    if status != 0:
        raise JepaError(status, _lib.jepa_last_error().decode(errors="replace"))


def _ptr(x) -> int | None:
    """Device (torch) or host (numpy / torch cpu) buffer -> address."""
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        if not x.flags["C_CONTIGUOUS"]:
            raise ValueError("array must be C-contiguous")
        return x.ctypes.data
    if not x.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def make_dims(d: dict) -> jepa_dims:
    return jepa_dims(d["dim"], d["depth"], d["heads"], d["mlp_dim"], d["patch"], d["tubelet"],
                     d["img_h"], d["img_w"], d["frames"], int(d["has_cls"]), MASK[d["mask"]],
                     DTYPE[d["act_dtype"]], float(d["ln_eps"]), (C.c_float * 3)(*d["mean"]),
                     (C.c_float * 3)(*d["std"]), int(d.get("rope", 0)), int(d.get("head_blocks", 0)),
                     int(d.get("head_classes", 0)))


def jepa_create(dims: dict, tensors: list[dict]) -> int:
    """dims: mapping of jepa_dims fields (mask / act_dtype by name); tensors:
    dicts with name, dtype (name), ne0, ne1 and data (a C-contiguous numpy
    array of the raw storage).  Returns the context handle."""
    arr = (jepa_tensor * len(tensors))()
    keep = []
    for i, t in enumerate(tensors):
        data = np.ascontiguousarray(t["data"])
        keep.append(data)
        name = t["name"].encode()
        keep.append(name)
        arr[i] = jepa_tensor(name, DTYPE[t["dtype"]], t["ne0"], t["ne1"], data.ctypes.data, data.nbytes)
    ctx = C.c_void_p()
    d = make_dims(dims)
    _check(_lib.jepa_create(C.byref(d), arr, len(tensors), C.byref(ctx)))
    return ctx.value


def dims_to_dict(d: jepa_dims) -> dict:
    inv_mask = {v: k for k, v in MASK.items()}
    inv_dt = {v: k for k, v in DTYPE.items()}
    return dict(dim=d.dim, depth=d.depth, heads=d.heads, mlp_dim=d.mlp_dim, patch=d.patch,
                tubelet=d.tubelet, img_h=d.img_h, img_w=d.img_w, frames=d.frames,
                has_cls=d.has_cls, mask=inv_mask.get(d.mask, d.mask),
                act_dtype=inv_dt.get(d.act_dtype, d.act_dtype), ln_eps=d.ln_eps,
                mean=tuple(d.mean), std=tuple(d.std), rope=d.rope, head_blocks=d.head_blocks,
                head_classes=d.head_classes)


def jepa_gguf_read_info(path: str) -> dict:
    info = jepa_gguf_info()
    _check(_lib.jepa_gguf_read_info(os.fsencode(path), C.byref(info)))
    return dict(dims=dims_to_dict(info.dims), version=info.version, file_type=info.file_type,
                n_tensors=info.n_tensors, n_kv=info.n_kv, alignment=info.alignment,
                data_offset=info.data_offset, tensor_bytes=info.tensor_bytes)


def jepa_create_from_gguf(path: str, act_dtype: str | None = None) -> int:
    ctx = C.c_void_p()
    _check(_lib.jepa_create_from_gguf(os.fsencode(path), -1 if act_dtype is None else DTYPE[act_dtype],
                                      C.byref(ctx)))
    return ctx.value


def jepa_file_type_name(code: int) -> str | None:
    r = _lib.jepa_file_type_name(code)
    return r.decode() if r is not None else None


def jepa_encode(ctx: int, frames, batch: int, tokens_out=None, stream=None) -> None:
    """frames: uint8 [batch, T, H, W, 3], a CUDA tensor (device) or a numpy
    array / CPU tensor (host).  tokens_out: f32 CUDA tensor [batch, N, D] or None."""
    on_dev = int(hasattr(frames, "is_cuda") and frames.is_cuda)
    _check(_lib.jepa_encode(ctx, _ptr(frames), batch, on_dev, _ptr(tokens_out), _stream(stream)))


# bytes of the static device array jepa_encode_noalloc works in
NOALLOC_SCRATCH_BYTES = 64 << 20


def jepa_encode_noalloc(ctx: int, frames, batch: int, tokens_out, stream=None) -> None:
    """frames: uint8 CUDA tensor [batch, T, H, W, 3]; tokens_out: f32 CUDA
    tensor [batch, N, D] (required).  Allocates nothing on the device."""
    if not (hasattr(frames, "is_cuda") and frames.is_cuda):
        raise ValueError("jepa_encode_noalloc takes frames in device memory")
    _check(_lib.jepa_encode_noalloc(ctx, _ptr(frames), batch, _ptr(tokens_out), _stream(stream)))


def jepa_pool(ctx: int, mode: str | int, out, stream=None) -> None:
    m = POOL[mode] if isinstance(mode, str) else mode
    _check(_lib.jepa_pool(ctx, m, _ptr(out), _stream(stream)))


def jepa_classify(ctx: int, logits_out, stream=None) -> None:
    """Class scores [batch, classes] of the last encode's token map."""
    _check(_lib.jepa_classify(ctx, _ptr(logits_out), _stream(stream)))


def jepa_free(ctx: int) -> None:
    _lib.jepa_free(ctx)


def jepa_last_error() -> str:
    return _lib.jepa_last_error().decode()


def jepa_last_compute_ms(ctx: int) -> float:
    return float(_lib.jepa_last_compute_ms(ctx))


def jepa_model_n_bytes(ctx: int) -> int:
    return int(_lib.jepa_model_n_bytes(ctx))


def jepa_device_weight_bytes(ctx: int) -> int:
    return int(_lib.jepa_device_weight_bytes(ctx))


def jepa_workspace_bytes(ctx: int, batch: int) -> int:
    return int(_lib.jepa_workspace_bytes(ctx, batch))


def jepa_dequant_tensor(ctx: int, name: str, out, stream=None) -> None:
    _check(_lib.jepa_dequant_tensor(ctx, name.encode(), _ptr(out), _stream(stream)))


def jepa_quantize(dtype: str, x: np.ndarray) -> np.ndarray:
    """Host quantizer: f32 [rows, cols] -> uint8 blocks [rows, cols/32*(34|18)]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    bb = {"q8_0": 34, "q4_0": 18}[dtype]
    out = np.empty((rows, cols // 32 * bb), np.uint8)
    _check(_lib.jepa_quantize(DTYPE[dtype], x.ctypes.data, rows, cols, out.ctypes.data))
    return out


def jepa_set_batch_parts(ctx: int, parts: int) -> None:
    """Encode the batch as `parts` concurrent groups of items (0 = default)."""
    _check(_lib.jepa_set_batch_parts(ctx, parts))


def jepa_set_int8_matmul(ctx: int, enable: bool) -> None:
    """Run q8_0 / q4_0 products on int8 MFMA with quantised inputs (or not)."""
    _check(_lib.jepa_set_int8_matmul(ctx, 1 if enable else 0))


def jepa_set_profiling(ctx: int, class_mask: int) -> None:
    """class_mask: bit i times kernel class i (0 = off, 0xffffffff = all)."""
    _check(_lib.jepa_set_profiling(ctx, class_mask & 0xFFFFFFFF))


def jepa_kernel_stats(ctx: int) -> dict:
    cap = 64
    buf = (jepa_kernel_stat * cap)()
    n = _lib.jepa_kernel_stats(ctx, buf, cap)
    if n < 0:
        _check(n)
    return {buf[i].name.decode(): dict(launches=buf[i].launches, total_ms=buf[i].total_ms)
            for i in range(min(n, cap))}


def jepa_reset_kernel_stats(ctx: int) -> None:
    _lib.jepa_reset_kernel_stats(ctx)


# ---------------------------------------------------------------------------
# single kernels (include/jepa_mi355x_ops.h)
# ---------------------------------------------------------------------------
EPI = {"store": 0, "gelu": 1, "resid": 2}


def jepa_op_patchify(act_dtype: str, frames, tubelet: int, patch: int, mean, std, out, ld: int,
                     stream=None) -> None:
    B, T, H, W, _ = frames.shape
    m = (C.c_float * 3)(*mean)
    sd = (C.c_float * 3)(*std)
    _check(_lib.jepa_op_patchify(DTYPE[act_dtype], _ptr(frames), B, T, H, W, tubelet, patch, m, sd,
                                 _ptr(out), ld, _stream(stream)))


def jepa_op_layernorm(x, gamma, beta, eps: float, y, y_dtype: str, stream=None) -> None:
    rows, dim = x.shape
    _check(_lib.jepa_op_layernorm(_ptr(x), rows, dim, _ptr(gamma), _ptr(beta), eps, _ptr(y),
                                  DTYPE[y_dtype], _stream(stream)))


def jepa_op_gemm(act_dtype: str, a, w, w_dtype: str, n: int, bias, epilogue: str, out,
                 w_scale=None, stream=None) -> None:
    M, K = a.shape
    _check(_lib.jepa_op_gemm(DTYPE[act_dtype], _ptr(a), M, K, _ptr(w), DTYPE[w_dtype], _ptr(w_scale),
                             n, _ptr(bias), EPI[epilogue], _ptr(out), out.shape[1], _stream(stream)))


def jepa_op_quantize_act(act_dtype: str, x, codes_out, scales_out, stream=None) -> None:
    """x act [rows, k] -> codes_out int8 [rows, k], scales_out f32 [rows, k/32]."""
    rows, k = x.shape
    _check(_lib.jepa_op_quantize_act(DTYPE[act_dtype], _ptr(x), rows, k, _ptr(codes_out), _ptr(scales_out),
                                     _stream(stream)))


def jepa_op_gemm_i8(act_dtype: str, a_codes, a_scales, w, w_dtype: str, n: int, bias, epilogue: str, out,
                    w_scale, stream=None) -> None:
    M, K = a_codes.shape
    _check(_lib.jepa_op_gemm_i8(DTYPE[act_dtype], _ptr(a_codes), _ptr(a_scales), M, K, _ptr(w),
                                DTYPE[w_dtype], _ptr(w_scale), n, _ptr(bias), EPI[epilogue], _ptr(out),
                                out.shape[1], _stream(stream)))


def jepa_op_gemm_qkv(act_dtype: str, a, w, w_dtype: str, heads: int, bias, n_tokens: int, qk_out, vt,
                     w_scale=None, q_scale: float = 0.0, rope=None, head_dim: int = 64,
                     stream=None) -> None:
    """q, k columns -> qk_out [M, ld] (rotated by the rope table [n_tokens,
    head_dim/2, 2] if given, then q times q_scale if nonzero); v columns
    transposed -> vt [M/n_tokens, heads*head_dim, npad]."""
    M, K = a.shape
    _check(_lib.jepa_op_gemm_qkv(DTYPE[act_dtype], _ptr(a), M, K, _ptr(w), DTYPE[w_dtype], _ptr(w_scale),
                                 heads, head_dim, _ptr(bias), n_tokens, _ptr(qk_out), qk_out.shape[1],
                                 _ptr(vt), vt.shape[-1], _ptr(rope), float(q_scale), _stream(stream)))


def jepa_rope_table(dims: dict) -> np.ndarray:
    """Host: the 3-D rotary table of dims' token grid, f32 [N, dh/2, 2] (cos, sin)."""
    d = make_dims(dims)
    n = (dims["frames"] // dims["tubelet"]) * (dims["img_h"] // dims["patch"]) * \
        (dims["img_w"] // dims["patch"]) + int(dims["has_cls"])
    out = np.empty((n, dims["dim"] // dims["heads"] // 2, 2), np.float32)
    _check(_lib.jepa_rope_table(C.byref(d), out.ctypes.data))
    return out


# log2(e) / sqrt(head_dim): JEPA_ATTN_Q_SCALE and _32, the factor
# jepa_op_gemm_qkv folds into q
ATTN_Q_SCALE = 0.18033688011112042
ATTN_Q_SCALE_32 = 0.25503486164919736


def attn_q_scale(head_dim: int) -> float:
    return ATTN_Q_SCALE_32 if head_dim == 32 else ATTN_Q_SCALE


def jepa_op_attention(act_dtype: str, qk, vt, batch: int, n_tokens: int, heads: int, has_cls: bool,
                      mask: str, tokens_per_slot: int, out, q_prescaled: bool = False, head_dim: int = 64,
                      stream=None) -> None:
    """qk: [batch*n_tokens, ld] (q | k columns first; q times
    attn_q_scale(head_dim) if q_prescaled); vt: [batch, heads*head_dim, npad]."""
    _check(_lib.jepa_op_attention(DTYPE[act_dtype], _ptr(qk), qk.shape[1], _ptr(vt), vt.shape[-1],
                                  batch, n_tokens, heads, head_dim, int(has_cls), MASK[mask], tokens_per_slot,
                                  int(q_prescaled), _ptr(out), _stream(stream)))


def jepa_op_transpose_v(act_dtype: str, qkv, batch: int, n_tokens: int, heads: int, vt,
                        head_dim: int = 64, stream=None) -> None:
    _check(_lib.jepa_op_transpose_v(DTYPE[act_dtype], _ptr(qkv), batch, n_tokens, heads, head_dim,
                                    _ptr(vt), vt.shape[-1], _stream(stream)))


def jepa_op_mfma_probe(workgroups: int, iters: int, out, operands: int = 0, stream=None) -> int:
    """Dense bf16 MFMA calibration launch (operands 0: constant, 1: random);
    returns its flops."""
    _check(_lib.jepa_op_mfma_probe(workgroups, iters, operands, _ptr(out), _stream(stream)))
    return workgroups * 4 * iters * 8 * 32 * 32 * 16 * 2


def jepa_op_patch_embed(act_dtype: str, frames, tubelet: int, patch: int, mean, std, w, bias, pos,
                        has_cls: bool, out, stream=None) -> None:
    """Patch embedding gathered from device frames [B, T, H, W, 3]; w [n, k_pitch]; out f32 [B, N_tok, n]."""
    B, T, H, W, _ = frames.shape
    m = (C.c_float * 3)(*mean)
    sd = (C.c_float * 3)(*std)
    _check(_lib.jepa_op_patch_embed(DTYPE[act_dtype], _ptr(frames), B, T, H, W, tubelet, patch, m, sd, _ptr(w),
                                    w.shape[1], w.shape[0], _ptr(bias), _ptr(pos), int(has_cls), _ptr(out),
                                    _stream(stream)))


def jepa_op_mfma_i8_probe(workgroups: int, iters: int, mode: int, out, stream=None) -> int:
    """int8 MFMA calibration launch (mode 0 plain, 1 / 2 rescaled); returns its ops."""
    _check(_lib.jepa_op_mfma_i8_probe(workgroups, iters, mode, _ptr(out), _stream(stream)))
    return workgroups * 4 * iters * 4 * 32 * 32 * 32 * 2


def jepa_pack_blocks(dtype: str, blocks: np.ndarray, rows: int, cols: int):
    """Host: blocks -> (codes uint8, scales uint16) in the GEMM's device layout."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    ncode = rows * cols if dtype == "q8_0" else rows * cols // 2
    codes = np.empty(ncode, np.uint8)
    scales = np.empty(rows * cols // 32, np.uint16)
    _check(_lib.jepa_pack_blocks(DTYPE[dtype], blocks.ctypes.data, rows, cols, codes.ctypes.data,
                                 scales.ctypes.data))
    return codes, scales
