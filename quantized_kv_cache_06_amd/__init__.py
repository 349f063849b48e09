"""Python binding of libkvq, the quantized KV cache library for MI355X.

Thin ctypes layer with the C entry points' names; it marshals arguments and
checks buffer sizes, and runs no part of the computation. Device buffers may
be given as torch tensors (on the GPU, contiguous) or as integer addresses.
The shared library is built in-tree by ``build.build()``; importing works
without it, but the first call raises if ``libkvq.so`` is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "FMT_FP8_E4M3", "FMT_INT8", "FMT_KIVI", "FMT_BF16", "FMT_INT4", "FMT_FP8_STATIC", "FMT_INT4_HADAMARD", "FMT_KIVI_F16", "DT_F32",
    "DT_BF16",
    "KvqConfig", "KvqLayout", "KvqError", "LIB_PATH", "lib", "make_config",
    "kvq_status_string", "kvq_version", "kvq_get_layout", "kvq_quantize_append",
    "kvq_decode_workspace_bytes", "kvq_decode_attention", "kvq_append_decode", "kvq_append_decode_noalloc",
    "STATIC_WORKSPACE_BYTES",
]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

FMT_FP8_E4M3, FMT_INT8, FMT_KIVI, FMT_BF16, FMT_INT4, FMT_FP8_STATIC, FMT_INT4_HADAMARD, FMT_KIVI_F16 = range(1, 9)
DT_F32, DT_BF16 = 0, 1
OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
STATIC_WORKSPACE_BYTES = 64 << 20  # KVQ_STATIC_WORKSPACE_BYTES of include/kvq.h


class KvqConfig(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "format", "bits", "group", "residual", "batch", "n_kv_heads", "n_q_heads",
        "head_dim", "max_tokens", "in_dtype")]


class KvqLayout(ctypes.Structure):
    _fields_ = [(name, ctypes.c_uint64) for name in (
        "total_bytes", "k_codes_off", "v_codes_off", "k_scale_off", "v_scale_off",
        "k_zero_off", "v_zero_off", "k_resid_off", "v_resid_off")] + [
        (name, ctypes.c_int32) for name in ("token_capacity", "resid_slots", "row_bytes", "elem_bytes")]


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {kvq_status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkvq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libkvq.so not found at {LIB_PATH}; build it with "
                               "quantized_kv_cache_06_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        cfgp = ctypes.POINTER(KvqConfig)
        L.kvq_status_string.argtypes = [ctypes.c_int32]
        L.kvq_status_string.restype = ctypes.c_char_p
        L.kvq_version.argtypes = []
        L.kvq_version.restype = ctypes.c_int32
        L.kvq_get_layout.argtypes = [cfgp, ctypes.POINTER(KvqLayout)]
        L.kvq_get_layout.restype = ctypes.c_int32
        L.kvq_quantize_append.argtypes = [cfgp, P, P, P, P, ctypes.c_int32, P, P, P]
        L.kvq_quantize_append.restype = ctypes.c_int32
        L.kvq_decode_workspace_bytes.argtypes = [cfgp, ctypes.c_int32, ctypes.POINTER(ctypes.c_uint64)]
        L.kvq_decode_workspace_bytes.restype = ctypes.c_int32
        L.kvq_decode_attention.argtypes = [cfgp, P, P, P, ctypes.c_float, P, P, ctypes.c_uint64,
                                           ctypes.c_int32, P]
        L.kvq_decode_attention.restype = ctypes.c_int32
        L.kvq_append_decode.argtypes = [cfgp, P, P, P, P, P, ctypes.c_float, P, P, ctypes.c_uint64,
                                        ctypes.c_int32, P, P]
        L.kvq_append_decode.restype = ctypes.c_int32
        L.kvq_append_decode_noalloc.argtypes = [cfgp, P, P, P, P, P, ctypes.c_float, P, ctypes.c_int32, P, P]
        L.kvq_append_decode_noalloc.restype = ctypes.c_int32
        _lib = L
    return _lib


def make_config(fmt: int, bits: int, group: int, residual: int, batch: int, n_kv_heads: int,
                n_q_heads: int, head_dim: int, max_tokens: int, in_dtype: int) -> KvqConfig:
    return KvqConfig(fmt, bits, group, residual, batch, n_kv_heads, n_q_heads, head_dim, max_tokens, in_dtype)


def _check(status: int, where: str) -> None:
    if status != OK:
        raise KvqError(status, where)


def _check_types(*args) -> None:
    """(tensor, element type, name) triples: raises ValueError for a tensor
    of another element type. None and raw integer addresses pass. Every
    entry point runs this before it takes any address, so a wrong type is
    reported whatever the device."""
    for x, dtype, what in args:
        if x is None or isinstance(x, int):
            continue
        if x.dtype != dtype:
            raise ValueError(f"{what} must be {dtype}, got {x.dtype}")


def _addr(x, min_bytes: Optional[int] = None, what: str = "buffer") -> Optional[int]:
    """Device address of a tensor or integer; None stays NULL. For tensors,
    checks device residency, contiguity and (when given) the byte size. Raw
    integer addresses are passed unchecked."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not getattr(x, "is_cuda", False):
        raise ValueError(f"{what} must be a GPU tensor")
    if not x.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if min_bytes is not None and x.numel() * x.element_size() < min_bytes:
        raise ValueError(f"{what} holds {x.numel() * x.element_size()} bytes, needs {min_bytes}")
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def kvq_status_string(status: int) -> str:
    return lib().kvq_status_string(int(status)).decode()


def kvq_version() -> int:
    return lib().kvq_version()


def kvq_get_layout(cfg: KvqConfig) -> KvqLayout:
    out = KvqLayout()
    _check(lib().kvq_get_layout(ctypes.byref(cfg), ctypes.byref(out)), "kvq_get_layout")
    return out


def _elem(cfg: KvqConfig) -> int:
    return 2 if cfg.in_dtype == DT_BF16 else 4


def _in_dtype(cfg: KvqConfig):
    """torch element type of K/V inputs and q for cfg.in_dtype."""
    import torch
    return torch.bfloat16 if cfg.in_dtype == DT_BF16 else torch.float32


def _i32():
    import torch
    return torch.int32


def _f32():
    import torch
    return torch.float32


def kvq_quantize_append(cfg: KvqConfig, cache, seq_lens, k_new, v_new, t_new: int,
                        append_lens=None, skipped=None, stream=None) -> None:
    """Quantize and append t_new tokens per sequence (see include/kvq.h).
    skipped: optional int32 [B] device tensor, set to 1 for each sequence the
    append leaves unchanged (over capacity or a malformed length), else 0."""
    _check_types((seq_lens, _i32(), "seq_lens"), (k_new, _in_dtype(cfg), "k_new"),
                 (v_new, _in_dtype(cfg), "v_new"), (append_lens, _i32(), "append_lens"),
                 (skipped, _i32(), "skipped"))
    lay = kvq_get_layout(cfg)
    n_in = cfg.batch * cfg.n_kv_heads * t_new * cfg.head_dim * _elem(cfg)
    st = lib().kvq_quantize_append(
        ctypes.byref(cfg), _addr(cache, lay.total_bytes, "cache"),
        _addr(seq_lens, 4 * cfg.batch, "seq_lens"),
        _addr(k_new, n_in, "k_new"), _addr(v_new, n_in, "v_new"), int(t_new),
        _addr(append_lens, 4 * cfg.batch, "append_lens"), _addr(skipped, 4 * cfg.batch, "skipped"),
        _stream(stream))
    _check(st, "kvq_quantize_append")


def kvq_decode_workspace_bytes(cfg: KvqConfig, split_tokens: int = 0) -> int:
    out = ctypes.c_uint64()
    _check(lib().kvq_decode_workspace_bytes(ctypes.byref(cfg), int(split_tokens), ctypes.byref(out)),
           "kvq_decode_workspace_bytes")
    return out.value


def kvq_decode_attention(cfg: KvqConfig, cache, seq_lens, q, sm_scale: float, out, workspace,
                         workspace_bytes: Optional[int] = None, split_tokens: int = 0, stream=None) -> None:
    """Decode attention of one query token per sequence over the cache.
    The workspace must be zero-filled before its first use (its leading
    arrival counters are left zero by every call)."""
    _check_types((seq_lens, _i32(), "seq_lens"), (q, _in_dtype(cfg), "q"), (out, _f32(), "out"))
    lay = kvq_get_layout(cfg)
    if workspace_bytes is None:
        workspace_bytes = (workspace.numel() * workspace.element_size()
                           if not isinstance(workspace, int) else kvq_decode_workspace_bytes(cfg, split_tokens))
    n_q = cfg.batch * cfg.n_q_heads * cfg.head_dim
    st = lib().kvq_decode_attention(
        ctypes.byref(cfg), _addr(cache, lay.total_bytes, "cache"),
        _addr(seq_lens, 4 * cfg.batch, "seq_lens"),
        _addr(q, n_q * _elem(cfg), "q"), ctypes.c_float(sm_scale),
        _addr(out, n_q * 4, "out"),
        _addr(workspace, workspace_bytes, "workspace"), int(workspace_bytes), int(split_tokens),
        _stream(stream))
    _check(st, "kvq_decode_attention")


def kvq_append_decode(cfg: KvqConfig, cache, seq_lens, k_new, v_new, q, sm_scale: float, out, workspace,
                      workspace_bytes: Optional[int] = None, split_tokens: int = 0, skipped=None,
                      stream=None) -> None:
    """One decode step in one launch: append the one new K/V token per
    sequence (k_new, v_new shaped [B, Hkv, 1, d]) and attend over the grown
    cache; seq_lens advances on the device. Same workspace rules as
    kvq_decode_attention. skipped: optional int32 [B] device tensor, set to
    1 for each sequence that takes no token (at capacity or a negative
    length), else 0."""
    _check_types((seq_lens, _i32(), "seq_lens"), (k_new, _in_dtype(cfg), "k_new"),
                 (v_new, _in_dtype(cfg), "v_new"), (q, _in_dtype(cfg), "q"), (out, _f32(), "out"),
                 (skipped, _i32(), "skipped"))
    lay = kvq_get_layout(cfg)
    if workspace_bytes is None:
        workspace_bytes = (workspace.numel() * workspace.element_size()
                           if not isinstance(workspace, int) else kvq_decode_workspace_bytes(cfg, split_tokens))
    n_q = cfg.batch * cfg.n_q_heads * cfg.head_dim
    n_in = cfg.batch * cfg.n_kv_heads * cfg.head_dim * _elem(cfg)
    st = lib().kvq_append_decode(
        ctypes.byref(cfg), _addr(cache, lay.total_bytes, "cache"),
        _addr(seq_lens, 4 * cfg.batch, "seq_lens"),
        _addr(k_new, n_in, "k_new"), _addr(v_new, n_in, "v_new"),
        _addr(q, n_q * _elem(cfg), "q"), ctypes.c_float(sm_scale),
        _addr(out, n_q * 4, "out"), _addr(workspace, workspace_bytes, "workspace"),
        int(workspace_bytes), int(split_tokens), _addr(skipped, 4 * cfg.batch, "skipped"), _stream(stream))
    _check(st, "kvq_append_decode")


def kvq_append_decode_noalloc(cfg: KvqConfig, cache, seq_lens, k_new, v_new, q, sm_scale: float, out,
                              split_tokens: int = 0, skipped=None, stream=None) -> None:
    """kvq_append_decode with the library's fixed device workspace instead of
    a caller's (for callers that cannot allocate): same arguments without
    the workspace; raises KvqError(ERR_WORKSPACE) when the call's split plan
    does not fit STATIC_WORKSPACE_BYTES. Calls that overlap in time on one
    device race (they share the device's array)."""
    _check_types((seq_lens, _i32(), "seq_lens"), (k_new, _in_dtype(cfg), "k_new"),
                 (v_new, _in_dtype(cfg), "v_new"), (q, _in_dtype(cfg), "q"), (out, _f32(), "out"),
                 (skipped, _i32(), "skipped"))
    lay = kvq_get_layout(cfg)
    n_q = cfg.batch * cfg.n_q_heads * cfg.head_dim
    n_in = cfg.batch * cfg.n_kv_heads * cfg.head_dim * _elem(cfg)
    st = lib().kvq_append_decode_noalloc(
        ctypes.byref(cfg), _addr(cache, lay.total_bytes, "cache"),
        _addr(seq_lens, 4 * cfg.batch, "seq_lens"),
        _addr(k_new, n_in, "k_new"), _addr(v_new, n_in, "v_new"),
        _addr(q, n_q * _elem(cfg), "q"), ctypes.c_float(sm_scale),
        _addr(out, n_q * 4, "out"), int(split_tokens), _addr(skipped, 4 * cfg.batch, "skipped"),
        _stream(stream))
    _check(st, "kvq_append_decode_noalloc")
