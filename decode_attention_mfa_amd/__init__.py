"""Python binding of libmfa.so, the MI355X (gfx950) decode step of
Multi-Matrix Factorization Attention.

Argument marshalling only: every computation runs in the library's HIP
kernels. Tensors may be passed as torch tensors (their device pointer is
used) or as raw integer device pointers. The names mirror the C ABI in
include/mfa.h. Importing fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
# MFA_LIBRARY may name another build of the same library (for A/B timing)
LIB_PATH = os.environ.get("MFA_LIBRARY") or os.path.join(_PKG, "libmfa.so")

MFA_OK = 0
MFA_ERR_INVALID = -1
MFA_ERR_UNSUPPORTED = -2
MFA_ERR_NOMEM = -3
MFA_ERR_HIP = -4
MFA_DTYPE_BF16 = 0
MFA_DTYPE_FP8_E4M3 = 1
MFA_SPLIT_BALANCED = -1
MFA_ATTN_BF16_MFMA = 0
MFA_ATTN_FP8_MFMA = 1
KERNEL_KINDS = ("attention", "combine", "qproj_down", "rmsnorm", "qproj_up", "kv_proj", "kv_write")


class MfaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class mfa_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("q_rank", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_batch", ctypes.c_int32), ("max_context", ctypes.c_int32),
                ("split_tokens", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("softmax_scale", ctypes.c_float), ("attn_math", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("kv_latent", ctypes.c_int32)]


class mfa_kv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("seq_lens", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
                ("pt_stride", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("kv_stride", ctypes.c_int64), ("max_seq_len", ctypes.c_int32),
                ("min_seq_len", ctypes.c_int32)]


def _load_lib():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'` "
                          "or `python decode_attention_mfa_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.mfa_create.argtypes = [ctypes.POINTER(mfa_config), ctypes.POINTER(P)]
    lib.mfa_create.restype = ctypes.c_int
    lib.mfa_qproj.argtypes = [P, P, P, P, P, P, I32, P]
    lib.mfa_qproj.restype = ctypes.c_int
    lib.mfa_decode.argtypes = [P, P, ctypes.POINTER(mfa_kv), P, P, I32, P]
    lib.mfa_decode_mtp.argtypes = [P, P, ctypes.POINTER(mfa_kv), I32, P, P, I32, P]
    lib.mfa_decode_mtp.restype = ctypes.c_int
    lib.mfa_kv_append.argtypes = [P, P, P, P, ctypes.POINTER(mfa_kv), I32, P]
    lib.mfa_kv_append.restype = ctypes.c_int
    lib.mfa_decode.restype = ctypes.c_int
    lib.mfa_decode_noalloc.argtypes = [ctypes.POINTER(mfa_config), P, ctypes.POINTER(mfa_kv), P, P, I32, P]
    lib.mfa_decode_noalloc.restype = ctypes.c_int
    lib.mfa_split_tokens.argtypes = [P, I32, I32, I32]
    lib.mfa_split_tokens.restype = I32
    lib.mfa_split_tokens_mtp.argtypes = [P, I32, I32, I32]
    lib.mfa_split_tokens_mtp.restype = I32
    lib.mfa_head_groups.argtypes = [P, I32, I32, I32]
    lib.mfa_head_groups.restype = I32
    lib.mfa_debug_gather_kv.argtypes = [P, ctypes.POINTER(mfa_kv), I32, P, P, P]
    lib.mfa_debug_gather_kv.restype = ctypes.c_int
    lib.mfa_debug_fp8_mfma.argtypes = [P, P, P, P, I32, P]
    lib.mfa_debug_fp8_mfma.restype = ctypes.c_int
    lib.mfa_debug_mfma_rate.argtypes = [I32, I32, P, P, P]
    lib.mfa_debug_mfma_rate.restype = ctypes.c_int
    lib.mfa_profile_enable.argtypes = [P, ctypes.c_int]
    lib.mfa_profile_enable.restype = ctypes.c_int
    lib.mfa_profile_read.argtypes = [P, P, P]
    lib.mfa_profile_read.restype = ctypes.c_int
    lib.mfa_destroy.argtypes = [P]
    lib.mfa_destroy.restype = ctypes.c_int
    lib.mfa_status_string.argtypes = [ctypes.c_int]
    lib.mfa_status_string.restype = ctypes.c_char_p
    lib.mfa_last_error.argtypes = []
    lib.mfa_last_error.restype = ctypes.c_char_p
    return lib


lib = _load_lib()


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, fn: str) -> int:
    if status < 0:
        raise MfaError(status, f"{fn}: {lib.mfa_last_error().decode()}")
    return status


def mfa_status_string(status: int) -> str:
    return lib.mfa_status_string(status).decode()


def mfa_last_error() -> str:
    return lib.mfa_last_error().decode()


def make_config(*, hidden=7168, q_rank=2048, num_heads=64, head_dim=256, kv_dtype=MFA_DTYPE_BF16,
                page_size=0, max_batch=1, max_context=4096, split_tokens=0, rms_eps=1e-6,
                softmax_scale=1.0 / 16.0, attn_math=MFA_ATTN_BF16_MFMA, kv_heads=1, kv_latent=0) -> mfa_config:
    if isinstance(kv_dtype, str):
        kv_dtype = MFA_DTYPE_FP8_E4M3 if kv_dtype == "fp8" else MFA_DTYPE_BF16
    return mfa_config(hidden, q_rank, num_heads, head_dim, kv_dtype, page_size, max_batch,
                      max_context, split_tokens, rms_eps, softmax_scale, attn_math, kv_heads, kv_latent)


def make_kv(k, v, seq_lens, *, page_table=None, k_scale=1.0, v_scale=1.0, kv_stride=0,
            pt_stride=0, num_pages=0, max_seq_len=0, min_seq_len=0) -> mfa_kv:
    """Describe a KV cache. For torch tensors the strides default from the
    shapes: contiguous k [B, S, 256] (or grouped [B, G, S, 256]) -> kv_stride
    S; paged k [P, 64, 256] (or [P, G, 64, 256]) -> num_pages P; page_table
    [B, n] -> pt_stride n."""
    if page_table is not None:
        if not pt_stride and hasattr(page_table, "shape"):
            pt_stride = int(page_table.shape[1])
        if not num_pages and hasattr(k, "shape"):
            num_pages = int(k.shape[0])
    elif not kv_stride and hasattr(k, "shape"):
        kv_stride = int(k.shape[-2])
    return mfa_kv(_ptr(k), _ptr(v), k_scale, v_scale, _ptr(seq_lens), _ptr(page_table),
                  pt_stride, num_pages, kv_stride, max_seq_len, min_seq_len)


def mfa_create(cfg: Optional[mfa_config] = None, **kw) -> int:
    """Create a handle (an opaque integer). kwargs go to make_config."""
    if cfg is None:
        cfg = make_config(**kw)
    h = ctypes.c_void_p()
    _check(lib.mfa_create(ctypes.byref(cfg), ctypes.byref(h)), "mfa_create")
    return h.value


def mfa_qproj(h: int, x, w_qa, rms_w, w_qb, q_out, batch: int, stream=None) -> None:
    _check(lib.mfa_qproj(h, _ptr(x), _ptr(w_qa), _ptr(rms_w), _ptr(w_qb), _ptr(q_out), batch,
                         _stream(stream)), "mfa_qproj")


def mfa_decode(h: int, q, kv: mfa_kv, out, lse_out, batch: int, stream=None) -> None:
    _check(lib.mfa_decode(h, _ptr(q), ctypes.byref(kv), _ptr(out), _ptr(lse_out), batch,
                          _stream(stream)), "mfa_decode")


def mfa_decode_noalloc(cfg: mfa_config, q, kv: mfa_kv, out, lse_out, batch: int, stream=None) -> None:
    """mfa_decode without a handle: the library's static device workspace
    (allocates nothing)."""
    _check(lib.mfa_decode_noalloc(ctypes.byref(cfg), _ptr(q), ctypes.byref(kv), _ptr(out), _ptr(lse_out), batch,
                                  _stream(stream)), "mfa_decode_noalloc")


def mfa_decode_mtp(h: int, q, kv: mfa_kv, num_tokens: int, out, lse_out, batch: int, stream=None) -> None:
    """num_tokens query tokens per sequence: q, out [batch, num_tokens, 64, 256]."""
    _check(lib.mfa_decode_mtp(h, _ptr(q), ctypes.byref(kv), num_tokens, _ptr(out), _ptr(lse_out), batch,
                              _stream(stream)), "mfa_decode_mtp")


def mfa_kv_append(h: int, x, w_k, w_v, kv: mfa_kv, batch: int, stream=None) -> None:
    """Writes the new token's K and V rows into kv's cache at row seq_lens[b]."""
    _check(lib.mfa_kv_append(h, _ptr(x), _ptr(w_k), _ptr(w_v), ctypes.byref(kv), batch,
                             _stream(stream)), "mfa_kv_append")


def mfa_split_tokens(h: int, batch: int, max_seq_len: int = 0, min_seq_len: int = 0) -> int:
    return _check(lib.mfa_split_tokens(h, batch, max_seq_len, min_seq_len), "mfa_split_tokens")


def mfa_split_tokens_mtp(h: int, batch: int, num_tokens: int, max_seq_len: int = 0) -> int:
    return _check(lib.mfa_split_tokens_mtp(h, batch, num_tokens, max_seq_len), "mfa_split_tokens_mtp")


def mfa_head_groups(h: int, batch: int, max_seq_len: int = 0, min_seq_len: int = 0) -> int:
    return _check(lib.mfa_head_groups(h, batch, max_seq_len, min_seq_len), "mfa_head_groups")


def mfa_debug_gather_kv(h: int, kv: mfa_kv, b: int, k_dst, v_dst, stream=None) -> None:
    _check(lib.mfa_debug_gather_kv(h, ctypes.byref(kv), b, _ptr(k_dst), _ptr(v_dst),
                                   _stream(stream)), "mfa_debug_gather_kv")


def mfa_debug_fp8_mfma(a, b, c, d, n_tiles: int, stream=None) -> None:
    """d = a . b + c per tile on the FP8 MFMA of the FP8-MFMA mode (a [n,16,128],
    b [n,128,16] E4M3 codes; c (or None), d [n,16,16] fp32)."""
    _check(lib.mfa_debug_fp8_mfma(_ptr(a), _ptr(b), _ptr(c), _ptr(d), n_tiles, _stream(stream)),
           "mfa_debug_fp8_mfma")


def mfa_debug_mfma_rate(kind: int, iters: int, sink, stream=None) -> float:
    """Launch the matrix-core rate microbenchmark (kind 0: bf16 16x16x32
    MFMAs, 1: E4M3 16x16x128) on the stream; returns the launch's flop count."""
    flops = ctypes.c_double(0.0)
    _check(lib.mfa_debug_mfma_rate(kind, iters, _ptr(sink), ctypes.byref(flops), _stream(stream)),
           "mfa_debug_mfma_rate")
    return flops.value


def mfa_profile_enable(h: int, enable: bool = True) -> None:
    _check(lib.mfa_profile_enable(h, int(bool(enable))), "mfa_profile_enable")


def mfa_profile_read(h: int) -> dict:
    """{kind: (launches, total_ms)} for the launches since the last read."""
    n = (ctypes.c_int32 * len(KERNEL_KINDS))()
    ms = (ctypes.c_double * len(KERNEL_KINDS))()
    _check(lib.mfa_profile_read(h, ctypes.cast(n, ctypes.c_void_p), ctypes.cast(ms, ctypes.c_void_p)),
           "mfa_profile_read")
    return {k: (int(n[i]), float(ms[i])) for i, k in enumerate(KERNEL_KINDS)}


def mfa_destroy(h: Optional[int]) -> None:
    _check(lib.mfa_destroy(h), "mfa_destroy")
