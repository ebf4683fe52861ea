"""Python access to the fp64 CPU oracle (``oracle/mfa_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline use it to check and time the GPU library. The product path never
imports it. It shares no code with the GPU library; the only code both sides
use is the seeded input generator in ``synth``.

Every function here is a thin ctypes wrapper; the arithmetic is in the C file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mfa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

KV_BF16 = 0
KV_FP8 = 1


def build(force: bool = True) -> str:
    """Compile liboracle.so with the host C compiler (no fast-math: IEEE fp64)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        I64 = ctypes.c_int64
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = D
        lib.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_to_f64.restype = D
        lib.oracle_e4m3_table.argtypes = [P]
        lib.oracle_decode_bf16.argtypes = [P, P, I64]
        lib.oracle_decode_e4m3.argtypes = [P, P, I64]
        lib.oracle_max_threads.restype = I
        lib.oracle_qproj.argtypes = [I, I, I, I, P, P, P, P, D, P, P, P, I]
        lib.oracle_qproj.restype = I
        lib.oracle_attention.argtypes = [I, I, I, P, I, P, P, D, D, P, P, I, I, I64, D, I,
                                         P, P, I]
        lib.oracle_attention.restype = I
        lib.oracle_attention_grouped.argtypes = [I, I, I, I, P, I, P, P, D, D, P, P, I, I, I64, D, I,
                                                 P, P, I]
        lib.oracle_attention_grouped.restype = I
        lib.oracle_attention_fp8mma.argtypes = [I, I, I, P, P, P, D, D, P, P, I, I, I64, D, P, P, I]
        lib.oracle_attention_fp8mma.restype = I
        lib.oracle_fp8_q_exponent.argtypes = [D]
        lib.oracle_fp8_q_exponent.restype = I
        lib.oracle_weights.argtypes = [I, I, P, I, I, I, P, D, P, P, I, I, I64, D, P]
        lib.oracle_weights.restype = I
        lib.oracle_gather_kv.argtypes = [I, I, I, P, P, P, P, I, I, I64, P, P]
        lib.oracle_gather_kv.restype = I
        lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
        lib.oracle_f32_to_e4m3.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_e4m3.restype = ctypes.c_uint8
        lib.oracle_encode_bf16.argtypes = [P, P, I64]
        lib.oracle_encode_e4m3.argtypes = [P, P, I64]
        lib.oracle_kv_project.argtypes = [I, I, I, P, P, P, P, P, I]
        lib.oracle_kv_project.restype = I
        lib.oracle_kv_append.argtypes = [I, I, I, P, P, D, D, P, P, P, P, I, I, I64, I]
        lib.oracle_kv_append.restype = I
        _lib = lib
        return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def e4m3_table() -> np.ndarray:
    out = np.empty(256, dtype=np.float64)
    _load().oracle_e4m3_table(_ptr(out))
    return out


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oracle_decode_bf16(_ptr(bits), _ptr(out), bits.size)
    return out


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    _load().oracle_decode_e4m3(_ptr(codes), _ptr(out), codes.size)
    return out


def encode_bf16(x) -> np.ndarray:
    """float32 values -> bf16 bits, round to nearest even."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_encode_bf16(_ptr(x), _ptr(out), x.size)
    return out


def encode_e4m3(x) -> np.ndarray:
    """float32 values -> E4M3FN codes, round to nearest even, saturating at 448."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().oracle_encode_e4m3(_ptr(x), _ptr(out), x.size)
    return out


def kv_project(x, w_k, w_v, nthreads: int = 0):
    """x [B, hidden], w_k and w_v [hidden, D] as bf16 bits -> (k, v) [B, D] fp64."""
    x, w_k, w_v = (_c(a, np.uint16) for a in (x, w_k, w_v))
    B, hidden = x.shape
    D = w_k.shape[1]
    assert w_k.shape == (hidden, D) and w_v.shape == (hidden, D)
    k = np.empty((B, D), dtype=np.float64)
    v = np.empty((B, D), dtype=np.float64)
    rc = _load().oracle_kv_project(B, hidden, D, _ptr(x), _ptr(w_k), _ptr(w_v), _ptr(k), _ptr(v),
                                   nthreads)
    if rc:
        raise RuntimeError(f"oracle_kv_project failed: {rc}")
    return k, v


def kv_append(k_new, v_new, k, v, seq_lens, *, kv_dtype: int, k_scale: float = 1.0,
              v_scale: float = 1.0, page_table=None, page_size: int = 64) -> int:
    """Write the encoded rows k_new, v_new [B, D] (fp64) into the caches k, v
    (raw bits, modified in place: contiguous [B, S, D] or paged [P, page, D])
    at row seq_lens[b]. Returns the number of sequences written."""
    k_new = _c(k_new, np.float64)
    v_new = _c(v_new, np.float64)
    B, D = k_new.shape
    raw = np.uint16 if kv_dtype == KV_BF16 else np.uint8
    for a in (k, v):
        assert a.dtype == raw and a.flags.c_contiguous and a.shape[-1] == D
    L = _c(seq_lens, np.int32)
    assert L.shape == (B,)
    if page_table is not None:
        pt = _c(page_table, np.int32)
        pt_stride, kv_stride, num_pages = pt.shape[1], 0, k.shape[0]
        assert k.shape[1] == page_size
    else:
        pt, pt_stride, kv_stride, num_pages = None, 0, k.shape[1], 0
        assert k.shape[0] == B
    return int(_load().oracle_kv_append(B, D, kv_dtype, _ptr(k_new), _ptr(v_new), float(k_scale),
                                        float(v_scale), _ptr(k), _ptr(v), _ptr(L), _ptr(pt),
                                        pt_stride, page_size, kv_stride, num_pages))


def qproj(x, w_qa, gamma, w_qb, eps: float = 1e-6, nthreads: int = 0, return_c: bool = False):
    """x [B, hidden], w_qa [hidden, rank], gamma [rank], w_qb [rank, nq] as bf16
    bits -> q [B, nq] fp64 (and c, chat when ``return_c``)."""
    x, w_qa, gamma, w_qb = (_c(a, np.uint16) for a in (x, w_qa, gamma, w_qb))
    B, hidden = x.shape
    rank = w_qa.shape[1]
    nq = w_qb.shape[1]
    assert w_qa.shape[0] == hidden and gamma.shape == (rank,) and w_qb.shape[0] == rank
    q = np.empty((B, nq), dtype=np.float64)
    c = np.empty((B, rank), dtype=np.float64) if return_c else None
    chat = np.empty((B, rank), dtype=np.float64) if return_c else None
    rc = _load().oracle_qproj(B, hidden, rank, nq, _ptr(x), _ptr(w_qa), _ptr(gamma), _ptr(w_qb),
                              float(eps), _ptr(c), _ptr(chat), _ptr(q), nthreads)
    if rc:
        raise RuntimeError(f"oracle_qproj failed: {rc}")
    return (q, c, chat) if return_c else q


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_lens, *, kv_dtype: int,
              k_scale: float = 1.0, v_scale: float = 1.0, page_table=None, page_size: int = 64,
              softmax_scale: float = 1.0 / 16.0, chunk: int = 0, nthreads: int = 0, kv_heads: int = 1):
    """q [B, H, D] fp64; k, v contiguous [B, S, D] or paged [P, page, D] as raw
    bits (uint16 bf16 or uint8 E4M3). With kv_heads = G > 1 (grouped-query
    attention): k, v contiguous [B, G, S, D] or paged [P, G, page, D], query
    head h reading KV head h // (H // G). Returns (o [B, H, D], lse [B, H])
    fp64."""
    q = _c(q, np.float64)
    B, H, D = q.shape
    G = int(kv_heads)
    raw = np.uint16 if kv_dtype == KV_BF16 else np.uint8
    k = _c(k, raw)
    v = _c(v, raw)
    L = _c(seq_lens, np.int32)
    assert L.shape == (B,)
    if k.ndim == 4:   # grouped layout [., G, ., D] (G may be 1)
        assert k.shape[1] == G, "grouped caches are [., G, ., D]"
    else:
        assert G == 1, "grouped caches are [., G, ., D]"
    rows_axis = 2 if k.ndim == 4 else 1
    if page_table is not None:
        pt = _c(page_table, np.int32)
        pt_stride = pt.shape[1]
        kv_stride = 0
        page_size = k.shape[rows_axis]
    else:
        pt = None
        pt_stride = 0
        kv_stride = k.shape[rows_axis]
    assert k.shape[-1] == D and v.shape == k.shape
    o = np.empty((B, H, D), dtype=np.float64)
    lse = np.empty((B, H), dtype=np.float64)
    rc = _load().oracle_attention_grouped(B, H, G, D, _ptr(q), kv_dtype, _ptr(k), _ptr(v), float(k_scale),
                                          float(v_scale), _ptr(L), _ptr(pt), pt_stride, page_size,
                                          kv_stride, float(softmax_scale), int(chunk), _ptr(o), _ptr(lse),
                                          nthreads)
    if rc:
        raise RuntimeError(f"oracle_attention_grouped failed: {rc}")
    return o, lse


def fp8_q_exponent(amax: float) -> int:
    """The power of two 2^e that puts a head's largest |q| in [128, 256)
    (e = 0 for an all-zero head, e limited to [-100, 100])."""
    return int(_load().oracle_fp8_q_exponent(float(amax)))


def attention_fp8mma(q_bits: np.ndarray, k: np.ndarray, v: np.ndarray, seq_lens, *, k_scale: float = 1.0,
                     v_scale: float = 1.0, page_table=None, page_size: int = 64,
                     softmax_scale: float = 1.0 / 16.0, nthreads: int = 0):
    """Attention in FP8 arithmetic (E4M3 query per head with a power-of-two
    scale, E4M3 weights 4P against an integer reference, applied-weight
    normalisation; see oracle_attention_fp8mma in the C file). q_bits [B, H, D]
    bf16 bits; k, v E4M3 codes, contiguous [B, S, D] or paged [P, page, D].
    Returns (o [B, H, D], lse [B, H]) fp64."""
    q_bits = _c(q_bits, np.uint16)
    B, H, D = q_bits.shape
    k = _c(k, np.uint8)
    v = _c(v, np.uint8)
    L = _c(seq_lens, np.int32)
    assert L.shape == (B,) and k.shape == v.shape and k.shape[-1] == D and k.ndim == 3
    if page_table is not None:
        pt = _c(page_table, np.int32)
        pt_stride, kv_stride, page_size = pt.shape[1], 0, k.shape[1]
    else:
        pt, pt_stride, kv_stride = None, 0, k.shape[1]
    o = np.empty((B, H, D), dtype=np.float64)
    lse = np.empty((B, H), dtype=np.float64)
    rc = _load().oracle_attention_fp8mma(B, H, D, _ptr(q_bits), _ptr(k), _ptr(v), float(k_scale),
                                         float(v_scale), _ptr(L), _ptr(pt), pt_stride, page_size, kv_stride,
                                         float(softmax_scale), _ptr(o), _ptr(lse), nthreads)
    if rc:
        raise RuntimeError(f"oracle_attention_fp8mma failed: {rc}")
    return o, lse


def attention_mtp(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_lens, *, kv_dtype: int,
                  k_scale: float = 1.0, v_scale: float = 1.0, page_table=None, page_size: int = 64,
                  softmax_scale: float = 1.0 / 16.0, nthreads: int = 0):
    """Multi-token decode: q [B, t, H, D] fp64, the cache holding the t new
    tokens as its last rows; token j of sequence b attends to the rows
    s < L_b - (t-1-j) (itself and all before it). Returns (o [B, t, H, D],
    lse [B, t, H]). Each (sequence, token) is one call of ``attention``."""
    q = _c(q, np.float64)
    B, t, H, D = q.shape
    L = _c(seq_lens, np.int32)
    Lv = np.maximum(0, np.repeat(L, t) - np.tile(np.arange(t - 1, -1, -1), B)).astype(np.int32)
    if page_table is not None:
        pt = np.repeat(_c(page_table, np.int32), t, axis=0)
        kk, vv = k, v
    else:
        pt = None
        kk = np.repeat(np.ascontiguousarray(k), t, axis=0)
        vv = np.repeat(np.ascontiguousarray(v), t, axis=0)
    o, lse = attention(q.reshape(B * t, H, D), kk, vv, Lv, kv_dtype=kv_dtype, k_scale=k_scale,
                       v_scale=v_scale, page_table=pt, page_size=page_size, softmax_scale=softmax_scale,
                       nthreads=nthreads)
    return o.reshape(B, t, H, D), lse.reshape(B, t, H)


def weights(q: np.ndarray, k: np.ndarray, seq_lens, b: int, h: int, *, kv_dtype: int,
            k_scale: float = 1.0, page_table=None, softmax_scale: float = 1.0 / 16.0):
    """Softmax weights of head h of sequence b over its L_b tokens."""
    q = _c(q, np.float64)
    B, H, D = q.shape
    raw = np.uint16 if kv_dtype == KV_BF16 else np.uint8
    k = _c(k, raw)
    L = _c(seq_lens, np.int32)
    pt = _c(page_table, np.int32)
    w = np.empty(max(int(L[b]), 1), dtype=np.float64)
    n = _load().oracle_weights(H, D, _ptr(q), b, h, kv_dtype, _ptr(k), float(k_scale), _ptr(L),
                               _ptr(pt), 0 if pt is None else pt.shape[1],
                               k.shape[1] if pt is not None else 64,
                               0 if pt is not None else k.shape[1], float(softmax_scale), _ptr(w))
    return w[:n]


def gather_kv(k: np.ndarray, v: np.ndarray, seq_lens, b: int, page_table=None):
    """Logical K/V rows t < L_b of sequence b, contiguous, same dtype as k."""
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    L = _c(seq_lens, np.int32)
    D = k.shape[-1]
    pt = _c(page_table, np.int32)
    n = int(L[b])
    kd = np.empty((n, D), dtype=k.dtype)
    vd = np.empty((n, D), dtype=v.dtype)
    _load().oracle_gather_kv(b, D, k.dtype.itemsize, _ptr(k), _ptr(v), _ptr(L), _ptr(pt),
                             0 if pt is None else pt.shape[1],
                             k.shape[1] if pt is not None else 64,
                             0 if pt is not None else k.shape[1], _ptr(kd), _ptr(vd))
    return kd, vd


def case_q(case) -> np.ndarray:
    """fp64 queries of a ``synth.Case``: decoded bf16 Q, or the oracle's own Q
    projection when the case carries the projection weights."""
    from synth import NUM_HEADS, HEAD_DIM
    if case.q is not None:
        return decode_bf16(case.q)
    q = qproj(case.x, case.w_qa, case.gamma, case.w_qb, eps=case.rms_eps)
    return q.reshape(case.batch, NUM_HEADS, HEAD_DIM)


def case_attention_fp8mma(case, nthreads: int = 0):
    """Oracle output (o, lse) of a ``synth.Case`` with an FP8 cache in the FP8
    attention arithmetic (its Q is the given bf16 Q)."""
    assert case.kv_dtype == "fp8" and case.q is not None
    return attention_fp8mma(case.q, case.k, case.v, case.seq_lens, k_scale=case.k_scale,
                            v_scale=case.v_scale, page_table=case.page_table,
                            softmax_scale=case.softmax_scale, nthreads=nthreads)


def case_attention(case, q: Optional[np.ndarray] = None, chunk: int = 0, nthreads: int = 0):
    """Oracle output (o, lse) of a ``synth.Case``."""
    if q is None:
        q = case_q(case)
    return attention(q, case.k, case.v, case.seq_lens,
                     kv_dtype=KV_FP8 if case.kv_dtype == "fp8" else KV_BF16,
                     k_scale=case.k_scale, v_scale=case.v_scale, page_table=case.page_table,
                     softmax_scale=case.softmax_scale, chunk=chunk, nthreads=nthreads,
                     kv_heads=getattr(case, "kv_heads", 1))
