"""The C ABI on the CPU: the library loads, exports every entry point its
header declares, and rejects bad arguments on the host with the documented
status and a message, before touching any device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "mfa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|int32_t|const char\*)\s+(mfa_\w+)\s*\(", src, re.M)))


def test_header_declares_the_boundary():
    names = _header_functions()
    for n in ("mfa_create", "mfa_qproj", "mfa_decode", "mfa_destroy", "mfa_status_string",
              "mfa_last_error", "mfa_debug_gather_kv", "mfa_split_tokens", "mfa_split_tokens_mtp",
              "mfa_kv_append"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import decode_attention_mfa_amd as m
    lib = ctypes.CDLL(m.LIB_PATH)
    missing = [n for n in _header_functions() if not hasattr(lib, n)]
    assert not missing, missing


def _create(**kw):
    import decode_attention_mfa_amd as m
    cfg = m.make_config(**kw)
    h = ctypes.c_void_p()
    st = m.lib.mfa_create(ctypes.byref(cfg), ctypes.byref(h))
    return st, m.mfa_last_error(), h.value


@pytest.mark.parametrize("kw,status,needle", [
    (dict(num_heads=32), -2, "64 heads"),
    (dict(head_dim=128), -2, "64 heads x 256"),
    (dict(page_size=16), -2, "page_size"),
    (dict(kv_dtype=7), -1, "kv_dtype"),
    (dict(max_batch=0), -1, "max_batch"),
    (dict(split_tokens=100), -1, "split_tokens"),
    (dict(split_tokens=-2), -1, "split_tokens"),
    (dict(attn_math=5), -1, "attn_math"),
    (dict(attn_math=1, kv_dtype="bf16"), -2, "FP8 cache"),
    (dict(q_rank=8192), -2, "q_rank"),
    (dict(page_size=64, split_tokens=8256), -2, "paged cache"),
    (dict(softmax_scale=0.0), -1, "softmax_scale"),
    (dict(softmax_scale=float("inf")), -1, "softmax_scale"),
    (dict(rms_eps=-1.0), -1, "rms_eps"),
    (dict(hidden=1000), -2, "hidden"),
    (dict(q_rank=100), -2, "q_rank"),
    (dict(kv_heads=3, kv_dtype="fp8"), -1, "kv_heads"),
    (dict(kv_heads=8, kv_dtype="fp8"), -1, "kv_heads"),
    (dict(kv_heads=2, kv_dtype="fp8", attn_math=1), -2, "kv_heads > 1"),
    (dict(kv_heads=4, kv_dtype="fp8", split_tokens=-1), -2, "kv_heads > 1"),
    (dict(kv_latent=256, kv_dtype="fp8"), -1, "kv_latent"),
    (dict(kv_latent=512, kv_dtype="bf16"), -2, "kv_latent"),
    (dict(kv_latent=512, kv_dtype="fp8", kv_heads=2), -2, "kv_latent"),
    (dict(kv_latent=512, kv_dtype="fp8", split_tokens=-1), -2, "kv_latent"),
    (dict(kv_latent=512, kv_dtype="fp8", attn_math=1), -2, "kv_latent"),
])
def test_create_rejects_bad_config(kw, status, needle):
    st, msg, h = _create(**kw)
    assert st == status and h is None
    assert needle in msg


def test_null_arguments_are_rejected():
    import decode_attention_mfa_amd as m
    assert m.lib.mfa_create(None, None) == m.MFA_ERR_INVALID
    assert "null" in m.mfa_last_error()
    kv = m.mfa_kv()
    assert m.lib.mfa_decode(None, None, ctypes.byref(kv), None, None, 1, None) == m.MFA_ERR_INVALID
    assert "handle" in m.mfa_last_error()
    assert m.lib.mfa_qproj(None, None, None, None, None, None, 1, None) == m.MFA_ERR_INVALID
    assert m.lib.mfa_debug_gather_kv(None, ctypes.byref(kv), 0, None, None, None) == m.MFA_ERR_INVALID
    assert m.lib.mfa_debug_fp8_mfma(None, None, None, None, 1, None) == m.MFA_ERR_INVALID
    assert m.lib.mfa_debug_fp8_mfma(1, 1, None, 1, -1, None) == m.MFA_ERR_INVALID
    assert m.lib.mfa_kv_append(None, None, None, None, ctypes.byref(kv), 1, None) == m.MFA_ERR_INVALID
    assert "handle" in m.mfa_last_error()
    assert m.lib.mfa_destroy(None) == m.MFA_OK
    with pytest.raises(m.MfaError):
        m.mfa_decode(None, 0, kv, 0, 0, 1, stream=0)


def test_status_strings():
    import decode_attention_mfa_amd as m
    assert m.mfa_status_string(0) == "ok"
    assert m.mfa_status_string(-2) == "unsupported configuration"
    assert m.mfa_status_string(-99) == "unknown status"
