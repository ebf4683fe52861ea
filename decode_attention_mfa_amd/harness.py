"""Device-side marshalling for host workloads: copies host arrays (bf16 bit
patterns, E4M3 codes, int32 lengths and page tables) into torch device
tensors and calls the C ABI through the binding. No arithmetic of the method
happens here.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import (MFA_DTYPE_BF16, MFA_DTYPE_FP8_E4M3, make_config, make_kv, mfa_create,
               mfa_decode, mfa_destroy, mfa_kv_append, mfa_qproj)

HEADS, HEAD_DIM = 64, 256


def _dev(a: Optional[np.ndarray], device) -> Optional[torch.Tensor]:
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


@dataclasses.dataclass
class DeviceCase:
    batch: int
    kv_dtype: str
    k: torch.Tensor
    v: torch.Tensor
    seq_lens: torch.Tensor
    max_len: int
    q: Optional[torch.Tensor] = None
    page_table: Optional[torch.Tensor] = None
    k_scale: float = 1.0
    v_scale: float = 1.0
    x: Optional[torch.Tensor] = None
    w_qa: Optional[torch.Tensor] = None
    gamma: Optional[torch.Tensor] = None
    w_qb: Optional[torch.Tensor] = None
    w_k: Optional[torch.Tensor] = None
    w_v: Optional[torch.Tensor] = None
    softmax_scale: float = 1.0 / 16.0
    rms_eps: float = 1e-6
    split_tokens: int = 0
    min_len: int = 0             # lower bound of the lengths (as a scheduler knows it), 0 = unknown
    kv_heads: int = 1            # K/V heads per token (grouped-query caches: 2 or 4)
    kv_latent: int = 0           # 512: latent-cache mode (q, out [B, 64, 512])

    @property
    def paged(self) -> bool:
        return self.page_table is not None

    def kv(self, max_seq_len: int = 0):
        return make_kv(self.k, self.v, self.seq_lens, page_table=self.page_table,
                       k_scale=self.k_scale, v_scale=self.v_scale,
                       max_seq_len=max_seq_len or self.max_len, min_seq_len=self.min_len)


def to_device(case, device="cuda") -> DeviceCase:
    """``case`` is any object with the fields of ``synth.Case``."""
    return DeviceCase(
        batch=case.batch, kv_dtype=case.kv_dtype, k=_dev(case.k, device), v=_dev(case.v, device),
        seq_lens=_dev(case.seq_lens.astype(np.int32), device), max_len=max(1, int(case.seq_lens.max())),
        q=_dev(case.q, device), page_table=_dev(case.page_table, device), k_scale=case.k_scale,
        v_scale=case.v_scale, x=_dev(case.x, device), w_qa=_dev(case.w_qa, device),
        gamma=_dev(case.gamma, device), w_qb=_dev(case.w_qb, device),
        w_k=_dev(getattr(case, "w_k", None), device), w_v=_dev(getattr(case, "w_v", None), device),
        softmax_scale=case.softmax_scale, rms_eps=case.rms_eps, split_tokens=case.split_tokens,
        min_len=max(0, int(case.seq_lens.min())) if case.batch else 0,
        kv_heads=getattr(case, "kv_heads", 1), kv_latent=getattr(case, "kv_latent", 0))


def create_handle(dc: DeviceCase, *, max_batch: Optional[int] = None, max_context: Optional[int] = None,
                  split_tokens: Optional[int] = None, attn_math: int = 0) -> int:
    return mfa_create(make_config(
        kv_dtype=MFA_DTYPE_FP8_E4M3 if dc.kv_dtype == "fp8" else MFA_DTYPE_BF16,
        page_size=64 if dc.paged else 0, max_batch=max_batch or dc.batch,
        max_context=max_context or dc.max_len,
        split_tokens=dc.split_tokens if split_tokens is None else split_tokens,
        rms_eps=dc.rms_eps, softmax_scale=dc.softmax_scale, attn_math=attn_math,
        kv_heads=dc.kv_heads, kv_latent=dc.kv_latent))


def alloc_outputs(dc: DeviceCase):
    out = torch.empty((dc.batch, HEADS, dc.kv_latent or HEAD_DIM), dtype=torch.int16, device=dc.k.device)
    lse = torch.empty((dc.batch, HEADS), dtype=torch.float32, device=dc.k.device)
    return out, lse


def qproj(h: int, dc: DeviceCase, q_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    if q_out is None:
        q_out = torch.empty((dc.batch, HEADS, HEAD_DIM), dtype=torch.int16, device=dc.x.device)
    mfa_qproj(h, dc.x, dc.w_qa, dc.gamma, dc.w_qb, q_out, dc.batch, stream)
    return q_out


def kv_append(h: int, dc: DeviceCase, stream=None, max_seq_len: int = 0) -> None:
    """Write the new token's K and V rows at row seq_lens[b] of dc's cache."""
    mfa_kv_append(h, dc.x, dc.w_k, dc.w_v, dc.kv(max_seq_len), dc.batch, stream)


def decode(h: int, dc: DeviceCase, q: Optional[torch.Tensor] = None, out=None, lse=None,
           stream=None, max_seq_len: int = 0):
    if out is None or lse is None:
        out, lse = alloc_outputs(dc)
    mfa_decode(h, dc.q if q is None else q, dc.kv(max_seq_len), out, lse, dc.batch, stream)
    return out, lse


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.bfloat16).float().cpu().numpy().astype(np.float64)


def run_case(dc: DeviceCase, **handle_kw):
    """Full layer step for a case: Q projection when the case carries the
    weights, then decode. Returns (out bf16 as int16, lse fp32, q)."""
    h = create_handle(dc, **handle_kw)
    try:
        q = qproj(h, dc) if dc.q is None else dc.q
        out, lse = decode(h, dc, q=q)
        torch.cuda.synchronize()
    finally:
        mfa_destroy(h)
    return out, lse, q
