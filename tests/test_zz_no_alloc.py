"""The allocation-free decode entry point (mfa_decode_noalloc) against
mfa_decode on a handle created with the same configuration: the same kernels
and split, so the outputs are compared bit for bit, over two calls in a row
(the second with a smaller input) that share the library's static
workspace."""
import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _mfa():
    import decode_attention_mfa_amd as m
    from decode_attention_mfa_amd import harness
    return m, harness


def _cfg(m, dc, max_batch, max_context, split):
    return m.make_config(kv_dtype=m.MFA_DTYPE_FP8_E4M3 if dc.kv_dtype == "fp8" else m.MFA_DTYPE_BF16,
                         page_size=64 if dc.paged else 0, max_batch=max_batch, max_context=max_context,
                         split_tokens=split, softmax_scale=dc.softmax_scale)


def _both(m, hz, case, cfg):
    dc = hz.to_device(case)
    kv = dc.kv()
    o1, l1 = hz.alloc_outputs(dc)
    o2, l2 = hz.alloc_outputs(dc)
    h = m.mfa_create(cfg)
    try:
        m.mfa_decode(h, dc.q, kv, o1, l1, dc.batch)
        torch.cuda.synchronize()
    finally:
        m.mfa_destroy(h)
    free0 = torch.cuda.mem_get_info()[0]
    m.mfa_decode_noalloc(cfg, dc.q, kv, o2, l2, dc.batch)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    return (o1.cpu().numpy(), l1.cpu().numpy()), (o2.cpu().numpy(), l2.cpu().numpy()), free0 - free1


@pytest.mark.parametrize("kind", ["fp8_two_chunks", "bf16_combine", "fp8_paged_balanced"])
def test_noalloc_matches_decode_twice(kind):
    m, hz = _mfa()
    if kind == "fp8_two_chunks":      # in-kernel merge of two chunks
        big = synth.make_case("na1", 6, [4096, 4000, 2049, 4096, 100, 0], "fp8", seed=301)
        small = synth.make_case("na2", 2, [1000, 4096], "fp8", seed=302)
        mk = lambda dc: _cfg(m, dc, 8, 4096, 2048)
    elif kind == "bf16_combine":      # many chunks, merged by the combine kernel
        big = synth.make_case("na3", 3, [8192, 5000, 1], "bf16", seed=303)
        small = synth.make_case("na4", 1, [3000], "bf16", seed=304)
        mk = lambda dc: _cfg(m, dc, 4, 8192, 512)
    else:                             # balanced split over a paged cache
        big = synth.make_case("na5", 12, [3000, 64, 1, 700, 8192, 129, 2048, 65, 4000, 0, 5, 1000], "fp8",
                              seed=305, paged=True)
        small = synth.make_case("na6", 3, [100, 2000, 64], "fp8", seed=306, paged=True)
        mk = lambda dc: _cfg(m, dc, 16, 8192, m.MFA_SPLIT_BALANCED)
    for i, case in enumerate((big, small)):
        dc = hz.to_device(case)
        _say(f"[noalloc] {kind}: B={case.batch} L=[{case.seq_lens.min()},{case.seq_lens.max()}]")
        (o1, l1), (o2, l2), dfree = _both(m, hz, case, mk(dc))
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2, equal_nan=True)
        # the first call in a process loads the library's static workspace
        # (64 MiB, at set-up); no call allocates anything after that
        assert dfree <= (72 << 20 if i == 0 else 0), f"device memory shrank by {dfree} bytes across the call"


def test_noalloc_rejects_what_the_scratch_cannot_hold():
    m, hz = _mfa()
    case = synth.make_case("na7", 1, [64], "fp8", seed=307)
    dc = hz.to_device(case)
    o, l = hz.alloc_outputs(dc)
    # 3000 sequences of 8192 tokens in 256-token chunks need 96000 partial slots
    cfg = _cfg(m, dc, 3000, 8192, 256)
    q = torch.zeros((3000, 64, 256), dtype=torch.int16, device="cuda")
    out = torch.empty_like(q)
    lens = torch.full((3000,), 8192, dtype=torch.int32, device="cuda")
    k = torch.zeros((1, 64, 256), dtype=torch.uint8, device="cuda")
    kv = m.make_kv(k, k, lens, kv_stride=8192, max_seq_len=8192)
    with pytest.raises(m.MfaError) as ei:
        m.mfa_decode_noalloc(cfg, q, kv, out, None, 3000)
    assert ei.value.status == m.MFA_ERR_UNSUPPORTED and "partial slots" in str(ei.value)
    with pytest.raises(m.MfaError) as ei:
        m.mfa_decode_noalloc(_cfg(m, dc, 70000, 64, 0), dc.q, dc.kv(), o, l, 1)
    assert ei.value.status == m.MFA_ERR_UNSUPPORTED
