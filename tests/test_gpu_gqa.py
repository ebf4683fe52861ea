"""GPU parity of grouped-query attention (mfa_config.kv_heads = G > 1: query
head h reads K/V head h / (64/G)) against the fp64 oracle, through the C
ABI. Same row-wise metric and bars as the single-head tests."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 1e-2
LSE_TOL = 1e-3


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _mfa():
    import decode_attention_mfa_amd as m
    from decode_attention_mfa_amd import harness
    return m, harness


def _check(case, split, label, sample=None):
    m, hz = _mfa()
    _say(f"[gqa] {label}: G={case.kv_heads} B={case.batch} paged={case.paged} "
         f"L=[{case.seq_lens.min()},{case.seq_lens.max()}] split={split}")
    dc = hz.to_device(case)
    h = hz.create_handle(dc, split_tokens=split)
    try:
        groups = m.mfa_head_groups(h, dc.batch, dc.max_len, dc.min_len)
        o, lse = hz.decode(h, dc)
        torch.cuda.synchronize()
    finally:
        m.mfa_destroy(h)
    assert groups == case.kv_heads
    o = hz.bf16_to_f64(o)
    lse = lse.cpu().numpy().astype(np.float64)
    idx = np.arange(case.batch) if sample is None else sample
    sub = case
    if sample is not None:
        sub = synth.Case(name="s", batch=len(idx), kv_dtype=case.kv_dtype, seq_lens=case.seq_lens[idx],
                         k=case.k[idx], v=case.v[idx], q=case.q[idx], k_scale=case.k_scale,
                         v_scale=case.v_scale, kv_heads=case.kv_heads)
    o_ref, lse_ref = oracle.case_attention(sub)
    o, lse = o[idx], lse[idx]
    nz = sub.seq_lens > 0
    err = np.abs(o - o_ref).max(axis=-1) / np.maximum(np.abs(o_ref).max(axis=-1), 1e-30)
    e = float(err[nz].max()) if nz.any() else 0.0
    el = float(np.abs(lse[nz] - lse_ref[nz]).max()) if nz.any() else 0.0
    _say(f"    row-rel err {e:.3e}  lse abs err {el:.3e}")
    assert e <= TOL and el <= LSE_TOL
    if (~nz).any():
        assert np.all(o[~nz] == 0) and np.all(np.isneginf(lse[~nz]))


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("G", [2, 4])
@pytest.mark.parametrize("split", [0, 256, 1024])
def test_gqa_contiguous(kv, G, split):
    """Ragged tails, an empty sequence, one and two chunks (merged in the
    kernel) and many chunks (combine kernel)."""
    L = [0, 1, 63, 64, 65, 300, 1000, 2049]
    case = synth.make_case("gqa", len(L), L, kv, seed=400 + G, kv_slack=5, kv_heads=G)
    _check(case, split, f"contiguous {kv}")


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("G", [2, 4])
def test_gqa_paged(kv, G):
    L = [5, 64, 129, 700, 1500, 0]
    case = synth.make_case("gqa_paged", len(L), L, kv, seed=410 + G, paged=True, kv_heads=G)
    _check(case, 256, f"paged {kv}")
    _check(case, 0, f"paged {kv}, auto split")


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_gqa_groups_are_independent(kv):
    """Changing K/V head 1's rows changes only its query heads' outputs."""
    m, hz = _mfa()
    outs = []
    for variant in range(2):
        c = synth.make_case("gqa_ind", 2, [300, 77], kv, seed=420, kv_heads=2)
        if variant:
            # other finite values: E4M3 codes below NaN's, or bf16 bits of N(0,1) draws
            g = np.random.default_rng(421)
            if kv == "fp8":
                c.k[:, 1] = g.integers(0, 0x7e, size=c.k[:, 1].shape, dtype=np.uint8)
            else:
                c.k[:, 1] = synth.bf16_bits(g.standard_normal(c.k[:, 1].shape).astype(np.float32))
        dc = hz.to_device(c)
        h = hz.create_handle(dc, split_tokens=0)
        try:
            o, _ = hz.decode(h, dc)
            torch.cuda.synchronize()
        finally:
            m.mfa_destroy(h)
        outs.append(o.cpu())
    assert torch.equal(outs[0][:, :32], outs[1][:, :32])
    assert not torch.equal(outs[0][:, 32:], outs[1][:, 32:])


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("G", [2, 4])
def test_gqa_full_size(kv, G):
    """The comparison workloads at full size (B = 128, L = 4096, G K/V heads)
    in bench.py's configuration: sampled sequences against the oracle."""
    case = synth.gqa_case(G, kv_dtype=kv)
    _check(case, 0, f"full size {kv}", sample=np.array([0, 41, 86, 127]))


def test_gqa_rejected_where_unsupported():
    m, hz = _mfa()
    case = synth.make_case("gqa_rej", 1, [100], "fp8", seed=430, kv_heads=2)
    dc = hz.to_device(case)
    h = hz.create_handle(dc, max_batch=4)
    try:
        q = torch.zeros((1, 2, 64, 256), dtype=torch.int16, device="cuda")
        o = torch.empty_like(q)
        with pytest.raises(m.MfaError) as ei:
            m.mfa_decode_mtp(h, q, dc.kv(), 2, o, None, 1)
        assert ei.value.status == m.MFA_ERR_UNSUPPORTED
        k = torch.empty((100, 256), dtype=torch.uint8, device="cuda")
        with pytest.raises(m.MfaError) as ei:
            m.mfa_debug_gather_kv(h, dc.kv(), 0, k, k)
        assert ei.value.status == m.MFA_ERR_UNSUPPORTED
    finally:
        m.mfa_destroy(h)
