"""GPU parity of the latent-cache (MLA-style) mode (mfa_config.kv_latent =
512: one 512-wide E4M3 latent row per token, key and value of all 64 heads,
q and out [B, 64, 512]) against the fp64 oracle (multi-query attention over
the latent rows, pinned as MLA's absorbed attention in
tests/test_oracle_latent.py), through the C ABI. Same row-wise metric and
bars as the MFA tests: the latent codes decode exactly, Q is bf16 on both
sides, the GPU rounds P and the output (and a piece's partial) to bf16."""
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


def _run(case, split):
    m, hz = _mfa()
    dc = hz.to_device(case)
    h = hz.create_handle(dc, split_tokens=split)
    try:
        assert m.mfa_head_groups(h, dc.batch, dc.max_len, dc.min_len) == 2
        o, lse = hz.decode(h, dc)
        torch.cuda.synchronize()
    finally:
        m.mfa_destroy(h)
    return o, lse


def _check(case, split, label, sample=None):
    _say(f"[latent] {label}: B={case.batch} paged={case.paged} L=[{case.seq_lens.min()},{case.seq_lens.max()}] "
         f"split={split}")
    m, hz = _mfa()
    o, lse = _run(case, split)
    o = hz.bf16_to_f64(o)
    lse = lse.cpu().numpy().astype(np.float64)
    idx = np.arange(case.batch) if sample is None else sample
    sub = case
    if sample is not None:
        sub = synth.Case(name="s", batch=len(idx), kv_dtype="fp8", seq_lens=case.seq_lens[idx], k=case.k[idx],
                         v=case.k[idx], q=case.q[idx], k_scale=case.k_scale, v_scale=case.k_scale, kv_latent=512)
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


@pytest.mark.parametrize("split", [0, 256, 1024])
def test_latent_contiguous(split):
    """Ragged tails, an empty sequence, one chunk and several (merge kernel)."""
    L = [0, 1, 63, 64, 65, 300, 1000, 2049]
    _check(synth.latent_case("lat", len(L), L, seed=500, kv_slack=5), split, "contiguous")


def test_latent_paged():
    L = [5, 64, 129, 700, 1500, 0]
    case = synth.latent_case("lat_paged", len(L), L, seed=510, paged=True)
    _check(case, 256, "paged")
    _check(case, 0, "paged, auto split")


def test_latent_paged_equals_contiguous_bitwise():
    m, hz = _mfa()
    L = [77, 1000, 300]
    cc = synth.latent_case("lat_c", len(L), L, seed=520)
    cp = synth.latent_case("lat_p", len(L), L, seed=520, paged=True)
    for b in range(len(L)):   # the same logical rows in the pool
        for j in range((L[b] + 63) // 64):
            n = min(64, L[b] - 64 * j)
            cp.k[cp.page_table[b, j], :n] = cc.k[b, 64 * j:64 * j + n]
    cp.v = cp.k
    cp.k_scale = cp.v_scale = cc.k_scale
    cp.q = cc.q
    for split in (0, 256):
        oc, lc = _run(cc, split)
        op, lp = _run(cp, split)
        assert torch.equal(oc.cpu(), op.cpu()) and torch.equal(lc.cpu(), lp.cpu())


def test_latent_deterministic():
    case = synth.latent_case("lat_det", 4, [4096, 3000, 2049, 65], seed=530)
    o1, l1 = _run(case, 512)
    o2, l2 = _run(case, 512)
    assert torch.equal(o1.cpu(), o2.cpu()) and torch.equal(l1.cpu(), l2.cpu())


def test_latent_full_size():
    """The comparison workload at full size (B = 128, L = 4096, FP8 latent) in
    bench.py's configuration: sampled sequences against the oracle."""
    case = synth.latent_case("fp8_mla", 128, 4096, seed=1300)
    _check(case, 0, "full size", sample=np.array([0, 41, 86, 127]))


def test_latent_rejected_where_unsupported():
    m, hz = _mfa()
    case = synth.latent_case("lat_rej", 1, [100], seed=540)
    dc = hz.to_device(case)
    h = hz.create_handle(dc, max_batch=4)
    try:
        q = torch.zeros((1, 2, 64, 512), dtype=torch.int16, device="cuda")
        o = torch.empty_like(q)
        for call in (lambda: m.mfa_decode_mtp(h, q, dc.kv(), 2, o, None, 1),
                     lambda: m.mfa_debug_gather_kv(h, dc.kv(), 0, o, o)):
            with pytest.raises(m.MfaError) as ei:
                call()
            assert ei.value.status == m.MFA_ERR_UNSUPPORTED
    finally:
        m.mfa_destroy(h)
