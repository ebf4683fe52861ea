"""GPU parity of mfa_decode_mtp (several query tokens per sequence against the
same cache, the last t rows being the new tokens') against the fp64 oracle,
through the C ABI, with the row-wise metric of the single-token tests."""
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


def _q(B, t, seed, std=1.0):
    rng = np.random.default_rng(seed)
    return synth.bf16_bits((rng.standard_normal((B, t, 64, 256)) * std).astype(np.float32))


def _run_mtp(case, q_bits, t, split):
    m, hz = _mfa()
    dc = hz.to_device(case)
    q = torch.from_numpy(q_bits.view(np.int16)).cuda()
    B = case.batch
    out = torch.empty((B, t, 64, 256), dtype=torch.int16, device="cuda")
    lse = torch.empty((B, t, 64), dtype=torch.float32, device="cuda")
    h = hz.create_handle(dc, max_batch=B * t, split_tokens=split)
    try:
        m.mfa_decode_mtp(h, q, dc.kv(), t, out, lse, B)
        torch.cuda.synchronize()
    finally:
        m.mfa_destroy(h)
    return out, lse


def _check(case, t, split, seed, label, std=1.0):
    _, hz = _mfa()
    _say(f"[mtp] {label}: B={case.batch} t={t} kv={case.kv_dtype} paged={case.paged} "
         f"L=[{case.seq_lens.min()},{case.seq_lens.max()}] split={split}")
    qb = _q(case.batch, t, seed, std)
    out, lse = _run_mtp(case, qb, t, split)
    o_ref, lse_ref = oracle.attention_mtp(oracle.decode_bf16(qb), case.k, case.v, case.seq_lens,
                                          kv_dtype=oracle.KV_FP8 if case.kv_dtype == "fp8" else oracle.KV_BF16,
                                          k_scale=case.k_scale, v_scale=case.v_scale,
                                          page_table=case.page_table, softmax_scale=case.softmax_scale)
    o = hz.bf16_to_f64(out)
    lg = lse.cpu().numpy().astype(np.float64)
    seen = np.isfinite(lse_ref)
    err = np.abs(o - o_ref).max(axis=-1) / np.maximum(np.abs(o_ref).max(axis=-1), 1e-30)
    e = float(err[seen].max()) if seen.any() else 0.0
    el = float(np.abs(lg[seen] - lse_ref[seen]).max()) if seen.any() else 0.0
    _say(f"    row-rel err {e:.3e}  lse abs err {el:.3e}")
    assert e <= TOL and el <= LSE_TOL
    # tokens that see no row: out 0, lse -inf
    assert np.all(o[~seen] == 0) and np.all(np.isneginf(lg[~seen]))
    return out, lse


@pytest.mark.parametrize("t", [2, 3, 4])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_mtp_contiguous(t, kv):
    L = [1, 2, 63, 64, 65, 300, 1000]
    case = synth.make_case("mtp", len(L), L, kv, seed=100 + t)
    _check(case, t, 256, 200 + t, f"contiguous {kv}")


@pytest.mark.parametrize("split", [0, 128, 1024])
def test_mtp_paged_ragged(split):
    case = synth.config_case(4, batch=20, scale_len=1 / 16)
    _check(case, 2, split, 210, "paged ragged fp8")


def test_mtp_fused_merge_and_combine():
    """Two chunks (merged in the attention kernel) and many chunks (combine
    kernel), t = 3."""
    case = synth.config_case(3, batch=4, scale_len=0.25)          # L = 1024
    _check(case, 3, 512, 220, "two chunks")
    _check(case, 3, 128, 221, "eight chunks")


def test_mtp_one_token_equals_decode():
    m, hz = _mfa()
    case = synth.config_case(3, batch=5, scale_len=0.25)
    dc = hz.to_device(case)
    h = hz.create_handle(dc, split_tokens=256)
    try:
        o1, l1 = hz.alloc_outputs(dc)
        o2, l2 = hz.alloc_outputs(dc)
        m.mfa_decode(h, dc.q, dc.kv(), o1, l1, dc.batch)
        m.mfa_decode_mtp(h, dc.q, dc.kv(), 1, o2, l2, dc.batch)
        torch.cuda.synchronize()
    finally:
        m.mfa_destroy(h)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_mtp_tokens_equal_single_decodes():
    """Token j of a t-token call is bitwise the single-token decode of the same
    query over the first L - (t-1-j) rows (same chunking)."""
    m, hz = _mfa()
    t = 3
    case = synth.make_case("mtp_eq", 6, [5, 64, 130, 700, 2, 1500], "fp8", seed=230, paged=True)
    qb = _q(case.batch, t, 231)
    out, lse = _run_mtp(case, qb, t, 256)
    for j in range(t):
        single = synth.make_case("mtp_eq", 6, [5, 64, 130, 700, 2, 1500], "fp8", seed=230, paged=True)
        single.seq_lens = np.maximum(0, case.seq_lens - (t - 1 - j)).astype(np.int32)
        single.q = np.ascontiguousarray(qb[:, j])
        dc = hz.to_device(single)
        h = hz.create_handle(dc, split_tokens=256, max_context=int(case.seq_lens.max()))
        try:
            o, l = hz.alloc_outputs(dc)
            m.mfa_decode(h, dc.q, dc.kv(max_seq_len=int(case.seq_lens.max())), o, l, dc.batch)
            torch.cuda.synchronize()
        finally:
            m.mfa_destroy(h)
        _say(f"[mtp] token {j} against single decodes")
        assert torch.equal(o, out[:, j].contiguous()) and torch.equal(l, lse[:, j].contiguous())


def test_mtp_rejects_bad_arguments():
    m, hz = _mfa()
    case = synth.config_case(1)
    dc = hz.to_device(case)
    h = hz.create_handle(dc, max_batch=2)
    try:
        o = torch.empty((1, 3, 64, 256), dtype=torch.int16, device="cuda")
        for t, needle in ((0, "num_tokens"), (17, "num_tokens"), (3, "max_batch")):
            with pytest.raises(m.MfaError) as ei:
                m.mfa_decode_mtp(h, dc.q, dc.kv(), t, o, None, 1)
            assert needle in str(ei.value)
    finally:
        m.mfa_destroy(h)


def test_mtp_full_size_fp8():
    """The FP8 contiguous workload's size (B = 128, L = 4096) with two query
    tokens, in bench.py's configuration: sampled sequences against the oracle."""
    _, hz = _mfa()
    case = synth.config_case(3)
    t = 2
    qb = _q(case.batch, t, 240)
    _say(f"[mtp full size] B={case.batch} t={t}")
    out, lse = _run_mtp(case, qb, t, 0)
    o = hz.bf16_to_f64(out)
    idx = np.array([0, 37, 64, 127])
    sub = synth.Case(name="s", batch=len(idx), kv_dtype="fp8", seq_lens=case.seq_lens[idx], k=case.k[idx],
                     v=case.v[idx], k_scale=case.k_scale, v_scale=case.v_scale)
    o_ref, lse_ref = oracle.attention_mtp(oracle.decode_bf16(qb[idx]), sub.k, sub.v, sub.seq_lens,
                                          kv_dtype=oracle.KV_FP8, k_scale=sub.k_scale, v_scale=sub.v_scale)
    err = np.abs(o[idx] - o_ref).max(axis=-1) / np.maximum(np.abs(o_ref).max(axis=-1), 1e-30)
    el = np.abs(lse.cpu().numpy()[idx] - lse_ref).max()
    _say(f"    row-rel err {err.max():.3e}  lse abs err {el:.3e}")
    assert err.max() <= TOL and el <= LSE_TOL
    assert np.isfinite(o).all()


def test_mtp_split_policy():
    """The chunk mfa_split_tokens_mtp reports: 128 x 4096 with 2 or 4 tokens
    per sequence takes each sequence whole (4096), one token gives
    mfa_decode's chunked split (2048 here), a fixed split_tokens wins, and the
    argument checks hold."""
    m, hz = _mfa()
    case = synth.config_case(3, batch=2, scale_len=0.25)
    dc = hz.to_device(case)
    h = hz.create_handle(dc, max_context=4096, max_batch=512)
    try:
        assert m.mfa_split_tokens_mtp(h, 128, 2, 4096) == 4096
        assert m.mfa_split_tokens_mtp(h, 128, 4, 4096) == 4096
        assert m.mfa_split_tokens_mtp(h, 128, 1, 4096) == 2048
        assert m.mfa_split_tokens_mtp(h, 8, 2, 1000) == 256   # the smallest automatic chunk
        for bad in ((128, 0, 4096), (128, 17, 4096), (0, 2, 4096), (300, 2, 4096)):
            with pytest.raises(RuntimeError):
                m.mfa_split_tokens_mtp(h, *bad)
    finally:
        m.mfa_destroy(h)
    h = hz.create_handle(dc, split_tokens=512, max_context=4096, max_batch=512)
    try:
        assert m.mfa_split_tokens_mtp(h, 128, 2, 4096) == 512
    finally:
        m.mfa_destroy(h)
