"""GPU parity of the query path (mfa_qproj) and of the full layer (mfa_qproj
then mfa_decode) against the fp64 oracle, through the C ABI.

The query rows are compared head by head with the same row-wise normwise
metric as the attention output: ||q_gpu - q_ref||_inf / ||q_ref||_inf over
each (sequence, head) row of 256 values. The GPU rounds the normalised
bottleneck to bf16 before the second product and the query to bf16 at the
end (about 2^-9 relative each); the oracle keeps both in fp64.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _mfa():
    import decode_attention_mfa_amd as m
    from decode_attention_mfa_amd import harness
    return m, harness


def _row_err(a, b):
    err = np.abs(a - b).max(axis=-1) / np.maximum(np.abs(b).max(axis=-1), 1e-30)
    return float(err.max())


@pytest.mark.parametrize("batch", [1, 5, 32, 48, 70])
def test_qproj_parity_full_shape(batch):
    """hidden 7168 -> 2048 -> 64 x 256 at several batch sizes: one partial
    16-row MFMA tile (1, 5), exact tiles (32), one 64-row block (48) and two
    64-row blocks (70, with fewer K splits in the down-projection)."""
    m, hz = _mfa()
    case = synth.config_case(2, batch=batch, scale_len=1 / 64)
    _say(f"[qproj] B={batch} hidden=7168 rank=2048")
    dc = hz.to_device(case)
    h = hz.create_handle(dc)
    try:
        q = hz.qproj(h, dc)
        torch.cuda.synchronize()
    finally:
        m.mfa_destroy(h)
    q_ref = oracle.case_q(case)
    e = _row_err(hz.bf16_to_f64(q), q_ref)
    _say(f"    row-rel err {e:.3e}")
    assert e <= TOL, e


def test_qproj_repeat_calls_bitwise():
    """The down-projection's arrival counters return to zero after every
    call, and its split sums do not depend on which workgroup finishes last:
    the same inputs give the same bits on every call, across calls of other
    batch sizes (and so other K splits) on the same handle."""
    m, hz = _mfa()
    case = synth.config_case(2, batch=70, scale_len=1 / 64)
    _say(f"[qproj repeat] B=70/5/32 hidden=7168 rank=2048")
    dc = hz.to_device(case)
    h = hz.create_handle(dc)
    try:
        outs = {}
        for b in (5, 70, 5, 32, 5, 70, 32):
            q = torch.empty((b, 64, 256), dtype=torch.int16, device="cuda")
            m.mfa_qproj(h, dc.x[:b].contiguous(), dc.w_qa, dc.gamma, dc.w_qb, q, b)
            torch.cuda.synchronize()
            outs.setdefault(b, []).append(q.cpu())
    finally:
        m.mfa_destroy(h)
    for b, qs in outs.items():
        for q in qs[1:]:
            assert torch.equal(q, qs[0]), b
    # the first rows do not depend on how many rows the call has
    assert torch.equal(outs[5][0], outs[32][0][:5])
    q_ref = oracle.case_q(case)
    e = _row_err(hz.bf16_to_f64(outs[70][0]), q_ref)
    assert e <= TOL, e


def test_qproj_parity_small_shape():
    """A smaller layer shape through the same ABI: hidden 1024, rank 128,
    batch 17, a non-unit RMSNorm weight and eps 1e-3."""
    m, hz = _mfa()
    B, hidden, rank, nq = 17, 1024, 128, 64 * 256
    g = np.random.default_rng(4242)
    x = synth.bf16_bits(g.standard_normal((B, hidden), dtype=np.float32) * np.float32(3.0))
    wa = synth.bf16_bits(g.standard_normal((hidden, rank), dtype=np.float32) / np.float32(np.sqrt(hidden)))
    gamma = synth.bf16_bits(g.uniform(0.5, 1.5, rank).astype(np.float32))
    wb = synth.bf16_bits(g.standard_normal((rank, nq), dtype=np.float32) / np.float32(np.sqrt(rank)))
    dev = [torch.from_numpy(a.view(np.int16)).cuda() for a in (x, wa, gamma, wb)]
    q = torch.empty((B, nq), dtype=torch.int16, device="cuda")
    h = m.mfa_create(hidden=hidden, q_rank=rank, max_batch=B, max_context=64, rms_eps=1e-3)
    try:
        _say(f"[qproj] B={B} hidden={hidden} rank={rank}")
        m.mfa_qproj(h, *dev, q, B)
        torch.cuda.synchronize()
    finally:
        m.mfa_destroy(h)
    q_ref = oracle.qproj(x, wa, gamma, wb, eps=1e-3).reshape(B, 64, 256)
    e = _row_err(hz.bf16_to_f64(q).reshape(B, 64, 256), q_ref)
    _say(f"    row-rel err {e:.3e}")
    assert e <= TOL, e


def test_qproj_rejects_bad_arguments():
    m, hz = _mfa()
    h = m.mfa_create(hidden=1024, q_rank=128, max_batch=4, max_context=64)
    try:
        t = torch.zeros(16, dtype=torch.int16, device="cuda")
        with pytest.raises(m.MfaError):
            m.mfa_qproj(h, t, t, t, t, t, 5)          # batch > max_batch
        with pytest.raises(m.MfaError):
            m.mfa_qproj(h, None, t, t, t, t, 1)       # null input
    finally:
        m.mfa_destroy(h)


def test_full_layer_parity():
    """Q projection then decode attention (bf16 KV, split into chunks) against
    the oracle's fp64 projection and attention."""
    m, hz = _mfa()
    case = synth.config_case(2, batch=6, scale_len=1 / 4)
    _say(f"[full layer] B={case.batch} L={int(case.seq_lens[0])}")
    dc = hz.to_device(case)
    out, lse, _ = hz.run_case(dc, split_tokens=256)
    o_ref, lse_ref = oracle.case_attention(case)
    e = _row_err(hz.bf16_to_f64(out), o_ref)
    el = float(np.abs(lse.cpu().numpy() - lse_ref).max())
    _say(f"    row-rel err {e:.3e}  lse abs err {el:.3e}")
    assert e <= TOL, e
    assert el <= 1e-2, el
