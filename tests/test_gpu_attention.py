"""GPU parity of mfa_decode against the fp64 oracle, through the C ABI.

Metric (one reading of "max relative error 1e-2"): for every (sequence,
head) row, ||o_gpu - o_ref||_inf / ||o_ref||_inf; the test takes the max over
rows. Element-wise relative error is meaningless on near-zero entries of a
softmax average. The log-sum-exp is compared in absolute terms.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 1e-2        # row-wise normwise relative error of the bf16 output
LSE_TOL = 1e-3    # absolute, natural log


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _mfa():
    import decode_attention_mfa_amd as m
    from decode_attention_mfa_amd import harness
    return m, harness


def row_err(o_gpu, o_ref, lens=None):
    err = np.abs(o_gpu - o_ref).max(axis=-1) / np.maximum(np.abs(o_ref).max(axis=-1), 1e-30)
    if lens is not None:
        err = err[np.asarray(lens) > 0]
    return float(err.max()) if err.size else 0.0


def check_parity(case, split_tokens=None, label=""):
    m, hz = _mfa()
    _say(f"[parity] {label or case.name}: B={case.batch} kv={case.kv_dtype} paged={case.paged} "
         f"L=[{case.seq_lens.min()},{case.seq_lens.max()}] split={split_tokens}")
    dc = hz.to_device(case)
    out, lse, _ = hz.run_case(dc, split_tokens=split_tokens)
    o_ref, lse_ref = oracle.case_attention(case)
    o = hz.bf16_to_f64(out)
    lse_gpu = lse.cpu().numpy().astype(np.float64)
    nz = case.seq_lens > 0
    e = row_err(o, o_ref, case.seq_lens)
    el = float(np.abs(lse_gpu[nz] - lse_ref[nz]).max()) if nz.any() else 0.0
    _say(f"    row-rel err {e:.3e}  lse abs err {el:.3e}")
    assert e <= TOL, e
    assert el <= LSE_TOL, el
    if (~nz).any():
        assert np.all(o[~nz] == 0) and np.all(np.isneginf(lse_gpu[~nz]))
    return out, lse


def test_tiny_config():
    check_parity(synth.config_case(1), label="tiny B=1 L=256 bf16")


@pytest.mark.parametrize("split", [0, 64, 192, 512, 704, 1024, 4096])
def test_fp8_contiguous_splits(split):
    check_parity(synth.config_case(3, batch=3, scale_len=0.5), split_tokens=split,
                 label=f"fp8 contiguous B=3 L=2048 split={split}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_ragged_tails(kv):
    L = [1, 63, 64, 65, 127, 129, 1000, 2049]
    case = synth.make_case("ragged", len(L), L, kv, seed=77, kv_slack=5)
    check_parity(case, split_tokens=256, label=f"ragged tails {kv}")
    check_parity(case, split_tokens=0, label=f"ragged tails {kv} auto split")


@pytest.mark.parametrize("lens", [[256], [1, 700], [4096, 3000, 65]])
def test_bf16_head_groups(lens):
    """bf16 caches whose grid would use at most a quarter of the compute units
    run four workgroups of 16 heads per (sequence, chunk): parity with the
    oracle, and the output is bitwise the one of 64-head workgroups on the
    same chunks (the head groups change no arithmetic of a head), here from a
    batch repeated until its grid is large enough for 64-head workgroups."""
    m, hz = _mfa()
    case = synth.make_case("bf16_hg", len(lens), lens, "bf16", seed=81, kv_slack=3)
    dc = hz.to_device(case)
    h = hz.create_handle(dc, split_tokens=0)
    try:
        groups = m.mfa_head_groups(h, dc.batch, dc.max_len, dc.min_len)
        chunk = m.mfa_split_tokens(h, dc.batch, dc.max_len, dc.min_len)
    finally:
        m.mfa_destroy(h)
    _say(f"[bf16 head groups] lens={lens}: {groups} groups, chunk {chunk}")
    assert groups == 4
    out, _ = check_parity(case, split_tokens=0, label="bf16 head groups")
    reps = 1
    while True:
        reps *= 2
        big = synth.Case(name="rep", batch=case.batch * reps, kv_dtype="bf16", seq_lens=np.tile(case.seq_lens, reps),
                         k=np.tile(case.k, (reps, 1, 1)), v=np.tile(case.v, (reps, 1, 1)),
                         q=np.tile(case.q, (reps, 1, 1)), k_scale=case.k_scale, v_scale=case.v_scale)
        bdc = hz.to_device(big)
        h = hz.create_handle(bdc, split_tokens=chunk)
        try:
            g1 = m.mfa_head_groups(h, bdc.batch, bdc.max_len, bdc.min_len)
        finally:
            m.mfa_destroy(h)
        if g1 == 1:
            break
        assert reps < 4096
    out1, _, _ = hz.run_case(bdc, split_tokens=chunk)
    assert torch.equal(out.cpu(), out1.cpu()[:case.batch])


def test_empty_sequences():
    case = synth.make_case("empty", 4, [0, 5, 0, 300], "fp8", seed=78)
    check_parity(case, split_tokens=128, label="empty sequences")


def test_peaky_scores():
    """Q scaled by 8: logits with std ~8 exercise the running-max rescale."""
    case = synth.config_case(3, batch=2, scale_len=0.25, q_std=8.0)
    check_parity(case, split_tokens=256, label="peaky fp8")
    case = synth.config_case(5, batch=2, scale_len=1 / 32, q_std=8.0)
    check_parity(case, label="peaky bf16")


def test_paged_ragged_reduced():
    check_parity(synth.config_case(4, batch=24, scale_len=1 / 16), label="paged ragged B=24")
    check_parity(synth.config_case(4, batch=24, scale_len=1 / 16), split_tokens=128,
                 label="paged ragged B=24 split=128")


BAL = -1   # MFA_SPLIT_BALANCED


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("paged", [False, True])
def test_balanced_ragged(kv, paged):
    """Equal step ranges per workgroup over ragged lengths (empty, one token,
    page edges): pieces that start and end inside sequences."""
    L = [0, 1, 63, 64, 65, 127, 129, 1000, 2049, 0, 300]
    case = synth.make_case("bal", len(L), L, kv, seed=81, paged=paged, kv_slack=0 if paged else 5)
    check_parity(case, split_tokens=BAL, label=f"balanced ragged {kv} paged={paged}")


def test_balanced_many_short_sequences():
    """Several sequences per workgroup range (300 sequences of 0..299 tokens)."""
    L = np.random.default_rng(82).integers(0, 300, 300).astype(np.int32)
    case = synth.make_case("bal_short", len(L), L, "fp8", seed=83, paged=True)
    check_parity(case, split_tokens=BAL, label="balanced 300 short sequences fp8 paged")


def test_balanced_long_and_short():
    """One long sequence among short ones is cut into ~80 pieces, merged by
    the last piece to finish."""
    case = synth.make_case("bal_long", 4, [20000, 10, 5, 3000], "bf16", seed=84)
    check_parity(case, split_tokens=BAL, label="balanced long + short bf16")


def test_balanced_auto_for_large_batches():
    """The per-call choice takes the balanced split for a batch of 128 or
    more (fp8 paged ragged, reduced lengths)."""
    m, hz = _mfa()
    case = synth.config_case(4, batch=160, scale_len=1 / 32)
    dc = hz.to_device(case)
    h = hz.create_handle(dc, split_tokens=0)
    try:
        # lengths unknown, or known to differ in step count: balanced
        assert m.mfa_split_tokens(h, dc.batch, dc.max_len) == 0
        assert m.mfa_split_tokens(h, dc.batch, dc.max_len, dc.min_len) == 0
        # every sequence with the same number of steps: equal chunks
        assert m.mfa_split_tokens(h, dc.batch, 4096, 4033) > 0
    finally:
        m.mfa_destroy(h)
    check_parity(case, split_tokens=0, label="paged ragged B=160 auto (balanced)")


def test_long_splitk_reduced():
    check_parity(synth.config_case(5, batch=4, scale_len=1 / 16), label="long split-K B=4 L=2K/4K")


def test_paged_equals_contiguous_bitwise():
    """Same logical rows via a permuted page table and via a contiguous cache,
    same chunking: bitwise identical outputs."""
    m, hz = _mfa()
    for kv in ("fp8", "bf16"):
        pc = synth.make_case("p", 6, [1, 64, 65, 700, 1500, 333], kv, seed=79, paged=True,
                             max_context=1536)
        maxL = int(pc.seq_lens.max())
        kc = np.zeros((pc.batch, maxL, 256), pc.k.dtype)
        vc = np.zeros_like(kc)
        for b in range(pc.batch):
            t = np.arange(int(pc.seq_lens[b]))
            pages = pc.page_table[b, t // 64]
            kc[b, :len(t)] = pc.k[pages, t % 64]
            vc[b, :len(t)] = pc.v[pages, t % 64]
        cc = synth.Case(name="c", batch=pc.batch, kv_dtype=kv, seq_lens=pc.seq_lens, k=kc, v=vc,
                        q=pc.q, k_scale=pc.k_scale, v_scale=pc.v_scale)
        for split in (128, 512, BAL):
            _say(f"[bitwise] paged vs contiguous {kv} split={split}")
            o1, l1, _ = hz.run_case(hz.to_device(pc), split_tokens=split)
            o2, l2, _ = hz.run_case(hz.to_device(cc), split_tokens=split)
            assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("paged", [True, False])
def test_debug_gather_bit_exact(paged):
    """The page-table gather, bit for bit, through the attention kernel's own
    addressing (page indices of a piece of up to 128 steps in registers):
    lengths with partial pages and more than one such piece."""
    m, hz = _mfa()
    for kv in ("fp8", "bf16"):
        pc = synth.make_case("g", 8, [1, 63, 64, 200, 511, 8192, 8193, 20000], kv, seed=80, paged=paged)
        dc = hz.to_device(pc)
        h = hz.create_handle(dc)
        try:
            for b in range(pc.batch):
                _say(f"[gather] {kv} b={b}")
                kd = torch.zeros((dc.max_len, 256), dtype=dc.k.dtype, device="cuda")
                vd = torch.zeros_like(kd)
                m.mfa_debug_gather_kv(h, dc.kv(), b, kd, vd)
                torch.cuda.synchronize()
                kr, vr = oracle.gather_kv(pc.k, pc.v, pc.seq_lens, b, page_table=pc.page_table)
                n = int(pc.seq_lens[b])
                kg = kd[:n].cpu().numpy().view(kr.dtype)
                vg = vd[:n].cpu().numpy().view(vr.dtype)
                assert np.array_equal(kg, kr) and np.array_equal(vg, vr)
        finally:
            m.mfa_destroy(h)


def test_deterministic_run_twice():
    m, hz = _mfa()
    case = synth.config_case(4, batch=16, scale_len=1 / 16)
    dc = hz.to_device(case)
    _say("[determinism] paged fp8 B=16, two runs")
    for split in (128, BAL):
        o1, l1, _ = hz.run_case(dc, split_tokens=split)
        o2, l2, _ = hz.run_case(dc, split_tokens=split)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_in_kernel_merge_is_order_independent():
    """Two chunks per sequence merged inside the attention kernel by
    whichever workgroup of the pair finishes last: every run gives the same
    bits, whatever the finishing order was."""
    m, hz = _mfa()
    case = synth.config_case(3, batch=64, scale_len=0.5)   # FP8 contiguous, 2048 tokens
    dc = hz.to_device(case)
    _say("[determinism] fp8 contiguous B=64 L=2048, split 1024, five runs")
    o1, l1, _ = hz.run_case(dc, split_tokens=1024)
    for _ in range(4):
        o2, l2, _ = hz.run_case(dc, split_tokens=1024)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, lse_ref = oracle.case_attention(case)
    assert row_err(hz.bf16_to_f64(o1), o_ref) <= TOL


def test_lse_null_is_allowed():
    m, hz = _mfa()
    case = synth.config_case(1)
    dc = hz.to_device(case)
    h = hz.create_handle(dc)
    try:
        out = torch.empty((1, 64, 256), dtype=torch.int16, device="cuda")
        m.mfa_decode(h, dc.q, dc.kv(), out, None, 1)
        torch.cuda.synchronize()
        o_ref, _ = oracle.case_attention(case)
        assert row_err(hz.bf16_to_f64(out), o_ref) <= TOL
    finally:
        m.mfa_destroy(h)


def test_host_errors_enqueue_nothing():
    m, hz = _mfa()
    case = synth.config_case(1)
    dc = hz.to_device(case)
    h = hz.create_handle(dc)
    try:
        out = torch.full((1, 64, 256), 7, dtype=torch.int16, device="cuda")
        with pytest.raises(m.MfaError) as ei:
            m.mfa_decode(h, dc.q, dc.kv(), out, None, 2)          # batch > max_batch
        assert ei.value.status == m.MFA_ERR_INVALID
        with pytest.raises(m.MfaError):
            m.mfa_decode(h, dc.q, dc.kv(max_seq_len=100000), out, None, 1)
        with pytest.raises(m.MfaError):
            m.mfa_decode(h, None, dc.kv(), out, None, 1)
        torch.cuda.synchronize()
        assert torch.all(out == 7)
    finally:
        m.mfa_destroy(h)
    fp8 = synth.make_case("s", 1, 64, "fp8", seed=81)
    dc = hz.to_device(fp8)
    h = hz.create_handle(dc)
    try:
        kv = dc.kv()
        kv.k_scale = float("nan")
        with pytest.raises(m.MfaError) as ei:
            m.mfa_decode(h, dc.q, kv, torch.empty(1, 64, 256, dtype=torch.int16, device="cuda"), None, 1)
        assert "scale" in str(ei.value)
    finally:
        m.mfa_destroy(h)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_dominant_late_keys_restart(kv):
    """Keys planted late in a sequence whose scores exceed everything before
    them by far more than the kernel's headroom: the chunk must be redone with
    a higher reference (twice here) and still match the oracle."""
    B, L = 2, 1500
    case = synth.make_case("dominant", B, [L, 900], "bf16", seed=82)
    q = oracle.case_q(case)
    K = oracle.decode_bf16(case.k).astype(np.float32)
    for b, t, c in ((0, 700, 3.0), (0, 1300, 6.0), (1, 400, 5.0)):
        K[b, t] = (c * q[b, 5]).astype(np.float32)        # head 5: score ~ c*|q|^2/16
    if kv == "bf16":
        case.k = synth.bf16_bits(K)
    else:
        V = oracle.decode_bf16(case.v).astype(np.float32)
        ks = float(np.float32(np.abs(K).max() / 448.0))
        vs = float(np.float32(np.abs(V).max() / 448.0))
        case = synth.Case(name="dominant-fp8", batch=B, kv_dtype="fp8", seq_lens=case.seq_lens,
                          k=synth.e4m3_codes(K / np.float32(ks)), v=synth.e4m3_codes(V / np.float32(vs)),
                          q=case.q, k_scale=ks, v_scale=vs)
    for split in (0, 512):
        check_parity(case, split_tokens=split, label=f"dominant late keys {kv} split={split}")


@pytest.mark.parametrize("split", [1024, 256, -1])
def test_graph_replay_matches_eager(split):
    """mfa_decode captured into a HIP graph (through torch's capture on a side
    stream), replayed several times with other eager decodes in between: every
    replay equals the eager result bitwise. split 1024 merges the two chunks in
    the attention kernel, 256 uses the combine kernel, -1 (balanced) merges
    the pieces in the attention kernel."""
    m, hz = _mfa()
    case = synth.config_case(3, batch=3, scale_len=0.5)
    other = synth.config_case(3, batch=3, scale_len=0.5, q_std=2.0)
    dc, do = hz.to_device(case), hz.to_device(other)
    h = hz.create_handle(dc, split_tokens=split)
    try:
        st = torch.cuda.Stream()
        out, lse = hz.alloc_outputs(dc)
        oo, lo = hz.alloc_outputs(do)
        kv, kvo = dc.kv(), do.kv()
        with torch.cuda.stream(st):
            m.mfa_decode(h, dc.q, kv, out, lse, dc.batch, st)
        torch.cuda.synchronize()
        ref_o, ref_l = out.clone(), lse.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            m.mfa_decode(h, dc.q, kv, out, lse, dc.batch, st)
        for r in range(4):
            _say(f"[graph] split={split} replay {r}")
            out.zero_()
            lse.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
            with torch.cuda.stream(st):
                m.mfa_decode(h, do.q, kvo, oo, lo, do.batch, st)
            torch.cuda.synchronize()
        o_ref, _ = oracle.case_attention(case)
        assert row_err(hz.bf16_to_f64(out), o_ref) <= TOL
    finally:
        m.mfa_destroy(h)


@pytest.mark.parametrize("trial", range(8))
def test_seeded_random_configurations(trial):
    """Seeded random mixes of batch size, lengths (empty, one token, page
    boundaries, long), cache type and layout, and split (chunks of any page
    multiple, automatic, balanced) against the oracle, so that combinations
    no hand-written case covers still get checked."""
    rng = np.random.default_rng(900 + trial)
    B = int(rng.integers(1, 9))
    pool = [0, 1, 2, 63, 64, 65, 127, 128, 129, 500, 1024, 1500, 2048, 2100, 3000]
    L = [int(rng.choice(pool)) if rng.random() < 0.6 else int(rng.integers(1, 3200)) for _ in range(B)]
    if max(L) == 0:
        L[0] = 1
    kv = "fp8" if rng.random() < 0.6 else "bf16"
    paged = bool(rng.random() < 0.5)
    split = int(rng.choice([0, 64, 128, 320, 1024, -1]))
    case = synth.make_case("random", B, L, kv, seed=910 + trial, paged=paged, kv_slack=int(rng.integers(0, 9)))
    check_parity(case, split_tokens=split, label=f"random trial {trial}: L={L} {kv} paged={paged}")
