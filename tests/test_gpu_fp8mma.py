"""GPU parity of the FP8-MFMA attention mode (MFA_ATTN_FP8_MFMA: FP8 MFMAs on
the cache's codes, Q quantised per head and P quantised to E4M3).

The mode is compared with the oracle of its own arithmetic,
``oracle.attention_fp8mma`` (pinned in tests/test_oracle_fp8mma.py): the same
per-head power-of-two query scale, E4M3 round-to-nearest-even of the query
and of 4 P against an integer reference, normalisation by the sum of the
applied weights. The oracle sums products exactly; the FP8 MFMAs do not: they
add groups of products aligned to the group's largest one, with an error of
up to about 2^-12 of that product's binade (measured by
test_fp8_mfma_sum_accuracy below; the accumulator input is added exactly).

- On inputs whose products are exact in such sums (tests/fp8_inputs.py:
  integer E4M3 query values, keys 0, +-1/2, +-1, +-2, values 0, +-1; the
  quantisers still round, and the mode still differs from exact attention
  by about 6%), the GPU and the oracle take the same decisions. What remains
  is the bf16 rounding of the output and of a piece's partial before a merge
  (2^-9 each) and, for a weight below E4M3's smallest normal value, the
  finer grid the GPU may use when a piece's reference is below the oracle's
  (at most 2^-12 of the largest weight per such token): the bar is 2^-7
  row-wise and 1e-3 on the log-sum-exp. A round-toward-zero quantiser or a
  flush of the subnormal weights exceeds it (shown on the CPU).
- On N(0,1) inputs the inexact MFMA sums move scores by about 1e-3 (base 2)
  and outputs by up to a few percent: those cases are checked against the
  bars TOL_F8_HW and LSE_TOL_F8_HW, and the mode's distance from exact
  attention must stay within the modelled arithmetic's own distance plus
  that bar.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from fp8_inputs import exact_dot_case, subnormal_case

pytestmark = pytest.mark.gpu

TOL_F8 = 2.0 ** -7   # row-wise normwise, against the FP8-arithmetic oracle (exact-sum inputs)
LSE_TOL_F8 = 1e-3    # absolute, natural log, against the same
TOL_F8_HW = 6e-2     # the same on N(0,1) inputs, where the FP8 MFMAs' sums are inexact
LSE_TOL_F8_HW = 3e-2


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _mfa():
    import decode_attention_mfa_amd as m
    from decode_attention_mfa_amd import harness
    return m, harness


def _run(case, split, attn_math):
    m, hz = _mfa()
    dc = hz.to_device(case)
    h = hz.create_handle(dc, split_tokens=split, attn_math=attn_math)
    try:
        out, lse = hz.decode(h, dc)
        torch.cuda.synchronize()
    finally:
        m.mfa_destroy(h)
    return hz.bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)


def _rowerr(a, b, rows):
    if not rows.any():
        return 0.0
    e = np.abs(a - b).max(axis=-1) / np.maximum(np.abs(b).max(axis=-1), 1e-30)
    return float(e[rows].max())


def check_f8(case, split, label, exact_sums=False):
    m, _ = _mfa()
    _say(f"[fp8 mfma] {label}: B={case.batch} paged={case.paged} L=[{case.seq_lens.min()},"
         f"{case.seq_lens.max()}] split={split}")
    o, lse = _run(case, split, m.MFA_ATTN_FP8_MFMA)
    o_ref8, lse_ref8 = oracle.case_attention_fp8mma(case)
    nz = case.seq_lens > 0
    e8 = _rowerr(o, o_ref8, nz)
    el = float(np.abs(lse[nz] - lse_ref8[nz]).max()) if nz.any() else 0.0
    # budget report: the mode against exact attention, beside the modelled
    # arithmetic against exact attention
    o_ex, _ = oracle.case_attention(case)
    eg, em = _rowerr(o, o_ex, nz), _rowerr(o_ref8, o_ex, nz)
    _say(f"    vs FP8 oracle: row-rel {e8:.3e}  lse {el:.3e}   vs exact: gpu {eg:.3e}, oracle {em:.3e}")
    tol, ltol = (TOL_F8, LSE_TOL_F8) if exact_sums else (TOL_F8_HW, LSE_TOL_F8_HW)
    assert e8 <= tol and el <= ltol
    assert eg <= em + tol
    if (~nz).any():
        assert np.all(o[~nz] == 0) and np.all(np.isneginf(lse[~nz]))
    return o, lse


@pytest.mark.parametrize("split,paged", [(0, False), (256, False), (1024, False), (-1, False), (0, True),
                                         (128, True), (-1, True)])
def test_fp8_mma_exact_sums(split, paged):
    """Tight parity where the MFMA sums are exact (module docstring)."""
    lens = [4096, 2049, 1000, 130, 64, 1, 0, 3000]
    check_f8(exact_dot_case(31, lens, paged=paged), split, "exact sums", exact_sums=True)


def test_fp8_mfma_sum_accuracy():
    """The FP8 MFMA of the mode against exact sums: the accumulator input is
    added exactly; the products' sum is exact when its terms fit 12 bits below
    the largest product, and within 2^-10 of the largest product's binade
    otherwise (measured: about 2^-12 to 2^-11)."""
    m, _ = _mfa()
    tab = oracle.e4m3_table()
    g = np.random.default_rng(4)
    n = 64
    kinds = []
    a = np.empty((n, 16, 128), np.uint8)
    b = np.empty((n, 128, 16), np.uint8)
    c = np.zeros((n, 16, 16), np.float32)
    for t in range(n):
        kind = t % 4
        kinds.append(kind)
        if kind == 0:     # N(0,1)-like codes
            a[t] = synth.e4m3_codes(g.standard_normal((16, 128)) * 30)
            b[t] = synth.e4m3_codes(g.standard_normal((128, 16)) * 30)
        elif kind == 1:   # wide dynamic range
            a[t] = synth.e4m3_codes(np.sign(g.standard_normal((16, 128))) * 2.0 ** g.uniform(-9, 8.8, (16, 128)))
            b[t] = synth.e4m3_codes(np.sign(g.standard_normal((128, 16))) * 2.0 ** g.uniform(-9, 8.8, (128, 16)))
        elif kind == 2:   # small integers: exact sums, with a large accumulator input
            a[t] = synth.e4m3_codes(g.integers(-4, 5, (16, 128)).astype(np.float64))
            b[t] = synth.e4m3_codes(g.integers(-4, 5, (128, 16)).astype(np.float64))
            c[t] = (2.0 ** 20 + 0.5) * np.sign(g.standard_normal((16, 16)))
        else:             # the exact-sum attention inputs: weights' codes times +-1
            a[t] = synth.e4m3_codes(4.0 * 2.0 ** g.uniform(-12, 0, (16, 128)))
            b[t] = synth.e4m3_codes(g.choice([0.0, 1.0, -1.0], size=(128, 16)))
    dev = lambda x: torch.from_numpy(x).cuda()
    d = torch.empty((n, 16, 16), dtype=torch.float32, device="cuda")
    m.mfa_debug_fp8_mfma(dev(a), dev(b), dev(c), d, n)
    torch.cuda.synchronize()
    d = d.cpu().numpy().astype(np.float64)
    A, Bm = tab[a], tab[b]
    exact = np.einsum("tik,tkj->tij", A, Bm) + c
    prods = np.abs(A[:, :, :, None] * Bm[:, None, :, :])          # [t, i, k, j]
    binade = 2.0 ** np.floor(np.log2(np.maximum(prods.max(axis=2), 1e-300)))
    rel = np.abs(d - exact) / binade
    for kind in range(4):
        sel = np.array(kinds) == kind
        _say(f"[fp8 mfma sums] kind {kind}: max |d - exact| / binade(max product) = {rel[sel].max():.3e}")
    assert rel.max() <= 2.0 ** -10
    ex = np.isin(kinds, [2, 3])
    assert np.array_equal(d[ex], exact[ex])


@pytest.mark.parametrize("split", [0, 256, 1024])
def test_fp8_mma_contiguous(split):
    check_f8(synth.config_case(3, batch=3, scale_len=0.5), split, "fp8 contiguous B=3 L=2048")


@pytest.mark.parametrize("split", [0, 128, -1])
def test_fp8_mma_paged_ragged(split):
    check_f8(synth.config_case(4, batch=24, scale_len=1 / 16), split, "paged ragged")


def test_fp8_mma_ragged_tails_and_empty():
    L = [0, 1, 63, 64, 65, 127, 129, 1000, 2049, 0]
    case = synth.make_case("f8tails", len(L), L, "fp8", seed=120, kv_slack=3)
    check_f8(case, 256, "ragged tails")
    check_f8(case, -1, "ragged tails balanced")


def test_fp8_mma_peaky_scores_restart():
    """Q scaled by 4: later scores exceed the first step's maxima by more than
    the FP8 mode's bound (2^6), so the pieces restart with raised
    references (N(0,1) inputs: the hardware bar)."""
    check_f8(synth.config_case(3, batch=2, scale_len=0.25, q_std=4.0), 256, "peaky q")


@pytest.mark.parametrize("split", [0, 256, -1])
def test_fp8_mma_subnormal_weights(split):
    """Almost every weight's 4 P is an E4M3 subnormal and their share of the
    output is about 7%: a flush, or a threshold an octave off, moves the
    output by more than the bar (tests/test_oracle_fp8mma.py)."""
    q, k, v, ks, vs = subnormal_case(7, [4000, 4096, 1000])
    case = synth.Case(name="f8sub", batch=3, kv_dtype="fp8", seq_lens=np.array([4000, 4096, 1000], np.int32),
                      k=k, v=v, q=q, k_scale=ks, v_scale=vs)
    o, _ = check_f8(case, split, "subnormal weights", exact_sums=True)
    assert 0.03 < o[:, :, 128:].mean() < 0.15


def test_fp8_mma_differs_from_bf16_path():
    """The mode is really in effect (its rounding differs from the default
    path's), and the default path stays within its own 1e-2 bar."""
    m, _ = _mfa()
    case = synth.config_case(3, batch=2, scale_len=0.25)
    o8, _ = _run(case, 256, m.MFA_ATTN_FP8_MFMA)
    o16, _ = _run(case, 256, m.MFA_ATTN_BF16_MFMA)
    o_ref, _ = oracle.case_attention(case)
    e16 = (np.abs(o16 - o_ref).max(axis=-1) / np.abs(o_ref).max(axis=-1)).max()
    d = (np.abs(o8 - o16).max(axis=-1) / np.abs(o16).max(axis=-1)).max()
    _say(f"[fp8 mfma] default path err {e16:.3e}, fp8 vs default {d:.3e}")
    assert e16 <= 1e-2 and d > 1e-3


def test_fp8_mma_rejected_where_unsupported():
    m, hz = _mfa()
    with pytest.raises(m.MfaError) as ei:
        m.mfa_create(kv_dtype="bf16", attn_math=m.MFA_ATTN_FP8_MFMA)
    assert ei.value.status == m.MFA_ERR_UNSUPPORTED and "FP8 cache" in str(ei.value)
    case = synth.config_case(3, batch=1, scale_len=1 / 16)
    dc = hz.to_device(case)
    h = hz.create_handle(dc, max_batch=2, attn_math=m.MFA_ATTN_FP8_MFMA)
    try:
        q = torch.zeros((1, 2, 64, 256), dtype=torch.int16, device="cuda")
        o = torch.empty_like(q)
        with pytest.raises(m.MfaError) as ei:
            m.mfa_decode_mtp(h, q, dc.kv(), 2, o, None, 1)
        assert "bf16 MFMAs" in str(ei.value)
    finally:
        m.mfa_destroy(h)


@pytest.mark.parametrize("cfg", [3, 4])
def test_fp8_mma_full_size(cfg):
    """The FP8 workloads at full size in the FP8-MFMA mode: sampled sequences
    against the oracle."""
    m, hz = _mfa()
    case = synth.config_case(cfg)
    _say(f"[fp8 mfma full size] workload {cfg}: B={case.batch}")
    o, lse = _run(case, None, m.MFA_ATTN_FP8_MFMA)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    idx = np.unique(np.concatenate([np.linspace(0, case.batch - 1, 6).astype(int),
                                    [int(np.argmin(case.seq_lens)), int(np.argmax(case.seq_lens))]]))
    sub = synth.Case(name="s", batch=len(idx), kv_dtype="fp8", seq_lens=case.seq_lens[idx], k=None, v=None,
                     q=case.q[idx], k_scale=case.k_scale, v_scale=case.v_scale)
    if case.paged:
        sub.k, sub.v, sub.page_table = case.k, case.v, case.page_table[idx]
    else:
        sub.k, sub.v = case.k[idx], case.v[idx]
    o_ref, lse_ref = oracle.case_attention_fp8mma(sub)
    err = np.abs(o[idx] - o_ref).max(axis=-1) / np.maximum(np.abs(o_ref).max(axis=-1), 1e-30)
    el = np.abs(lse[idx] - lse_ref).max()
    _say(f"    vs FP8 oracle: row-rel err {err.max():.3e}  lse abs err {el:.3e}")
    assert err.max() <= TOL_F8_HW and el <= LSE_TOL_F8_HW


def test_head_split_policy():
    """FP8-MFMA mode at the FP8 workload's size: the 64 heads go to two
    workgroups per sequence (one chunk each, nothing to merge); with bf16
    MFMAs they stay together and each sequence takes two chunks."""
    m, hz = _mfa()
    case = synth.config_case(3, batch=1)
    dc = hz.to_device(case)
    for math, groups in ((m.MFA_ATTN_FP8_MFMA, 2), (m.MFA_ATTN_BF16_MFMA, 1)):
        h = hz.create_handle(dc, max_batch=128, attn_math=math)
        try:
            n_cu = torch.cuda.get_device_properties(0).multi_processor_count
            g = m.mfa_head_groups(h, 128, 4096, 4096)
            split = m.mfa_split_tokens(h, 128, 4096, 4096)
            _say(f"[head split] math={math} cu={n_cu} groups={g} split={split}")
            if n_cu == 256:
                assert g == groups
                assert split == (4096 if groups == 2 else 2048)
            assert g in (1, 2)
            if g == 2:   # the doubled grid fits on the compute units at once
                assert 2 * 128 * ((4096 + split - 1) // split) <= n_cu
        finally:
            m.mfa_destroy(h)
