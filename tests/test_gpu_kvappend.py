"""GPU parity of mfa_kv_append (the new token's K and V rows written into the
cache) against the fp64 oracle, through the C ABI.

Two kinds of check:
  - exact inputs: each sequence's hidden state has two nonzero entries, so
    every projection value is a sum of two bf16 products that is exact in
    fp32 on both sides; then the stored codes must equal the oracle's bit for
    bit, including values that sit exactly on a rounding tie, saturation and
    the subnormal codes, and every other byte of the cache must be unchanged;
  - the workloads' random recipe: the fp32 accumulation of 7168 products
    differs from the fp64 sum by rounding, so a code may differ from the
    oracle's only where the exact value lies within that rounding of a
    decision boundary (checked element by element), and rarely.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

D = synth.HEAD_DIM
HID = synth.HIDDEN
BF16, FP8 = oracle.KV_BF16, oracle.KV_FP8


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _mfa():
    import decode_attention_mfa_amd as m
    from decode_attention_mfa_amd import harness
    return m, harness


def _bits(a):
    return synth.bf16_bits(np.asarray(a, dtype=np.float32))


def _bf16_val(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def _exact_inputs(B, seed):
    """x [B, HID] with x[b, 2b] = x[b, 2b+1] = 1; W_k, W_v rows 2b and 2b+1
    chosen so that k[b] = W[2b] + W[2b+1] is exact in fp32 and covers E4M3
    and bf16 rounding ties, their neighbours, saturation and tiny values."""
    rng = np.random.default_rng(seed)
    x = np.zeros((B, HID), np.uint16)
    for b in range(B):
        x[b, 2 * b] = x[b, 2 * b + 1] = 0x3F80             # 1.0
    wk = _bits(rng.standard_normal((HID, D)) * 0.02)
    wv = _bits(rng.standard_normal((HID, D)) * 0.02)
    pos = oracle.e4m3_table()[:0x7F]
    mid = (pos[:-1] + pos[1:]) / 2
    mid_b = _bits(mid)
    assert np.array_equal(_bf16_val(mid_b).astype(np.float64), mid)   # ties are bf16 values
    ties = np.concatenate([mid_b, mid_b | 0x8000])                   # 252 values
    near = np.concatenate([mid_b + 1, mid_b - 1, (mid_b + 1) | 0x8000, (mid_b - 1) | 0x8000])
    special = _bits([448, 449, 464, 480, 1000, 1e4, 3e38, -448, -464, -1e4, -3e38,
                     2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -11, 2.0 ** -20, -2.0 ** -10, 0.0, 15 * 2.0 ** -10])
    pool = [ties, near, special]
    for b in range(B):
        kind = b % 4
        for which, w in (("k", wk), ("v", wv)):
            if kind == 0:                      # E4M3 ties and their bf16 neighbours
                vals = np.concatenate(pool)
                r0 = rng.permutation(vals)[:D] if vals.size >= D else np.resize(vals, D)
                r1 = np.zeros(D, np.uint16)
            elif kind == 1:                    # saturation, subnormals, the rest of the ties
                vals = np.concatenate([special, rng.permutation(np.concatenate(pool))])
                r0 = vals[:D]
                r1 = np.zeros(D, np.uint16)
            elif kind == 2:                    # generic fp32 values: |a| in [0.5, 4), |d| in [2^-9, 2^-8)
                a = rng.uniform(0.5, 4.0, D) * rng.choice([-1, 1], D)
                d = rng.uniform(1.0, 2.0, D) * 2.0 ** -9 * rng.choice([-1, 1], D)
                r0, r1 = _bits(a), _bits(d)
            else:                              # bf16 ties: a + half a bf16 step of a
                a = _bf16_val(_bits(rng.uniform(0.25, 64.0, D) * rng.choice([-1, 1], D)))
                e = np.floor(np.log2(np.abs(a.astype(np.float64))))
                half = 2.0 ** (e - 8) * np.sign(a) * rng.choice([-1, 1], D)
                r0, r1 = _bits(a), _bits(half)
            w[2 * b] = r0
            w[2 * b + 1] = r1
    return x, wk, wv


def _run_append(h, hz, dc):
    hz.kv_append(h, dc)
    torch.cuda.synchronize()
    k = dc.k.cpu().numpy()
    v = dc.v.cpu().numpy()
    return k, v


def _host_raw(a, kv_dtype):
    return np.ascontiguousarray(a).view(np.uint16) if kv_dtype == "bf16" else np.ascontiguousarray(a)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("scales", [(1.0, 2.0), (0.75, 3.0)])
def test_append_exact_inputs_bit_exact(kv, paged, scales):
    m, hz = _mfa()
    B = 8
    L = [0, 1, 63, 64, 127, 200, 5, 129]
    case = synth.make_case("append_exact", B, L, kv, seed=71, paged=paged, append_room=1)
    case.x, case.w_k, case.w_v = _exact_inputs(B, 72)
    if kv == "fp8":
        case.k_scale, case.v_scale = scales
    elif scales != (1.0, 2.0):
        pytest.skip("scales apply to the FP8 cache only")
    _say(f"[kv_append exact] kv={kv} paged={paged} scales={scales}")
    k0 = _host_raw(case.k, kv).copy()
    v0 = _host_raw(case.v, kv).copy()
    dc = hz.to_device(case)
    h = hz.create_handle(dc, max_context=int(max(L)) + 1)
    try:
        k, v = _run_append(h, hz, dc)
    finally:
        m.mfa_destroy(h)
    kn, vn = oracle.kv_project(case.x, case.w_k, case.w_v)
    kr, vr = k0.copy(), v0.copy()
    n = oracle.kv_append(kn, vn, kr, vr, case.seq_lens, kv_dtype=BF16 if kv == "bf16" else FP8,
                         k_scale=case.k_scale, v_scale=case.v_scale, page_table=case.page_table)
    assert n == B
    k = _host_raw(k, kv)
    v = _host_raw(v, kv)
    bad_k = int(np.count_nonzero(k != kr))
    bad_v = int(np.count_nonzero(v != vr))
    _say(f"    mismatched elements: K {bad_k}  V {bad_v}  (changed by the oracle: "
         f"{int(np.count_nonzero(kr != k0))}, {int(np.count_nonzero(vr != v0))})")
    assert bad_k == 0 and bad_v == 0


def _sum_abs(x, w):
    X = np.abs(_bf16_val(x).astype(np.float64))
    W = np.abs(_bf16_val(w).astype(np.float64))
    return X @ W


def _check_random(case, k_gpu, v_gpu, k0, v0, label):
    """Written rows: codes equal to the oracle's, or (rarely) a neighbour that
    is as close to the exact value up to the fp32 accumulation bound. Rows
    not written: unchanged."""
    kvd = BF16 if case.kv_dtype == "bf16" else FP8
    kn, vn = oracle.kv_project(case.x, case.w_k, case.w_v)
    kr, vr = k0.copy(), v0.copy()
    oracle.kv_append(kn, vn, kr, vr, case.seq_lens, kv_dtype=kvd, k_scale=case.k_scale,
                     v_scale=case.v_scale, page_table=case.page_table)
    dec = oracle.decode_bf16 if kvd == BF16 else oracle.decode_e4m3
    total = 0
    for name, got, ref, exact, w, scale in (("K", k_gpu, kr, kn, case.w_k, case.k_scale),
                                            ("V", v_gpu, vr, vn, case.w_v, case.v_scale)):
        diff = got != ref
        total_el = int(np.count_nonzero(ref != (k0 if name == "K" else v0)))
        if not diff.any():
            _say(f"    {label} {name}: all codes equal ({total_el} written elements differ from before)")
            continue
        # every mismatch lies in a written row
        flat = got.reshape(-1, D)
        rflat = ref.reshape(-1, D)
        rows = np.nonzero((flat != rflat).any(axis=1))[0]
        written = {}
        for b in range(case.batch):
            t = int(case.seq_lens[b])
            if case.paged:
                row = int(case.page_table[b, t // 64]) * 64 + t % 64
            else:
                row = b * got.shape[1] + t
            written[row] = b
        assert all(r in written for r in rows), f"{name}: rows outside the appended ones changed"
        bound = _sum_abs(case.x, w) * (HID * 2.0 ** -24) + 1e-30
        nbad = 0
        for r in rows:
            b = written[r]
            cols = np.nonzero(flat[r] != rflat[r])[0]
            z = exact[b, cols] / scale
            g = dec(flat[r, cols])
            o = dec(rflat[r, cols])
            slack = np.abs(g - z) - np.abs(o - z)
            assert np.all(slack <= bound[b, cols] / scale * 2), (name, b, cols, g, o, z)
            nbad += cols.size
        frac = nbad / max(total_el, 1)
        _say(f"    {label} {name}: {nbad} codes off by one rounding near a tie ({frac:.2e} of written)")
        assert frac <= 1e-2
        total += nbad
    return total


@pytest.mark.parametrize("cfg", ["bf16_contig", "fp8_paged"])
def test_append_random_recipe(cfg):
    m, hz = _mfa()
    if cfg == "bf16_contig":
        case = synth.make_case("append_bf16", 8, 300, "bf16", seed=73, append_room=1, with_kv_proj=True)
    else:
        g = np.random.default_rng(74)
        L = g.integers(60, 700, size=16).astype(np.int32)
        L[:3] = [64, 128, 0]
        case = synth.make_case("append_fp8", 16, L, "fp8", seed=75, paged=True, append_room=1,
                               with_kv_proj=True)
    _say(f"[kv_append random] {cfg}: B={case.batch} L=[{case.seq_lens.min()},{case.seq_lens.max()}]")
    k0 = _host_raw(case.k, case.kv_dtype).copy()
    v0 = _host_raw(case.v, case.kv_dtype).copy()
    dc = hz.to_device(case)
    h = hz.create_handle(dc, max_context=int(case.seq_lens.max()) + 1)
    try:
        k, v = _run_append(h, hz, dc)
    finally:
        m.mfa_destroy(h)
    _check_random(case, _host_raw(k, case.kv_dtype), _host_raw(v, case.kv_dtype), k0, v0, cfg)


@pytest.mark.parametrize("paged", [False, True])
def test_append_skips_rows_that_do_not_exist(paged):
    m, hz = _mfa()
    B = 6
    if paged:
        L = np.array([10, 64, 64 * 4, 5, 70, 200], np.int32)
        case = synth.make_case("append_skip", B, L, "fp8", seed=76, paged=True, append_room=1)
        P = case.k.shape[0]
        pt = case.page_table[:, :4].copy()   # 4 slots: enough to read every sequence
        pt[1, 1] = -1                    # sequence 1: its next page is not allocated
        # sequence 2: L / 64 = 4 >= pt_stride (4) -- no slot in the table
        pt[3, 0] = P                     # sequence 3: page number past the pool
        case.page_table = pt
        expect = [0, 4, 5]
        max_len = pt.shape[1] * 64
    else:
        case = synth.make_case("append_skip", B, 40, "bf16", seed=76, append_room=0)
        S = case.k.shape[1]
        case.seq_lens = np.array([-1, S, S + 5, 3, S - 1, 0], np.int32)
        expect = [3, 4, 5]
        max_len = S
    case.x, case.w_k, case.w_v = _exact_inputs(B, 77)
    _say(f"[kv_append skip] paged={paged} L={case.seq_lens.tolist()}")
    k0 = _host_raw(case.k, case.kv_dtype).copy()
    v0 = _host_raw(case.v, case.kv_dtype).copy()
    dc = hz.to_device(case)
    dc.max_len = max_len
    h = hz.create_handle(dc, max_context=max_len)
    try:
        k, v = _run_append(h, hz, dc)
    finally:
        m.mfa_destroy(h)
    kn, vn = oracle.kv_project(case.x, case.w_k, case.w_v)
    kr, vr = k0.copy(), v0.copy()
    n = oracle.kv_append(kn, vn, kr, vr, case.seq_lens, kv_dtype=BF16 if case.kv_dtype == "bf16" else FP8,
                         k_scale=case.k_scale, v_scale=case.v_scale, page_table=case.page_table)
    assert n == len(expect)
    assert np.array_equal(_host_raw(k, case.kv_dtype), kr)
    assert np.array_equal(_host_raw(v, case.kv_dtype), vr)


def _row_err(o_gpu, o_ref):
    err = np.abs(o_gpu - o_ref).max(axis=-1) / np.maximum(np.abs(o_ref).max(axis=-1), 1e-30)
    return float(err.max())


@pytest.mark.parametrize("cfg", ["fp8_paged", "full_layer"])
def test_decode_step_append_then_attend(cfg):
    """One decode step end to end: (Q projection,) KV append of the new
    token, then attention over L_b + 1 rows, against the oracle doing the
    same steps in fp64."""
    m, hz = _mfa()
    if cfg == "fp8_paged":
        g = np.random.default_rng(78)
        L = g.integers(100, 900, size=12).astype(np.int32)
        L[:2] = [63, 128]
        case = synth.make_case("step_fp8", 12, L, "fp8", seed=79, paged=True, append_room=1,
                               with_kv_proj=True)
    else:
        case = synth.make_case("step_layer", 4, 513, "bf16", seed=80, append_room=1, with_qproj=True,
                               with_kv_proj=True)
    kvd = BF16 if case.kv_dtype == "bf16" else FP8
    _say(f"[decode step] {cfg}: B={case.batch} L=[{case.seq_lens.min()},{case.seq_lens.max()}]")
    dc = hz.to_device(case)
    L1 = case.seq_lens + 1
    h = hz.create_handle(dc, max_context=int(L1.max()))
    try:
        q = hz.qproj(h, dc) if case.q is None else dc.q
        hz.kv_append(h, dc)
        dc.seq_lens = torch.from_numpy(L1.astype(np.int32)).to(dc.k.device)
        dc.max_len = int(L1.max())
        out, lse = hz.decode(h, dc, q=q)
        torch.cuda.synchronize()
    finally:
        m.mfa_destroy(h)
    kn, vn = oracle.kv_project(case.x, case.w_k, case.w_v)
    kr = _host_raw(case.k, case.kv_dtype).copy()
    vr = _host_raw(case.v, case.kv_dtype).copy()
    oracle.kv_append(kn, vn, kr, vr, case.seq_lens, kv_dtype=kvd, k_scale=case.k_scale,
                     v_scale=case.v_scale, page_table=case.page_table)
    qd = oracle.case_q(case)
    o_ref, lse_ref = oracle.attention(qd, kr, vr, L1, kv_dtype=kvd, k_scale=case.k_scale,
                                      v_scale=case.v_scale, page_table=case.page_table,
                                      softmax_scale=case.softmax_scale)
    o = hz.bf16_to_f64(out)
    e = _row_err(o, o_ref)
    el = float(np.abs(lse.cpu().numpy().astype(np.float64) - lse_ref).max())
    _say(f"    row-rel err {e:.3e}  lse abs err {el:.3e}")
    assert e <= 1e-2
    assert el <= (1e-2 if case.w_qa is not None else 1e-3)


@pytest.mark.parametrize("cfg", [2, 4])
def test_append_full_size(cfg):
    """The append at the workloads' full batch and cache sizes (the full
    layer's contiguous bf16 cache, the ragged batch's paged FP8 pool), with
    one row of room per sequence: written rows against the oracle, the rest
    of each cache unchanged (compared on the device)."""
    m, hz = _mfa()
    base = synth.config_case(cfg)
    case = synth.make_case(base.name + "_append", base.batch, base.seq_lens, base.kv_dtype, seed=base.seed,
                           paged=base.paged, append_room=1, with_kv_proj=True,
                           max_context=int(base.seq_lens.max()) + 1 if base.paged else 0)
    _say(f"[kv_append full size] workload {cfg}: B={case.batch} kv={case.kv_dtype} paged={case.paged}")
    dc = hz.to_device(case)
    k_before = dc.k.clone()
    v_before = dc.v.clone()
    h = hz.create_handle(dc, max_context=int(case.seq_lens.max()) + 1)
    try:
        hz.kv_append(h, dc)
        torch.cuda.synchronize()
    finally:
        m.mfa_destroy(h)
    # written rows, flat row index per sequence
    L = case.seq_lens.astype(np.int64)
    if case.paged:
        rows = case.page_table[np.arange(case.batch), L // 64].astype(np.int64) * 64 + L % 64
    else:
        rows = np.arange(case.batch) * case.k.shape[1] + L
    rows_t = torch.from_numpy(rows).to(dc.k.device)
    kf, vf = dc.k.view(-1, D), dc.v.view(-1, D)
    kbf, vbf = k_before.view(-1, D), v_before.view(-1, D)
    changed_k = (kf != kbf).any(dim=1)
    changed_v = (vf != vbf).any(dim=1)
    changed_k[rows_t] = False
    changed_v[rows_t] = False
    assert not bool(changed_k.any()) and not bool(changed_v.any()), "rows other than L_b changed"
    k_rows = kf[rows_t].cpu().numpy()
    v_rows = vf[rows_t].cpu().numpy()
    kb_rows = kbf[rows_t].cpu().numpy()
    vb_rows = vbf[rows_t].cpu().numpy()
    del dc, k_before, v_before
    torch.cuda.empty_cache()
    # the oracle appends into a contiguous one-row-per-sequence cache
    small = synth.Case(name="rows", batch=case.batch, kv_dtype=case.kv_dtype,
                       seq_lens=np.zeros(case.batch, np.int32), k=None, v=None)
    small.x, small.w_k, small.w_v = case.x, case.w_k, case.w_v
    small.k_scale, small.v_scale = case.k_scale, case.v_scale
    k0 = _host_raw(kb_rows, case.kv_dtype).reshape(case.batch, 1, D)
    v0 = _host_raw(vb_rows, case.kv_dtype).reshape(case.batch, 1, D)
    _check_random(small, _host_raw(k_rows, case.kv_dtype).reshape(case.batch, 1, D),
                  _host_raw(v_rows, case.kv_dtype).reshape(case.batch, 1, D), k0, v0, f"workload {cfg}")
