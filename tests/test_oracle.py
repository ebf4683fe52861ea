"""Pins for the fp64 CPU oracle (CPU only).

The oracle is pinned to things other than itself: library routines (numpy
dgemm, torch's scaled_dot_product_attention and float8_e4m3fn casts), closed
forms and invariants of softmax attention, and 50-digit decimal brute force
on tiny inputs. Each pin is chosen so that a plausible slip in the oracle (a
dropped scale, a wrong index, a transposed operand, a missing max-shift or
normalisation) fails at least one of them.
"""
import decimal
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BF16, FP8 = oracle.KV_BF16, oracle.KV_FP8


def _torch_decode_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(
        torch.float64).numpy()


def _torch_decode_e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ------------------------------------------------------------------ formats

def test_e4m3_table_matches_torch():
    t = oracle.e4m3_table()
    ref = _torch_decode_e4m3(np.arange(256, dtype=np.uint8))
    same = (t == ref) | (np.isnan(t) & np.isnan(ref))
    assert same.all(), np.nonzero(~same)


def test_e4m3_golden_values():
    # OCP 8-bit floating point specification (OFP8), E4M3 encoding table
    with open(os.path.join(GOLDEN, "e4m3_ocp_values.json")) as f:
        g = json.load(f)
    for code_hex, val in g["values"].items():
        got = oracle.decode_e4m3(np.array([int(code_hex, 16)], dtype=np.uint8))[0]
        if val == "nan":
            assert math.isnan(got), code_hex
        else:
            assert got == float(val), (code_hex, got, val)
    t = oracle.e4m3_table()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)               # finite positive codes increase
    assert np.all(t[0x80:0xFF] == -t[:0x7F])      # sign bit is a pure sign


def test_bf16_decode_matches_torch():
    bits = np.random.default_rng(5).integers(0, 1 << 16, size=20000, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]       # drop inf/nan patterns
    assert np.array_equal(oracle.decode_bf16(bits), _torch_decode_bf16(bits))


def test_generator_encoders_match_torch():
    a = np.random.default_rng(7).standard_normal(50000).astype(np.float32)
    for s in (1e-3, 1.0, 40.0):
        x = (a * s).astype(np.float32)
        ref = torch.from_numpy(x).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(synth.e4m3_codes(x), ref)
    assert np.array_equal(synth.bf16_bits(a),
                          torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    # saturation instead of NaN
    assert synth.e4m3_codes(np.array([1e6, -1e6], dtype=np.float32)).tolist() == [0x7E, 0xFE]


# ------------------------------------------------------------------ attention

def _small_case(B=2, L=(37, 70), kv="bf16", seed=3, paged=False, q_std=1.0):
    return synth.make_case("t", B, list(L), kv, seed=seed, paged=paged, q_std=q_std)


def _kv_decoded(case):
    dec = oracle.decode_bf16 if case.kv_dtype == "bf16" else oracle.decode_e4m3
    return dec(case.k) * case.k_scale, dec(case.v) * case.v_scale


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_matches_torch_sdpa_mqa(kv):
    """MQA structure: one shared K/V head broadcast to all 64 query heads is
    textbook per-head softmax attention (torch SDPA, float64, CPU)."""
    case = _small_case(kv=kv)
    q = oracle.case_q(case)
    o, lse = oracle.case_attention(case)
    K, V = _kv_decoded(case)
    for b in range(case.batch):
        L = int(case.seq_lens[b])
        qt = torch.from_numpy(q[b])[None]                              # [1, H, D] as [B, L=H, D]
        kt = torch.from_numpy(K[b, :L])[None]
        vt = torch.from_numpy(V[b, :L])[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=1.0 / 16)[0]
        assert _rel(o[b], ref.numpy()) < 1e-12
        s = (torch.from_numpy(q[b]) @ torch.from_numpy(K[b, :L]).T) / 16.0
        assert np.max(np.abs(lse[b] - torch.logsumexp(s, dim=1).numpy())) < 1e-12


def test_weights_sum_to_one():
    case = _small_case(L=(1, 4096), seed=11)
    q = oracle.case_q(case)
    for b, h in [(0, 0), (1, 5), (1, 63)]:
        w = oracle.weights(q, case.k, case.seq_lens, b, h, kv_dtype=BF16)
        assert len(w) == case.seq_lens[b]
        assert abs(w.sum() - 1.0) < 1e-12
        assert (w >= 0).all()


def test_identical_keys_give_mean_v():
    case = _small_case(L=(50, 129), seed=12)
    case.k[:] = case.k[:, :1, :]                  # every row = row 0
    o, _ = oracle.case_attention(case)
    _, V = _kv_decoded(case)
    for b in range(case.batch):
        L = int(case.seq_lens[b])
        mean = V[b, :L].mean(axis=0)
        assert np.max(np.abs(o[b] - mean[None, :])) < 1e-13


def test_one_token_returns_v_exactly():
    case = _small_case(L=(1, 1), kv="fp8", seed=13)
    q = oracle.case_q(case)
    o, lse = oracle.case_attention(case)
    K, V = _kv_decoded(case)
    for b in range(case.batch):
        assert np.array_equal(o[b], np.broadcast_to(V[b, 0], o[b].shape))
        assert np.allclose(lse[b], (q[b] @ K[b, 0]) / 16.0, rtol=0, atol=1e-13)


def test_permutation_invariance():
    case = _small_case(L=(200, 333), seed=14)
    o, lse = oracle.case_attention(case)
    rng = np.random.default_rng(99)
    for b in range(case.batch):
        L = int(case.seq_lens[b])
        p = rng.permutation(L)
        case.k[b, :L] = case.k[b, p]
        case.v[b, :L] = case.v[b, p]
    o2, lse2 = oracle.case_attention(case)
    assert _rel(o2, o) < 1e-13
    assert np.max(np.abs(lse2 - lse)) < 1e-12


def test_scale_zero_gives_mean_v():
    case = _small_case(L=(17, 301), seed=15)
    case.softmax_scale = 0.0
    o, lse = oracle.case_attention(case)
    _, V = _kv_decoded(case)
    for b in range(case.batch):
        L = int(case.seq_lens[b])
        assert np.max(np.abs(o[b] - V[b, :L].mean(axis=0)[None])) < 1e-13
        assert np.allclose(lse[b], math.log(L), rtol=0, atol=1e-13)


def test_dominant_key_returns_its_v_row():
    case = _small_case(B=1, L=(64,), seed=16)
    q = np.zeros((1, 64, 256))
    q[0, :, 0] = 1.0
    K = np.zeros((1, case.k.shape[1], 256), dtype=np.float32)
    K[0, :, 0] = 0.5
    K[0, 23, 0] = 0.5 + 60.0 * 16.0                # logit +60 above the rest
    case.k = synth.bf16_bits(K)
    o, _ = oracle.attention(q, case.k, case.v, case.seq_lens, kv_dtype=BF16)
    _, V = _kv_decoded(case)
    assert np.max(np.abs(o[0] - V[0, 23][None])) < 1e-20


def test_empty_sequence():
    case = _small_case(L=(0, 5), seed=17)
    o, lse = oracle.case_attention(case)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))


def _decimal_attention(q, K, V, scale):
    decimal.getcontext().prec = 50
    Dd = decimal.Decimal
    H, D = q.shape
    L = K.shape[0]
    o = np.zeros((H, D))
    lse = np.zeros(H)
    for h in range(H):
        s = [Dd(scale) * sum(Dd(float(q[h, d])) * Dd(float(K[t, d])) for d in range(D))
             for t in range(L)]
        m = max(s)
        e = [(x - m).exp() for x in s]
        tot = sum(e)
        for d in range(D):
            o[h, d] = float(sum(e[t] / tot * Dd(float(V[t, d])) for t in range(L)))
        lse[h] = float(m + tot.ln())
    return o, lse


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_tiny_brute_force_decimal(kv):
    rng = np.random.default_rng(21)
    for trial in range(6):
        H, D, L = int(rng.integers(1, 4)), int(rng.integers(1, 5)), int(rng.integers(1, 9))
        q = synth.bf16_bits(rng.standard_normal((1, H, D)).astype(np.float32) * 3)
        qd = _torch_decode_bf16(q)
        Kf = rng.standard_normal((1, L, D)).astype(np.float32) * 2
        Vf = rng.standard_normal((1, L, D)).astype(np.float32)
        if kv == "bf16":
            K, V, ks, vs, code = synth.bf16_bits(Kf), synth.bf16_bits(Vf), 1.0, 1.0, BF16
            Kd, Vd = _torch_decode_bf16(K), _torch_decode_bf16(V)
        else:
            K, V, ks, vs, code = synth.e4m3_codes(Kf), synth.e4m3_codes(Vf), 0.375, 1.25, FP8
            Kd, Vd = _torch_decode_e4m3(K) * ks, _torch_decode_e4m3(V) * vs
        scale = 0.7
        o, lse = oracle.attention(qd, K, V, np.array([L], np.int32), kv_dtype=code,
                                  k_scale=ks, v_scale=vs, softmax_scale=scale)
        ro, rl = _decimal_attention(qd[0], Kd[0], Vd[0], scale)
        assert np.max(np.abs(o[0] - ro)) <= 1e-14 * max(1.0, np.max(np.abs(ro)))
        assert np.max(np.abs(lse[0] - rl)) <= 1e-14 * max(1.0, np.max(np.abs(rl)))


@pytest.mark.parametrize("chunk", [1, 7, 64, 512])
def test_split_equals_unsplit(chunk):
    case = _small_case(L=(1000, 513), seed=22, kv="fp8")
    o, lse = oracle.case_attention(case)
    o2, lse2 = oracle.case_attention(case, chunk=chunk)
    assert _rel(o2, o) < 1e-13
    assert np.max(np.abs(lse2 - lse)) < 1e-12


def test_paged_equals_contiguous_bitwise():
    """Same logical data through a permuted page table gives identical fp64
    results (the same operations in the same order)."""
    pc = synth.make_case("p", 3, [64, 130, 1], "fp8", seed=23, paged=True)
    P = pc.k.shape[0]
    maxL = int(pc.seq_lens.max())
    kc = np.zeros((3, maxL, 256), np.uint8)
    vc = np.zeros((3, maxL, 256), np.uint8)
    for b in range(3):
        for t in range(int(pc.seq_lens[b])):
            p = pc.page_table[b, t // 64]
            kc[b, t] = pc.k[p, t % 64]
            vc[b, t] = pc.v[p, t % 64]
    q = oracle.case_q(pc)
    o1, l1 = oracle.case_attention(pc)
    o2, l2 = oracle.attention(q, kc, vc, pc.seq_lens, kv_dtype=FP8, k_scale=pc.k_scale,
                              v_scale=pc.v_scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert P == 1 + 3 + 1


def test_gather_matches_numpy_indexing():
    pc = synth.make_case("p", 4, [1, 63, 64, 200], "bf16", seed=24, paged=True)
    for b in range(4):
        L = int(pc.seq_lens[b])
        t = np.arange(L)
        pages = pc.page_table[b, t // 64]
        kd, vd = oracle.gather_kv(pc.k, pc.v, pc.seq_lens, b, page_table=pc.page_table)
        assert np.array_equal(kd, pc.k[pages, t % 64])
        assert np.array_equal(vd, pc.v[pages, t % 64])


def test_page_table_is_permutation():
    c = synth.config_case(4, batch=24, scale_len=1 / 16)
    npg = (c.seq_lens + 63) // 64
    used = np.concatenate([c.page_table[b, :npg[b]] for b in range(c.batch)])
    assert np.array_equal(np.sort(used), np.arange(c.k.shape[0]))
    assert c.seq_lens.min() >= 64 and c.seq_lens.max() <= 512


# ------------------------------------------------------------------ Q projection

def _tiny_qproj_inputs(B, hidden, rank, nq, seed):
    rng = np.random.default_rng(seed)
    x = synth.bf16_bits(rng.standard_normal((B, hidden)).astype(np.float32))
    wa = synth.bf16_bits((rng.standard_normal((hidden, rank)) / math.sqrt(hidden)).astype(np.float32))
    wb = synth.bf16_bits((rng.standard_normal((rank, nq)) / math.sqrt(rank)).astype(np.float32))
    g = synth.bf16_bits((1.0 + 0.25 * rng.standard_normal(rank)).astype(np.float32))
    return x, wa, g, wb


def test_qproj_matches_numpy_dgemm():
    x, wa, g, wb = _tiny_qproj_inputs(5, 96, 48, 80, 31)
    q, c, chat = oracle.qproj(x, wa, g, wb, eps=1e-6, return_c=True)
    X, WA, G, WB = (_torch_decode_bf16(a) for a in (x, wa, g, wb))
    c_ref = X @ WA                                       # library dgemm
    assert _rel(c, c_ref) < 1e-13
    q_ref = chat @ WB
    assert _rel(q, q_ref) < 1e-13
    # chat is c scaled per row by a positive factor times gamma
    ratio = chat / (c * G[None, :])
    assert np.allclose(ratio, ratio[:, :1], rtol=1e-13, atol=0)


def test_rmsnorm_closed_form_and_gamma():
    x, wa, g, wb = _tiny_qproj_inputs(4, 64, 32, 16, 32)
    ones = synth.bf16_bits(np.ones(32, np.float32))
    eps = 1e-3
    _, c, chat = oracle.qproj(x, wa, ones, wb, eps=eps, return_c=True)
    m = (c * c).mean(axis=1)
    assert np.allclose((chat * chat).sum(axis=1), 32 * m / (m + eps), rtol=1e-13, atol=0)
    twos = synth.bf16_bits(np.full(32, 2.0, np.float32))
    _, _, chat2 = oracle.qproj(x, wa, twos, wb, eps=eps, return_c=True)
    assert np.array_equal(chat2, 2 * chat)


def test_rmsnorm_scale_invariance_exact():
    """With eps = 0, scaling x by 4 (exact in bf16 and fp64) leaves chat and q
    bit-identical: the norm divides the scale out."""
    x, wa, g, wb = _tiny_qproj_inputs(3, 64, 32, 24, 33)
    x4 = synth.bf16_bits(_torch_decode_bf16(x).astype(np.float32) * 4)
    q1 = oracle.qproj(x, wa, g, wb, eps=0.0)
    q4 = oracle.qproj(x4, wa, g, wb, eps=0.0)
    assert np.array_equal(q1, q4)
    qe = oracle.qproj(x, wa, g, wb, eps=1e-6)
    assert not np.array_equal(q1, qe) and _rel(qe, q1) < 1e-5


def test_qproj_tiny_decimal():
    decimal.getcontext().prec = 50
    Dd = decimal.Decimal
    x, wa, g, wb = _tiny_qproj_inputs(2, 8, 4, 6, 34)
    X, WA, G, WB = (_torch_decode_bf16(a) for a in (x, wa, g, wb))
    eps = 1e-6
    q = oracle.qproj(x, wa, g, wb, eps=eps)
    for b in range(2):
        c = [sum(Dd(float(X[b, i])) * Dd(float(WA[i, j])) for i in range(8)) for j in range(4)]
        r = 1 / (sum(v * v for v in c) / 4 + Dd(eps)).sqrt()
        ch = [c[j] * r * Dd(float(G[j])) for j in range(4)]
        for n in range(6):
            ref = float(sum(ch[j] * Dd(float(WB[j, n])) for j in range(4)))
            assert abs(q[b, n] - ref) <= 1e-14 * max(1.0, abs(ref))


def test_config_recipes():
    c1 = synth.config_case(1)
    assert c1.q.shape == (1, 64, 256) and c1.k.shape == (1, 256, 256) and c1.kv_dtype == "bf16"
    c3 = synth.config_case(3, batch=2, scale_len=1 / 64)
    assert c3.kv_dtype == "fp8" and c3.k.dtype == np.uint8 and 0 < c3.k_scale < 1
    c5 = synth.config_case(5, batch=4, scale_len=1 / 256)
    assert c5.seq_lens.tolist() == [128, 128, 256, 256] and c5.split_tokens == 512
    c2 = synth.config_case(2, batch=2, scale_len=1 / 256)
    assert c2.x.shape == (2, 7168) and c2.w_qa.shape == (7168, 2048) and c2.w_qb.shape == (2048, 16384)
    # seeded: same seed, same bytes
    assert np.array_equal(synth.config_case(1).k, c1.k)


# ------------------------------------------------------------------ KV append

def _e4m3_finite_positive():
    t = oracle.e4m3_table()
    return t[:0x7F]                                      # codes 0x00 .. 0x7e


def test_encode_e4m3_matches_torch_in_range():
    rng = np.random.default_rng(41)
    for s in (1e-3, 0.1, 1.0, 30.0, 200.0):
        x = (rng.standard_normal(40000) * s).astype(np.float32)
        x = x[np.abs(x) < 448]
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(oracle.encode_e4m3(x), ref)


def test_encode_e4m3_round_trip_ties_and_saturation():
    pos = _e4m3_finite_positive()
    codes = np.arange(0x7F, dtype=np.uint8)
    # every finite code decodes and encodes back to itself, both signs
    assert np.array_equal(oracle.encode_e4m3(pos.astype(np.float32)), codes)
    assert np.array_equal(oracle.encode_e4m3(-pos.astype(np.float32)), codes | 0x80)
    # midpoints between neighbours (exact in float32) go to the even code,
    # points just inside either side go to that side
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    even = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])
    assert np.array_equal(oracle.encode_e4m3(mid), even)
    lo = np.nextafter(mid, np.float32(0))
    hi = np.nextafter(mid, np.float32(np.inf))
    assert np.array_equal(oracle.encode_e4m3(lo), codes[:-1])
    assert np.array_equal(oracle.encode_e4m3(hi), codes[1:])
    # no infinities in the format: everything at or past 448 saturates
    big = np.array([448, 449, 464, 1e4, 3e38, np.inf], dtype=np.float32)
    assert np.all(oracle.encode_e4m3(big) == 0x7E)
    assert np.all(oracle.encode_e4m3(-big) == 0xFE)
    assert oracle.encode_e4m3(np.array([np.nan], np.float32))[0] & 0x7F == 0x7F
    # below half the smallest subnormal: zero with the sign
    assert oracle.encode_e4m3(np.array([2.0 ** -11, -2.0 ** -11], np.float32)).tolist() == [0, 0x80]


def test_encode_bf16_matches_torch_and_ties():
    rng = np.random.default_rng(42)
    x = (rng.standard_normal(50000) * np.exp(rng.uniform(-20, 20, 50000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.encode_bf16(x), ref)
    # exact halfway points: bf16 value with low half 0x8000 rounds to even
    hi = rng.integers(0x0080, 0x7F00, size=4000, dtype=np.uint32)
    tie = ((hi << 16) | 0x8000).view(np.float32)
    assert np.array_equal(oracle.encode_bf16(tie), (hi + (hi & 1)).astype(np.uint16))
    assert oracle.encode_bf16(np.array([np.inf, -np.inf], np.float32)).tolist() == [0x7F80, 0xFF80]


def test_encode_monotone():
    x = np.sort(np.random.default_rng(43).standard_normal(20000).astype(np.float32) * 50)
    d8 = oracle.decode_e4m3(oracle.encode_e4m3(x))
    assert np.all(np.diff(d8) >= 0)
    d16 = oracle.decode_bf16(oracle.encode_bf16(x))
    assert np.all(np.diff(d16) >= 0)


def _tiny_kv_inputs(B, hidden, D, seed):
    rng = np.random.default_rng(seed)
    x = synth.bf16_bits(rng.standard_normal((B, hidden)).astype(np.float32))
    wk = synth.bf16_bits((rng.standard_normal((hidden, D)) / math.sqrt(hidden)).astype(np.float32))
    wv = synth.bf16_bits((rng.standard_normal((hidden, D)) / math.sqrt(hidden)).astype(np.float32))
    return x, wk, wv


def test_kv_project_matches_numpy_dgemm():
    x, wk, wv = _tiny_kv_inputs(6, 160, 48, 44)
    k, v = oracle.kv_project(x, wk, wv)
    X, WK, WV = (_torch_decode_bf16(a) for a in (x, wk, wv))
    assert _rel(k, X @ WK) < 1e-13
    assert _rel(v, X @ WV) < 1e-13
    # swapping the two weights swaps the outputs
    k2, v2 = oracle.kv_project(x, wv, wk)
    assert np.array_equal(k2, v) and np.array_equal(v2, k)


def test_kv_project_tiny_decimal():
    decimal.getcontext().prec = 50
    Dd = decimal.Decimal
    x, wk, wv = _tiny_kv_inputs(2, 7, 3, 45)
    X, WK, WV = (_torch_decode_bf16(a) for a in (x, wk, wv))
    k, v = oracle.kv_project(x, wk, wv)
    for b in range(2):
        for j in range(3):
            rk = float(sum(Dd(float(X[b, i])) * Dd(float(WK[i, j])) for i in range(7)))
            rv = float(sum(Dd(float(X[b, i])) * Dd(float(WV[i, j])) for i in range(7)))
            assert abs(k[b, j] - rk) <= 1e-15 * max(1.0, abs(rk))
            assert abs(v[b, j] - rv) <= 1e-15 * max(1.0, abs(rv))


@pytest.mark.parametrize("kv", [BF16, FP8])
def test_kv_append_contiguous_writes_one_row(kv):
    B, S, D = 4, 10, 16
    raw = np.uint16 if kv == BF16 else np.uint8
    rng = np.random.default_rng(46)
    k = rng.integers(0, 0x7E, size=(B, S, D)).astype(raw)
    v = rng.integers(0, 0x7E, size=(B, S, D)).astype(raw)
    k0, v0 = k.copy(), v.copy()
    kn = rng.standard_normal((B, D)) * 3
    vn = rng.standard_normal((B, D)) * 3
    L = np.array([0, 5, 9, 10], np.int32)                # the last is past the capacity
    ks, vs = (0.5, 0.25) if kv == FP8 else (1.0, 1.0)
    n = oracle.kv_append(kn, vn, k, v, L, kv_dtype=kv, k_scale=ks, v_scale=vs)
    assert n == 3
    enc = ((lambda a, s: oracle.encode_bf16(a.astype(np.float32))) if kv == BF16 else
           (lambda a, s: oracle.encode_e4m3(a.astype(np.float32) / np.float32(s))))
    for b in range(B):
        for t in range(S):
            if b < 3 and t == L[b]:
                assert np.array_equal(k[b, t], enc(kn[b], ks))
                assert np.array_equal(v[b, t], enc(vn[b], vs))
            else:
                assert np.array_equal(k[b, t], k0[b, t]) and np.array_equal(v[b, t], v0[b, t])
    # the written row decodes to the value within half a step of the format
    dec = oracle.decode_bf16 if kv == BF16 else oracle.decode_e4m3
    got = dec(k[1, 5]) * ks
    rel = 2.0 ** -8 if kv == BF16 else 2.0 ** -4           # half a unit in the last place
    assert np.all(np.abs(got - kn[1]) <= rel * np.abs(kn[1]) + (2.0 ** -10) * ks)


@pytest.mark.parametrize("kv", [BF16, FP8])
def test_kv_append_paged_matches_contiguous(kv):
    """Appending through a page table and gathering the pages back gives the
    same cache as appending to the contiguous layout."""
    case = synth.make_case("t", 3, [63, 64, 130], "bf16" if kv == BF16 else "fp8", seed=47,
                           paged=True, append_room=1)
    B, D = case.batch, case.k.shape[-1]
    rng = np.random.default_rng(48)
    kn, vn = rng.standard_normal((B, D)), rng.standard_normal((B, D))
    kp, vp = case.k.copy(), case.v.copy()
    n = oracle.kv_append(kn, vn, kp, vp, case.seq_lens, kv_dtype=kv, k_scale=case.k_scale,
                         v_scale=case.v_scale, page_table=case.page_table)
    assert n == B
    for b in range(B):
        L1 = case.seq_lens[b] + 1
        kc, vc = oracle.gather_kv(kp, vp, [L1], 0, page_table=case.page_table[b:b + 1])
        kc0, vc0 = oracle.gather_kv(case.k, case.v, [L1], 0, page_table=case.page_table[b:b + 1])
        kk, vv = kc0[None].copy(), vc0[None].copy()
        oracle.kv_append(kn[b:b + 1], vn[b:b + 1], kk, vv, case.seq_lens[b:b + 1], kv_dtype=kv,
                         k_scale=case.k_scale, v_scale=case.v_scale)
        assert np.array_equal(kc, kk[0]) and np.array_equal(vc, vv[0])
    # pages no sequence owns are untouched
    owned = np.unique(case.page_table[case.page_table >= 0])
    free = np.setdiff1d(np.arange(case.k.shape[0]), owned)
    assert np.array_equal(kp[free], case.k[free]) and np.array_equal(vp[free], case.v[free])


# ------------------------------------------------------------------ multi-token decode

def test_mtp_matches_torch_sdpa_with_causal_mask():
    """t query tokens per sequence, the last t cache rows being theirs: against
    torch's scaled_dot_product_attention with an explicit boolean mask
    (query j may see keys s < L - (t-1-j)), K and V broadcast to the heads."""
    t, H, D = 3, 64, 256
    for L in (3, 10, 70):
        case = synth.make_case("mtp", 1, L, "bf16", seed=90 + L)
        rng = np.random.default_rng(91)
        q = _torch_decode_bf16(synth.bf16_bits(rng.standard_normal((1, t, H, D)).astype(np.float32)))
        o, lse = oracle.attention_mtp(q, case.k, case.v, case.seq_lens, kv_dtype=BF16)
        K, V = _kv_decoded(case)
        Kt = torch.from_numpy(K[0, :L]).to(torch.float64)
        Vt = torch.from_numpy(V[0, :L]).to(torch.float64)
        qt = torch.from_numpy(q[0]).permute(1, 0, 2)                     # [H, t, D]
        mask = torch.arange(L)[None, :] < (L - (t - 1) + torch.arange(t))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, Kt[None].expand(H, L, D), Vt[None].expand(H, L, D), attn_mask=mask, scale=1.0 / 16.0)
        assert _rel(o[0], ref.permute(1, 0, 2).numpy()) < 1e-12
        s = torch.einsum("htd,ld->htl", qt, Kt) / 16.0
        lse_ref = torch.logsumexp(s.masked_fill(~mask[None], float("-inf")), dim=-1).permute(1, 0).numpy()
        assert np.abs(lse[0] - lse_ref).max() < 1e-12


def test_mtp_token_with_no_rows():
    """A sequence shorter than t: its first tokens see no row (out 0, lse -inf)."""
    case = synth.make_case("mtp0", 1, 2, "fp8", seed=95)
    q = np.random.default_rng(96).standard_normal((1, 4, 64, 256))
    o, lse = oracle.attention_mtp(q, case.k, case.v, case.seq_lens, kv_dtype=FP8, k_scale=case.k_scale,
                                  v_scale=case.v_scale)
    assert np.all(o[0, :2] == 0) and np.all(np.isneginf(lse[0, :2]))
    assert np.all(np.isfinite(lse[0, 2:]))


# ------------------------------------------------------- grouped KV heads (GQA)
def _gqa_inputs(B, G, L, kv, seed, H=16, D=8, paged=False):
    """Small grouped caches: q [B, H, D] fp64, K/V raw [B, G, S, D] (or paged
    pools [P, G, 64, D] with a permuted page table)."""
    rng = np.random.default_rng(seed)
    q = _torch_decode_bf16(synth.bf16_bits(rng.standard_normal((B, H, D)).astype(np.float32)))
    S = max(L)
    Kf = rng.standard_normal((B, G, S, D)).astype(np.float32)
    Vf = rng.standard_normal((B, G, S, D)).astype(np.float32)
    if kv == "bf16":
        K, V, ks, vs, code = synth.bf16_bits(Kf), synth.bf16_bits(Vf), 1.0, 1.0, BF16
        dec = _torch_decode_bf16
    else:
        K, V, ks, vs, code = synth.e4m3_codes(Kf), synth.e4m3_codes(Vf), 0.5, 0.75, FP8
        dec = _torch_decode_e4m3
    Kd, Vd = dec(K) * ks, dec(V) * vs
    return q, K, V, Kd, Vd, ks, vs, code


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("G", [1, 2, 4, 16])
def test_gqa_matches_torch_sdpa_enable_gqa(kv, G):
    """Grouped-query attention against torch's own grouped SDPA (float64,
    CPU, enable_gqa: query head h uses KV head h // (H // G)); G = H is
    multi-head attention, G = 1 MFA's single shared head."""
    L = [5, 33, 64]
    q, K, V, Kd, Vd, ks, vs, code = _gqa_inputs(3, G, L, kv, seed=300 + G)
    o, lse = oracle.attention(q, K, V, np.array(L, np.int32), kv_dtype=code, k_scale=ks, v_scale=vs,
                              softmax_scale=0.3, kv_heads=G)
    for b, n in enumerate(L):
        qt = torch.from_numpy(q[b])[None, :, None, :]                 # [1, H, 1, D]
        kt = torch.from_numpy(Kd[b, :, :n])[None]                      # [1, G, n, D]
        vt = torch.from_numpy(Vd[b, :, :n])[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.3, enable_gqa=True)
        assert _rel(o[b], ref[0, :, 0].numpy()) < 1e-12
        grp = np.arange(q.shape[1]) // (q.shape[1] // G)
        s = np.einsum("hd,htd->ht", q[b], Kd[b, grp, :n]) * 0.3
        assert np.max(np.abs(lse[b] - torch.logsumexp(torch.from_numpy(s), dim=1).numpy())) < 1e-12


def test_gqa_is_independent_mqa_per_group():
    """Each group is MFA's single-head attention of its own query heads
    against its own K/V head: the grouped result equals G separate calls."""
    G, H = 4, 16
    L = [17, 40]
    q, K, V, Kd, Vd, ks, vs, code = _gqa_inputs(2, G, L, "fp8", seed=310, H=H)
    o, lse = oracle.attention(q, K, V, np.array(L, np.int32), kv_dtype=code, k_scale=ks, v_scale=vs,
                              softmax_scale=0.25, kv_heads=G)
    hg = H // G
    for g in range(G):
        og, lg = oracle.attention(np.ascontiguousarray(q[:, g * hg:(g + 1) * hg]), np.ascontiguousarray(K[:, g]),
                                  np.ascontiguousarray(V[:, g]), np.array(L, np.int32), kv_dtype=code,
                                  k_scale=ks, v_scale=vs, softmax_scale=0.25)
        assert np.array_equal(og, o[:, g * hg:(g + 1) * hg]) and np.array_equal(lg, lse[:, g * hg:(g + 1) * hg])


def test_gqa_paged_equals_contiguous_bitwise():
    """Paged grouped pools [P, G, 64, D] through a permuted page table give
    the contiguous grouped result bit for bit."""
    G, L = 2, [70, 129, 1]
    q, K, V, _, _, ks, vs, code = _gqa_inputs(3, G, L, "fp8", seed=320, H=8)
    npg = [(n + 63) // 64 for n in L]
    P = sum(npg)
    perm = np.random.default_rng(321).permutation(P).astype(np.int32)
    pt = np.zeros((3, max(npg)), np.int32)
    Kp = np.zeros((P, G, 64, K.shape[-1]), np.uint8)
    Vp = np.zeros_like(Kp)
    i = 0
    S = K.shape[2]
    for b, n in enumerate(L):
        for j in range(npg[b]):
            page = perm[i]
            i += 1
            pt[b, j] = page
            rows = min(64, S - 64 * j)
            Kp[page, :, :rows] = K[b, :, 64 * j:64 * j + rows]
            Vp[page, :, :rows] = V[b, :, 64 * j:64 * j + rows]
    oc, lc = oracle.attention(q, K, V, np.array(L, np.int32), kv_dtype=code, k_scale=ks, v_scale=vs, kv_heads=G)
    op, lp = oracle.attention(q, Kp, Vp, np.array(L, np.int32), kv_dtype=code, k_scale=ks, v_scale=vs,
                              page_table=pt, kv_heads=G)
    assert np.array_equal(oc, op) and np.array_equal(lc, lp)


def test_gqa_tiny_brute_force_decimal():
    """50-digit decimal softmax per query head against its group's K/V."""
    G, H, D, L = 2, 4, 3, [6]
    q, K, V, Kd, Vd, ks, vs, code = _gqa_inputs(1, G, L, "bf16", seed=330, H=H, D=D)
    o, lse = oracle.attention(q, K, V, np.array(L, np.int32), kv_dtype=code, softmax_scale=0.6, kv_heads=G)
    for h in range(H):
        g = h // (H // G)
        ro, rl = _decimal_attention(q[0, h:h + 1], Kd[0, g, :6], Vd[0, g, :6], 0.6)
        assert np.max(np.abs(o[0, h] - ro[0])) <= 1e-14 * max(1.0, np.max(np.abs(ro)))
        assert abs(lse[0, h] - rl[0]) <= 1e-14 * max(1.0, abs(rl[0]))
