"""Pins for the oracle of the FP8 attention arithmetic (CPU only).

``oracle.attention_fp8mma`` quantises each head's query to E4M3 after a
power-of-two scale that puts its largest |q| in [128, 256), takes exact dot
products with the E4M3 key codes, rounds 4 P = 4 * 2^(s2 - ceil(max s2)) to
E4M3 and normalises by the sum of the rounded weights. It is pinned here
against:

- the exact oracle, on inputs where every quantiser is the identity (a
  dropped scale, a wrong reference or normalisation, a transposed operand
  shows up as a difference);
- a 50-digit decimal brute force whose E4M3 rounding is an exhaustive
  nearest-value search over torch's float8_e4m3fn values, ties to the even
  code (an independent statement of round-to-nearest-even, subnormals
  included);
- a float64 re-implementation at full head size whose quantiser is torch's
  float8_e4m3fn cast;
- invariants: power-of-two query scaling, token order, paging, one-token and
  equal-key contexts, the empty sequence.

It also shows that the GPU test's bar (``TOL_F8``, tests/test_gpu_fp8mma.py)
would catch a round-toward-zero quantiser or a flush of the subnormal weights.
"""
import decimal
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from fp8_inputs import exact_case, subnormal_case

TOL_F8 = 2.0 ** -7   # the GPU parity bar against this oracle (row-wise normwise)


def _rowerr(a, b):
    return float((np.abs(a - b).max(axis=-1) / np.maximum(np.abs(b).max(axis=-1), 1e-300)).max())


def _e4m3_values():
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)   # positive finite codes
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ------------------------------------------------------------ the query scale

def test_q_exponent_puts_amax_in_128_256():
    rng = np.random.default_rng(1)
    vals = np.concatenate([2.0 ** rng.uniform(-60, 60, 500), 2.0 ** np.arange(-90, 91, dtype=np.float64),
                           np.nextafter(2.0 ** np.arange(-90, 91, dtype=np.float64), 0)])
    for a in vals:
        e = oracle.fp8_q_exponent(a)
        assert 128.0 <= a * 2.0 ** e < 256.0, (a, e)
    assert oracle.fp8_q_exponent(0.0) == 0
    assert oracle.fp8_q_exponent(1.0) == 7 and oracle.fp8_q_exponent(255.9) == 0
    assert oracle.fp8_q_exponent(2.0 ** -120) == 100     # limited to [-100, 100]
    assert oracle.fp8_q_exponent(2.0 ** 120) == -100


# ------------------------------------------------- identity quantisers: exact

@pytest.mark.parametrize("q_pow2", [0, -20, 9])
def test_reduces_to_exact_attention_when_quantisers_are_identity(q_pow2):
    q, k, v, scale = exact_case(3, B=2, H=8, D=64, L=200, q_pow2=q_pow2)
    L = np.array([200, 131], dtype=np.int32)
    o8, l8 = oracle.attention_fp8mma(q, k, v, L, k_scale=1.0, v_scale=0.375, softmax_scale=scale)
    o, l = oracle.attention(oracle.decode_bf16(q), k, v, L, kv_dtype=oracle.KV_FP8, k_scale=1.0,
                            v_scale=0.375, softmax_scale=scale)
    assert _rowerr(o8, o) < 1e-12
    assert np.abs(l8 - l).max() < 1e-12
    # a k_scale is folded into the score scale exactly like softmax_scale
    o8b, l8b = oracle.attention_fp8mma(q, k, v, L, k_scale=0.5, v_scale=0.375, softmax_scale=2 * scale)
    assert _rowerr(o8b, o) < 1e-12 and np.abs(l8b - l).max() < 1e-12


# ----------------------------------------------------- decimal brute force

def _nearest_e4m3(x: Fraction, table, mode="rne") -> Fraction:
    """Nearest E4M3 value by exhaustive search, ties to the even code (the
    code's last bit is the mantissa's); mode 'rtz' takes the largest value
    not above |x| instead."""
    s = -1 if x < 0 else 1
    a = abs(x)
    if mode == "rtz":
        best = max(i for i in range(len(table)) if table[i] <= a)
        return s * table[best]
    d = [abs(t - a) for t in table]
    m = min(d)
    cands = [i for i in range(len(table)) if d[i] == m]
    best = [i for i in cands if i % 2 == 0][0] if len(cands) > 1 else cands[0]
    return s * table[best]


def _brute(qf, kf, vf, L, scale, k_scale, v_scale, mode="rne"):
    """qf [H, D] (exact bf16 values), kf, vf [L, D] (E4M3 values) as floats."""
    ctx = decimal.Context(prec=50)
    table = [Fraction(float(t)) for t in _e4m3_values()]
    ln2 = ctx.ln(decimal.Decimal(2))
    H, D = qf.shape
    o = np.zeros((H, D))
    lse = np.zeros(H)
    for h in range(H):
        qh = [Fraction(float(x)) for x in qf[h]]
        amax = max(abs(x) for x in qh)
        e = 0
        if amax > 0:
            while amax * Fraction(2) ** e < 128:
                e += 1
            while amax * Fraction(2) ** e >= 256:
                e -= 1
        q8 = [_nearest_e4m3(x * Fraction(2) ** e, table, mode) for x in qh]
        s2 = []
        for t in range(L):
            dot = sum(q8[d] * Fraction(float(kf[t, d])) for d in range(D))
            dd = decimal.Decimal(dot.numerator) / decimal.Decimal(dot.denominator)
            s2.append(ctx.divide(ctx.multiply(dd, decimal.Decimal(scale * k_scale)),
                                 ctx.multiply(ln2, decimal.Decimal(2) ** e)))
        r = max(s2).to_integral_value(rounding=decimal.ROUND_CEILING)
        p8 = []
        for t in range(L):
            p = ctx.multiply(4, ctx.exp(ctx.multiply(s2[t] - r, ln2)))
            pf = Fraction(p)
            p8.append(_nearest_e4m3(pf, table, mode) / 4)
        S8 = sum(p8)
        for d in range(D):
            o[h, d] = float(sum(p8[t] * Fraction(float(vf[t, d])) for t in range(L)) / S8) * v_scale
        lse[h] = float(ln2 * r + ctx.ln(decimal.Decimal(S8.numerator) / decimal.Decimal(S8.denominator)))
    return o, lse


@pytest.mark.parametrize("q_std", [1.0, 5.0])
def test_tiny_brute_force_decimal(q_std):
    """H = 3, D = 16, L = 37 N(0,1) inputs; q_std = 5 spreads the scores so
    that weights fall into E4M3's subnormal range and to zero."""
    g = np.random.default_rng(11)
    H, D, L = 3, 16, 37
    q = synth.bf16_bits((g.standard_normal((1, H, D)) * q_std).astype(np.float32))
    k = synth.e4m3_codes(g.standard_normal((1, L, D)) * 20.0)
    v = synth.e4m3_codes(g.standard_normal((1, L, D)) * 3.0)
    scale, ks, vs = 0.25, 0.7, 1.3
    o8, l8 = oracle.attention_fp8mma(q, k, v, np.array([L], np.int32), k_scale=ks, v_scale=vs,
                                     softmax_scale=scale)
    ob, lb = _brute(oracle.decode_bf16(q[0]), oracle.decode_e4m3(k[0]), oracle.decode_e4m3(v[0]), L,
                    scale, ks, vs)
    assert _rowerr(o8[0], ob) < 1e-12
    assert np.abs(l8[0] - lb).max() < 1e-12
    # a round-toward-zero quantiser gives another result
    orz, _ = _brute(oracle.decode_bf16(q[0]), oracle.decode_e4m3(k[0]), oracle.decode_e4m3(v[0]), L,
                    scale, ks, vs, mode="rtz")
    assert _rowerr(orz, ob) > 1e-3


# --------------------------------------- float64 re-implementation (torch cast)

def _torch_q8(x64, flush_below=0.0, rtz=False):
    """x -> E4M3 value of float32(x): torch's cast (round to nearest even), or
    truncation toward zero, optionally flushing results below flush_below to
    zero."""
    x32 = torch.from_numpy(np.asarray(x64, dtype=np.float32))
    if rtz:
        tab = _e4m3_values()
        a = np.abs(x32.numpy().astype(np.float64))
        idx = np.searchsorted(tab, a, side="right") - 1
        val = np.sign(x32.numpy()) * tab[np.clip(idx, 0, None)]
    else:
        val = x32.to(torch.float8_e4m3fn).to(torch.float64).numpy()
    if flush_below > 0:
        val = np.where(np.abs(val) < flush_below, 0.0, val)
    return val


def _torch_impl(q_bits, k, v, L, scale, k_scale, v_scale, **quant):
    qf = oracle.decode_bf16(q_bits)             # [B, H, D]
    kf = oracle.decode_e4m3(k)
    vf = oracle.decode_e4m3(v)
    B, H, D = qf.shape
    o = np.zeros((B, H, D))
    lse = np.zeros((B, H))
    for b in range(B):
        n = int(L[b])
        amax = np.abs(qf[b]).max(axis=1)
        e = np.where(amax > 0, 7 - np.floor(np.log2(np.where(amax > 0, amax, 1.0))), 0.0)
        q8 = _torch_q8(qf[b] * 2.0 ** e[:, None], **quant)
        s2 = (q8 @ kf[b, :n].T) * scale * k_scale / math.log(2.0) * 2.0 ** -e[:, None]
        r = np.ceil(s2.max(axis=1, keepdims=True))
        p8 = _torch_q8(4.0 * np.exp2(s2 - r), **quant) / 4.0
        S8 = p8.sum(axis=1)
        o[b] = (p8 @ vf[b, :n]) * v_scale / S8[:, None]
        lse[b] = math.log(2.0) * r[:, 0] + np.log(S8)
    return o, lse


def test_matches_torch_cast_reimplementation_full_heads():
    case = synth.config_case(3, batch=2, scale_len=0.25)
    L = np.array([1000, 640], dtype=np.int32)
    o8, l8 = oracle.attention_fp8mma(case.q, case.k, case.v, L, k_scale=case.k_scale, v_scale=case.v_scale)
    ot, lt = _torch_impl(case.q, case.k, case.v, L, 1 / 16, case.k_scale, case.v_scale)
    assert _rowerr(o8, ot) < 1e-12 and np.abs(l8 - lt).max() < 1e-12
    # the bar of the GPU test catches a round-toward-zero quantiser
    orz, _ = _torch_impl(case.q, case.k, case.v, L, 1 / 16, case.k_scale, case.v_scale, rtz=True)
    assert _rowerr(orz, o8) > 2 * TOL_F8
    # the mode's own error against exact attention (its budget, not a pin)
    o, _ = oracle.attention(oracle.decode_bf16(case.q), case.k, case.v, L, kv_dtype=oracle.KV_FP8,
                            k_scale=case.k_scale, v_scale=case.v_scale)
    assert 1e-2 < _rowerr(o8, o) < 0.2


def test_subnormal_weights_are_rounded_not_flushed():
    q, k, v, ks, vs = subnormal_case(5, [4000, 1000])
    L = np.array([4000, 1000], dtype=np.int32)
    o8, l8 = oracle.attention_fp8mma(q, k, v, L, k_scale=ks, v_scale=vs)
    ot, lt = _torch_impl(q, k, v, L, 1 / 16, ks, vs)
    assert _rowerr(o8, ot) < 1e-12 and np.abs(l8 - lt).max() < 1e-12
    # the second half of each row is the subnormal weights' share
    share = o8[:, :, 128:].mean()
    assert 0.03 < share < 0.15
    # flushing every subnormal weight, or only those an octave below the
    # smallest normal value, moves the output by more than the GPU bar
    of, _ = _torch_impl(q, k, v, L, 1 / 16, ks, vs, flush_below=2.0 ** -6)
    assert np.all(of[:, :, 128:] == 0)
    assert _rowerr(of, o8) > 2 * TOL_F8
    of, _ = _torch_impl(q, k, v, L, 1 / 16, ks, vs, flush_below=2.0 ** -7)
    assert _rowerr(of, o8) > 2 * TOL_F8


# ---------------------------------------------------------------- invariants

def _f8case(seed=21, B=3, L=(300, 1, 77)):
    case = synth.make_case("f8inv", B, list(L), "fp8", seed=seed)
    return case


def test_power_of_two_query_scaling_is_exact():
    case = _f8case()
    o8, l8 = oracle.case_attention_fp8mma(case)
    qf = oracle.decode_bf16(case.q)
    for s in (4.0, 1 / 8, 2.0 ** 30):
        q2 = synth.bf16_bits((qf * s).astype(np.float32))
        assert np.array_equal(oracle.decode_bf16(q2), qf * s)
        o2, l2 = oracle.attention_fp8mma(q2, case.k, case.v, case.seq_lens, k_scale=case.k_scale / s,
                                         v_scale=case.v_scale)
        # the query's own scale is undone exactly: only the score scale moves
        assert _rowerr(o2, o8) < 1e-13 and np.abs(l2 - l8).max() < 1e-12


def test_token_order_invariance():
    case = _f8case(B=1, L=(500,))
    o8, l8 = oracle.case_attention_fp8mma(case)
    perm = np.random.default_rng(2).permutation(500)
    k2 = case.k.copy()
    v2 = case.v.copy()
    k2[0, :500] = case.k[0, perm]
    v2[0, :500] = case.v[0, perm]
    o2, l2 = oracle.attention_fp8mma(case.q, k2, v2, case.seq_lens, k_scale=case.k_scale, v_scale=case.v_scale)
    assert _rowerr(o2, o8) < 1e-13 and np.abs(l2 - l8).max() < 1e-13


def test_paged_equals_contiguous_bitwise():
    case = synth.make_case("f8pg", 3, [300, 64, 129], "fp8", seed=23, paged=True)
    o8, l8 = oracle.case_attention_fp8mma(case)
    kc = np.zeros((3, 320, 256), np.uint8)
    vc = np.zeros_like(kc)
    for b, n in enumerate(case.seq_lens):
        kk, vv = oracle.gather_kv(case.k, case.v, case.seq_lens, b, page_table=case.page_table)
        kc[b, :n], vc[b, :n] = kk, vv
    oc, lc = oracle.attention_fp8mma(case.q, kc, vc, case.seq_lens, k_scale=case.k_scale, v_scale=case.v_scale)
    assert np.array_equal(o8, oc) and np.array_equal(l8, lc)


def test_one_token_equal_keys_and_empty():
    case = _f8case(B=3, L=(1, 200, 0))
    k = case.k.copy()
    k[1, :200] = k[1, 0]                      # equal keys in sequence 1
    o8, l8 = oracle.attention_fp8mma(case.q, k, case.v, case.seq_lens, k_scale=case.k_scale,
                                     v_scale=case.v_scale)
    vf = oracle.decode_e4m3(case.v)
    # one token: its V row exactly (the weight divides out)
    assert np.array_equal(o8[0], np.broadcast_to(vf[0, 0] * case.v_scale, (64, 256)))
    # equal keys: equal weights, the mean of V
    assert _rowerr(o8[1], np.broadcast_to(vf[1, :200].mean(axis=0) * case.v_scale, (64, 256))) < 1e-13
    # empty: zero output, -inf lse
    assert np.all(o8[2] == 0) and np.all(np.isneginf(l8[2]))


def test_exact_sum_inputs_still_round_and_catch_rtz():
    """The GPU's tight parity inputs (tests/fp8_inputs.exact_dot_case): every
    product sum is exact, yet the quantisers round (the result is several
    percent from exact attention), and a round-toward-zero quantiser moves it
    by more than the GPU bar."""
    from fp8_inputs import exact_dot_case
    case = exact_dot_case(31, [4096, 1000, 130])
    o8, l8 = oracle.case_attention_fp8mma(case)
    o, _ = oracle.case_attention(case)
    assert _rowerr(o8, o) > 2e-2
    ot, lt = _torch_impl(case.q, case.k, case.v, case.seq_lens, 1 / 16, case.k_scale, case.v_scale)
    assert _rowerr(ot, o8) < 1e-12 and np.abs(lt - l8).max() < 1e-12
    orz, _ = _torch_impl(case.q, case.k, case.v, case.seq_lens, 1 / 16, case.k_scale, case.v_scale, rtz=True)
    assert _rowerr(orz, o8) > 2 * TOL_F8
    # every E4M3 query value is an integer (or zero) of at most 256 and every
    # product an integer of at most 512: exact in any accumulator keeping 12
    # bits below its largest product
    qf = oracle.decode_bf16(case.q)
    q8 = np.array([[oracle.decode_e4m3(oracle.encode_e4m3(qf[b, h] * 2.0 ** oracle.fp8_q_exponent(
        np.abs(qf[b, h]).max()))) for h in range(64)] for b in range(case.batch)])
    assert np.all(q8 == np.round(q8)) and np.abs(q8).max() <= 256
