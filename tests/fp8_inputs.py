"""Hand-built inputs for the FP8 attention arithmetic (test helpers, no
arithmetic of the method): queries and E4M3 key codes placed so that the
scores land where a check needs them.
"""
from __future__ import annotations

import numpy as np

import synth

ONE = 0x38          # E4M3 code of 1.0
MINUS_ONE = 0xB8    # E4M3 code of -1.0
BF16_ONE = 0x3F80   # bf16 bits of 1.0


def exact_case(seed: int, B: int, H: int, D: int, L: int, q_pow2: int = 0):
    """Every quantiser is the identity: each head's query has four entries
    +-2^q_pow2 on dims of its own (the rest zero), each key is -1, 0 or +1 on
    those dims, so with softmax_scale * k_scale = ln 2 * 2^-q_pow2 the
    base-2 scores are integers spanning at most 8 octaves and every 4 P is an
    E4M3 value. Returns (q bits [B, H, D], k, v codes [B, L, D], softmax
    scale)."""
    g = np.random.default_rng(seed)
    assert 4 * H <= D
    qf = np.zeros((B, H, D), dtype=np.float32)
    k = synth.e4m3_codes(g.standard_normal((B, L, D)) * 8.0)   # dims no query reads
    for h in range(H):
        dims = slice(4 * h, 4 * h + 4)
        qf[:, h, dims] = g.choice([-1.0, 1.0], size=(B, 4)) * 2.0 ** q_pow2
    ks = g.choice([MINUS_ONE, 0, ONE], size=(B, L, 4 * H)).astype(np.uint8)
    k[:, :, :4 * H] = ks
    v = synth.e4m3_codes(g.standard_normal((B, L, D)))
    return synth.bf16_bits(qf), k, v, float(np.log(2.0)) * 2.0 ** -q_pow2


def subnormal_case(seed: int, lens, H: int = 64, D: int = 256):
    """Scores that put almost every weight below E4M3's smallest normal value.
    Every query is 1 on dims 0 and 1. The first token of every 64-token step
    has keys 0 there (score 0, the maximum, so every piece's first step holds
    its maximum); every other token has key codes k0 in {-448, -416, -384}
    and k1 in [-60, 0], which with softmax_scale 1/16 and k_scale 0.24 gives
    base-2 scores in [-11, -8.3]: 4 P in [2^-9, 2^-6.3], all E4M3
    subnormals. V is 1 on dims [0, 128) for the maximal tokens and on
    [128, 256) for the others, so the output's second half is the share of
    the subnormal weights (about 7%). Returns (q bits [B, H, D], k, v codes
    [B, S, D], k_scale, v_scale)."""
    g = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    B, S = len(lens), max(1, int(lens.max()))
    q = np.zeros((B, H, D), dtype=np.uint16)
    q[:, :, 0] = BF16_ONE
    q[:, :, 1] = BF16_ONE
    k = synth.e4m3_codes(g.standard_normal((B, S, D)))
    k0 = g.choice([-448.0, -416.0, -384.0], size=(B, S))
    k1 = -g.uniform(0.0, 60.0, size=(B, S))
    k[:, :, 0] = synth.e4m3_codes(k0)
    k[:, :, 1] = synth.e4m3_codes(k1)
    top = (np.arange(S) % 64) == 0
    k[:, top, 0] = 0
    k[:, top, 1] = 0
    v = np.zeros((B, S, D), dtype=np.uint8)
    v[:, top, :128] = ONE
    v[:, ~top, 128:] = ONE
    return q, k, v, 0.24, 1.0


def exact_dot_case(seed: int, lens, H: int = 64, D: int = 256, paged: bool = False):
    """Inputs on which every FP8 dot product of the FP8-MFMA mode is exact in
    any accumulator that keeps 12 bits below its largest product, while the
    quantisers still round: each head's query has one entry in [128, 256) and
    the others in [16, 256) or zero, as bf16 values that are mostly not E4M3
    values, so with e = 0 every E4M3 query value is an integer of at most
    256; keys take the values 0, +-1/2, +-1, +-2 (integer products of at most
    512); values are 0 or +-1 (products are the weights' codes, multiples of
    2^-9).
    k_scale puts the base-2 scores at a standard deviation of about 1, so the
    weights spread widely but almost none lies more than 8 octaves below the
    largest (where E4M3's subnormal grid would make the result depend on
    each piece's own reference). Returns a synth.Case."""
    g = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    B, S = len(lens), max(1, int(lens.max()))
    mag = g.uniform(16.0, 255.0, (B, H, D))
    mag[:, :, 0] = g.uniform(128.0, 255.0, (B, H))
    mag *= g.choice([-1.0, 1.0], size=mag.shape)
    mag[:, :, 1:][g.random((B, H, D - 1)) < 0.2] = 0.0
    q = synth.bf16_bits(mag.astype(np.float32))
    kv = synth.e4m3_codes(g.choice([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0], size=(B, S, D)))
    vv = synth.e4m3_codes(g.choice([0.0, 1.0, -1.0], size=(B, S, D), p=[0.2, 0.4, 0.4]))
    case = synth.Case(name="f8exact", batch=B, kv_dtype="fp8", seq_lens=lens, k=kv, v=vv, q=q,
                      k_scale=1.0 / 240.0, v_scale=0.3)
    if paged:
        pages = (lens + 63) // 64
        P = int(pages.sum())
        perm = g.permutation(P).astype(np.int32)
        pt = np.zeros((B, max(1, int(pages.max()))), dtype=np.int32)
        kp = np.zeros((P, 64, D), dtype=np.uint8)
        vp = np.zeros_like(kp)
        j = 0
        for b in range(B):
            for i in range(int(pages[b])):
                pt[b, i] = perm[j]
                n = min(64, int(lens[b]) - 64 * i)
                kp[perm[j], :n] = kv[b, 64 * i:64 * i + n]
                vp[perm[j], :n] = vv[b, 64 * i:64 * i + n]
                j += 1
        case.k, case.v, case.page_table = kp, vp, pt
    return case
