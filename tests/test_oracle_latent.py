"""Pins of the latent-cache (MLA-style) reading (CPU only).

The latent-cache mode computes, for every head, softmax attention of a
512-wide query against the token's latent row used as key and value
(multi-query attention over the latent, ``oracle.attention`` with D = 512 and
k = v). The pin here is the identity that makes that MLA's attention: with
per-head key and value up-projections W_uk,h and W_uv,h of the latent rows,
explicit attention (keys c_t W_uk,h, values c_t W_uv,h) equals the absorbed
form (query W_uk,h q_h in the latent space, output (sum_t p_t c_t) W_uv,h),
weights and log-sum-exp included, checked in fp64 on small random inputs.
"""
import numpy as np
import pytest

import oracle
import synth


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_absorbed_latent_attention_equals_explicit(seed):
    rng = np.random.default_rng(seed)
    H, dc, dh, L = 3, 16, 4, 9
    C = synth.bf16_bits(rng.standard_normal((1, L, dc)).astype(np.float32))   # latent rows, bf16 bits
    Cf = oracle.decode_bf16(C)[0]
    Wuk = rng.standard_normal((H, dc, dh))
    Wuv = rng.standard_normal((H, dc, dh))
    q = rng.standard_normal((H, dh))
    scale = 0.37
    o_exp = np.empty((H, dh))
    lse_exp = np.empty(H)
    for h in range(H):   # explicit: every head's own keys and values
        K, V = Cf @ Wuk[h], Cf @ Wuv[h]
        s = scale * (K @ q[h])
        m = s.max()
        w = np.exp(s - m)
        o_exp[h] = (w / w.sum()) @ V
        lse_exp[h] = m + np.log(w.sum())
    # absorbed: queries in the latent space, one shared latent row per token
    qt = np.stack([Wuk[h] @ q[h] for h in range(H)])[None]
    ot, lt = oracle.attention(qt, C, C, np.array([L], dtype=np.int32), kv_dtype=oracle.KV_BF16,
                              softmax_scale=scale)
    o_abs = np.stack([ot[0, h] @ Wuv[h] for h in range(H)])
    assert np.abs(o_abs - o_exp).max() < 1e-12
    assert np.abs(lt[0] - lse_exp).max() < 1e-12


def test_latent_case_shapes_and_identical_rows():
    """The generator's latent case: k and v are the same rows; a context whose
    latent rows are all equal returns that row (decoded, times the scale)."""
    c = synth.latent_case("t", 2, [5, 64], seed=3, kv_slack=1)
    assert c.k is c.v and c.k.shape == (2, 65, 512) and c.q.shape == (2, 64, 512) and c.kv_latent == 512
    c.k[0, :5] = c.k[0, 0]
    o, _ = oracle.case_attention(c)
    row = oracle.decode_e4m3(c.k[0, 0]) * c.k_scale
    assert np.abs(o[0] - row[None]).max() < 1e-12
