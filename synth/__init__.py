"""Seeded synthetic inputs for the MFA decode step.

This module is shared by the CPU oracle and the GPU path. It holds none of
the attention arithmetic: it draws numbers, rounds them into the storage
formats (bf16 bit patterns, OCP FP8-E4M3FN codes) and lays out the KV cache
and page table. Decoding those formats is left to each consumer.

Shapes follow the Step-3 summary page ("Step-3 is Large yet Affordable",
Key points): hidden size 7168, a 2048-wide query bottleneck, 64 query heads
sharing one key head and one value head of dimension 256.

Every tensor draws from its own child of ``SeedSequence(seed)`` (numpy
PCG64), so adding a tensor never shifts the numbers of another.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

HIDDEN = 7168
Q_RANK = 2048
NUM_HEADS = 64
HEAD_DIM = 256
PAGE_SIZE = 64
FP8_MAX = 448.0

# fixed order of per-tensor random streams; append only
_STREAMS = ("q", "k", "v", "seq_lens", "perm", "x", "w_qa", "w_qb", "gamma", "w_k", "w_v")


def _streams(seed: int) -> dict:
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {n: np.random.Generator(np.random.PCG64(s)) for n, s in zip(_STREAMS, kids)}


# --------------------------------------------------------------------------- formats

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def e4m3_codes(a: np.ndarray, block: int = 1 << 22) -> np.ndarray:
    """float -> OCP FP8 E4M3FN codes (uint8), round to nearest even, saturating
    at +-448 (the format's largest finite value). Never produces the NaN code."""
    a = np.asarray(a)
    flat = a.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for s in range(0, flat.size, block):
        x = flat[s:s + block].astype(np.float64)
        sign = np.signbit(x)
        m = np.minimum(np.abs(x), FP8_MAX)
        _, e2 = np.frexp(m)                     # m = f * 2**e2, f in [0.5, 1)
        e = np.maximum(e2 - 1, -6)              # unbiased exponent, subnormals at -6
        q = np.rint(np.ldexp(m, 3 - e))         # 3 mantissa bits, ties to even
        carry = q >= 16                         # rounding overflowed the mantissa
        e = np.where(carry, e + 1, e)
        q = np.where(carry, q / 2, q)
        q = q.astype(np.int64)
        normal = q >= 8
        code = np.where(normal, ((e + 7) << 3) | (q - 8), q)  # subnormal: exp field 0
        code = np.where(m == 0, 0, code)
        code = np.minimum(code, 0x7E)           # saturate (448 = 0x7E)
        out[s:s + block] = (code | (sign.astype(np.int64) << 7)).astype(np.uint8)
    return out.reshape(a.shape)


# --------------------------------------------------------------------------- cases

@dataclasses.dataclass
class Case:
    """One decode-step workload, host side.

    q      uint16 [B, H, D] bf16 bits (None when the case runs the Q projection)
    k, v   contiguous: [B, kv_stride, D]; paged: [num_pages, PAGE_SIZE, D];
           uint16 (bf16 bits) or uint8 (E4M3FN codes). With kv_heads = G > 1
           (grouped-query caches): [B, G, kv_stride, D] / [num_pages, G,
           PAGE_SIZE, D]
    seq_lens int32 [B]; page_table int32 [B, pt_stride] or None
    k_scale, v_scale  float32 dequant scales (1.0 for bf16)
    x, w_qa, gamma, w_qb  bf16 bits for the Q projection, or None
    w_k, w_v  bf16 bits [HIDDEN, D] for the new token's K and V, or None
    """
    name: str
    batch: int
    kv_dtype: str                  # "bf16" | "fp8"
    seq_lens: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q: Optional[np.ndarray] = None
    page_table: Optional[np.ndarray] = None
    k_scale: float = 1.0
    v_scale: float = 1.0
    x: Optional[np.ndarray] = None
    w_qa: Optional[np.ndarray] = None
    gamma: Optional[np.ndarray] = None
    w_qb: Optional[np.ndarray] = None
    w_k: Optional[np.ndarray] = None
    w_v: Optional[np.ndarray] = None
    softmax_scale: float = 1.0 / 16.0
    rms_eps: float = 1e-6
    kv_latent: int = 0             # 512: latent-cache case (k = v = latent rows [., 512], q [B, 64, 512])
    split_tokens: int = 0
    seed: int = 0
    kv_heads: int = 1

    @property
    def paged(self) -> bool:
        return self.page_table is not None

    @property
    def max_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    @property
    def kv_stride(self) -> int:
        return 0 if self.paged else int(self.k.shape[1])

    def kv_bytes_read(self) -> int:
        """Bytes of K and V the method has to read: every cached row t < L_b."""
        per_tok = 2 * HEAD_DIM * (1 if self.kv_dtype == "fp8" else 2)
        return int(self.seq_lens.astype(np.int64).sum()) * per_tok


def _normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _kv_tensor(g, shape, kv_dtype):
    a = _normal(g, shape)
    if kv_dtype == "bf16":
        return bf16_bits(a), 1.0
    amax = float(np.abs(a).max()) if a.size else 1.0
    scale = float(np.float32(amax / FP8_MAX)) if amax > 0 else 1.0
    codes = e4m3_codes(a / np.float32(scale))
    return codes, scale


def make_case(name: str, batch: int, seq_lens, kv_dtype: str = "bf16", *,
              seed: int = 0, paged: bool = False, with_qproj: bool = False,
              q_std: float = 1.0, split_tokens: int = 0, max_context: int = 0,
              kv_slack: int = 0, append_room: int = 0, with_kv_proj: bool = False,
              kv_heads: int = 1) -> Case:
    """Build a case. ``seq_lens`` is an int or a sequence of B ints.

    Contiguous caches have ``kv_stride = max(L) + kv_slack`` token slots per
    sequence; slots past L_b hold random data that must be ignored. Paged
    caches hold P = sum_b ceil(L_b/64) pages; page_table[b][j] = perm[off_b+j]
    with perm a seeded permutation of [0, P), assigned in (b, j) order. Unused
    page-table entries and cache rows past L_b hold 0 / random data.

    ``append_room`` tokens of room past L_b are reserved for appended rows
    (contiguous: added to the slack; paged: pages cover L_b + append_room).
    ``with_kv_proj`` adds the hidden state x and the K and V projection
    weights, drawn like the Q projection's (std 1/sqrt(HIDDEN)).
    ``kv_heads`` = G > 1 gives grouped-query caches with G K/V heads per token
    (head axis after the sequence or page axis), drawn like the others.
    """
    st = _streams(seed)
    L = np.broadcast_to(np.asarray(seq_lens, dtype=np.int32), (batch,)).copy()
    maxL = int(L.max()) if batch else 0
    case = Case(name=name, batch=batch, kv_dtype=kv_dtype, seq_lens=L,
                k=None, v=None, seed=seed, split_tokens=split_tokens, kv_heads=kv_heads)
    heads = (kv_heads,) if kv_heads > 1 else ()
    if paged:
        npg = (L.astype(np.int64) + append_room + PAGE_SIZE - 1) // PAGE_SIZE
        P = int(npg.sum())
        pt_stride = max(1, (max(maxL + append_room, max_context) + PAGE_SIZE - 1) // PAGE_SIZE)
        perm = st["perm"].permutation(P).astype(np.int32)
        pt = np.zeros((batch, pt_stride), dtype=np.int32)
        off = 0
        for b in range(batch):
            n = int(npg[b])
            pt[b, :n] = perm[off:off + n]
            off += n
        case.page_table = pt
        shape = (max(P, 1), *heads, PAGE_SIZE, HEAD_DIM)
    else:
        shape = (batch, *heads, maxL + kv_slack + append_room, HEAD_DIM)
    case.k, case.k_scale = _kv_tensor(st["k"], shape, kv_dtype)
    case.v, case.v_scale = _kv_tensor(st["v"], shape, kv_dtype)
    if with_qproj:
        case.x = bf16_bits(_normal(st["x"], (batch, HIDDEN)))
        case.w_qa = bf16_bits(_normal(st["w_qa"], (HIDDEN, Q_RANK), 1.0 / math.sqrt(HIDDEN)))
        case.w_qb = bf16_bits(_normal(st["w_qb"], (Q_RANK, NUM_HEADS * HEAD_DIM),
                                      1.0 / math.sqrt(Q_RANK)))
        case.gamma = bf16_bits(np.ones(Q_RANK, dtype=np.float32))
    else:
        case.q = bf16_bits(_normal(st["q"], (batch, NUM_HEADS, HEAD_DIM), q_std))
    if with_kv_proj:
        if case.x is None:
            case.x = bf16_bits(_normal(st["x"], (batch, HIDDEN)))
        case.w_k = bf16_bits(_normal(st["w_k"], (HIDDEN, HEAD_DIM), 1.0 / math.sqrt(HIDDEN)))
        case.w_v = bf16_bits(_normal(st["w_v"], (HIDDEN, HEAD_DIM), 1.0 / math.sqrt(HIDDEN)))
    return case


# The five workloads: (1) tiny, (2) full layer with Q projection, (3) FP8
# contiguous, (4) FP8 paged ragged, (5) long-context split-K. Seeds 1000+i.

def config_case(i: int, *, batch: Optional[int] = None, scale_len: float = 1.0,
                q_std: float = 1.0, append: bool = False) -> Case:
    """Workload ``i`` (1..5). ``batch`` and ``scale_len`` shrink it for tests
    (same recipe, smaller sizes); the defaults give the full size.
    ``append`` adds the new token's K/V projection weights (and x) and one
    row of cache room per sequence, for the KV-append step; the other tensors
    are unchanged except a paged pool's page count and permutation."""
    if append:
        return _with_append(config_case(i, batch=batch, scale_len=scale_len, q_std=q_std))
    seed = 1000 + i
    if i == 1:
        B = batch or 1
        return make_case("tiny", B, max(1, int(256 * scale_len)), "bf16", seed=seed, q_std=q_std)
    if i == 2:
        B = batch or 32
        return make_case("full_layer", B, max(1, int(4096 * scale_len)), "bf16", seed=seed,
                         with_qproj=True)
    if i == 3:
        B = batch or 128
        return make_case("fp8_contig", B, max(1, int(4096 * scale_len)), "fp8", seed=seed,
                         q_std=q_std)
    if i == 4:
        B = batch or 384
        lo, hi = max(1, int(1024 * scale_len)), max(1, int(8192 * scale_len))
        g = _streams(seed)["seq_lens"]
        L = g.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
        return make_case("paged_ragged", B, L, "fp8", seed=seed, paged=True, q_std=q_std,
                         max_context=hi)
    if i == 5:
        B = batch or 8
        half = B // 2
        L = np.array([int(32768 * scale_len)] * half + [int(65536 * scale_len)] * (B - half),
                     dtype=np.int32)
        return make_case("long_splitk", B, L, "bf16", seed=seed, q_std=q_std, split_tokens=512)
    raise ValueError(f"no workload {i}")


def gqa_case(kv_heads: int, *, batch: Optional[int] = None, scale_len: float = 1.0,
             paged: bool = False, kv_dtype: str = "fp8") -> Case:
    """The FP8 workload's recipe (B = 128, L = 4096, N(0,1) Q and K/V, E4M3
    codes with per-tensor amax scales) with ``kv_heads`` K/V heads per token,
    for comparing head-sharing schemes at equal query shape. Seed 1003 for
    one head (the FP8 workload itself), 1100 + G otherwise. kv_dtype "bf16":
    the same shapes with a bf16 cache (seed 1200 + G), the BF16-attention
    setting of the comparison."""
    B = batch or 128
    if kv_dtype == "bf16":
        return make_case(f"bf16_gqa{kv_heads}", B, max(1, int(4096 * scale_len)), "bf16", seed=1200 + kv_heads,
                         paged=paged, kv_heads=kv_heads)
    seed = 1003 if kv_heads == 1 else 1100 + kv_heads
    return make_case(f"fp8_gqa{kv_heads}", B, max(1, int(4096 * scale_len)), "fp8", seed=seed,
                     paged=paged, kv_heads=kv_heads)


LATENT = 512


def latent_case(name: str, batch: int, seq_lens, *, seed: int = 0, paged: bool = False, kv_slack: int = 0,
                q_std: float = 1.0, split_tokens: int = 0) -> Case:
    """A latent-cache (MLA-style) case: one 512-wide latent row per token,
    N(0,1) encoded to E4M3 with a per-tensor amax scale, serving as key and
    value of all 64 heads (k and v are the same array); Q [B, 64, 512] bf16
    N(0, q_std). Contiguous [B, max(L) + kv_slack, 512] or pages [P, 64, 512]
    with the page table of make_case."""
    st = _streams(seed)
    L = np.broadcast_to(np.asarray(seq_lens, dtype=np.int32), (batch,)).copy()
    maxL = int(L.max()) if batch else 0
    case = Case(name=name, batch=batch, kv_dtype="fp8", seq_lens=L, k=None, v=None, seed=seed,
                split_tokens=split_tokens, kv_latent=LATENT)
    if paged:
        npg = (L.astype(np.int64) + PAGE_SIZE - 1) // PAGE_SIZE
        P = int(npg.sum())
        pt_stride = max(1, (maxL + PAGE_SIZE - 1) // PAGE_SIZE)
        perm = st["perm"].permutation(P).astype(np.int32)
        pt = np.zeros((batch, pt_stride), dtype=np.int32)
        off = 0
        for b in range(batch):
            n = int(npg[b])
            pt[b, :n] = perm[off:off + n]
            off += n
        case.page_table = pt
        shape = (max(P, 1), PAGE_SIZE, LATENT)
    else:
        shape = (batch, maxL + kv_slack, LATENT)
    case.k, case.k_scale = _kv_tensor(st["k"], shape, "fp8")
    case.v, case.v_scale = case.k, case.k_scale
    case.q = bf16_bits(_normal(st["q"], (batch, NUM_HEADS, LATENT), q_std))
    return case


def _with_append(base: Case) -> Case:
    c = make_case(base.name + "_append", base.batch, base.seq_lens, base.kv_dtype, seed=base.seed,
                  paged=base.paged, with_qproj=base.q is None, q_std=1.0, split_tokens=base.split_tokens,
                  max_context=int(base.seq_lens.max()) + 1 if base.paged else 0, append_room=1,
                  with_kv_proj=True)
    if base.q is not None:
        c.q = base.q
    return c


def mtp_queries(batch: int, t: int, seed: int) -> np.ndarray:
    """Queries of multi-token decode: bf16 bits [batch, t, 64, 256], N(0,1),
    from the "q" stream of ``seed``'s streams (t = 1 gives the single-token Q
    of a case built with the same seed)."""
    g = _streams(seed)["q"]
    return bf16_bits(_normal(g, (batch, t, NUM_HEADS, HEAD_DIM)))
