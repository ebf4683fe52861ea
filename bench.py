#!/usr/bin/env python3
"""Benchmark of the MFA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup W] [--workload fp8_contig]

A step is one pass of the hot path over one batch: the decode attention
(chunked scores, online softmax, P.V, log-sum-exp merge) and, for the
full-layer workload, the Q projection with RMSNorm before it. The two
"+append" workloads add the KV append of the new token before the attention
(its K and V projections, encoded and written at row L_b), which then reads
L_b + 1 rows: the full layer as a complete decode step, and the ragged paged
FP8 batch writing into its pool. Inputs are
seeded synthetic tensors already resident in HBM; several copies are rotated
so that consecutive steps do not find their KV cache in the 256 MB MALL.

Prints one JSON line: tokens/s per layer (batch / step time), the attention
kernel's achieved algorithmic HBM bandwidth against 8 TB/s, its MFMA rate
against the dense peak, and the fp64 CPU oracle timed on a bounded sample on
the host cores (with the largest row error of the GPU's output against it on
that sample). The step time is the wall time of the timed steps between two
device synchronisations; a HIP event pair on the launch stream brackets the
same steps. When a step is one kernel, the kernel's duration is that event
time per step (never more than the wall step). Otherwise per-kernel
durations come from a later pass in which the library attaches a HIP event
pair to each launch (hipExtLaunchKernel stamps the kernel's own start and
end); those pairs add launch gaps, so that pass is not the throughput pass.
A third pass with an event pair around every step gives the median and the
10th and 90th percentiles of the step time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MFA decode tokens/s per layer (1 GPU) + achieved HBM GB/s vs roofline"
HBM_PEAK_GBPS = 8000.0
WORKLOADS = {"tiny": 1, "full_layer": 2, "fp8_contig": 3, "paged_ragged": 4, "long_splitk": 5,
             "decode_step": 2, "paged_append": 4, "fp8_mtp2": 3, "fp8_mtp4": 3, "fp8_gqa2": 3, "fp8_gqa4": 3,
             "bf16_contig": 3, "bf16_gqa2": 3, "bf16_gqa4": 3, "fp8_mla": 3}
APPEND = ("decode_step", "paged_append")
MTP = {"fp8_mtp2": 2, "fp8_mtp4": 4}   # query tokens per sequence
GQA = {"fp8_gqa2": 2, "fp8_gqa4": 4}   # K/V heads (head-sharing comparison)
GQA_BF16 = {"bf16_contig": 1, "bf16_gqa2": 2, "bf16_gqa4": 4}   # the same with a bf16 cache
LATENT = ("fp8_mla",)   # latent-cache (MLA-style) comparison
DESCRIPTION = {
    "tiny": "B=1, L=256, bf16 KV, contiguous, decode only",
    "full_layer": "B=32, L=4096, bf16 KV, contiguous, Q projection 7168->2048 (RMSNorm)->64x256 + decode",
    "fp8_contig": "B=128, L=4096, FP8-E4M3 KV (per-tensor scales), contiguous, decode only",
    "paged_ragged": "B=384, L~U[1024,8192], FP8-E4M3 KV, 64-token pages, permuted page table, decode only",
    "long_splitk": "B=8, L=32768 x4 + 65536 x4, bf16 KV, split-K 512-token chunks, decode only",
    "decode_step": "B=32, L=4096, bf16 KV, contiguous: Q projection + KV append (7168->256 x2, row L_b) "
                   "+ decode over L_b+1",
    "paged_append": "B=384, L~U[1024,8192], FP8-E4M3 KV, 64-token pages: KV append (7168->256 x2, E4M3, "
                    "row L_b) + decode over L_b+1",
    "fp8_mtp2": "B=128, L=4096, FP8-E4M3 KV, contiguous, 2 query tokens per sequence (multi-token decode)",
    "fp8_mtp4": "B=128, L=4096, FP8-E4M3 KV, contiguous, 4 query tokens per sequence (multi-token decode)",
    "fp8_gqa2": "B=128, L=4096, FP8-E4M3 KV, contiguous, 64 query heads on 2 K/V heads (grouped-query comparison)",
    "fp8_gqa4": "B=128, L=4096, FP8-E4M3 KV, contiguous, 64 query heads on 4 K/V heads (grouped-query comparison)",
    "bf16_contig": "B=128, L=4096, bf16 KV, contiguous, 64 query heads on 1 K/V head (MFA, BF16-attention setting)",
    "bf16_gqa2": "B=128, L=4096, bf16 KV, contiguous, 64 query heads on 2 K/V heads (grouped-query comparison)",
    "bf16_gqa4": "B=128, L=4096, bf16 KV, contiguous, 64 query heads on 4 K/V heads (grouped-query comparison)",
    "fp8_mla": "B=128, L=4096, one 512-wide FP8-E4M3 latent row per token as key and value of 64 heads of 512 "
               "(absorbed MLA-style latent cache, same cache bytes per token as MFA), contiguous",
}
# sources that decide the attention kernel's memory traffic (kernel, launch
# shape, split and merge policy); the stored HBM counters hold for this hash
ATTN_SOURCES = ("decode_attention_mfa_amd/csrc/mfa_attn.hip", "decode_attention_mfa_amd/csrc/mfa_attn_ws.inc",
                "decode_attention_mfa_amd/csrc/mfa_device.h",
                "decode_attention_mfa_amd/csrc/mfa_internal.h", "decode_attention_mfa_amd/csrc/mfa_api.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # MI355X dense matrix peaks
WARMUP_SECONDS = 0.5


def attn_kernel_name(split: int, fp8: bool, latent: bool = False) -> str:
    """The attention kernel a launch runs: balanced split, chunks, or the
    latent-cache kernel."""
    if latent:
        return "mfa_mla_kernel"
    return "mfa_attn_balanced_kernel" if split == 0 else "mfa_attn_ws_split_kernel"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attn_source_sha() -> str:
    h = hashlib.sha256()
    for p in ATTN_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(case, attention_writes_out: bool, append: bool = False, qtok: int = 1):
    """(attention-kernel bytes, whole-step bytes) the method must move.
    Attention: every cached K and V row t < L_b (512 B per token and K/V
    head with FP8, 1024 B with bf16; t <= L_b after an append), Q (32 KB per sequence), the
    lengths and (paged) the page-table entries it reads, and the bf16 output
    (32 KB per sequence) when the attention kernel writes it (no separate
    merge launch). Step: all of that plus the output; with the Q projection,
    x, gamma and both projection weights (Q is then produced on the device,
    not read); with the append, x, W_k, W_v, the lengths and page-table
    entries it reads and the K and V rows it writes."""
    import numpy as np
    B = case.batch
    L = case.seq_lens.astype(np.int64) + (1 if append else 0)
    elem = 1 if case.kv_dtype == "fp8" else 2
    latent = getattr(case, "kv_latent", 0)
    if latent:   # one latent row per token, read once as key and value; 512-wide Q and output rows
        kv = int(L.sum()) * latent * elem
    else:
        kv = int(L.sum()) * 2 * 256 * elem * getattr(case, "kv_heads", 1)
    width = latent or 256
    q = B * qtok * 64 * width * 2
    o = B * qtok * 64 * width * 2
    meta = B * 4
    if case.paged:
        meta += int(((L + 63) // 64).sum()) * 4
    attn = kv + q + meta + (o if attention_writes_out else 0)
    step = kv + q + meta + o
    if case.w_qa is not None:
        step += case.x.nbytes + case.w_qa.nbytes + case.w_qb.nbytes + case.gamma.nbytes
        attn -= q
        step -= q
    if append:
        step += case.w_k.nbytes + case.w_v.nbytes + B * 4 + B * 2 * 256 * elem
        step += case.x.nbytes if case.w_qa is None else 0
        step += B * 4 if case.paged else 0
    return attn, step


def append_bytes(case):
    """Bytes the KV append must move: x, W_k, W_v, the lengths (and page-table
    entries) it reads and the two rows per sequence it writes."""
    elem = 1 if case.kv_dtype == "fp8" else 2
    return (case.x.nbytes + case.w_k.nbytes + case.w_v.nbytes + case.batch * (8 if case.paged else 4)
            + case.batch * 2 * 256 * elem)


def sample_case(case, n):
    """The first n sequences of a workload (same cache pool when paged)."""
    import copy
    s = copy.copy(case)
    s.batch = n
    s.seq_lens = case.seq_lens[:n]
    if case.q is not None:
        s.q = case.q[:n]
    if case.x is not None:
        s.x = case.x[:n]
    if case.paged:
        s.page_table = case.page_table[:n]
    else:
        s.k = case.k[:n]
        s.v = case.v[:n]
    return s


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(case, budget_s: float, gpu_out=None, gpu_lse=None):
    """The fp64 oracle, as it stands, on the first n sequences; n chosen from
    a one-sequence probe so that the run takes about budget_s seconds. With
    the GPU's output of the workload (gpu_out bf16 bits, gpu_lse), also the
    largest row error of the GPU against the oracle on that sample (row-wise
    max |o_gpu - o_ref| / max |o_ref|; absolute on the log-sum-exp)."""
    import numpy as np
    import oracle

    qtok = case.q.shape[1] if case.q is not None and case.q.ndim == 4 else 1

    def work(s):
        if s.w_k is not None:
            oracle.kv_project(s.x, s.w_k, s.w_v)
        if qtok > 1:
            return oracle.attention_mtp(oracle.decode_bf16(s.q), s.k, s.v, s.seq_lens,
                                        kv_dtype=oracle.KV_FP8 if s.kv_dtype == "fp8" else oracle.KV_BF16,
                                        k_scale=s.k_scale, v_scale=s.v_scale, page_table=s.page_table)
        return oracle.case_attention(s)

    t0 = time.perf_counter()
    work(sample_case(case, 1))
    t1 = time.perf_counter() - t0
    n = max(1, min(case.batch, int(budget_s / max(t1, 1e-3))))
    s = sample_case(case, n)
    t0 = time.perf_counter()
    ref = work(s)
    dt = time.perf_counter() - t0
    what = " + ".join(w for w, on in (("Q projection", case.w_qa is not None),
                                       ("K/V projection", case.w_k is not None), ("attention", True)) if on)
    res = {"value": n * qtok / dt, "unit": "tokens/s/layer", "cores": oracle.max_threads(), "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{what} of the first {n} of {case.batch} sequences, fp64, {dt:.1f} s"}
    if ref is not None and gpu_out is not None:
        o_ref, lse_ref = ref
        o = oracle.decode_bf16(gpu_out[:n].reshape(o_ref.shape))
        lse = gpu_lse[:n].reshape(lse_ref.shape).astype(np.float64)
        live = np.isfinite(lse_ref)
        den = np.maximum(np.abs(o_ref).max(axis=-1), 1e-30)
        err = (np.abs(o - o_ref).max(axis=-1) / den)[live]
        res["parity"] = {"max_row_err": float(err.max()) if err.size else 0.0,
                         "max_lse_err": float(np.abs(lse - lse_ref)[live].max()) if err.size else 0.0,
                         "vs": "exact fp64 oracle", "rows": int(err.size)}
    return res


def context_rates(mfa, torch) -> dict:
    """Rates measured on this GPU to set beside the data-sheet peaks that the
    roofline and MFMA fractions divide by: a device copy of 1 GiB (bytes read
    plus bytes written over its time) and the matrix-core microbenchmark
    (mfa_debug_mfma_rate) for the two MFMA shapes the path uses."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        dst.copy_(src)
    reps = 10
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * n * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    rates = {}
    for kind, name in ((0, "bf16"), (1, "fp8")):
        iters = 1 << 14
        mfa.mfa_debug_mfma_rate(kind, iters, sink)   # warm-up
        fl = 0.0
        e0.record()
        for _ in range(5):
            fl += mfa.mfa_debug_mfma_rate(kind, iters, sink)
        e1.record()
        torch.cuda.synchronize()
        rates[name] = round(fl / (e0.elapsed_time(e1) / 1e3) / 1e12, 1)
    return {"stream_copy_gbps": round(copy_gbps, 1),
            "stream_copy": "device copy of 1 GiB, (read + written bytes) / time, 10 copies",
            "mfma_rate_tflops": rates,
            "mfma_rate": "mfa_debug_mfma_rate: independent v_mfma_f32_16x16x32_bf16 / unit-scaled "
                         "v_mfma_f32_16x16x128_f8f6f4 on register operands, two waves per SIMD, 5 launches"}


def traffic_key(workload: str, attn_math: str) -> str:
    """Key of a workload's stored HBM counters (per attention arithmetic)."""
    return workload if attn_math == "bf16" else f"{workload}/{attn_math}"


def load_traffic(workload: str, sha: str):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("source_sha") != sha:
        return None
    return float(e["traffic_bytes_per_launch"])


def load_counters(workload: str, sha: str):
    """Stored rocprofv3 counter figures of a workload's attention kernel, if
    taken on the current sources."""
    try:
        with open(COUNTERS_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("source_sha") != sha:
        return None
    return e


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=-1,
                    help="untimed steps first; default: as many as take %.1f s" % 0.5)
    ap.add_argument("--workload", default="fp8_contig", choices=sorted(WORKLOADS))
    ap.add_argument("--split", type=int, default=None, help="override the split-K chunk (tokens)")
    ap.add_argument("--attn-math", default="bf16", choices=("bf16", "fp8"),
                    help="attention arithmetic: bf16 MFMAs (default) or FP8 MFMAs (FP8 caches only)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-baseline budget; 0 skips it")
    ap.add_argument("--context", type=int, default=1,
                    help="1 (default): also measure a device copy and the MFMA rate microbenchmark")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a device copy of known size (for HBM counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the MFA decode path runs on one GPU; --gpus {args.gpus} is not supported "
              "(there is no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = 512 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))
        return

    import decode_attention_mfa_amd as mfa
    from decode_attention_mfa_amd import harness
    import synth

    wl = args.workload
    log(f"[bench] generating workload {wl}: {DESCRIPTION[wl]}")
    t0 = time.perf_counter()
    append = wl in APPEND
    qtok = MTP.get(wl, 1)
    if wl in GQA:
        case = synth.gqa_case(GQA[wl])
    elif wl in GQA_BF16:
        case = synth.gqa_case(GQA_BF16[wl], kv_dtype="bf16")
    elif wl in LATENT:
        case = synth.latent_case(wl, 128, 4096, seed=1300)
    else:
        case = synth.config_case(WORKLOADS[wl], append=append)
    if qtok > 1:
        case.q = synth.mtp_queries(case.batch, qtok, case.seed)
    log(f"[bench] generated in {time.perf_counter() - t0:.1f} s")
    _, step_bytes = algorithmic_bytes(case, True, append, qtok)

    dc = harness.to_device(case)
    # rotate copies of the per-step inputs so that no step finds them in the MALL
    nrot = max(2, min(8, math.ceil(768e6 / max(step_bytes, 1)) + 1))
    if step_bytes * nrot > 6e9:
        nrot = 2
    sets = [dc]
    for _ in range(nrot - 1):
        c = harness.DeviceCase(**{f: getattr(dc, f) for f in dc.__dataclass_fields__})
        c.k, c.v = dc.k.clone(), dc.v.clone()
        if dc.q is not None:
            c.q = dc.q.clone()
        if dc.x is not None:
            c.x = dc.x.clone()
        if dc.w_qa is not None:
            c.w_qa, c.w_qb = dc.w_qa.clone(), dc.w_qb.clone()
        if dc.w_k is not None:
            c.w_k, c.w_v = dc.w_k.clone(), dc.w_v.clone()
        sets.append(c)
    cold = nrot * step_bytes > 512e6

    # after the append the attention reads L_b + 1 rows
    attn_lens = dc.seq_lens + 1 if append else dc.seq_lens
    attn_max = dc.max_len + 1 if append else dc.max_len
    attn_min = dc.min_len + 1 if append else dc.min_len
    attn_math = mfa.MFA_ATTN_FP8_MFMA if args.attn_math == "fp8" else mfa.MFA_ATTN_BF16_MFMA
    h = harness.create_handle(dc, split_tokens=args.split, max_context=attn_max, max_batch=dc.batch * qtok,
                              attn_math=attn_math)
    # multi-token decode: its own chunked split, one workgroup per (sequence,
    # token, chunk)
    if qtok > 1:
        split = mfa.mfa_split_tokens_mtp(h, dc.batch, qtok, attn_max)
        head_groups = 1
    else:
        split = mfa.mfa_split_tokens(h, dc.batch, attn_max, attn_min)
        head_groups = mfa.mfa_head_groups(h, dc.batch, attn_max, attn_min)
    stream = torch.cuda.Stream()
    if qtok > 1:
        outs = [(torch.empty((dc.batch, qtok, 64, 256), dtype=torch.int16, device="cuda"),
                 torch.empty((dc.batch, qtok, 64), dtype=torch.float32, device="cuda")) for _ in range(nrot)]
    else:
        outs = [harness.alloc_outputs(dc) for _ in range(nrot)]
    qbufs = [torch.empty((dc.batch, 64, 256), dtype=torch.int16, device="cuda") for _ in range(nrot)]

    kvs = [c.kv() for c in sets]
    attn_kvs = [mfa.make_kv(c.k, c.v, attn_lens, page_table=c.page_table, k_scale=c.k_scale,
                            v_scale=c.v_scale, max_seq_len=attn_max, min_seq_len=attn_min) for c in sets]

    def step(i):
        s = sets[i % nrot]
        o, l = outs[i % nrot]
        q = s.q
        if s.q is None:
            q = qbufs[i % nrot]
            mfa.mfa_qproj(h, s.x, s.w_qa, s.gamma, s.w_qb, q, s.batch, stream)
        if append:
            # writes row L_b (the same row every step: the cache stays as it is)
            mfa.mfa_kv_append(h, s.x, s.w_k, s.w_v, kvs[i % nrot], s.batch, stream)
        if qtok > 1:
            mfa.mfa_decode_mtp(h, q, attn_kvs[i % nrot], qtok, o, l, s.batch, stream)
        else:
            mfa.mfa_decode(h, q, attn_kvs[i % nrot], o, l, s.batch, stream)

    def run(n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            step(i)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    with torch.cuda.stream(stream):
        # warm-up: W steps, or at least WARMUP_SECONDS of them when W is not
        # given, so that clocks and caches reach their steady state
        warmup = args.warmup
        if warmup < 0:
            t = run(10)
            warmup = max(20, int(math.ceil(WARMUP_SECONDS / (t / 10))))
        run(warmup)
        # timed steps (the reported throughput), no per-launch events: wall
        # time between two synchronisations, and an event pair on the launch
        # stream around the same steps
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(args.steps):
            step(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        gpu_ms = ev0.elapsed_time(ev1)
        # the step-time distribution: an event pair around every step
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.steps)]
        for i, (a, b) in enumerate(pairs):
            a.record(stream)
            step(i)
            b.record(stream)
        torch.cuda.synchronize()
        step_ms = sorted(a.elapsed_time(b) for a, b in pairs)
        # per-kernel durations: an event pair attached to every launch
        mfa.mfa_profile_enable(h, True)
        mfa.mfa_profile_read(h)
        run(args.steps)
        prof = mfa.mfa_profile_read(h)
        mfa.mfa_profile_enable(h, False)
    mfa.mfa_destroy(h)
    args.warmup = warmup

    ms_per_step = dt * 1e3 / args.steps
    value = dc.batch * qtok / (ms_per_step / 1e3)
    attn_bytes, _ = algorithmic_bytes(case, prof["combine"][0] == 0, append, qtok)
    n_attn, ms_attn = prof["attention"]
    one_kernel = all(n == 0 for k, (n, _) in prof.items() if k != "attention")
    if one_kernel:
        # the step is the attention kernel alone: its duration is the event
        # time of the timed steps per step (launch gaps included)
        attn_ms = gpu_ms / args.steps
        timing = "HIP event pair on the launch stream around the timed steps (one kernel per step)"
    else:
        attn_ms = ms_attn / max(n_attn, 1)
        timing = ("hipExtLaunchKernel event pairs on the launch stream (the kernel's own start and end), "
                  "over a later pass of the same steps")
    if attn_ms > ms_per_step:   # a kernel cannot outlast the step it belongs to
        attn_ms = ms_per_step
        timing += "; capped at the step time"
    achieved = attn_bytes / (attn_ms / 1e3) / 1e9
    # MFMA work: scores and P.V, 2 x 64 x 256 multiply-adds per (query token, cached token)
    # (2 x 64 x 512 with a latent cache)
    flops = 4 * 64 * (getattr(case, "kv_latent", 0) or 256) * \
        int((case.seq_lens.astype(np.int64) + (1 if append else 0)).sum()) * qtok
    mfma_kind = "fp8" if args.attn_math == "fp8" else "bf16"
    mfma_tflops = flops / (attn_ms / 1e3) / 1e12
    counters = load_counters(traffic_key(wl, args.attn_math), attn_source_sha())
    pct = lambda q: step_ms[min(len(step_ms) - 1, int(q * len(step_ms)))] * 1e3
    sha = attn_source_sha()
    traffic = load_traffic(traffic_key(wl, args.attn_math), sha)
    kernels = {k: {"launches": n, "avg_us": round(ms * 1e3 / n, 2)} for k, (n, ms) in prof.items() if n}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s/layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": f"synthetic: seeded N(0,1) (numpy PCG64, seed {case.seed}), FP8 codes by RNE with "
                "per-tensor amax scales",
        "config": {"workload": wl, "description": DESCRIPTION[wl], "batch": case.batch,
                   "context_min": int(case.seq_lens.min()), "context_max": int(case.seq_lens.max()),
                   "kv_dtype": "fp8_e4m3" if case.kv_dtype == "fp8" else "bf16",
                   "layout": "paged64" if case.paged else "contiguous", "split_tokens": split,
                   "query_tokens": qtok,
                   "attn_math": "fp8 MFMA (quantised Q and P)" if args.attn_math == "fp8" else "bf16 MFMA",
                   "work_split": ("balanced ranges of steps" if split == 0 else f"chunks of {split} tokens")
                   + (f", heads in {head_groups} workgroups of {64 // head_groups}" if head_groups > 1 else ""),
                   "kv_heads": getattr(case, "kv_heads", 1),
                   "input_sets_rotated": nrot, "mall": "cold" if cold else "warm"},
        "step_hbm_gbps": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": attn_kernel_name(split, case.kv_dtype == "fp8",
                                                                bool(getattr(case, "kv_latent", 0))),
                     "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": attn_bytes,
                     "avg_launch_us": round(attn_ms * 1e3, 2), "source_sha": sha, "timing": timing},
        "mfma": {"dtype": mfma_kind, "flops_per_launch": flops, "achieved_tflops": round(mfma_tflops, 1),
                 "peak_tflops": MFMA_PEAK_TFLOPS[mfma_kind],
                 "frac": round(mfma_tflops / MFMA_PEAK_TFLOPS[mfma_kind], 4),
                 "busy_frac": counters.get("mfma_busy_frac") if counters else None,
                 "busy_source": "rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs), "
                                "profiles/counters.json" if counters else None},
        "step_us": {"median": round(pct(0.5), 2), "p10": round(pct(0.1), 2), "p90": round(pct(0.9), 2),
                    "n": len(step_ms), "timing": "HIP event pair around each step, a later pass"},
        "kernels": kernels,
    }
    if append:
        n_p, ms_p = prof["kv_proj"]
        n_w, ms_w = prof["kv_write"]
        ab = append_bytes(case)
        app_us = (ms_p / max(n_p, 1) + ms_w / max(n_w, 1)) * 1e3
        result["kv_append"] = {"algorithmic_bytes": ab, "kernels_us": round(app_us, 2),
                               "achieved_gbps": round(ab / (app_us / 1e6) / 1e9, 1),
                               "frac": round(ab / (app_us / 1e6) / 1e9 / HBM_PEAK_GBPS, 4)}
    if args.context:
        log("[bench] context: device copy and matrix-core rates")
        result["context"] = context_rates(mfa, torch)
    if args.cpu_seconds > 0:
        log("[bench] timing the fp64 CPU oracle on a bounded sample")
        o_last, l_last = outs[(args.steps - 1) % nrot]
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds,
                                              None if append else o_last.cpu().numpy().view(np.uint16),
                                              None if append else l_last.cpu().numpy())
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
