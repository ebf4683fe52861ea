"""bench.py's contract on the CPU: it refuses more than one GPU with a clear
message, and the algorithmic byte counts its roofline divides by follow the
definitions (K and V rows, Q, lengths, page-table entries, output when the
attention kernel writes it) at the workloads' shapes."""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _case(lens, kv="fp8", paged=False, **kw):
    base = dict(batch=len(lens), seq_lens=np.asarray(lens, dtype=np.int32), kv_dtype=kv, paged=paged,
                w_qa=None, kv_heads=1, kv_latent=0)
    base.update(kw)
    return SimpleNamespace(**base)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout


def test_fp8_contig_bytes():
    # 128 x 4096 tokens x (256 K + 256 V) bytes, 32 KB of Q and of output and
    # 4 B of length per sequence
    attn, step = bench.algorithmic_bytes(_case([4096] * 128), attention_writes_out=True)
    assert attn == step == 128 * 4096 * 512 + 128 * 32768 * 2 + 128 * 4 == 276_824_576


def test_long_splitk_bytes_exclude_the_combined_output():
    # bf16 rows (1 KB per token); the combine kernel writes the output, so
    # the attention kernel's bytes hold Q and the lengths only
    attn, step = bench.algorithmic_bytes(_case([32768] * 4 + [65536] * 4, kv="bf16"), attention_writes_out=False)
    assert attn == 393216 * 1024 + 8 * 32768 + 8 * 4 == 402_915_360
    assert step == attn + 8 * 32768


def test_paged_bytes_count_page_table_entries():
    attn, _ = bench.algorithmic_bytes(_case([1, 64, 65], paged=True), attention_writes_out=True)
    assert attn == 130 * 512 + 3 * 32768 * 2 + 3 * 4 + (1 + 1 + 2) * 4


def test_grouped_and_latent_bytes():
    attn, _ = bench.algorithmic_bytes(_case([100], kv_heads=2), attention_writes_out=True)
    assert attn == 100 * 512 * 2 + 32768 * 2 + 4
    # one 512-wide FP8 latent row per token, 64 KB of q and of output
    attn, _ = bench.algorithmic_bytes(_case([100], kv_latent=512), attention_writes_out=True)
    assert attn == 100 * 512 + 65536 * 2 + 4
    # multi-token decode: the rows once, Q and output per token
    attn, _ = bench.algorithmic_bytes(_case([100]), attention_writes_out=True, qtok=3)
    assert attn == 100 * 512 + 3 * 32768 * 2 + 4
