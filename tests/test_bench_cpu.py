"""CPU tests of bench.py's contract: it refuses more than one GPU, and its
algorithmic byte counts (the numerator of the reported GB/s and of
roofline.achieved) equal closed forms written out here from the cache
layout: per token and KV head, FP8/INT8 store d codes of one byte per K and
V row plus one fp32 scale each; KIVI stores d*bits/8 bytes of codes per row,
fp32 scale and zero-point per channel per G tokens (Key) and per G channels
per token (Value), and keeps the residual tokens in the input type."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from kvq_workloads import WORKLOADS, context_lengths  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _closed_form_decode_bytes(fmt, bits, G, R, B, Hkv, Hq, d, n, elem):
    if fmt in ("fp8", "int8"):
        cache = B * Hkv * n * 2 * (d + 4)
    else:
        nq = G * ((n - R) // G) if n > R else 0
        per_token = 2 * d * bits // 8 + (8 * d) // G + 8 * (d // G)
        cache = B * Hkv * (nq * per_token + (n - nq) * 2 * d * elem)
    return cache + B * Hq * d * (elem + 4)


@pytest.mark.parametrize("idx,expect_mb", [(2, 138.8), (3, 1110.4), (4, 1087.9)])
def test_decode_bytes_match_closed_form(idx, expect_mb):
    w = WORKLOADS[idx]
    lens = context_lengths(w).numpy()
    assert (lens == w.context).all()
    ref = _closed_form_decode_bytes(w.fmt, w.bits, w.group, w.residual, w.batch, w.n_kv_heads, w.n_q_heads,
                                    w.head_dim, w.context, 2)
    assert bench.decode_bytes(w, lens) == ref
    assert round(ref / 1e6, 1) == expect_mb


def test_long_context_decode_bytes_per_sequence():
    """Ragged workload: the byte count is the sum of each sequence's own
    closed form (quantized prefix plus its residual window)."""
    w = WORKLOADS[5]
    lens = context_lengths(w).numpy()
    assert lens.min() >= 65536 and lens.max() <= 131072
    ref = sum(_closed_form_decode_bytes("kivi", w.bits, w.group, w.residual, 1, w.n_kv_heads, w.n_q_heads,
                                        w.head_dim, int(n), 2) for n in lens)
    assert bench.decode_bytes(w, lens) == ref
    mean_n = float(np.mean(lens))
    assert abs(ref / len(lens) / (w.n_kv_heads * mean_n) - 160) < 1.0  # about 160 B per token per KV head


def test_per_token_append_bytes_closed_form():
    """Bulk append of n tokens into an empty FP8 cache: bf16 K and V read,
    codes and scales written."""
    w = WORKLOADS[2]
    lens0 = np.zeros(w.batch, dtype=np.int64)
    t = w.context
    ref = w.batch * w.n_kv_heads * t * (2 * w.head_dim * 2 + 2 * (w.head_dim + 4))
    assert bench.append_bytes(w, lens0, t) == ref
