"""GPU test of kvq_append_decode_noalloc, the fused decode step that keeps
its split-K partial states in the library's fixed device workspace instead
of a caller's: through the C ABI it must leave the same cache, seq_lens and
skipped flags and write the same output, bit for bit, as kvq_append_decode
on a twin cache (same kernel, same split plan), and that output must agree
with the oracle within the attention tolerance. Two calls in a row per
format, the second on a smaller input, so that the second finds the first
call's contents in the shared array."""
import sys

import numpy as np
import pytest
import torch

import quantized_kv_cache_06_amd as kvq
import kvq_testlib as T
from kvq_workloads import WORKLOADS, context_lengths, kv_tokens, queries
from oracle import kvq_oracle as O

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _filled(w, cap, seed_stream=0):
    lens = context_lengths(w) if w.ragged else torch.full((w.batch,), w.context, dtype=torch.int32)
    k, v = kv_tokens(w, int(lens.max()), stream=seed_stream, device="cuda")
    caches = []
    for _ in range(2):
        c = T.GpuCache(T.config(w, cap))
        c.append(k, v, lens if w.ragged else None)
        caches.append(c)
    seqs = []
    kf, vf = T.as_f32(k), T.as_f32(v)
    for b in range(w.batch):
        n = int(lens[b])
        seqs.append([T.oracle_sequence(w, [kf[b, h, :n]], [vf[b, h, :n]]) for h in range(w.n_kv_heads)])
    return caches, seqs, lens


CASES = {
    "kivi": (WORKLOADS[5].scaled(batch=3, n_kv_heads=2, n_q_heads=16, context=1500, context_min=700, layers=1),
             WORKLOADS[5].scaled(batch=2, n_kv_heads=1, n_q_heads=8, context=500, context_min=300, layers=1)),
    "fp8": (WORKLOADS[2].scaled(batch=4, n_kv_heads=2, n_q_heads=8, context=1000, context_min=1000),
            WORKLOADS[2].scaled(batch=2, n_kv_heads=2, n_q_heads=4, context=333, context_min=333)),
}


@pytest.mark.parametrize("fmt", sorted(CASES))
def test_noalloc_step_equals_fused_step(fmt):
    for i, w in enumerate(CASES[fmt]):
        cap = w.context + 8
        _log(f"[noalloc {fmt} call {i}: B={w.batch} Hkv={w.n_kv_heads} Hq={w.n_q_heads} n<={w.context}]")
        (ca, cb), seqs, lens = _filled(w, cap, seed_stream=i)
        k1, v1 = kv_tokens(w, 1, stream=7 + i, device="cuda")
        q = queries(w, step=3 + i, device="cuda")
        sm = float(O.default_sm_scale(w.head_dim))
        out_a = torch.full((w.batch, w.n_q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        out_b = torch.full_like(out_a, float("nan"))
        sk_a = torch.full((w.batch,), 7, dtype=torch.int32, device="cuda")
        sk_b = torch.full_like(sk_a, 7)
        kvq.kvq_append_decode(ca.cfg, ca.buf, ca.seq_lens, k1.contiguous(), v1.contiguous(), q, sm, out_a, ca.ws,
                              skipped=sk_a)
        kvq.kvq_append_decode_noalloc(cb.cfg, cb.buf, cb.seq_lens, k1.contiguous(), v1.contiguous(), q, sm, out_b,
                                      skipped=sk_b)
        torch.cuda.synchronize()
        assert torch.equal(ca.seq_lens, cb.seq_lens)
        assert torch.equal(cb.seq_lens.cpu(), lens + 1)
        assert torch.equal(sk_a, sk_b) and int(sk_b.sum()) == 0
        assert torch.equal(ca.buf, cb.buf), "cache bytes differ"
        a, b = out_a.cpu().numpy(), out_b.cpu().numpy()
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
        k1f, v1f, qf = T.as_f32(k1), T.as_f32(v1), T.as_f32(q)
        for bi in range(w.batch):
            for h in range(w.n_kv_heads):
                seqs[bi][h].append(k1f[bi, h], v1f[bi, h])
            ref = O.decode_attention(seqs[bi], qf[bi], sm)
            ma, rel = T.attention_errors(b[bi], ref)
            assert ma <= T.MAX_ABS_TOL and rel <= T.REL_L2_TOL, f"b={bi}: {ma:.3g} {rel:.3g}"
        _log("  bit-identical to kvq_append_decode, within tolerance of the oracle")


def test_noalloc_step_refuses_plans_beyond_the_fixed_workspace():
    """An explicit split length whose partial states exceed the fixed array
    is refused (KVQ_ERR_WORKSPACE) and launches nothing."""
    w = WORKLOADS[2].scaled(batch=16, n_kv_heads=8, n_q_heads=64, context=64, context_min=64)
    cache = T.GpuCache(T.config(w, 8192))
    k1, v1 = kv_tokens(w, 1, device="cuda")
    q = queries(w, device="cuda")
    out = torch.zeros((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    before = cache.buf.clone()
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_append_decode_noalloc(cache.cfg, cache.buf, cache.seq_lens, k1.contiguous(), v1.contiguous(), q,
                                      0.088, out, split_tokens=64)
    assert e.value.status == kvq.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(cache.buf, before) and int(cache.seq_lens.sum()) == 0
