"""GPU parity of the decode's split plan at its edges: batches above 64
sequences (lengths beyond the first 64 are read from memory rather than from
the one-round-trip preload), KIVI's splits of decreasing size handed out
through the work-item counter (with sequences of every kind: empty,
residual-only, a group just flushed, long), the per-token formats' static
plan, explicit split lengths, one fused step, and the workspace counters
back at zero after every call."""
import numpy as np
import pytest
import torch

import quantized_kv_cache_06_amd as kvq
import kvq_testlib as T
from kvq_workloads import WORKLOADS, kv_tokens, queries
from oracle import kvq_oracle as O

pytestmark = pytest.mark.gpu

B = 70
# lengths: empty, a single token, residual-only, exactly one group past the
# window, then a seeded spread up to 3000 tokens
_rng = np.random.default_rng(1234)
LENS = np.concatenate([[0, 1, 15, 16 + 32, 3000], _rng.integers(0, 3001, B - 5)]).astype(np.int32)

CASES = {
    # KIVI INT4, G 32, R 16, d 64: with 70 pairs the plan has 16 splits per
    # pair (10 large, 2 medium, 4 small) on MI355X
    "kivi": WORKLOADS[1].scaled(batch=B, n_kv_heads=1, n_q_heads=4, context=3000, context_min=0),
    # FP8 per token, d 128, bf16 inputs: equal static splits
    "fp8": WORKLOADS[2].scaled(batch=B, n_kv_heads=1, n_q_heads=4, context=3000, context_min=0),
}


def _counters_zero(cache):
    n = cache.cfg.batch * (cache.cfg.n_kv_heads + 1) + 1
    return torch.count_nonzero(cache.ws[:4 * n].view(torch.int32)).item() == 0


@pytest.mark.parametrize("fmt", sorted(CASES))
def test_large_batch_plans_match_oracle(fmt):
    w = CASES[fmt]
    print(f"[large batch {fmt}: B {B}]", flush=True)
    cache = T.GpuCache(T.config(w, 4096))
    k, v = kv_tokens(w, 3000, device="cuda")
    lens = torch.from_numpy(LENS)
    cache.append(k, v, lens)
    torch.cuda.synchronize()
    assert np.array_equal(cache.seq_lens.cpu().numpy(), LENS)
    kf, vf = T.as_f32(k), T.as_f32(v)
    seqs = [[T.oracle_sequence(w, [kf[b, 0, :LENS[b]]], [vf[b, 0, :LENS[b]]])] for b in range(B)]
    contents = T.CacheContents(cache)
    for b in range(0, B, 7):
        T.assert_cache_matches(contents, b, 0, seqs[b][0], w)
    q = queries(w, device="cuda")
    qf = T.as_f32(q)
    sm = O.default_sm_scale(w.head_dim)
    for st in (0, 256, 1024):
        out = cache.decode(q, sm, st).cpu().numpy()
        for b in range(B):
            ref = O.decode_attention(seqs[b], qf[b], sm)
            ma, rel = T.attention_errors(out[b], ref)
            assert ma <= T.MAX_ABS_TOL and rel <= T.REL_L2_TOL, f"split {st} b={b} n={LENS[b]}: {ma:.3g} {rel:.3g}"
        assert _counters_zero(cache) or st != 0
    assert _counters_zero(cache)
    # two fused steps
    for step in range(2):
        k1, v1 = kv_tokens(w, 1, stream=5 + step, device="cuda")
        out = torch.empty((B, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
        kvq.kvq_append_decode(cache.cfg, cache.buf, cache.seq_lens, k1.contiguous(), v1.contiguous(),
                              q.contiguous(), float(sm), out, cache.ws)
        out = out.cpu().numpy()
        k1f, v1f = T.as_f32(k1), T.as_f32(v1)
        for b in range(B):
            seqs[b][0].append(k1f[b, 0], v1f[b, 0])
            ref = O.decode_attention(seqs[b], qf[b], sm)
            ma, rel = T.attention_errors(out[b], ref)
            assert ma <= T.MAX_ABS_TOL and rel <= T.REL_L2_TOL, f"fused {step} b={b}: {ma:.3g} {rel:.3g}"
        assert np.array_equal(cache.seq_lens.cpu().numpy(), LENS + step + 1)
        assert _counters_zero(cache)
