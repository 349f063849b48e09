"""GPU parity of the unquantized bf16 cache (KVQ_FMT_BF16, the 16-bit
baseline) against the CPU oracle: stored bf16 patterns bit-exact (bf16
inputs unchanged, fp32 inputs rounded to nearest even), attention within
the tolerance of the quantized formats, through bulk appends, single-token
appends and the fused decode step."""
import sys

import numpy as np
import pytest
import torch

import quantized_kv_cache_06_amd as kvq
import kvq_testlib as T
from kvq_workloads import WORKLOADS, kv_tokens, queries
from oracle import kvq_oracle as O
from test_gpu_parity import _check_decode, _oracle_all

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bf16(w, **kw):
    return w.scaled(fmt="bf16", bits=16, group=0, residual=0, **kw)


CASES = {
    "w2-bf16": _bf16(WORKLOADS[2], batch=3, n_kv_heads=2, n_q_heads=8, context=1000, context_min=1000),
    "w3-f32-d64": _bf16(WORKLOADS[3], batch=2, n_kv_heads=2, n_q_heads=16, head_dim=64, dtype="f32", context=777,
                        context_min=777),
    "w5-ragged": _bf16(WORKLOADS[5], batch=3, n_kv_heads=2, n_q_heads=16, context=1500, context_min=700, layers=1),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_bf16_cache_append_decode_stream_and_fused(name):
    w = CASES[name]
    _log(f"[bf16 cache {name}: d={w.head_dim} {w.dtype} B={w.batch} Hkv={w.n_kv_heads} Hq={w.n_q_heads} "
         f"n<={w.context}]")
    steps = 40
    cache = T.GpuCache(T.config(w, w.context + 2 * steps + 8))
    k, v = kv_tokens(w, w.context, device="cuda")
    from kvq_workloads import context_lengths
    lens = context_lengths(w) if w.ragged else torch.full((w.batch,), w.context, dtype=torch.int32)
    cache.append(k, v, lens if w.ragged else None)
    torch.cuda.synchronize()
    seqs = _oracle_all(w, k, v, lens)
    contents = T.CacheContents(cache)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            T.assert_cache_matches(contents, b, h, seqs[b][h], w)
    q = queries(w, device="cuda")
    sm = O.default_sm_scale(w.head_dim)
    for st in (0, 64, 512):
        _check_decode(w, cache, seqs, q, sm, st, f"split{st}")
    # single-token appends, then fused steps
    kk, vv = kv_tokens(w, 2 * steps, stream=1, device="cuda")
    kf, vf = T.as_f32(kk), T.as_f32(vv)
    for s in range(steps):
        cache.append(kk[:, :, s:s + 1], vv[:, :, s:s + 1])
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            seqs[b][h].append(kf[b, h, :steps], vf[b, h, :steps])
    for s in range(steps, 2 * steps):
        qs = queries(w, step=s, device="cuda")
        out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
        kvq.kvq_append_decode(cache.cfg, cache.buf, cache.seq_lens, kk[:, :, s:s + 1].contiguous(),
                              vv[:, :, s:s + 1].contiguous(), qs, float(sm), out, cache.ws)
        out = out.cpu().numpy()
        qf = T.as_f32(qs)
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                seqs[b][h].append(kf[b, h, s:s + 1], vf[b, h, s:s + 1])
            ref = O.decode_attention(seqs[b], qf[b], sm)
            ma, rel = T.attention_errors(out[b], ref)
            assert ma <= T.MAX_ABS_TOL and rel <= T.REL_L2_TOL, f"fused step {s} b={b}: {ma:.3g} {rel:.3g}"
    torch.cuda.synchronize()
    contents = T.CacheContents(cache)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            T.assert_cache_matches(contents, b, h, seqs[b][h], w)
    _log(f"  {steps} appends + {steps} fused steps: bit-exact cache, attention in tolerance")


def test_bf16_cache_rounds_fp32_ties_to_even():
    """fp32 inputs whose low 16 bits are exactly half an ulp of bf16 (and one
    unit either side): the stored patterns equal the oracle's rounding."""
    w = _bf16(WORKLOADS[3], batch=1, n_kv_heads=1, n_q_heads=2, head_dim=64, dtype="f32", context=96,
              context_min=96)
    _log("[bf16 cache: fp32 rounding ties]")
    rng = np.random.default_rng(11)
    upper = rng.integers(0x3C00, 0x4400, (96, 64)).astype(np.uint32) | (rng.integers(0, 2, (96, 64)) << 15).astype(
        np.uint32)
    low = rng.choice(np.array([0x7FFF, 0x8000, 0x8001, 0x0000, 0xFFFF], dtype=np.uint32), (96, 64))
    x = ((upper << 16) | low).view(np.float32)
    k = torch.from_numpy(x.copy()).reshape(1, 1, 96, 64).cuda()
    v = torch.from_numpy((-x).copy()).reshape(1, 1, 96, 64).cuda()
    cache = T.GpuCache(T.config(w, 96))
    cache.append(k, v)
    torch.cuda.synchronize()
    ref = T.oracle_sequence(w, [x], [-x])
    T.assert_cache_matches(T.CacheContents(cache), 0, 0, ref, w)
