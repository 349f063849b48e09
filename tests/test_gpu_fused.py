"""GPU parity of the fused decode step (kvq_append_decode: append one token
per sequence, then attend, in one launch) against the CPU oracle, which
appends the same token and then attends. The cache (codes, scales,
zero-points, residual rows) and seq_lens must be bit-exact, the attention
within the same tolerance as the plain decode; the cache buffer must also
equal, byte for byte, what the two separate calls leave."""
import sys

import numpy as np
import pytest
import torch

import quantized_kv_cache_06_amd as kvq
import kvq_testlib as T
from kvq_workloads import WORKLOADS, kv_tokens, queries
from oracle import kvq_oracle as O
from test_gpu_parity import SMALL, _lens, _oracle_all

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _fused(cache, k1, v1, q, sm, skipped=None):
    out = torch.empty((cache.cfg.batch, cache.cfg.n_q_heads, cache.cfg.head_dim), dtype=torch.float32,
                      device=cache.buf.device)
    kvq.kvq_append_decode(cache.cfg, cache.buf, cache.seq_lens, k1.contiguous(), v1.contiguous(), q.contiguous(),
                          float(sm), out, cache.ws, split_tokens=cache.split_tokens, skipped=skipped)
    return out


def _counters_zero(cache):
    # [B][Hkv] arrival counters, [B] per-sequence counters, the work-item counter
    n = cache.cfg.batch * (cache.cfg.n_kv_heads + 1) + 1
    return torch.count_nonzero(cache.ws[:4 * n].view(torch.int32)).item() == 0


# The five small workloads, plus KIVI with no residual window (every 32nd
# new token completes a group by itself) and a d = 64 fp32 INT8 case.
CASES = dict(SMALL)
CASES[6] = WORKLOADS[1].scaled(residual=0, context=200, context_min=200)
CASES[7] = WORKLOADS[3].scaled(batch=2, n_kv_heads=3, n_q_heads=6, head_dim=64, dtype="f32", context=300,
                               context_min=300)


@pytest.mark.parametrize("idx", sorted(CASES))
def test_fused_steps_match_oracle(idx):
    w = CASES[idx]
    steps = 70 if w.fmt == "kivi" else 40
    _log(f"[fused steps, case {idx}: {w.name} {w.fmt} bits={w.bits} G={w.group} R={w.residual} d={w.head_dim} "
         f"{w.dtype} B={w.batch} Hkv={w.n_kv_heads} Hq={w.n_q_heads} n<={w.context}, {steps} steps]")
    cache = T.GpuCache(T.config(w, w.context + steps + 8))
    k, v = kv_tokens(w, w.context, device="cuda")
    lens = _lens(w)
    cache.append(k, v, lens if w.ragged else None)
    torch.cuda.synchronize()
    seqs = _oracle_all(w, k, v, lens)
    kk, vv = kv_tokens(w, steps, stream=3, device="cuda")
    kf, vf = T.as_f32(kk), T.as_f32(vv)
    sm = O.default_sm_scale(w.head_dim)
    worst = (0.0, 0.0)
    for s in range(steps):
        q = queries(w, step=s + 1, device="cuda")
        out = _fused(cache, kk[:, :, s:s + 1], vv[:, :, s:s + 1], q, sm).cpu().numpy()
        qf = T.as_f32(q)
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                seqs[b][h].append(kf[b, h, s:s + 1], vf[b, h, s:s + 1])
            ref = O.decode_attention(seqs[b], qf[b], sm)
            ma, rel = T.attention_errors(out[b], ref)
            worst = (max(worst[0], ma), max(worst[1], rel))
            assert ma <= T.MAX_ABS_TOL and rel <= T.REL_L2_TOL, f"step {s} b={b}: max-abs {ma:.3g} rel-L2 {rel:.3g}"
    torch.cuda.synchronize()
    assert _counters_zero(cache)
    contents = T.CacheContents(cache)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            T.assert_cache_matches(contents, b, h, seqs[b][h], w)
    _log(f"  cache bit-exact after {steps} fused steps; attention worst max-abs {worst[0]:.3g} "
         f"rel-L2 {worst[1]:.3g}")


@pytest.mark.parametrize("idx", [1, 2, 5, 6])
def test_fused_step_equals_append_then_decode(idx):
    """The same steps through the two separate calls and through the fused
    call leave byte-identical cache buffers and seq_lens."""
    w = CASES[idx]
    steps = 66
    _log(f"[fused vs two calls, case {idx}]")
    two = T.GpuCache(T.config(w, w.context + steps + 8))
    one = T.GpuCache(T.config(w, w.context + steps + 8))
    k, v = kv_tokens(w, w.context, device="cuda")
    lens = _lens(w)
    for c in (two, one):
        c.append(k, v, lens if w.ragged else None)
    kk, vv = kv_tokens(w, steps, stream=4, device="cuda")
    sm = O.default_sm_scale(w.head_dim)
    worst = 0.0
    for s in range(steps):
        q = queries(w, step=s + 1, device="cuda")
        two.append(kk[:, :, s:s + 1], vv[:, :, s:s + 1])
        o2 = two.decode(q, sm)
        o1 = _fused(one, kk[:, :, s:s + 1], vv[:, :, s:s + 1], q, sm)
        worst = max(worst, float((o1 - o2).abs().max()))
    torch.cuda.synchronize()
    assert torch.equal(two.seq_lens, one.seq_lens)
    assert torch.equal(two.buf, one.buf), "cache buffers differ"
    assert worst <= 2 * T.MAX_ABS_TOL
    _log(f"  byte-identical caches; outputs differ by at most {worst:.3g}")


EDGE_FORMATS = {
    "kivi": lambda: SMALL[5],
    "fp8": lambda: SMALL[2],
    "int8": lambda: SMALL[3],
    "kivi16": lambda: SMALL[4].scaled(fmt="kivi16"),
    "int4": lambda: SMALL[3].scaled(fmt="int4", bits=4, group=32, residual=0),
    "int4h": lambda: SMALL[2].scaled(fmt="int4h", bits=4, group=128, residual=0),
    "fp8s": lambda: SMALL[2].scaled(fmt="fp8s"),
    "bf16": lambda: SMALL[2].scaled(fmt="bf16", bits=16, group=0, residual=0),
}


@pytest.mark.parametrize("fmt", sorted(EDGE_FORMATS))
def test_fused_capacity_and_empty_sequences(fmt):
    """Ragged lengths 0, 1, cap - 1 and cap: the first three take the token
    (an empty sequence then attends to the new token alone), the full one is
    left unchanged and attended as it is."""
    base = EDGE_FORMATS[fmt]()
    cap = 300
    w = base.scaled(batch=4, context=cap, context_min=cap)
    _log(f"[fused capacity edges, {fmt}]")
    cache = T.GpuCache(T.config(w, cap))
    k, v = kv_tokens(w, cap, device="cuda")
    lens = torch.tensor([0, 1, cap - 1, cap], dtype=torch.int32)
    cache.append(k, v, lens)
    seqs = _oracle_all(w, k, v, lens)
    sm = O.default_sm_scale(w.head_dim)
    kk, vv = kv_tokens(w, 2, stream=5, device="cuda")
    kf, vf = T.as_f32(kk), T.as_f32(vv)
    skipped = torch.full((w.batch,), 7, dtype=torch.int32, device="cuda")
    for s in range(2):
        q = queries(w, step=s + 1, device="cuda")
        out = _fused(cache, kk[:, :, s:s + 1], vv[:, :, s:s + 1], q, sm, skipped).cpu().numpy()
        # the full sequence (and, after the first step, the one at cap - 1) takes no token
        assert skipped.cpu().tolist() == ([0, 0, 0, 1] if s == 0 else [0, 0, 1, 1])
        qf = T.as_f32(q)
        for b in range(w.batch):
            if seqs[b][0].n < cap:
                for h in range(w.n_kv_heads):
                    seqs[b][h].append(kf[b, h, s:s + 1], vf[b, h, s:s + 1])
            ref = O.decode_attention(seqs[b], qf[b], sm)
            ma, rel = T.attention_errors(out[b], ref)
            assert ma <= T.MAX_ABS_TOL and rel <= T.REL_L2_TOL, f"step {s} b={b}: {ma:.3g} {rel:.3g}"
    torch.cuda.synchronize()
    assert cache.seq_lens.cpu().tolist() == [2, 3, cap, cap]
    assert _counters_zero(cache)
    contents = T.CacheContents(cache)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            T.assert_cache_matches(contents, b, h, seqs[b][h], w)


def test_fused_steps_in_a_graph_replay():
    """Fused steps captured once in a HIP graph and replayed: seq_lens
    advances on the device every replay; results match eager fused calls."""
    w = SMALL[5]
    _log("[fused steps in a graph]")
    steps = 3
    caches = [T.GpuCache(T.config(w, w.context + 16)) for _ in range(2)]
    k, v = kv_tokens(w, w.context, device="cuda")
    lens = _lens(w)
    for c in caches:
        c.append(k, v, lens)
    kk, vv = kv_tokens(w, 1, stream=6, device="cuda")
    k1, v1 = kk.contiguous(), vv.contiguous()
    q = queries(w, step=1, device="cuda").contiguous()
    sm = O.default_sm_scale(w.head_dim)
    out_g = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            kvq.kvq_append_decode(caches[0].cfg, caches[0].buf, caches[0].seq_lens, k1, v1, q, float(sm), out_g,
                                  caches[0].ws)
    torch.cuda.synchronize()
    # capture does not run the kernel: the cache is untouched
    assert torch.equal(caches[0].seq_lens, caches[1].seq_lens)
    for s in range(steps):
        g.replay()
        torch.cuda.synchronize()
        out_e = _fused(caches[1], k1, v1, q, sm)
        torch.cuda.synchronize()
        assert torch.equal(caches[0].seq_lens, caches[1].seq_lens), f"replay {s}"
        assert torch.equal(caches[0].buf, caches[1].buf), f"replay {s}"
        assert float((out_g - out_e).abs().max()) <= 1e-6, f"replay {s}"
    assert caches[0].seq_lens.cpu().tolist() == (lens + steps).tolist()


@pytest.mark.parametrize("split", [64, 512])
@pytest.mark.parametrize("idx", [2, 5, 6])
def test_fused_steps_with_explicit_split_lengths(idx, split):
    """The fused step with a caller-chosen split length (more, shorter splits;
    some sequences then hold fewer splits than the grid has): attention
    in tolerance, cache bit-exact, counters back to zero."""
    w = CASES[idx]
    steps = 35
    _log(f"[fused steps, case {idx}, split {split}]")
    cache = T.GpuCache(T.config(w, w.context + steps + 8), split_tokens=split)
    k, v = kv_tokens(w, w.context, device="cuda")
    lens = _lens(w)
    cache.append(k, v, lens if w.ragged else None)
    seqs = _oracle_all(w, k, v, lens)
    kk, vv = kv_tokens(w, steps, stream=7, device="cuda")
    kf, vf = T.as_f32(kk), T.as_f32(vv)
    sm = O.default_sm_scale(w.head_dim)
    for s in range(steps):
        q = queries(w, step=s + 1, device="cuda")
        out = _fused(cache, kk[:, :, s:s + 1], vv[:, :, s:s + 1], q, sm).cpu().numpy()
        qf = T.as_f32(q)
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                seqs[b][h].append(kf[b, h, s:s + 1], vf[b, h, s:s + 1])
            ref = O.decode_attention(seqs[b], qf[b], sm)
            ma, rel = T.attention_errors(out[b], ref)
            assert ma <= T.MAX_ABS_TOL and rel <= T.REL_L2_TOL, f"step {s} b={b}: {ma:.3g} {rel:.3g}"
    torch.cuda.synchronize()
    assert _counters_zero(cache)
    contents = T.CacheContents(cache)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            T.assert_cache_matches(contents, b, h, seqs[b][h], w)
