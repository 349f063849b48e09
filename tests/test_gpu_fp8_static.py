"""GPU parity of FP8 with the static per-tensor scale 1.0 (KVQ_FMT_FP8_STATIC)
against the CPU oracle: E4M3 codes bit-exact (values beyond +-448 saturate),
no scale arrays, attention within tolerance, through bulk appends and the
fused decode step."""
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


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "f32")])
def test_fp8_static_append_decode_and_fused(d, dtype):
    w = WORKLOADS[2].scaled(fmt="fp8s", batch=2, n_kv_heads=2, n_q_heads=8, head_dim=d, dtype=dtype, context=500,
                            context_min=500)
    print(f"[fp8 static scale d={d} {dtype}]", flush=True)
    cache = T.GpuCache(T.config(w, w.context + 40))
    k, v = kv_tokens(w, w.context, device="cuda")
    # a few tokens far beyond the E4M3 range: they saturate to +-448
    k[:, :, 7] *= 100.0
    v[:, :, 300] *= 300.0
    lens = torch.full((w.batch,), w.context, dtype=torch.int32)
    cache.append(k, v)
    torch.cuda.synchronize()
    seqs = _oracle_all(w, k, v, lens)
    contents = T.CacheContents(cache)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            T.assert_cache_matches(contents, b, h, seqs[b][h], w)
    assert np.any(np.abs(T.as_f32(k)) > 448)
    q = queries(w, device="cuda") * 0.05   # keep the saturated keys from dominating every head
    sm = O.default_sm_scale(w.head_dim)
    for st in (0, 64):
        _check_decode(w, cache, seqs, q, sm, st, f"split{st}")
    kk, vv = kv_tokens(w, 20, stream=1, device="cuda")
    kf, vf = T.as_f32(kk), T.as_f32(vv)
    for s in range(20):
        qs = queries(w, step=s + 1, device="cuda")
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
