"""Benchmark of the quantized KV cache hot path on one MI355X.

A step is one decode iteration over every cache copy ("layer"): append one
new K/V token per sequence (quantize, or residual write + group flush) and
run decode attention over the whole cache, as one fused launch per layer
(kvq_append_decode; --unfused times the two separate calls instead). Workload 2 (FP8 E4M3 per-token,
batch 16, 8 KV heads, 32 query heads, head_dim 128, 4096 tokens) is the
default; its 139 MB cache fits in the 256 MB Infinity Cache, so the step
rotates over enough independent copies to touch >= 2 GB. Workload 5 runs its
80 layers instead. Inputs are seeded synthetic data already resident in HBM.

Prints one JSON line: value = algorithmic bytes of the timed steps (cache
bytes read by decode + q + out, plus append input and cache writes) per
second of the timed region; "roofline" covers the decode-attention call
(one launch of the split-K kernel, whose last split per (sequence, KV head)
merges the partials) timed with HIP events on its stream;
"cpu_baseline" times the CPU oracle on a bounded sample of the same work;
"stream_read_ceiling" is the read rate of a plain streaming kernel on the
same device, measured first, for context.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", type=int, default=2, help="workload index 1..5")
    p.add_argument("--split", type=int, default=0, help="longest decode split in tokens (0 = library choice)")
    p.add_argument("--min-bytes", type=float, default=2.0e9, help="bytes the rotated copies must span")
    p.add_argument("--layers", type=int, default=0, help="override the number of cache copies")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--decode-rounds", type=int, default=20, help="passes over all copies in the decode-only timing")
    p.add_argument("--cache-format", choices=("native", "bf16", "int4", "int4h", "fp8s", "kivi16"), default="native",
                   help="bf16: the same workload shapes and inputs with the unquantized 16-bit cache "
                        "(the baseline the quantized formats save bytes against); int4: with the "
                        "group-wise symmetric INT4 cache (--group channels per scale); int4h: the same "
                        "with Walsh-Hadamard rotated Keys; kivi16: a KIVI workload with fp16 scales and "
                        "zero-points; fp8s: FP8 with "
                        "the static per-tensor scale 1.0")
    p.add_argument("--group", type=int, default=32, help="channels per scale of --cache-format int4")
    p.add_argument("--unfused", action="store_true",
                   help="time the step as kvq_quantize_append + kvq_decode_attention (two calls per layer)")
    p.add_argument("--stream-ref", type=float, default=0.0,
                   help="instead of the hot path: time torch's copy and sum over this many GiB (the "
                        "attainable streaming bandwidth, and the plain copy used to scale HBM counters)")
    return p.parse_args()


def bytes_per_token_head(w):
    """Algorithmic bytes of one quantized token for one KV head (K + V)."""
    d = w.head_dim
    if w.fmt == "bf16":
        return 2 * d * 2
    if w.fmt in ("int4", "int4h"):
        return 2 * d // 2 + 2 * 4 * (d // w.group)
    if w.fmt == "fp8s":
        return 2 * d
    if w.fmt in ("fp8", "int8"):
        return 2 * d + 2 * 4
    codes = 2 * d * w.bits // 8
    mb = 2 if w.fmt == "kivi16" else 4    # bytes per scale or zero-point
    key_meta = 2 * mb * d / w.group       # per-channel scale + zero, amortized over G tokens
    val_meta = 2 * mb * (d // w.group)    # per-token scale + zero per channel group
    return codes + key_meta + val_meta


def resid_bytes_per_token_head(w):
    return 2 * w.head_dim * (2 if w.dtype == "bf16" else 4)


def is_kivi(w):
    return w.fmt in ("kivi", "kivi16")


def nq_of(w, n):
    if not is_kivi(w):
        return n
    return w.group * (max(n - w.residual, 0) // w.group)


def decode_bytes(w, lens):
    """Cache bytes read for sequences of the given lengths, plus q and out."""
    total = 0.0
    for n in lens:
        nq = nq_of(w, int(n))
        total += w.n_kv_heads * (nq * bytes_per_token_head(w) + (int(n) - nq) * resid_bytes_per_token_head(w))
    elem = 2 if w.dtype == "bf16" else 4
    total += len(lens) * w.n_q_heads * w.head_dim * (elem + 4)
    return total


def append_bytes(w, lens_before, t):
    """Input read + cache bytes written when t tokens are appended to
    sequences of the given lengths (KIVI: ring writes and group flushes)."""
    elem = 2 if w.dtype == "bf16" else 4
    d = w.head_dim
    total = 0.0
    for n in lens_before:
        n = int(n)
        per_head = 2 * t * d * elem                       # read new K and V
        if not is_kivi(w):
            per_head += t * bytes_per_token_head(w)       # codes + scales written
        else:
            q0, q1 = nq_of(w, n), nq_of(w, n + t)
            flushed = q1 - q0
            from_ring = max(0, min(n, q1) - q0)
            per_head += from_ring * 2 * d * elem          # old residual tokens read back
            per_head += flushed * bytes_per_token_head(w)  # codes + metadata written
            per_head += (n + t - max(n, q1)) * 2 * d * elem  # tokens left in the ring
        total += w.n_kv_heads * per_head
    return total


def workload_key(w):
    """File-name key of a workload's profile summaries under profiles/."""
    fmt = w.fmt if w.fmt != "kivi" else f"kivi{w.bits}_g{w.group}_r{w.residual}"
    ctx = w.context if not w.ragged else f"{w.context_min}-{w.context}"
    return f"{fmt}_b{w.batch}_hkv{w.n_kv_heads}_hq{w.n_q_heads}_d{w.head_dim}_n{ctx}"


DECODE_SOURCES = ("quantized_kv_cache_06_amd/csrc/kvq_decode.hip", "quantized_kv_cache_06_amd/csrc/kvq_device.h",
                  "quantized_kv_cache_06_amd/csrc/kvq_quant.h",
                  "quantized_kv_cache_06_amd/csrc/kvq_internal.h", "include/kvq.h")


def profiled_traffic(w):
    """HBM bytes per decode launch from the committed rocprofv3 counter
    summary of this workload (FETCH_SIZE and WRITE_SIZE per dispatch, scaled
    by what they read for a plain 1 GiB copy), or None when there is none or
    the decode kernel's sources have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"decode_split_{workload_key(w)}.hbm_counters.md")
    if not os.path.exists(path):
        return None, None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith('{"kernel": '):
                r = json.loads(line)
                if r["kernel"] == "decode_split":  # the plain decode call (not the fused step)
                    rec = r
    if rec is None:
        return None, None
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, name), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["kernel_source_sha256"]:
        return None, os.path.relpath(path, ROOT) + " (stale: kernel sources changed)"
    return float(rec["traffic_bytes_per_launch"]), os.path.relpath(path, ROOT)


def cpu_baseline(w, k_host, v_host, q_host, lens, seconds):
    """Time the CPU oracle (as it is) on whole sequences of copy 0: append
    every token, then decode, until about `seconds` of work is done."""
    from threadpoolctl import threadpool_limits

    from oracle import kvq_oracle as O
    sm = O.default_sm_scale(w.head_dim)
    done_bytes, done_seqs, t_used = 0.0, 0, 0.0
    with threadpool_limits(limits=1):
        for b in range(w.batch):
            n = int(lens[b])
            t0 = time.perf_counter()
            seqs = []
            for h in range(w.n_kv_heads):
                s = O.SequenceCache(w.fmt, w.head_dim, w.bits, w.group, w.residual)
                s.append(k_host[b, h, :n], v_host[b, h, :n])
                seqs.append(s)
            O.decode_attention(seqs, q_host[b], sm)
            t_used += time.perf_counter() - t0
            done_bytes += append_bytes(w, [0], n) + decode_bytes(w, [n])
            done_seqs += 1
            if t_used >= seconds:
                break
    return {"value": done_bytes / t_used / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done_seqs} of {w.batch} sequences of copy 0 (bulk append of n tokens + one decode, "
                      f"all {w.n_kv_heads} KV heads), numpy with one BLAS thread, {t_used:.1f} s"}


def stream_reference(torch, gib):
    """Plain streaming kernels of known size: a device-to-device copy (reads
    and writes n bytes) and a sum (reads n bytes), each timed with events over
    10 runs. Prints one JSON line."""
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    res = {}
    for name, fn, nbytes in (("copy", lambda: dst.copy_(src), 8 * n), ("sum", lambda: src.sum(), 4 * n)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        res[name] = {"bytes": nbytes, "us": round(ms * 1e3, 2), "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    print(json.dumps({"stream_reference": res, "gib": gib}), flush=True)


def stream_ceiling(torch, gib=2.0):
    """Read rate of a plain streaming kernel over gib GiB of fp32 in HBM
    (more than the Infinity Cache holds), timed with events over 10 runs, as
    the attainable read rate the decode kernel is set against. The kernel is
    torch's row sum over rows of 4096 floats: one block per row streams the
    buffer once; a full sum to one scalar streams markedly slower on this
    device. Taken before the caches are allocated; the buffer is freed again."""
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    rows = src.view(-1, 4096)
    rows.sum(1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        rows.sum(1)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    del src, rows
    torch.cuda.empty_cache()
    return {"kernel": f"torch row sum over {gib:g} GiB fp32, rows of 4096 (plain streaming read)", "bytes": 4 * n,
            "us": round(ms * 1e3, 2), "gbps": round(4 * n / (ms * 1e-3) / 1e9, 1)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the quantized KV cache path here is single-GPU "
              "(sequence/head sharding across GPUs is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    # 80 layers of long-context cache fill most of HBM: let the caching
    # allocator grow segments instead of fragmenting on the large temporaries
    os.environ.setdefault("PYTORCH_ALLOC_CONF", "expandable_segments:True")
    import torch

    import quantized_kv_cache_06_amd as kvq
    from kvq_workloads import WORKLOADS, context_lengths, kv_tokens, queries
    if not os.path.exists(kvq.LIB_PATH):
        from quantized_kv_cache_06_amd import build as _b
        _b.build()

    if args.stream_ref > 0:
        stream_reference(torch, args.stream_ref)
        return
    ceiling = stream_ceiling(torch)

    w = WORKLOADS[args.config]
    if args.cache_format == "bf16":
        w = w.scaled(fmt="bf16", bits=16, group=0, residual=0)
    elif args.cache_format == "int4":
        w = w.scaled(fmt="int4", bits=4, group=args.group, residual=0)
    elif args.cache_format == "int4h":
        w = w.scaled(fmt="int4h", bits=4, group=args.group, residual=0)
    elif args.cache_format == "kivi16":
        if w.fmt != "kivi":
            sys.exit("--cache-format kivi16 needs a KIVI workload (4 or 5)")
        w = w.scaled(fmt="kivi16")
    elif args.cache_format == "fp8s":
        w = w.scaled(fmt="fp8s", bits=8, group=0, residual=0)
    dev = torch.device("cuda:0")
    lens0 = context_lengths(w)
    n_max = int(lens0.max())
    grow = args.warmup + 2 * args.steps + 1  # warm-up steps, an untimed and a timed replay of the steps
    fmt = {"fp8": kvq.FMT_FP8_E4M3, "int8": kvq.FMT_INT8, "kivi": kvq.FMT_KIVI, "bf16": kvq.FMT_BF16,
           "int4": kvq.FMT_INT4, "fp8s": kvq.FMT_FP8_STATIC, "int4h": kvq.FMT_INT4_HADAMARD,
           "kivi16": kvq.FMT_KIVI_F16}[w.fmt]
    cfg = kvq.make_config(fmt, w.bits, w.group, w.residual, w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim,
                          n_max + grow, kvq.DT_BF16 if w.dtype == "bf16" else kvq.DT_F32)
    lay = kvq.kvq_get_layout(cfg)
    if args.layers:
        copies = args.layers
    elif w.layers > 1:
        copies = w.layers
    else:
        # enough copies to span min_bytes, at most 64 (the tiny workload's
        # 0.1 MB cache would otherwise need ~20000 copies and graphs of
        # hundreds of thousands of launches)
        copies = min(64, max(1, math.ceil(args.min_bytes / lay.total_bytes)))
    # the bf16 cache of the long-context workload is 8.6 GB per layer at
    # capacity: keep the copies within 250 GB of the 288 GB of HBM (the 80
    # layers of every quantized workload fit)
    fit = max(2, int(250e9 // lay.total_bytes))
    if copies > fit:
        print(f"bench: {copies} cache copies of {lay.total_bytes / 1e9:.1f} GB do not fit; using {fit}",
              file=sys.stderr)
        copies = fit
    ws_bytes = kvq.kvq_decode_workspace_bytes(cfg, args.split)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)  # arrival counters start at zero
    stream = torch.cuda.current_stream()

    caches, seq_lens, qs, outs = [], [], [], []
    fill_ms = []
    k_host = v_host = None
    for c in range(copies):
        buf = torch.zeros(lay.total_bytes, dtype=torch.uint8, device=dev)
        sl = torch.zeros(w.batch, dtype=torch.int32, device=dev)
        k, v = kv_tokens(w, n_max, layer=c, device=dev)
        al = lens0.to(dev) if w.ragged else None
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kvq.kvq_quantize_append(cfg, buf, sl, k, v, n_max, al)
        e1.record(stream)
        torch.cuda.synchronize()
        fill_ms.append(e0.elapsed_time(e1))
        if c == 0 and not args.no_cpu_baseline:
            k_host = k.float().cpu().numpy()
            v_host = v.float().cpu().numpy()
        del k, v
        torch.cuda.empty_cache()
        caches.append(buf)
        seq_lens.append(sl)
        qs.append(queries(w, layer=c, device=dev))
        outs.append(torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    bulk_tokens = float(lens0.sum())
    bulk_bytes = sum(append_bytes(w, [0], int(n)) for n in lens0)
    bulk_ms = float(np.median(fill_ms))

    # new tokens for every step and copy (small), generated up front
    steps_total = args.warmup + args.steps
    new_k, new_v = [], []
    for c in range(copies):
        k, v = kv_tokens(w, steps_total, layer=c, stream=1, device=dev)
        new_k.append([k[:, :, s:s + 1].contiguous() for s in range(steps_total)])
        new_v.append([v[:, :, s:s + 1].contiguous() for s in range(steps_total)])
    sm = 1.0 / math.sqrt(w.head_dim)

    ws_list = [ws]

    def decode(c):
        kvq.kvq_decode_attention(cfg, caches[c], seq_lens[c], qs[c], sm, outs[c], ws_list[0], ws_bytes, args.split)

    def step(s):
        for c in range(copies):
            if args.unfused:
                kvq.kvq_quantize_append(cfg, caches[c], seq_lens[c], new_k[c][s], new_v[c][s], 1)
                decode(c)
            else:
                kvq.kvq_append_decode(cfg, caches[c], seq_lens[c], new_k[c][s], new_v[c][s], qs[c], sm, outs[c],
                                      ws_list[0], ws_bytes, args.split)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    lens_start = lens0.numpy().astype(np.int64) + args.warmup

    # The timed steps are captured into one HIP graph first, so the host's
    # per-launch cost stays outside the timed region (all arguments are
    # device pointers and sizes; seq_lens advance on the device).
    steps_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(steps_graph):
        for s in range(args.warmup, steps_total):
            step(s)
    torch.cuda.synchronize()
    # an untimed replay first (the first launch of a graph also uploads it);
    # it appends the same new tokens once more, which the capacity allows
    steps_graph.replay()
    torch.cuda.synchronize()
    lens_start += args.steps
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    steps_graph.replay()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)

    # Decode call alone (one kernel launch per call), rotating over the
    # copies: a graph of `rounds` passes, timed with events on its stream.
    rounds = max(1, args.decode_rounds)
    dec_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(dec_graph):
        for _ in range(rounds):
            for c in range(copies):
                decode(c)
    torch.cuda.synchronize()
    dec_graph.replay()  # untimed pass
    torch.cuda.synchronize()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record()
    dec_graph.replay()
    d1.record()
    torch.cuda.synchronize()
    dec_avg_ms = d0.elapsed_time(d1) / (rounds * copies)

    lens_end = lens_start + args.steps
    dec_bytes_total, app_bytes_total = 0.0, 0.0
    for i in range(args.steps):
        before = lens_start + i
        app_bytes_total += copies * append_bytes(w, before, 1)
        dec_bytes_total += copies * decode_bytes(w, before + 1)
    dec_bytes_per_call = decode_bytes(w, lens_end)
    achieved = dec_bytes_per_call / (dec_avg_ms * 1e-3) / 1e9
    value = (dec_bytes_total + app_bytes_total) / (total_ms * 1e-3) / 1e9
    ms_per_step = total_ms / args.steps

    traffic, traffic_src = profiled_traffic(w) if args.split == 0 else (None, None)
    result = {
        "metric": "decode-attn effective HBM GB/s (% of peak) + appended KV tokens/s, 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "e4m3", "fp8s": "e4m3", "int8": "i8", "bf16": "bf16", "int4": "s4",
                  "int4h": "s4"}.get(w.fmt, f"u{w.bits}") +
                 " codes, bf16 MFMA (hi+lo), f32 accumulate",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_kv_heads": w.n_kv_heads, "n_q_heads": w.n_q_heads,
                   "head_dim": w.head_dim, "context": w.context if not w.ragged else
                   f"ragged {w.context_min}..{w.context}", "group": w.group, "residual": w.residual,
                   "input_dtype": w.dtype, "cache_format": w.fmt, "cache_copies": copies,
                   "split_tokens": args.split,
                   "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "decode_gbps": round(achieved, 2),
        "decode_pct_of_peak": round(100 * achieved / HBM_PEAK_GBPS, 2),
        "decode_us_per_call": round(dec_avg_ms * 1e3, 2),
        "step": "one launch per layer (append + decode fused)" if not args.unfused else
                "two calls per layer (append, then decode)",
        "step_us_per_layer": round(total_ms * 1e3 / (args.steps * copies), 2),
        "decode_tokens_per_s_per_layer": round(w.batch * copies * args.steps / (total_ms * 1e-3), 1),
        "append_tokens_per_s_streaming": round(w.batch * copies * args.steps / (total_ms * 1e-3), 1),
        "append_bulk_tokens_per_s": round(bulk_tokens / (bulk_ms * 1e-3), 1),
        "append_bulk_gbps": round(bulk_bytes / (bulk_ms * 1e-3) / 1e9, 2),
        "wall_s_timed": round(wall, 3),
        "decode_calls_timed": rounds * copies,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": round(traffic) if traffic is not None else None,
                     "kernel": "decode_split (one launch per decode call, merge fused)",
                     "bytes_per_launch": round(dec_bytes_per_call, 1),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE, WRITE_SIZE scaled by a 1 GiB copy)",
                     "traffic_source": traffic_src},
    }
    ceiling["decode_frac_of_ceiling"] = round(achieved / ceiling["gbps"], 4)
    result["stream_read_ceiling"] = ceiling
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, k_host, v_host, qs[0].float().cpu().numpy(), lens0.numpy(),
                                              args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
