"""Benchmark of the quantized KV cache hot path on one MI355X.

A step is one decode iteration over every cache copy ("layer"): append one
new K/V token per sequence (quantize, or residual write + group flush) and
run decode attention over the whole cache, as one fused launch per layer
(kvq_append_decode; --unfused times the two separate calls instead). The
default workload is the long-context one (workload 5: KIVI INT4, group 64,
residual 128, batch 16, 8 KV heads, 64 query heads, head_dim 128, ragged
contexts of 64K-128K tokens, 80 layers with their own seeds): the largest
configuration, on which the INT4 KIVI half of the decode target is set.
The FP8 workload (workload 2: batch 16, 8 KV heads, 32 query heads, 4096
tokens) is measured after it in the same run and reported under
"fp8_workload"; its 139 MB cache fits in the 256 MB Infinity Cache, so its
timing rotates over enough independent copies to touch >= 2 GB. Inputs are
seeded synthetic data already resident in HBM.

Prints one JSON line: value = algorithmic bytes of the timed steps (cache
bytes read by decode + q + out, plus append input and cache writes) per
second of the timed region; "roofline" covers the decode-attention call
(one launch of the split-K kernel, whose last split per (sequence, KV head)
merges the partials) timed with HIP events on its stream;
"cpu_baseline" times the CPU oracle on a bounded sample of the same work,
on every host core the process may use (one worker process each) and on
one core; "stream_read_ceiling" is the read rate of a plain streaming
kernel on the same device, measured first, for context.
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
    p.add_argument("--config", type=int, default=5, help="workload index 1..5")
    p.add_argument("--no-fp8-extra", action="store_true",
                   help="with the default workload 5, skip the FP8 workload 2 measurement after it")
    p.add_argument("--split", type=int, default=0, help="longest decode split in tokens (0 = library choice)")
    p.add_argument("--min-bytes", type=float, default=2.0e9, help="bytes the rotated copies must span")
    p.add_argument("--layers", type=int, default=0, help="override the number of cache copies")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="wall-clock budget of the all-cores oracle timing")
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


DECODE_SOURCES = ("quantized_kv_cache_06_amd/csrc/kvq_decode.hip", "quantized_kv_cache_06_amd/csrc/kvq_api.cpp",
                  "quantized_kv_cache_06_amd/csrc/kvq_device.h", "quantized_kv_cache_06_amd/csrc/kvq_wave.h",
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


# --- CPU baseline: the oracle as it is, on the host cores ------------------
# Worker processes are started fresh (spawn) and import only numpy and the
# oracle; each runs one BLAS thread. A task is one (sequence, KV head) pair:
# append its n tokens through the oracle, then decode its g query heads
# (what the oracle's decode_attention does per KV head). The pair's bf16
# inputs come from shared memory when the host allows it, else with the task.
_WORKER = {}


def _cpu_worker_init(shm_names):
    from threadpoolctl import threadpool_limits
    _WORKER["limits"] = threadpool_limits(limits=1)
    _WORKER["shm"] = {}
    if shm_names:
        from multiprocessing import shared_memory
        for key, name in shm_names.items():
            _WORKER["shm"][key] = shared_memory.SharedMemory(name=name)


def _as_f32(x):
    """Input rows as float32: bf16 (held as uint16 bit patterns) widens
    exactly; float32 passes."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    return np.asarray(x, dtype=np.float32)


def _cpu_pair(task):
    """Returns the seconds the oracle took for one pair (input widening and
    transfer excluded)."""
    from oracle import kvq_oracle as O
    wdesc, b, h, n, q_rows, sm, arrays = task
    fmt, d, bits, group, residual, shape, dt = wdesc
    if arrays is None:
        views = [np.ndarray(shape, dtype=dt, buffer=_WORKER["shm"][key].buf) for key in ("k", "v")]
        kb, vb = views[0][b, h, :n], views[1][b, h, :n]
    else:
        kb, vb = arrays
    k, v = _as_f32(kb), _as_f32(vb)
    t0 = time.perf_counter()
    s = O.SequenceCache(fmt, d, bits, group, residual)
    s.append(k, v)
    K, V = s.dequantized()
    for qr in q_rows:
        O.attention_one_head(qr, K, V, sm)
    return time.perf_counter() - t0


def cpu_workers():
    """Host cores the process may use, capped at the 16-core share of one GPU
    on the benchmark machines."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_baseline(w, k_in, v_in, q_host, lens, seconds):
    """Time the CPU oracle (as it is) on copy 0's (sequence, KV head) pairs:
    first on one core in this process (until ~2 s of work), then on every
    core with one worker process per core over as many pairs as fit the
    wall-clock budget (the whole copy when it fits). GB/s use the same
    algorithmic byte counts as the GPU figures."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    from threadpoolctl import threadpool_limits

    from oracle import kvq_oracle as O
    sm = O.default_sm_scale(w.head_dim)
    g = w.n_q_heads // w.n_kv_heads
    wdesc = (w.fmt, w.head_dim, w.bits, w.group, w.residual, tuple(k_in.shape), k_in.dtype.str)
    pairs = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]

    def pair_bytes(b):
        n = int(lens[b])
        return (append_bytes(w, [0], n) + decode_bytes(w, [n])) / w.n_kv_heads

    def task(b, h, inline):
        n = int(lens[b])
        arrays = (k_in[b, h, :n], v_in[b, h, :n]) if inline else None
        return (wdesc, b, h, n, q_host[b, h * g:(h + 1) * g], sm, arrays)

    # one core, in this process
    _WORKER["shm"] = {}
    one_s, one_bytes, one_pairs = 0.0, 0.0, 0
    with threadpool_limits(limits=1):
        for b, h in pairs:
            one_s += _cpu_pair(task(b, h, True))
            one_bytes += pair_bytes(b)
            one_pairs += 1
            if one_s >= 2.0:
                break
    t_pair = one_s / one_pairs
    workers = cpu_workers()
    n_par = min(len(pairs), workers * max(1, int(seconds / t_pair)))
    sample = pairs[:n_par] if n_par == len(pairs) else pairs[::max(1, len(pairs) // n_par)][:n_par]

    shms, names = [], {}
    try:
        try:
            from multiprocessing import shared_memory
            for key, arr in (("k", k_in), ("v", v_in)):
                sh = shared_memory.SharedMemory(create=True, size=arr.nbytes)
                shms.append(sh)
                np.ndarray(arr.shape, dtype=arr.dtype, buffer=sh.buf)[...] = arr
                names[key] = sh.name
            inline = False
        except OSError:
            names, inline = {}, True
        ctx = mp.get_context("spawn")
        with ProcessPoolExecutor(max_workers=workers, mp_context=ctx, initializer=_cpu_worker_init,
                                 initargs=(names,)) as ex:
            list(ex.map(time.sleep, [0.05] * workers))  # workers started before the clock runs
            t0 = time.perf_counter()
            busy = list(ex.map(_cpu_pair, [task(b, h, inline) for b, h in sample]))
            wall = time.perf_counter() - t0
    finally:
        for sh in shms:
            sh.close()
            sh.unlink()
    par_bytes = sum(pair_bytes(b) for b, _ in sample)
    whole = n_par == len(pairs)
    out = {"value": par_bytes / wall / 1e9, "unit": "GB/s", "cores": workers, "kind": "oracle",
           "sample": f"{n_par} of {len(pairs)} (sequence, KV head) pairs of copy 0 (bulk append of each "
                     f"sequence's n tokens + one decode of its {g} query heads), numpy oracle, "
                     f"{workers} worker processes with one BLAS thread each, {wall:.1f} s wall "
                     f"({sum(busy):.1f} s of oracle work)",
           "single_core_value": one_bytes / one_s / 1e9,
           "single_core_sample": f"{one_pairs} pairs in this process, one BLAS thread, {one_s:.1f} s"}
    if whole:
        out["copy_seconds_all_cores"] = round(wall, 2)
        if w.layers > 1:
            out["all_layers_seconds_extrapolated"] = round(wall * w.layers, 1)
    return out


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


def resolve_workload(WORKLOADS, idx, args):
    w = WORKLOADS[idx]
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
    return w


def compute_label(w):
    """What the decode kernel computes in, for the JSON line's dtype."""
    codes = {"fp8": "e4m3", "fp8s": "e4m3", "int8": "i8", "bf16": "bf16", "int4": "s4",
             "int4h": "s4"}.get(w.fmt, f"u{w.bits}") + " codes"
    if is_kivi(w):
        return codes + ", Key scores on f16 MFMA (query x scale split hi+lo), values on bf16 MFMA " \
                       "(probabilities split hi+lo), f32 accumulate and softmax"
    return codes + ", bf16 MFMA (query and probabilities split hi+lo), f32 accumulate and softmax"


def run_workload(torch, kvq, w, args, copies_override=0, want_host=False):
    """Fill the caches of workload w, time the fused steps and the decode
    call, and return (result dict, host inputs of copy 0 or None)."""
    from kvq_workloads import context_lengths, kv_tokens, queries
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
    if copies_override:
        copies = copies_override
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

    # one untimed append through the same kernels on a one-sequence cache of
    # the same format first: the first launch of a kernel also loads its
    # code, which would otherwise count against the first copy's fill
    wcfg = kvq.make_config(fmt, w.bits, w.group, w.residual, 1, w.n_kv_heads, w.n_q_heads, w.head_dim,
                           2 * (w.group or 32) + w.residual, cfg.in_dtype)
    wbuf = torch.zeros(kvq.kvq_get_layout(wcfg).total_bytes, dtype=torch.uint8, device=dev)
    wsl = torch.zeros(1, dtype=torch.int32, device=dev)
    wk, wv = kv_tokens(w, wcfg.max_tokens, device=dev, batch=1)
    kvq.kvq_quantize_append(wcfg, wbuf, wsl, wk, wv, wcfg.max_tokens)
    torch.cuda.synchronize()
    del wbuf, wsl, wk, wv

    caches, seq_lens, qs, outs = [], [], [], []
    fill_ms = []
    host = None
    t_fill = time.perf_counter()
    for c in range(copies):
        buf = torch.zeros(lay.total_bytes, dtype=torch.uint8, device=dev)
        sl = torch.zeros(w.batch, dtype=torch.int32, device=dev)
        # the lengths' host-to-device copy waits for the host; made before the
        # inputs are generated, so that the device is still busy with those
        # while the host issues the append (the window then holds device
        # work only, not the binding's marshalling)
        al = lens0.to(dev) if w.ragged else None
        k, v = kv_tokens(w, n_max, layer=c, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kvq.kvq_quantize_append(cfg, buf, sl, k, v, n_max, al)
        e1.record(stream)
        torch.cuda.synchronize()
        fill_ms.append(e0.elapsed_time(e1))
        if c == 0 and want_host:
            if w.dtype == "bf16":
                host = (k.view(torch.int16).cpu().numpy().view(np.uint16),
                        v.view(torch.int16).cpu().numpy().view(np.uint16))
            else:
                host = (k.cpu().numpy(), v.cpu().numpy())
        del k, v
        torch.cuda.empty_cache()  # the 4 GB input temporaries would otherwise fragment HBM
        caches.append(buf)
        seq_lens.append(sl)
        qs.append(queries(w, layer=c, device=dev))
        outs.append(torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev))
        if c % 16 == 15:
            print(f"bench: {w.name}: {c + 1} of {copies} caches filled "
                  f"({time.perf_counter() - t_fill:.0f} s)", file=sys.stderr, flush=True)
    torch.cuda.empty_cache()
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

    def decode(c):
        kvq.kvq_decode_attention(cfg, caches[c], seq_lens[c], qs[c], sm, outs[c], ws, ws_bytes, args.split)

    def step(s):
        for c in range(copies):
            if args.unfused:
                kvq.kvq_quantize_append(cfg, caches[c], seq_lens[c], new_k[c][s], new_v[c][s], 1)
                decode(c)
            else:
                kvq.kvq_append_decode(cfg, caches[c], seq_lens[c], new_k[c][s], new_v[c][s], qs[c], sm, outs[c],
                                      ws, ws_bytes, args.split)

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
        "value": round(value, 2),
        "ms_per_step": round(ms_per_step, 4),
        "dtype": compute_label(w),
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
        "append_bulk_us_per_copy": round(bulk_ms * 1e3, 1),
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
    q_host = qs[0].float().cpu().numpy() if want_host else None
    return result, (host, q_host, lens0.numpy()) if want_host else None


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
    from kvq_workloads import WORKLOADS
    if not os.path.exists(kvq.LIB_PATH):
        from quantized_kv_cache_06_amd import build as _b
        _b.build()

    if args.stream_ref > 0:
        stream_reference(torch, args.stream_ref)
        return
    ceiling = stream_ceiling(torch)

    w = resolve_workload(WORKLOADS, args.config, args)
    want_cpu = not args.no_cpu_baseline
    res, host = run_workload(torch, kvq, w, args, copies_override=args.layers, want_host=want_cpu)
    result = {
        "metric": "decode-attn effective HBM GB/s (% of peak) + appended KV tokens/s, 1 GPU",
        "value": res.pop("value"),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res.pop("dtype"),
        "data": "synthetic",
        "config": res.pop("config"),
    }
    result.update(res)
    ceiling["decode_frac_of_ceiling"] = round(res["decode_gbps"] / ceiling["gbps"], 4)
    result["stream_read_ceiling"] = ceiling
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    if args.config == 5 and not args.no_fp8_extra:
        # the FP8 half of the decode target, in the same run: workload 2's
        # own copies (the long-context caches are freed first)
        print("bench: FP8 workload 2", file=sys.stderr, flush=True)
        w2 = resolve_workload(WORKLOADS, 2, args)
        r2, _ = run_workload(torch, kvq, w2, args)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        result["fp8_workload"] = {
            "config": r2["config"], "dtype": r2["dtype"], "value": r2["value"],
            "decode_us_per_call": r2["decode_us_per_call"], "decode_gbps": r2["decode_gbps"],
            "decode_pct_of_peak": r2["decode_pct_of_peak"], "step_us_per_layer": r2["step_us_per_layer"],
            "append_bulk_gbps": r2["append_bulk_gbps"], "roofline": r2["roofline"]}

    if want_cpu:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        (k_host, v_host), q_host, lens = host
        result["cpu_baseline"] = cpu_baseline(w, k_host, v_host, q_host, lens, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
