"""Seeded synthetic inputs for the quantized KV cache workloads.

Shared by the tests, the benchmark and the CPU oracle's callers. This module
only draws random numbers with torch generators; it holds none of the
method's arithmetic (no quantization, no attention).

Five workloads, all with bf16 inputs except the tiny one (fp32):

1. tiny KIVI INT4: 1 layer, batch 1, 2 KV heads, 8 query heads, head_dim 64,
   256 tokens, group 32, residual 16. K ~ N(0,1) with channels 3 and 40
   (0-based) scaled by 20; V rows ~ N(0,1) * exp(N(0,1)); q ~ N(0,1).
2. FP8 E4M3 per-token: batch 16, 8 KV heads, 32 query heads, head_dim 128,
   4096 tokens; K, V ~ N(0,1) with 4 fixed K outlier channels scaled by 10.
3. INT8 per-token: batch 64, 8 KV heads, 64 query heads, head_dim 128, 8192
   tokens; K with 4 outlier channels x30, V rows N(0,1) * exp(N(0,1)).
4. KIVI INT2, group 32, residual 128: batch 32, 8 KV heads, 64 query heads,
   head_dim 128, 32768 tokens; distributions as workload 3.
5. KIVI INT4, group 64, residual 128, long context: batch 16, 8 KV heads, 64
   query heads, head_dim 128, per-sequence context uniform in [65536, 131072],
   80 layers each with its own seed (1000 + layer); distributions as 3.

Outlier channels for workloads 2-5 are the first four entries of a seeded
permutation of the head_dim channels, fixed across batch, heads and tokens
of a layer.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    fmt: str                  # "fp8", "int8", "kivi"
    bits: int
    group: int
    residual: int
    layers: int
    batch: int
    n_kv_heads: int
    n_q_heads: int
    head_dim: int
    context: int              # tokens per sequence (upper end when ragged)
    context_min: int          # lower end of the ragged range (== context when fixed)
    dtype: str                # "f32" or "bf16"
    k_outliers: Tuple[int, ...] = ()   # fixed channels (workload 1); else drawn
    n_k_outliers: int = 0
    k_outlier_mul: float = 1.0
    v_lognormal: bool = False

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def ragged(self) -> bool:
        return self.context_min != self.context

    def scaled(self, **kw) -> "Workload":
        """Same distributions at other sizes (for small parity cases)."""
        return replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "tiny-kivi-int4-g32-r16", "kivi", 4, 32, 16, 1, 1, 2, 8, 64, 256, 256, "f32",
                k_outliers=(3, 40), k_outlier_mul=20.0, v_lognormal=True),
    2: Workload(2, "fp8-e4m3-per-token", "fp8", 8, 0, 0, 1, 16, 8, 32, 128, 4096, 4096, "bf16",
                n_k_outliers=4, k_outlier_mul=10.0, v_lognormal=False),
    3: Workload(3, "int8-sym-per-token", "int8", 8, 0, 0, 1, 64, 8, 64, 128, 8192, 8192, "bf16",
                n_k_outliers=4, k_outlier_mul=30.0, v_lognormal=True),
    4: Workload(4, "kivi-int2-g32-r128", "kivi", 2, 32, 128, 1, 32, 8, 64, 128, 32768, 32768, "bf16",
                n_k_outliers=4, k_outlier_mul=30.0, v_lognormal=True),
    5: Workload(5, "kivi-int4-g64-r128-long-ragged", "kivi", 4, 64, 128, 80, 16, 8, 64, 128,
                131072, 65536, "bf16", n_k_outliers=4, k_outlier_mul=30.0, v_lognormal=True),
}


def layer_seed(w: Workload, layer: int) -> int:
    """Base seed of one layer: 1000 + layer for the 80-layer workload,
    100 * workload index otherwise."""
    return 1000 + layer if w.layers > 1 else 100 * w.index + layer


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def outlier_channels(w: Workload, layer: int = 0) -> Tuple[int, ...]:
    if w.k_outliers:
        return tuple(c for c in w.k_outliers if c < w.head_dim)
    if w.n_k_outliers == 0:
        return ()
    perm = torch.randperm(w.head_dim, generator=_gen("cpu", layer_seed(w, layer) * 7 + 4))
    return tuple(int(c) for c in perm[: w.n_k_outliers])


def context_lengths(w: Workload, layer: int = 0) -> torch.Tensor:
    """int32 [batch] tokens per sequence (CPU tensor). Ragged workloads draw
    uniformly from [context_min, context]; the draw is shared by all layers."""
    if not w.ragged:
        return torch.full((w.batch,), w.context, dtype=torch.int32)
    g = _gen("cpu", 10_000 + w.index)
    return torch.randint(w.context_min, w.context + 1, (w.batch,), generator=g, dtype=torch.int64).to(torch.int32)


def kv_tokens(w: Workload, t: int, layer: int = 0, stream: int = 0, device="cpu",
              batch: Optional[int] = None):
    """(K, V) [batch, n_kv_heads, t, head_dim] in the workload dtype.

    ``stream`` selects independent draws (0 = the bulk prefill, s > 0 = the
    tokens appended at decode step s). Sampled per batch element to bound
    temporary memory."""
    B = w.batch if batch is None else batch
    base = layer_seed(w, layer) * 7919 + stream * 104729
    ch = list(outlier_channels(w, layer))
    ks, vs = [], []
    for b in range(B):
        gk = _gen(device, base + 2 * b)
        gv = _gen(device, base + 2 * b + 1)
        k = torch.randn((w.n_kv_heads, t, w.head_dim), generator=gk, device=device, dtype=torch.float32)
        if ch:
            k[..., ch] *= w.k_outlier_mul
        v = torch.randn((w.n_kv_heads, t, w.head_dim), generator=gv, device=device, dtype=torch.float32)
        if w.v_lognormal:
            mag = torch.randn((w.n_kv_heads, t, 1), generator=gv, device=device, dtype=torch.float32).exp_()
            v *= mag
        ks.append(k.to(w.torch_dtype))
        vs.append(v.to(w.torch_dtype))
    return torch.stack(ks), torch.stack(vs)


def queries(w: Workload, layer: int = 0, step: int = 0, device="cpu", batch: Optional[int] = None):
    """q [batch, n_q_heads, head_dim] ~ N(0,1) in the workload dtype."""
    B = w.batch if batch is None else batch
    g = _gen(device, layer_seed(w, layer) * 7919 + 31 + step * 104729)
    return torch.randn((B, w.n_q_heads, w.head_dim), generator=g, device=device,
                       dtype=torch.float32).to(w.torch_dtype)
