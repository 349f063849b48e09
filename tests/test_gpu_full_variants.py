"""GPU parity at the benchmark sizes for the cache-format variants and the
fused decode step: the full workload shapes that bench.py measures, sampled
(b, kv head) pairs bit-exact against the oracle and their attention within
tolerance."""
import pytest

from kvq_workloads import WORKLOADS
from test_gpu_parity import _sampled_full

pytestmark = pytest.mark.gpu

VARIANTS = {
    "bf16-w2": (2, dict(fmt="bf16", bits=16, group=0, residual=0)),
    "fp8s-w2": (2, dict(fmt="fp8s", bits=8, group=0, residual=0)),
    "int4-g32-w3": (3, dict(fmt="int4", bits=4, group=32, residual=0)),
    "int4h-g128-w3": (3, dict(fmt="int4h", bits=4, group=128, residual=0)),
    "kivi16-w4": (4, dict(fmt="kivi16")),
}


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_full_size_format_variant_sampled(name):
    idx, kw = VARIANTS[name]
    _sampled_full(idx, pairs=2, n_decode_pairs=1, w=WORKLOADS[idx].scaled(**kw))


@pytest.mark.parametrize("idx", [2, 3, 4])
def test_full_size_fused_step_sampled(idx):
    _sampled_full(idx, pairs=2, n_decode_pairs=2, fused=True)


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_full_size_format_variant_fused_step_sampled(name):
    """One fused append + decode step on each variant at its full workload
    size: the appended token's codes (and, for KIVI, a completed group)
    bit-exact on the sampled pairs, attention in tolerance."""
    idx, kw = VARIANTS[name]
    _sampled_full(idx, pairs=2, n_decode_pairs=1, w=WORKLOADS[idx].scaled(**kw), fused=True)


def test_full_size_long_context_fused_step_sampled():
    _sampled_full(5, pairs=2, n_decode_pairs=2, layer=0, fused=True)
