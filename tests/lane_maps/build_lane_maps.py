"""Builds tests/lane_maps/liblanemaps.so (test-only) with libkvq's compiler
flags and headers."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "liblanemaps.so")


def build() -> str:
    sys.path.insert(0, ROOT)
    from quantized_kv_cache_06_amd import build as B
    tmp = LIB + ".tmp"
    B._run([B.HIPCC, *B.COMMON, "-shared", "-x", "hip", os.path.join(HERE, "lane_maps.hip"), "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
