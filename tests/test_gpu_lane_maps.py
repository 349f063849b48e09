"""Lane maps and exact conversions of the wave-level building blocks
(kvq_wave.h, kvq_quant.h), run on one wave by a test-only kernel
(tests/lane_maps/lane_maps.hip) and compared with their definitions:
the DPP controls (quad_perm, row_ror by 8 under bank masks, half-row and row
mirrors), the cross-row shuffles, the order-preserving float keys, the byte
transpose, the FP8 E4M3 byte conversions (every byte to bf16; the
integers 0..15 to f16 through the scale 2^9), the FP4 E2M1 nibble
conversion (the integers 0..3 to f16 through the scale 2) and the bf16 dot
product that subtracts one half of a bf16 pair."""
import ctypes
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "lane_maps", "liblanemaps.so")
L = np.arange(64)
X = ((37 * L) % 64 + 0.25).astype(np.float32)
SX = ((37 * L) % 64 - 31.5).astype(np.float32)
ROR8 = (L & ~15) | (((L & 15) + 8) & 15)  # row_ror by 8: lane k of a row reads lane (k + 8) mod 16


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def _runs(a, n, f):
    return np.repeat(f(a.reshape(-1, n), axis=1), n)


@pytest.fixture(scope="module")
def out():
    import torch
    if not os.path.exists(LIB):
        from tests.lane_maps import build_lane_maps  # noqa: F401  (built in-tree when missing)
        build_lane_maps.build()
    lib = ctypes.CDLL(LIB)
    lib.kvq_test_lane_maps.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.kvq_test_lane_maps.restype = ctypes.c_int
    buf = torch.zeros(30 * 64, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    assert lib.kvq_test_lane_maps(buf.data_ptr(), ctypes.c_void_p(s.cuda_stream)) == 0
    torch.cuda.synchronize()
    return buf.cpu().numpy().view(np.uint32).reshape(30, 64)


@pytest.mark.gpu
def test_row_rotation_and_cross_row_reductions(out):
    np.testing.assert_array_equal(out[0], _bits(X + X[ROR8]))
    np.testing.assert_array_equal(out[1], _bits(np.maximum(X, X[ROR8])))
    rows = X.reshape(4, 16)  # lanes l, l ^ 16, l ^ 32, l ^ 48 share l mod 16
    np.testing.assert_array_equal(out[2], _bits(np.tile(rows.max(axis=0), 4)))
    np.testing.assert_array_equal(out[3], _bits(np.tile(rows.sum(axis=0, dtype=np.float32), 4)))
    np.testing.assert_array_equal(out[4], _bits(np.full(64, X[:32].max())))


@pytest.mark.gpu
def test_bank_masked_swaps(out):
    bank = (L & 15) >> 2
    take_hi = np.isin(bank, (2, 3))  # bank mask 0xc: lanes 8-15 of each row
    np.testing.assert_array_equal(out[5], np.where(take_hi, 2000 + ROR8, 1000 + L))
    take_lo = np.isin(bank, (0, 1))  # bank mask 0x3: lanes 0-7 of each row
    np.testing.assert_array_equal(out[6], np.where(take_lo, 2000 + ROR8, 1000 + L))
    np.testing.assert_array_equal(out[13], 1000 + (L ^ 2))  # quad_perm [2, 3, 0, 1]


@pytest.mark.gpu
def test_run_reductions(out):
    np.testing.assert_array_equal(out[7], _bits(_runs(X, 8, np.max)))
    np.testing.assert_array_equal(out[8], _bits(_runs(X, 16, np.max)))
    np.testing.assert_array_equal(out[9], _bits(_runs(SX, 4, np.min)))
    np.testing.assert_array_equal(out[10], _bits(_runs(SX, 4, np.max)))
    np.testing.assert_array_equal(out[11], _bits(_runs(SX, 8, np.min)))
    np.testing.assert_array_equal(out[12], _bits(_runs(SX, 8, np.max)))


@pytest.mark.gpu
def test_float_keys_preserve_order(out):
    keys = out[22]
    assert np.array_equal(np.argsort(keys, kind="stable"), np.argsort(SX, kind="stable"))
    np.testing.assert_array_equal(out[23], _bits(SX))


@pytest.mark.gpu
def test_byte_transpose(out):
    for e in range(4):
        want = sum(((16 * j + 4 * e + (L & 3)).astype(np.uint32) << (8 * j)) for j in range(4))
        np.testing.assert_array_equal(out[14 + e], want)


@pytest.mark.gpu
def test_e4m3_bytes_to_bf16_every_code(out):
    """Each lane converts bytes 4l .. 4l+3: all 256 E4M3 codes. The low half
    of each result holds the lower byte's value."""
    from oracle.kvq_oracle import e4m3_decode
    got = np.stack([out[18] & 0xFFFF, out[18] >> 16, out[19] & 0xFFFF, out[19] >> 16], axis=1).reshape(-1)
    want = e4m3_decode(np.arange(256)).astype(np.float32)
    nan = np.isnan(want)
    np.testing.assert_array_equal(got[~nan], _bits(want[~nan]) >> 16)  # every value is exact in bf16
    assert np.all(((got[nan] >> 7) & 0xFF) == 0xFF) and np.all((got[nan] & 0x7F) != 0)


@pytest.mark.gpu
def test_small_integers_through_the_scaled_e4m3_to_f16_conversion(out):
    """A byte c in 0..15 (the E4M3 pattern of c * 2^-9) converts with scale
    2^9 to the f16 value c exactly; the low half holds the lower byte."""
    c = (L[:, None] + np.arange(4)[None, :]) % 16
    got = np.stack([out[20] & 0xFFFF, out[20] >> 16, out[21] & 0xFFFF, out[21] >> 16], axis=1)
    np.testing.assert_array_equal(got, c.astype(np.float16).view(np.uint16))


@pytest.mark.gpu
def test_two_bit_integers_through_the_scaled_e2m1_to_f16_conversion(out):
    """A nibble c in 0..3 (the E2M1 pattern of c / 2) converts with scale 2 to
    the f16 value c exactly; byte k of the word gives result k, its low
    nibble in the low half."""
    for k in range(4):
        lo = (L + k) % 4
        hi = (L + 2 * k + 1) % 4
        got = np.stack([out[26 + k] & 0xFFFF, out[26 + k] >> 16], axis=1)
        want = np.stack([lo, hi], axis=1).astype(np.float16).view(np.uint16)
        np.testing.assert_array_equal(got, want)


@pytest.mark.gpu
def test_bf16_half_subtraction_by_dot_product(out):
    """y - float(bf16 half) as one bf16 dot product with the register units
    (-1, 0) and (0, -1): exact, and each unit picks its own half."""
    y = X * np.float32(1.0078125) + np.float32(2.0 ** -10)
    def trunc(a):
        return (_bits(a) & np.uint32(0xFFFF0000)).view(np.float32)
    np.testing.assert_array_equal(out[24], _bits(y - trunc(y)))
    np.testing.assert_array_equal(out[25], _bits(-y - trunc(-y)))
    assert np.all(out[24] != 0)
