"""Pins of the CPU oracle to facts fixed outside it: the pages' printed
numbers and worked examples, closed forms, library routines and brute force.

Each test names the passage it follows. A plausible slip in the oracle (a
transposed quantization axis, half-away rounding, a dropped zero-point, a
wrong GQA head mapping, a missing softmax scale) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import kvq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --- "KV Cache Quantization" (infra.bea.ai) §1 table --------------------------
def test_memory_table_matches_page():
    t = _golden("bea_memory_table.json")
    m = t["model"]
    for row in t["rows"]:
        per_token = O.kv_bytes_per_token(m["n_layers"], m["n_kv_heads"], m["head_dim"],
                                         row["bytes_per_element"])
        assert per_token == row["kv_per_token_kb"] * 1024
        ctx_gib = per_token * t["context_tokens"] / 2 ** 30
        # printed to two decimals, half up (0.625 -> 0.63)
        assert math.floor(ctx_gib * 100 + 0.5) / 100 == row["context_gb"]
        # the page divides the budget by its own rounded GB column
        assert math.floor(t["available_gb"] / row["context_gb"]) == row["max_requests"]


def test_memory_formula_llms_intro():
    # "Memory per Token = 2 x 2 x n_layers x n_kv_heads x d_head bytes" (16-bit)
    assert O.kv_bytes_per_token(80, 8, 128, 2) == 2 * 2 * 80 * 8 * 128
    # halving the element width halves the bytes (update section, capacity math)
    assert O.kv_bytes_per_token(80, 8, 128, 1) * 2 == O.kv_bytes_per_token(80, 8, 128, 2)


# --- §3 "Key: Per-Channel Quantization" worked example ----------------------
def test_key_example_per_channel_scale_is_page_value():
    g = _golden("bea_kivi_examples.json")
    K = np.array(g["key_matrix"], F32)                   # rows tokens, cols channels
    ch = g["key_outlier_channel_1based"] - 1
    num, den = g["key_outlier_scale"]["numerator"], g["key_outlier_scale"]["denominator"]
    # per channel = one symmetric absmax/127 scale per column
    codes, s = O.quantize_int8_per_token(K.T)
    assert s[ch] == F32(num) / F32(den)
    # the outlier does not affect the other channels' scales
    for c in range(K.shape[1]):
        if c != ch:
            assert s[c] == np.max(np.abs(K[:, c])) / F32(127)
            assert s[c] < s[ch] / 20
    # per-token scaling of the same matrix would mix the outlier into every row
    _, s_tok = O.quantize_int8_per_token(K)
    assert np.all(s_tok > F32(7.4) / F32(127))
    # largest element of each channel maps to the top code
    assert np.all(np.max(np.abs(codes.astype(int)), axis=1) == 127)


def test_key_example_kivi_asymmetric_int4():
    K = np.array(_golden("bea_kivi_examples.json")["key_matrix"], F32)
    codes, s, z = O.kivi_quantize_key_group(K, 4)
    # channel 3 (1-based): min 7.5, max 9.0 -> s = 1.5 / 15 = 0.1, z = 7.5
    assert s[2] == F32(1.5) / F32(15)
    assert z[2] == F32(7.5)
    assert list(codes[:, 2]) == [5, 15, 0]
    # channel 4: values 0.1, 0.2, 0.1 -> min 0.1, max 0.2 -> codes 0, 15, 0
    assert list(codes[:, 3]) == [0, 15, 0]
    assert np.all(codes <= 15)


def test_value_example_per_token():
    V = np.array(_golden("bea_kivi_examples.json")["value_matrix"], F32)
    codes, s, z = O.kivi_quantize_value_tokens(V, 4, group=4)
    assert s.shape == (3, 1) and z.shape == (3, 1)
    # each token gets its own range: [0.3, 0.6], [1.8, 2.1], [0.1, 0.3]
    np.testing.assert_array_equal(z[:, 0], F32([0.3, 1.8, 0.1]))
    np.testing.assert_allclose(s[:, 0], [0.3 / 15, 0.3 / 15, 0.2 / 15], rtol=1e-6)
    assert list(codes[0]) == [10, 0, 5, 15]
    assert list(codes[1]) == [10, 0, 15, 5]
    assert codes[2, 0] == 0 and codes[2, 3] == 15
    # per-token: scaling one token leaves the others' codes unchanged
    V2 = V.copy()
    V2[1] *= F32(64.0)
    c2, _, _ = O.kivi_quantize_value_tokens(V2, 4, group=4)
    np.testing.assert_array_equal(c2[[0, 2]], codes[[0, 2]])


def test_value_groups_split_channels():
    # two channel groups of 2: each has its own (s, z)
    v = np.array([[0.0, 3.0, 100.0, 130.0]], F32)
    codes, s, z = O.kivi_quantize_value_tokens(v, 2, group=2)
    assert list(s[0]) == [F32(1.0), F32(10.0)]
    assert list(z[0]) == [F32(0.0), F32(100.0)]
    assert list(codes[0]) == [0, 3, 0, 3]


# --- rounding mode: "Step 3" of the n4n.ai guide uses torch .round() -> half to even
def test_round_half_even_asymmetric():
    x = np.array([0.0, 15.0, 2.5, 3.5, 0.5, 14.5, 1.5], F32)[:, None]   # one channel, 7 tokens
    codes, s, z = O.kivi_quantize_key_group(x, 4)
    assert s[0] == F32(1.0) and z[0] == F32(0.0)
    assert list(codes[:, 0]) == [0, 15, 2, 4, 0, 14, 2]
    # same ties through torch's round (the routine the page calls)
    assert list(torch.round(torch.tensor([2.5, 3.5, 0.5, 14.5, 1.5])).int()) == [2, 4, 0, 14, 2]


def test_round_half_even_int8():
    x = np.array([[127.0, 62.5, -62.5, 63.5, 0.5, -0.5, 1.5]], F32)
    codes, s = O.quantize_int8_per_token(x)
    assert s[0] == F32(1.0)
    assert list(codes[0]) == [127, 62, -62, 64, 0, 0, 2]


def test_int8_range_is_symmetric_127():
    # "INT8 symmetric quantization maps values to [-127, 127]" (llms.blog, 2.)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((200, 128)).astype(F32)
    codes, s = O.quantize_int8_per_token(x)
    assert codes.min() >= -127 and codes.max() <= 127
    row_absmax = np.abs(codes.astype(int)).max(axis=1)
    assert np.all(row_absmax == 127)


# --- round-trip error bounds (integer formats: |x - xhat| <= s/2) ------------
def _fp32_slack(*mags):
    return 2.0 ** -20 * np.maximum.reduce([np.abs(np.asarray(m, np.float64)) for m in mags])


@pytest.mark.parametrize("bits", [2, 4])
def test_kivi_round_trip_bound(bits):
    rng = np.random.default_rng(bits)
    k = (rng.standard_normal((64, 128)) * np.exp(rng.standard_normal((1, 128)))).astype(F32)
    codes, s, z = O.kivi_quantize_key_group(k, bits)
    err = np.abs(O.kivi_dequantize_keys(codes, s, z) - k.astype(np.float64))
    bound = s.astype(np.float64)[None, :] / 2 + _fp32_slack(z, s)[None, :] + _fp32_slack(k)
    assert np.all(err <= bound)
    v = (rng.standard_normal((64, 128)) * np.exp(rng.standard_normal((64, 1)))).astype(F32)
    cv, sv, zv = O.kivi_quantize_value_tokens(v, bits, 32)
    errv = np.abs(O.kivi_dequantize_values(cv, sv, zv, 32) - v.astype(np.float64))
    sv_full = np.repeat(sv.astype(np.float64), 32, axis=1)
    zv_full = np.repeat(zv.astype(np.float64), 32, axis=1)
    assert np.all(errv <= sv_full / 2 + _fp32_slack(zv_full, sv_full) + _fp32_slack(v))


def test_int8_round_trip_bound():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((300, 128)) * 30).astype(F32)
    codes, s = O.quantize_int8_per_token(x)
    err = np.abs(O.dequantize_int8(codes, s) - x.astype(np.float64))
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 2.0 ** -20))


def test_fp8_round_trip_half_spacing():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((300, 128)) * np.exp(rng.standard_normal((300, 1)))).astype(F32)
    codes, s = O.quantize_fp8_per_token(x)
    xh = O.dequantize_fp8(codes, s)
    y = np.abs(x.astype(np.float64) / s.astype(np.float64)[:, None])
    # E4M3 spacing at |y|: 2**(e-3) for normals, 2**-9 below 2**-6
    e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
    half = 2.0 ** (e - 4)
    err = np.abs(xh - x.astype(np.float64)) / s.astype(np.float64)[:, None]
    assert np.all(err <= half * (1 + 2.0 ** -18) + 2.0 ** -20)
    # the row maximum reaches the top code 448 (0x7E / 0xFE)
    top = np.abs(O.e4m3_decode(codes)).max(axis=1)
    assert np.all(top == 448.0)


def test_grid_points_round_trip_exactly():
    s = F32(0.25)
    mn = F32(-3.0)
    ks = np.array([0, 3, 7, 15, 9, 1], F32)
    x = (mn + ks * s).astype(F32)[:, None]
    codes, s_, z_ = O.kivi_quantize_key_group(x, 4)
    assert s_[0] == s and z_[0] == mn
    np.testing.assert_array_equal(codes[:, 0], ks.astype(np.uint8))
    np.testing.assert_array_equal(O.kivi_dequantize_keys(codes, s_, z_)[:, 0], x[:, 0].astype(np.float64))


def test_degenerate_groups():
    c = np.full((32, 4), F32(1.25))
    codes, s, z = O.kivi_quantize_key_group(c, 4)
    assert np.all(s == 0) and np.all(codes == 0) and np.all(z == F32(1.25))
    np.testing.assert_array_equal(O.kivi_dequantize_keys(codes, s, z), c.astype(np.float64))
    zero = np.zeros((3, 16), F32)
    q8, s8 = O.quantize_int8_per_token(zero)
    qf, sf = O.quantize_fp8_per_token(zero)
    assert np.all(q8 == 0) and np.all(s8 == 0) and np.all(qf == 0) and np.all(sf == 0)
    # signed zeros are canonicalised in the stored zero-point and scale
    mixed = np.array([[-0.0], [0.0], [-0.0]], F32)
    _, s0, z0 = O.kivi_quantize_key_group(mixed, 2)
    assert not np.signbit(z0[0]) and not np.signbit(s0[0])


# --- E4M3 codec vs torch's float8_e4m3fn cast (a library routine) -----------
def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    assert O.e4m3_decode(np.uint8(0x7E)) == 448.0
    assert O.e4m3_decode(np.uint8(0x01)) == 2.0 ** -9


def _torch_e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, F32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_all_bf16_in_range_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.int16)
    vals = torch.from_numpy(bits).view(torch.bfloat16).float().numpy()
    m = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    np.testing.assert_array_equal(O.e4m3_encode(vals[m]), _torch_e4m3(vals[m]))


def test_e4m3_encode_midpoints_and_neighbours_match_torch():
    reps = O.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))     # non-negative finite codes
    reps = np.unique(reps)
    mids = ((reps[:-1] + reps[1:]) / 2).astype(F32)
    pts = [mids, np.nextafter(mids, F32(np.inf)), np.nextafter(mids, F32(-np.inf)), reps.astype(F32)]
    rng = np.random.default_rng(3)
    pts.append((rng.uniform(0, 448, 200000)).astype(F32))
    pts.append((2.0 ** rng.uniform(-14, -5, 100000)).astype(F32))
    x = np.concatenate(pts)
    x = x[np.abs(x) <= 448]
    x = np.concatenate([x, -x])
    np.testing.assert_array_equal(O.e4m3_encode(x), _torch_e4m3(x))
    # named cases: 3 * 2**-11 is the midpoint between 2**-10 and 2**-9 -> even mantissa (2**-9 has m=1... )
    assert O.e4m3_encode(np.array([3 * 2.0 ** -11], F32))[0] == _torch_e4m3(np.array([3 * 2.0 ** -11]))[0]


# --- flush rule: §3 "Residual Cache for Streaming" example ------------------
def test_residual_example_200_tokens_groups_of_64():
    ex = _golden("bea_kivi_examples.json")["residual_example"]
    n, G = ex["tokens"], ex["group"]
    lo, hi = ex["residual_tokens_1based"]
    n_resid = hi - lo + 1
    for R in range(0, n_resid + 1):
        nq = O.kivi_quantized_prefix(n, G, R)
        assert nq == ex["quantized_groups_1based"][-1][1]
        assert n - nq == n_resid
    seq = O.SequenceCache("kivi", 64, bits=4, group=G, residual=8)
    rng = np.random.default_rng(1)
    seq.append(rng.standard_normal((n, 64)).astype(F32), rng.standard_normal((n, 64)).astype(F32))
    assert seq.n_quantized == 192 and seq.resid_k.shape[0] == 8
    assert len(seq.k_codes) == 3


def test_flush_rule_workload_sizes():
    assert O.kivi_quantized_prefix(256, 32, 16) == 224      # tiny KIVI workload
    assert O.kivi_quantized_prefix(32768, 32, 128) == 32640
    assert O.kivi_quantized_prefix(100, 64, 128) == 0
    assert O.kivi_quantized_prefix(128 + 64, 64, 128) == 64


@pytest.mark.parametrize("fmt,bits,G,R", [("kivi", 4, 32, 16), ("kivi", 2, 32, 40), ("int8", 8, 0, 0),
                                          ("fp8", 8, 0, 0)])
def test_append_chunking_invariance(fmt, bits, G, R):
    rng = np.random.default_rng(11)
    k = (rng.standard_normal((257, 64)) * 3).astype(F32)
    v = rng.standard_normal((257, 64)).astype(F32)
    whole = O.SequenceCache(fmt, 64, bits, G, R)
    whole.append(k, v)
    single = O.SequenceCache(fmt, 64, bits, G, R)
    for t in range(257):
        single.append(k[t:t + 1], v[t:t + 1])
    mixed = O.SequenceCache(fmt, 64, bits, G, R)
    cuts = [0, 5, 6, 70, 71, 200, 257]
    for a, b in zip(cuts[:-1], cuts[1:]):
        mixed.append(k[a:b], v[a:b])
    for other in (single, mixed):
        Kw, Vw = whole.dequantized()
        Ko, Vo = other.dequantized()
        np.testing.assert_array_equal(Kw, Ko)
        np.testing.assert_array_equal(Vw, Vo)
        np.testing.assert_array_equal(whole.key_codes(), other.key_codes())
        np.testing.assert_array_equal(whole.value_codes(), other.value_codes())


# --- packing -----------------------------------------------------------------
def test_pack_known_bytes():
    assert list(O.pack_codes(np.array([1, 2, 3, 4], np.uint8), 4)) == [0x21, 0x43]
    assert list(O.pack_codes(np.array([1, 2, 3, 0, 3, 3, 3, 3], np.uint8), 2)) == [0x39, 0xFF]
    rng = np.random.default_rng(2)
    for bits in (2, 4):
        c = rng.integers(0, 2 ** bits, (5, 64)).astype(np.uint8)
        p = O.pack_codes(c, bits)
        assert p.shape == (5, 64 * bits // 8)
        np.testing.assert_array_equal(O.unpack_codes(p, bits), c)
        # brute force: bit j of element i sits at absolute bit bits*i + j
        for row in range(5):
            allbits = np.unpackbits(p[row], bitorder="little")
            for i in range(64):
                val = sum(int(allbits[bits * i + j]) << j for j in range(bits))
                assert val == c[row, i]


# --- attention: closed forms and a library softmax ----------------------------
def _seq_from_rows(K, V):
    """A float cache holding K, V exactly: KIVI with a residual window larger
    than the sequence keeps every token at full precision."""
    s = O.SequenceCache("kivi", K.shape[1], bits=4, group=32, residual=10 ** 6)
    s.append(K.astype(F32), V.astype(F32))
    return s


def test_attention_single_token_returns_its_value():
    rng = np.random.default_rng(4)
    K = rng.standard_normal((1, 8)).astype(F32)
    V = rng.standard_normal((1, 8)).astype(F32)
    out = O.decode_attention([_seq_from_rows(K, V)], rng.standard_normal((2, 8)), F32(0.3))
    np.testing.assert_array_equal(out, np.repeat(V.astype(np.float64), 2, axis=0))


def test_attention_zero_query_is_mean_of_values():
    rng = np.random.default_rng(5)
    K = rng.standard_normal((9, 8)).astype(F32)
    V = rng.standard_normal((9, 8)).astype(F32)
    out = O.decode_attention([_seq_from_rows(K, V)], np.zeros((1, 8)), F32(0.125))
    np.testing.assert_allclose(out[0], V.astype(np.float64).mean(axis=0), rtol=0, atol=1e-15)


def test_attention_two_tokens_log3_split_with_scale():
    # scores differ by ln 3 after the softmax scale -> weights 3/4, 1/4
    d = 4
    scale = F32(0.5)
    q = np.array([[1.0, 0, 0, 0]])
    K = np.array([[2 * math.log(3), 0, 0, 0], [0, 0, 0, 0]])
    V = np.array([[1.0, 0, 4, 8], [0, 1, 0, 8]], F32)
    seq = O.SequenceCache("kivi", d, bits=4, group=32, residual=100)
    seq.resid_k = K.astype(F32)            # the residual stores whatever precision it is given
    seq.resid_v = V
    seq.n = 2
    out = O.decode_attention([seq], q, scale)
    k_exact = np.float64(F32(2 * math.log(3)))
    w0 = 1 / (1 + math.exp(-np.float64(scale) * k_exact))
    V64 = V.astype(np.float64)
    np.testing.assert_allclose(out[0], w0 * V64[0] + (1 - w0) * V64[1], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(out[0], [0.75, 0.25, 3.0, 8.0], atol=1e-6)


def test_attention_gqa_head_mapping():
    rng = np.random.default_rng(6)
    seqs = []
    for h in range(2):
        K = rng.standard_normal((5, 8)).astype(F32)
        V = (np.ones((5, 8)) * (h + 1) * 10).astype(F32)   # each KV head's values are constant
        seqs.append(_seq_from_rows(K, V))
    out = O.decode_attention(seqs, rng.standard_normal((8, 8)), F32(0.3))
    # query heads 0..3 read KV head 0, 4..7 read KV head 1 (h // (Hq/Hkv))
    np.testing.assert_allclose(out[:4], 10.0, rtol=1e-14)
    np.testing.assert_allclose(out[4:], 20.0, rtol=1e-14)


def test_attention_matches_scipy_softmax_brute_force():
    rng = np.random.default_rng(9)
    for fmt, bits, G, R in (("kivi", 4, 32, 16), ("int8", 8, 0, 0), ("fp8", 8, 0, 0), ("kivi", 2, 32, 8)):
        hkv, hq, d, n = 2, 8, 64, 100
        seqs = [O.SequenceCache(fmt, d, bits, G, R) for _ in range(hkv)]
        raw = []
        for s in seqs:
            k = (rng.standard_normal((n, d)) * 2).astype(F32)
            v = rng.standard_normal((n, d)).astype(F32)
            s.append(k, v)
            raw.append(s.dequantized())
        q = rng.standard_normal((hq, d))
        scale = F32(1 / 8)
        out = O.decode_attention(seqs, q, scale)
        for h in range(hq):
            K, V = raw[h // (hq // hkv)]
            logits = [float(np.float64(scale) * sum(q[h, c] * K[t, c] for c in range(d))) for t in range(n)]
            w = scipy.special.softmax(logits)
            ref = np.array([sum(w[t] * V[t, c] for t in range(n)) for c in range(d)])
            np.testing.assert_allclose(out[h], ref, rtol=1e-12, atol=1e-12)


def test_attention_dominant_key():
    rng = np.random.default_rng(10)
    K = rng.standard_normal((50, 16)).astype(F32) * F32(0.01)
    K[17] = 40.0
    V = rng.standard_normal((50, 16)).astype(F32)
    out = O.decode_attention([_seq_from_rows(K, V)], np.ones((1, 16)), F32(1.0))
    np.testing.assert_allclose(out[0], V[17], atol=1e-12)


def test_kivi_dequantized_cache_orders_quantized_then_residual():
    rng = np.random.default_rng(12)
    k = rng.standard_normal((70, 32)).astype(F32)
    v = rng.standard_normal((70, 32)).astype(F32)
    s = O.SequenceCache("kivi", 32, 4, 32, 4)
    s.append(k, v)
    K, V = s.dequantized()
    assert K.shape == (70, 32)
    assert s.n_quantized == 64
    np.testing.assert_array_equal(K[64:], k[64:].astype(np.float64))   # residual untouched
    assert np.max(np.abs(K[:64] - k[:64])) < 0.5


# --- the unquantized 16-bit cache (the baseline the quantized formats save bytes against) ---
def test_round_bf16_matches_torch_cast_on_every_tie_and_neighbour():
    """round_bf16 against torch's CPU float32 -> bfloat16 cast (a library
    routine): every pattern whose low 16 bits are a tie (0x8000) or one ulp
    either side of it, over a spread of upper halves of both parities, plus
    random finite values."""
    rng = np.random.default_rng(7)
    upper = np.concatenate([np.arange(0x0000, 0x0100), np.arange(0x3F00, 0x4100),
                            rng.integers(0, 0x7F7F, 4000)]).astype(np.uint32)
    upper = np.concatenate([upper, upper | 0x8000])          # both signs
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    pats = (upper[:, None] << 16 | lows[None, :]).reshape(-1)
    pats = pats[(pats & 0x7F800000) != 0x7F800000]            # finite only
    x = pats.view(np.float32)
    x = np.concatenate([x, rng.standard_normal(20000).astype(np.float32) * 100])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.round_bf16(x), ref)


def test_round_bf16_ties_go_to_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: even is 1.0
    assert O.round_bf16(np.float32(1.0 + 2.0 ** -8)) == 0x3F80
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6: up
    assert O.round_bf16(np.float32(1.0 + 3 * 2.0 ** -8)) == 0x3F82
    assert O.round_bf16(np.float32(-0.0)) == 0x8000


def test_bf16_value_is_exact_and_bf16_cache_round_trips():
    """bf16 inputs are stored bit-unchanged and read back exactly; the 16-bit
    cache's decode attention equals attention over the bf16 values."""
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 0x7F00, (40, 64)).astype(np.uint16)
    bits |= (rng.integers(0, 2, bits.shape) << 15).astype(np.uint16)
    x = O.bf16_value(bits).astype(np.float32)
    np.testing.assert_array_equal(O.round_bf16(x), bits)
    s = O.SequenceCache("bf16", 64)
    s.append(x[:20], -x[:20])
    s.append(x[20:], -x[20:])
    K, V = s.dequantized()
    np.testing.assert_array_equal(K, x.astype(np.float64))
    np.testing.assert_array_equal(V, -x.astype(np.float64))
    assert s.n == 40 and s.key_codes().dtype == np.uint16
    q = rng.standard_normal(64)
    ref = O.attention_one_head(q, x.astype(np.float64), -x.astype(np.float64), np.float32(0.125))
    got = O.decode_attention([s], q[None, :], np.float32(0.125))[0]
    np.testing.assert_array_equal(got, ref)


def test_bf16_cache_halves_nothing_the_memory_table_says_2_bytes():
    # [BEA] §1: BF16 is the 2-byte row of the table (320 KB per token for the
    # 80-layer, 8-KV-head, d = 128 model); the bf16 cache stores exactly that
    assert O.kv_bytes_per_token(80, 8, 128, 2) == 327680


# --- group-wise symmetric INT4 (llms.blog "2. INT8 and INT4 Uniform Group-Wise Quantization") ---
def test_int4_groupwise_ties_and_closed_form():
    # max-abs 7 -> s = 1 exactly; ties round half to even
    x = np.array([[7.0, 3.5, -3.5, 2.5, 0.5, -0.5, 1.5, 0.0]], F32)
    codes, s = O.quantize_int4_groupwise(x, 8)
    assert s.shape == (1, 1) and s[0, 0] == F32(1.0)
    assert list(codes[0]) == [7, 4, -4, 2, 0, 0, 2, 0]
    # max-abs element of each group maps to +-7; the range never needs -8
    rng = np.random.default_rng(5)
    y = rng.standard_normal((300, 128)).astype(F32) * np.exp(rng.standard_normal((300, 1))).astype(F32)
    for G in (32, 64, 128):
        c, sc = O.quantize_int4_groupwise(y, G)
        assert sc.shape == (300, 128 // G)
        cg = np.abs(c.astype(int)).reshape(300, 128 // G, G)
        assert np.all(cg.max(axis=2) == 7) and c.min() >= -7
        np.testing.assert_array_equal(sc, np.max(np.abs(y.reshape(300, -1, G)), axis=2) / F32(7))


def test_int4_groupwise_isolates_outlier_channel_page_matrix():
    """The page: grouping isolates channel outliers to specific sub-vectors.
    On the worked Key matrix, one group over a token's 4 channels lets the
    outlier channel (8.0 .. 9.0) crush the small channels to code 0; groups
    of 2 keep the first two channels' resolution."""
    K = np.array(_golden("bea_kivi_examples.json")["key_matrix"], F32)
    c4, s4 = O.quantize_int4_groupwise(K, 4)
    np.testing.assert_array_equal(s4[:, 0], np.max(np.abs(K), axis=1) / F32(7))
    assert np.all(c4[:, [0, 1, 3]] == 0) and np.all(c4[:, 2] == 7)
    c2, s2 = O.quantize_int4_groupwise(K, 2)
    assert np.all(np.abs(c2[:, :2]).max(axis=1) == 7)          # small channels keep full range
    np.testing.assert_array_equal(s2[:, 0], np.max(np.abs(K[:, :2]), axis=1) / F32(7))
    # scaling the outlier group leaves the other group's codes unchanged
    K2 = K.copy()
    K2[:, 2:] *= F32(16.0)
    c2b, _ = O.quantize_int4_groupwise(K2, 2)
    np.testing.assert_array_equal(c2b[:, :2], c2[:, :2])


def test_int4_groupwise_round_trip_and_zero_groups():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((64, 128)) * 3).astype(F32)
    x[5, 32:64] = 0.0                                            # an all-zero group
    codes, s = O.quantize_int4_groupwise(x, 32)
    assert s[5, 1] == 0 and np.all(codes[5, 32:64] == 0)
    deq = O.dequantize_int4_groupwise(codes, s, 32)
    bound = np.repeat(s.astype(np.float64), 32, axis=1) / 2
    slack = 2.0 ** -20 * np.repeat(np.max(np.abs(x.reshape(64, 4, 32)), axis=2), 32, axis=1)
    assert np.all(np.abs(deq - x) <= bound + slack)
    # a sequence cache of this format appends chunk by chunk like the others
    seq = O.SequenceCache("int4", 128, 4, 32)
    seq.append(x[:10], -x[:10])
    seq.append(x[10:], -x[10:])
    K, V = seq.dequantized()
    np.testing.assert_array_equal(K, deq)
    np.testing.assert_array_equal(V, O.dequantize_int4_groupwise(*O.quantize_int4_groupwise(-x, 32), 32))


# --- static per-tensor FP8 (llms.blog "1. FP8 KV Cache": uncalibrated scale = 1.0) ---
def test_fp8_static_scale_one_saturates_and_matches_torch():
    """With scale 1.0 the code is E4M3 of the value itself: it equals torch's
    float8_e4m3fn cast (a library routine) inside the range, and values
    beyond +-448 saturate to the largest code instead of becoming NaN."""
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.standard_normal(5000) * 50, rng.standard_normal(200) * 1e-3,
                        [448.0, -448.0, 464.0 - 1e-3, 0.0]]).astype(F32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.quantize_fp8_static(x), ref)
    big = np.array([465.0, 1e4, -1e6], F32)
    np.testing.assert_array_equal(O.quantize_fp8_static(big), [0x7E, 0x7E, 0xFE])
    assert np.all(O.e4m3_decode(O.quantize_fp8_static(big)) == [448.0, 448.0, -448.0])
    # the sequence cache holds the codes and no scales
    s = O.SequenceCache("fp8s", 4)
    s.append(np.array([[1.0, 2.0, 3.0, 500.0]], F32), np.array([[0.5, -0.25, 0.0, 0.125]], F32))
    K, V = s.dequantized()
    np.testing.assert_array_equal(K, [[1.0, 2.0, 3.0, 448.0]])
    np.testing.assert_array_equal(V, [[0.5, -0.25, 0.0, 0.125]])
    assert s.k_scale == []


# --- Walsh-Hadamard rotated Keys (llms.blog "5. QuaRot and RotateKV") ---------
def test_fwht_equals_hadamard_matrix_and_is_exact_on_integers():
    for d in (2, 8, 64, 128):
        H = O.hadamard_f64(d)
        np.testing.assert_array_equal(H @ H, d * np.eye(d))          # orthogonal up to d, symmetric
        x = np.random.default_rng(d).integers(-50, 50, (7, d)).astype(F32)
        # small integers: every butterfly is exact, so the transform equals the matrix product
        np.testing.assert_array_equal(O.fwht_f32(x).astype(np.float64), x.astype(np.float64) @ H.T)
        np.testing.assert_array_equal(O.fwht_f32(O.fwht_f32(x)), d * x)
    # H_2 and H_4 written out
    np.testing.assert_array_equal(O.hadamard_f64(2), [[1, 1], [1, -1]])
    np.testing.assert_array_equal(O.hadamard_f64(4)[3], [1, -1, -1, 1])


def test_fwht_float_rounding_and_inner_products():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 128)).astype(F32)
    y = O.fwht_f32(x).astype(np.float64)
    ref = x.astype(np.float64) @ O.hadamard_f64(128).T
    assert np.max(np.abs(y - ref)) <= 7 * 2.0 ** -23 * np.max(np.abs(ref)) * 8
    # the rotation keeps inner products: (H q) . (H k) / d = q . k
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    H = O.hadamard_f64(128)
    assert abs((H @ q) @ (H @ k) / 128 - q @ k) < 1e-10


def test_rotation_spreads_an_outlier_channel():
    """The page: rotating spreads concentrated outlier energy over all
    dimensions. A one-hot row becomes flat; Keys with one outlier channel
    quantize per token to 4 bits with a smaller error after rotation."""
    e = np.zeros(64, F32)
    e[3] = 1.0
    np.testing.assert_array_equal(np.abs(O.fwht_f32(e)), np.ones(64, F32))
    rng = np.random.default_rng(8)
    K = rng.standard_normal((256, 128)).astype(F32)
    K[:, 5] *= 20
    plain = O.SequenceCache("int4", 128, 4, 128)
    rot = O.SequenceCache("int4h", 128, 4, 128)
    for s in (plain, rot):
        s.append(K, K)
    err_plain = np.linalg.norm(plain.dequantized()[0] - K) / np.linalg.norm(K)
    err_rot = np.linalg.norm(rot.dequantized()[0] - K) / np.linalg.norm(K)
    assert err_rot < 0.6 * err_plain
    # values are not rotated: both caches hold the same Value codes
    np.testing.assert_array_equal(plain.value_codes(), rot.value_codes())


# --- KIVI with half-precision scales and zero-points -------------------------
def test_kivi_f16_metadata_page_example_and_rounding():
    """The worked Key matrix (G = 3 tokens, INT4): channel 3's s = 0.1 is
    stored as the float16 nearest to it (numpy's float16 cast, a library
    routine), z = 7.5 is exact in float16, and the codes are taken against
    the stored values: 8.0 -> 5, 9.0 -> 15, 7.5 -> 0."""
    K = np.array(_golden("bea_kivi_examples.json")["key_matrix"], F32)
    codes, s16, z16 = O.asym_quantize_f16meta(K, 4, axis=0)
    assert s16.dtype == np.float16 and z16.dtype == np.float16
    assert s16[0, 2] == np.float16(F32(1.5) / F32(15)) and float(s16[0, 2]) != 0.1
    assert z16[0, 2] == np.float16(7.5)
    assert list(codes[:, 2]) == [5, 15, 0]
    # codes use the stored scale: a value exactly on the float16 grid round-trips
    x = np.array([[0.0], [15 * float(np.float16(0.3))], [3 * float(np.float16(0.3))]], F32)
    c, s, z = O.asym_quantize_f16meta(x, 4, axis=0)
    assert s[0, 0] == np.float16(0.3) and z[0, 0] == 0 and list(c[:, 0]) == [0, 15, 3]


def test_kivi_f16_metadata_round_trip_bound():
    rng = np.random.default_rng(13)
    for bits in (2, 4):
        x = (rng.standard_normal((64, 128)) * 4).astype(F32)
        c, s16, z16 = O.asym_quantize_f16meta(x, bits, axis=0)
        s, z = s16.astype(np.float64), z16.astype(np.float64)
        deq = c.astype(np.float64) * s + z
        mn = x.min(axis=0, keepdims=True).astype(np.float64)
        # within half a (stored) step, plus the zero-point's float16 rounding
        # at the bottom of the range, plus the top code's reach
        slack = np.abs(z - mn) + (2 ** bits - 1) * np.abs(s - (x.max(axis=0) - x.min(axis=0)) / (2 ** bits - 1))
        assert np.all(np.abs(deq - x) <= s / 2 + slack + 1e-6 * np.abs(x))
    # a sequence cache of this format flushes like plain KIVI, and its
    # stored metadata are float16
    seq = O.SequenceCache("kivi16", 64, 4, 32, 16)
    k = rng.standard_normal((100, 64)).astype(F32)
    seq.append(k[:50], k[:50])
    seq.append(k[50:], k[50:])
    assert seq.n_quantized == 64 and seq.k_scale[0].dtype == np.float16
    K, _ = seq.dequantized()
    np.testing.assert_array_equal(K[64:], k[64:].astype(np.float64))
