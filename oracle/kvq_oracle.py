"""CPU oracle for the quantized KV cache: plain, slow, obviously correct.

TEST INFRASTRUCTURE ONLY. The only code allowed to import this module is
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py``. The product (``quantized_kv_cache_06_amd``, ``libkvq``) never
imports, links or calls it, and it shares no code, tables or constants with
the HIP path. It takes inputs as numpy arrays and returns numpy arrays.

What it computes, and where the pages say so
---------------------------------------------
Sources (cited by title and section):

* [BEA]  "KV Cache Quantization", infra.bea.ai inference guide:
         §1 "The Memory Savings" (table), §3 "KIVI: Asymmetric Key/Value
         Quantization" (Key per-channel, Value per-token, "Residual Cache for
         Streaming"), §4 "FP8 KV Cache" (per-token scale from max-abs).
* [LLMS] "KV Cache Quantization in Production LLM Serving: Comparing FP8, INT8,
         INT4, KIVI, and KVQuant", llms.blog: intro (memory-per-token formula),
         "1. FP8 KV Cache (E4M3 vs. E5M2)", "2. INT8 and INT4 Uniform
         Group-Wise Quantization", "3. KIVI".
* [N4N]  "How KV cache quantization reduces GPU memory", n4n.ai blog:
         "Step 3: Implement quantization hooks" (x/scale, round half-to-even,
         clamp; (v - v_min)/v_scale for the asymmetric case; append/get).

Precision. Quantization follows fp32 formulas (numpy float32 arithmetic is
IEEE single precision with round-to-nearest-even and no fused multiply-add);
dequantized values and attention are evaluated in float64.

Readings where the pages are silent (each is also listed in the design notes):

* Asymmetric zero-point is the float minimum z = min (dequant q*s + z), not
  the integer round(-min/s) of [N4N] Step 3, so that the round-trip error
  stays within s/2.
* One group size G serves both tensors: G tokens per Key group (per channel),
  G channels per Value group (per token).
* Flush rule: after appending, a sequence of n tokens holds its first
  n_q = G * floor(max(n - R, 0) / G) tokens quantized and the rest in the
  full-precision residual window (whole groups only, and only tokens older
  than the R most recent). Keys and Values share this boundary.
* Degenerate groups (max == min, or an all-zero token) get scale 0 and
  codes 0. Signed zeros are canonicalised (+0.0 added) in scales and zeros.
* INT8 codes are clamped to [-127, 127]; FP8 inputs to the encoder are
  clamped to [-448, 448] before rounding.
* Decode attention: one query token per sequence attends to all n cached
  tokens; query head h reads KV head h // (Hq / Hkv); the softmax scale is an
  explicit float32 (1/sqrt(d) by default).

Pinned by ``tests/test_oracle_pins.py`` against the pages' worked examples and
printed numbers, closed forms, library routines (torch's float8_e4m3fn cast,
scipy's softmax) and brute force. Every public function below has a pin.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64


# ---------------------------------------------------------------------------
# Memory arithmetic  [BEA §1 table; LLMS intro "Memory per Token" formula]
# ---------------------------------------------------------------------------
def kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int,
                       bytes_per_element: float) -> float:
    """Bytes of K plus V for one token over all layers and KV heads.

    [LLMS intro] writes it for 16-bit caches as 2 x 2 x n_layers x n_kv_heads
    x d_head (one factor 2 for K and V, one for two bytes per element);
    [BEA §1] tabulates 2, 1 and 0.5 bytes per element.
    """
    return 2 * n_layers * n_kv_heads * head_dim * bytes_per_element


# ---------------------------------------------------------------------------
# OCP FP8 E4M3 codec  [LLMS "1. FP8 KV Cache": 1 sign, 4 exponent, 3 mantissa]
# ---------------------------------------------------------------------------
E4M3_BIAS = 7
E4M3_MAX = 448.0          # 1.75 * 2**8, code 0x7E; 0x7F/0xFF are NaN, no inf


def e4m3_decode(code) -> np.ndarray:
    """Value (float64) of each E4M3 byte: normals (1 + m/8) * 2**(e - 7),
    subnormals (e == 0) m * 2**-9, exponent-and-mantissa all ones is NaN."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** (1 - E4M3_BIAS - 3),
                   (1.0 + m / 8.0) * np.exp2((e - E4M3_BIAS).astype(F64)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def e4m3_encode(y) -> np.ndarray:
    """Round float32 values in [-448, 448] to the nearest E4M3 code, ties to
    even mantissa. The sign bit is kept (a negative value that rounds to zero
    gives 0x80). Callers clamp to +-448 first; out-of-range input raises."""
    y = np.asarray(y, dtype=F32).astype(F64)        # exact widening
    if np.any(np.isnan(y)) or np.any(np.abs(y) > E4M3_MAX):
        raise ValueError("e4m3_encode expects finite values within +-448")
    sign = np.signbit(y).astype(np.int64)
    a = np.abs(y)
    codes = np.zeros(a.shape, dtype=np.int64)

    # Subnormal range a < 2**-6: value m * 2**-9 with m in 0..8 (m == 8 is the
    # smallest normal 2**-6, whose code is also 8). Scaling by 2**9 is exact.
    sub = a < 2.0 ** -6
    codes[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)

    # Normal range: a = (1 + f) * 2**e with f in [0, 1); keep 3 mantissa bits.
    nrm = ~sub
    if np.any(nrm):
        frac, exp2 = np.frexp(a[nrm])              # a = frac * 2**exp2, frac in [0.5, 1)
        e = exp2.astype(np.int64) - 1
        m = np.rint((frac * 2.0 - 1.0) * 8.0).astype(np.int64)   # exact product, RNE
        carry = m == 8
        e = np.where(carry, e + 1, e)
        m = np.where(carry, 0, m)
        codes[nrm] = ((e + E4M3_BIAS) << 3) | m
    return ((sign << 7) | codes).astype(np.uint8)


# ---------------------------------------------------------------------------
# Per-token symmetric formats  [BEA §4: scale from max-abs, stored alongside;
# LLMS "2. INT8": symmetric, [-127, 127]; N4N Step 3: x / scale, round, clamp]
# ---------------------------------------------------------------------------
def quantize_int8_per_token(x):
    """x: float32 [..., d]. One scale per row: s = max|x| / 127; code =
    clamp(round_half_even(x / s), -127, 127); a zero row gets s = 0, codes 0."""
    x = np.asarray(x, dtype=F32)
    a = np.max(np.abs(x), axis=-1)
    s = (a / F32(127.0)) + F32(0.0)
    pos = s > 0
    div = np.where(pos, s, F32(1.0))[..., None]
    q = np.rint(x / div)
    q = np.where(pos[..., None], np.clip(q, F32(-127.0), F32(127.0)), F32(0.0))
    return q.astype(np.int8), s.astype(F32)


def quantize_fp8_per_token(x):
    """x: float32 [..., d]. One scale per row: s = max|x| / 448; code =
    E4M3(clamp(x / s, -448, 448)); a zero row gets s = 0 and y = 0."""
    x = np.asarray(x, dtype=F32)
    a = np.max(np.abs(x), axis=-1)
    s = (a / F32(E4M3_MAX)) + F32(0.0)
    pos = s > 0
    div = np.where(pos, s, F32(1.0))[..., None]
    y = np.where(pos[..., None], x / div, F32(0.0))
    y = np.clip(y, F32(-E4M3_MAX), F32(E4M3_MAX))
    return e4m3_encode(y), s.astype(F32)


# ---------------------------------------------------------------------------
# Unquantized 16-bit cache  [BEA §1 table: BF16 at 2 bytes per element, the
# baseline the quantized formats are measured against; LLMS intro: the
# 16-bit memory-per-token formula]
# ---------------------------------------------------------------------------
def round_bf16(x) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float32 values, rounded to nearest,
    ties to even: bfloat16 keeps the upper 16 bits of the binary32 pattern,
    so the lower 16 bits decide the rounding (below half: truncate, above:
    round up, exactly half: round to the even upper part). Finite inputs."""
    u = np.asarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    upper, lower = u >> np.uint64(16), u & np.uint64(0xFFFF)
    up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & np.uint64(1)) == 1))
    return (upper + up.astype(np.uint64)).astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """Value (float64) of bfloat16 bit patterns: the pattern shifted into the
    upper half of a binary32, widened exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(F32).astype(F64)


# ---------------------------------------------------------------------------
# Group-wise symmetric INT4  [LLMS "2. INT8 and INT4 Uniform Group-Wise
# Quantization": 4-bit codes in groups of 32, 64 or 128 elements along the
# channel dimension, one scale per group, symmetric like the INT8 entry of the
# same section]
# ---------------------------------------------------------------------------
def quantize_int4_groupwise(x, group: int):
    """x: float32 [T, d]. Per token and per group of ``group`` consecutive
    channels: s = max|x| / 7; code = clamp(round_half_even(x / s), -8, 7)
    (the codes stay within [-7, 7] since s is the group's max-abs over 7); a
    zero group gets s = 0 and codes 0. Returns codes int8 [T, d] and s
    float32 [T, d/group]."""
    x = np.asarray(x, dtype=F32)
    t, d = x.shape
    if group <= 0 or d % group:
        raise ValueError("channel groups must divide head_dim")
    xg = x.reshape(t, d // group, group)
    a = np.max(np.abs(xg), axis=2)
    s = (a / F32(7.0)) + F32(0.0)
    pos = s > 0
    div = np.where(pos, s, F32(1.0))[..., None]
    q = np.rint(xg / div)
    q = np.where(pos[..., None], np.clip(q, F32(-8.0), F32(7.0)), F32(0.0))
    return q.reshape(t, d).astype(np.int8), s.astype(F32)


def dequantize_int4_groupwise(codes, s, group: int):
    """codes [T, d] with per-token-group s [T, d/group] -> float64 [T, d]."""
    return np.asarray(codes, F64) * np.repeat(np.asarray(s, F64), group, axis=1)


def quantize_fp8_static(x):
    """Per-tensor FP8 without calibration [LLMS "1. FP8 KV Cache": scaling
    strategies, per-tensor uncalibrated scale = 1.0]: code = E4M3(clamp(x,
    -448, 448)); values beyond the E4M3 range saturate. No scale is stored."""
    x = np.asarray(x, dtype=F32)
    return e4m3_encode(np.clip(x, F32(-E4M3_MAX), F32(E4M3_MAX)))


# ---------------------------------------------------------------------------
# Walsh-Hadamard rotation of the Keys  [LLMS "5. QuaRot and RotateKV:
# Orthogonal Hadamard Dispersal": orthogonal Walsh-Hadamard rotations keep
# inner products, spread outlier energy over all dimensions so that uniform
# 4-bit codes suffice, and run online as fast transforms inside the kernels]
# ---------------------------------------------------------------------------
def fwht_f32(x) -> np.ndarray:
    """Unnormalized fast Walsh-Hadamard transform along the last axis
    (length a power of two) in float32: stages h = 1, 2, 4, ...; in each,
    every pair (i, i + h) with bit h of i clear becomes (a + b, a - b). The
    result is H x with H the Sylvester Hadamard matrix (entries +-1,
    H H = d I). Each output of a stage is one float32 add or subtract of the
    same two inputs, whatever the order the pairs are visited in."""
    y = np.array(x, dtype=F32, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("length must be a power of two")
    h = 1
    while h < d:
        z = y.reshape(*y.shape[:-1], d // (2 * h), 2, h)
        a, b = z[..., 0, :].copy(), z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(*y.shape[:-1], d)
        h *= 2
    return y


def hadamard_f64(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_d (+-1 entries), float64, by its closed
    form: entry (i, j) is (-1)^(popcount(i & j))."""
    i = np.arange(d)
    bits = np.bitwise_and(i[:, None], i[None, :])
    pop = np.zeros_like(bits)
    for k in range(int(np.log2(d)) + 1):
        pop += (bits >> k) & 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def dequantize_int8(codes, s):
    return np.asarray(codes, F64) * np.asarray(s, F64)[..., None]


def dequantize_fp8(codes, s):
    return e4m3_decode(codes) * np.asarray(s, F64)[..., None]


# ---------------------------------------------------------------------------
# KIVI asymmetric min/max quantization  [BEA §3; LLMS "3. KIVI";
# N4N Step 3 value path: (v - v_min) / v_scale, round, clamp to [0, 2^b - 1]]
# ---------------------------------------------------------------------------
def asym_quantize(x, bits: int, axis: int):
    """Asymmetric uniform quantization of float32 ``x`` along ``axis``.

    mn, mx = min, max along axis; s = (mx - mn) / (2^b - 1); z = mn;
    code = clamp(round_half_even((x - mn) / s), 0, 2^b - 1), and code 0
    where s == 0. Returns (codes uint8, s float32, z float32) with s and z
    keeping ``axis`` as a length-1 dimension."""
    x = np.asarray(x, dtype=F32)
    levels = F32(2 ** bits - 1)
    mn = np.min(x, axis=axis, keepdims=True)
    mx = np.max(x, axis=axis, keepdims=True)
    s = ((mx - mn) / levels) + F32(0.0)
    z = mn + F32(0.0)
    pos = s > 0
    div = np.where(pos, s, F32(1.0))
    q = np.rint((x - mn) / div)
    q = np.where(pos, np.clip(q, F32(0.0), levels), F32(0.0))
    return q.astype(np.uint8), s.astype(F32), z.astype(F32)


def asym_quantize_f16meta(x, bits: int, axis: int):
    """asym_quantize with half-precision metadata: s and z are computed as
    there in float32, rounded to float16 (to nearest even), and the codes are
    taken against the rounded values, clamp(round_half_even((x - z16) /
    s16), 0, 2^b - 1) in float32 (code 0 where s16 == 0), so that
    dequantization code * s16 + z16 uses exactly what is stored. Returns
    (codes uint8, s16 float16, z16 float16)."""
    x = np.asarray(x, dtype=F32)
    levels = F32(2 ** bits - 1)
    mn = np.min(x, axis=axis, keepdims=True)
    mx = np.max(x, axis=axis, keepdims=True)
    s16 = (((mx - mn) / levels) + F32(0.0)).astype(np.float16)
    z16 = (mn + F32(0.0)).astype(np.float16) + np.float16(0.0)
    s = s16.astype(F32)
    z = z16.astype(F32)
    pos = s > 0
    div = np.where(pos, s, F32(1.0))
    q = np.rint((x - z) / div)
    q = np.where(pos, np.clip(q, F32(0.0), levels), F32(0.0))
    return q.astype(np.uint8), s16, z16


def kivi_quantize_key_group(k_group, bits: int):
    """Key: per-channel [BEA §3 "Key: Per-Channel Quantization"]. k_group is
    [G tokens, d]; statistics run over the G tokens of each channel.
    Returns codes [G, d], s [d], z [d]."""
    q, s, z = asym_quantize(k_group, bits, axis=0)
    return q, s[0], z[0]


def kivi_quantize_value_tokens(v_tokens, bits: int, group: int):
    """Value: per-token [BEA §3 "Value: Per-Token Quantization"], in groups of
    ``group`` consecutive channels. v_tokens is [T, d].
    Returns codes [T, d], s [T, d/group], z [T, d/group]."""
    v = np.asarray(v_tokens, dtype=F32)
    t, d = v.shape
    if group <= 0 or d % group:
        raise ValueError("value channel groups must divide head_dim")
    q, s, z = asym_quantize(v.reshape(t, d // group, group), bits, axis=2)
    return q.reshape(t, d), s[..., 0], z[..., 0]


def kivi_dequantize_keys(codes, s, z):
    """codes [G, d] with per-channel s, z [d] -> float64 [G, d]."""
    return np.asarray(codes, F64) * np.asarray(s, F64)[None, :] + np.asarray(z, F64)[None, :]


def kivi_dequantize_values(codes, s, z, group: int):
    """codes [T, d] with per-token-group s, z [T, d/group] -> float64 [T, d]."""
    c = np.asarray(codes, F64)
    t, d = c.shape
    sc = np.repeat(np.asarray(s, F64), group, axis=1)
    zz = np.repeat(np.asarray(z, F64), group, axis=1)
    return c * sc + zz


def kivi_quantized_prefix(n: int, group: int, residual: int) -> int:
    """Tokens of a length-n sequence that sit in quantized groups:
    G * floor(max(n - R, 0) / G). [BEA §3 "Residual Cache for Streaming":
    recent tokens stay full precision until a whole group can be formed;
    LLMS "3. KIVI": tokens are quantized when they leave the window of the
    most recent R.]"""
    return group * (max(n - residual, 0) // group)


# ---------------------------------------------------------------------------
# Bit packing  [LLMS "3. KIVI": quantized and packed into memory blocks]
# ---------------------------------------------------------------------------
def pack_codes(codes, bits: int) -> np.ndarray:
    """Pack unsigned codes (< 2**bits) along the last axis, 8/bits per byte,
    element i of each byte's run in bits [bits*i, bits*(i+1)) (low bits first)."""
    c = np.asarray(codes, dtype=np.uint8)
    per = 8 // bits
    c = c.reshape(*c.shape[:-1], c.shape[-1] // per, per)
    out = np.zeros(c.shape[:-1], dtype=np.uint8)
    for i in range(per):
        out |= (c[..., i] << (bits * i)).astype(np.uint8)
    return out


def unpack_codes(packed, bits: int) -> np.ndarray:
    """Inverse of pack_codes."""
    p = np.asarray(packed, dtype=np.uint8)
    per = 8 // bits
    mask = (1 << bits) - 1
    parts = [(p >> (bits * i)) & mask for i in range(per)]
    return np.stack(parts, axis=-1).reshape(*p.shape[:-1], p.shape[-1] * per).astype(np.uint8)


# ---------------------------------------------------------------------------
# One (batch, KV head) stream of the cache: append and dequantized view
# [N4N Step 3 "append(layer_idx, k, v)" / "get(layer_idx)"]
# ---------------------------------------------------------------------------
class SequenceCache:
    """State of one sequence's cache for one KV head.

    fmt: "fp8", "fp8s" (FP8 with the static scale 1.0), "int8", "kivi",
    "kivi16" (kivi with float16 scales and zero-points, asym_quantize_f16meta),
    "int4h" (int4 whose Keys are stored rotated: the float32 FWHT of each
    Key row is what is quantized; dequantized() rotates them back, H x / d in
    float64, so attention sees the original coordinates),
    "int4" (group-wise symmetric, ``group``
    channels per scale, Key and Value alike) or "bf16" (the unquantized
    16-bit cache: codes are the bfloat16 patterns of the inputs, no scales). Inputs are
    float32 rows (bf16 inputs are widened exactly by the caller). For KIVI,
    flushed groups are kept as lists of arrays, the residual as float32 rows
    in arrival order.
    """

    def __init__(self, fmt: str, head_dim: int, bits: int = 8, group: int = 0,
                 residual: int = 0):
        if fmt not in ("fp8", "fp8s", "int8", "kivi", "kivi16", "int4", "int4h", "bf16"):
            raise ValueError(fmt)
        self.fmt, self.d, self.bits, self.group, self.residual = fmt, head_dim, bits, group, residual
        self.n = 0
        # per-token formats: lists of [T, d] codes and [T] scales
        self.k_codes, self.k_scale, self.v_codes, self.v_scale = [], [], [], []
        # KIVI
        self.k_zero, self.v_zero = [], []
        self.resid_k = np.zeros((0, head_dim), F32)
        self.resid_v = np.zeros((0, head_dim), F32)

    # -- append -----------------------------------------------------------
    def append(self, k, v):
        """k, v: float32 [T, d] new tokens, oldest first."""
        k = np.asarray(k, F32).reshape(-1, self.d)
        v = np.asarray(v, F32).reshape(-1, self.d)
        if k.shape[0] == 0:
            return
        if self.fmt == "int8":
            for x, codes, scales in ((k, self.k_codes, self.k_scale), (v, self.v_codes, self.v_scale)):
                q, s = quantize_int8_per_token(x)
                codes.append(q)
                scales.append(s)
        elif self.fmt == "fp8s":
            self.k_codes.append(quantize_fp8_static(k))
            self.v_codes.append(quantize_fp8_static(v))
        elif self.fmt in ("int4", "int4h"):
            if self.fmt == "int4h":
                k = fwht_f32(k)
            for x, codes, scales in ((k, self.k_codes, self.k_scale), (v, self.v_codes, self.v_scale)):
                q, s = quantize_int4_groupwise(x, self.group)
                codes.append(q)
                scales.append(s)
        elif self.fmt == "bf16":
            self.k_codes.append(round_bf16(k))
            self.v_codes.append(round_bf16(v))
        elif self.fmt == "fp8":
            for x, codes, scales in ((k, self.k_codes, self.k_scale), (v, self.v_codes, self.v_scale)):
                q, s = quantize_fp8_per_token(x)
                codes.append(q)
                scales.append(s)
        else:
            # New tokens enter the full-precision residual window; every whole
            # group of G tokens that is older than the R most recent leaves it,
            # oldest first, and is quantized (Key per channel, Value per token).
            self.resid_k = np.concatenate([self.resid_k, k])
            self.resid_v = np.concatenate([self.resid_v, v])
            G, R = self.group, self.residual
            while self.resid_k.shape[0] - R >= G:
                kg, self.resid_k = self.resid_k[:G], self.resid_k[G:]
                vg, self.resid_v = self.resid_v[:G], self.resid_v[G:]
                if self.fmt == "kivi16":
                    qk, sk, zk = asym_quantize_f16meta(kg, self.bits, axis=0)
                    qk, sk, zk = qk, sk[0], zk[0]
                    qv3, sv, zv = asym_quantize_f16meta(vg.reshape(G, self.d // G, G), self.bits, axis=2)
                    qv, sv, zv = qv3.reshape(G, self.d), sv[..., 0], zv[..., 0]
                else:
                    qk, sk, zk = kivi_quantize_key_group(kg, self.bits)
                    qv, sv, zv = kivi_quantize_value_tokens(vg, self.bits, G)
                self.k_codes.append(qk)
                self.k_scale.append(sk)
                self.k_zero.append(zk)
                self.v_codes.append(qv)
                self.v_scale.append(sv)
                self.v_zero.append(zv)
        self.n += k.shape[0]

    # -- views --------------------------------------------------------------
    @property
    def n_quantized(self) -> int:
        if self.fmt in ("kivi", "kivi16"):
            return len(self.k_codes) * self.group
        return self.n

    def key_codes(self):
        dt = np.uint16 if self.fmt == "bf16" else np.uint8
        return np.concatenate(self.k_codes) if self.k_codes else np.zeros((0, self.d), dt)

    def value_codes(self):
        dt = np.uint16 if self.fmt == "bf16" else np.uint8
        return np.concatenate(self.v_codes) if self.v_codes else np.zeros((0, self.d), dt)

    def dequantized(self):
        """(K, V) as float64 [n, d]: quantized tokens first, then the residual
        window as stored."""
        d = self.d
        if self.fmt in ("kivi", "kivi16"):
            ks = [kivi_dequantize_keys(c, s, z) for c, s, z in zip(self.k_codes, self.k_scale, self.k_zero)]
            vs = [kivi_dequantize_values(c, s, z, self.group)
                  for c, s, z in zip(self.v_codes, self.v_scale, self.v_zero)]
            ks.append(self.resid_k.astype(F64))
            vs.append(self.resid_v.astype(F64))
        elif self.fmt == "fp8s":
            ks = [e4m3_decode(c) for c in self.k_codes]
            vs = [e4m3_decode(c) for c in self.v_codes]
        elif self.fmt in ("int4", "int4h"):
            ks = [dequantize_int4_groupwise(c, s, self.group) for c, s in zip(self.k_codes, self.k_scale)]
            if self.fmt == "int4h":
                # back to the original coordinates: H (H k) = d k
                H = hadamard_f64(d)
                ks = [kr @ H / d for kr in ks]
            vs = [dequantize_int4_groupwise(c, s, self.group) for c, s in zip(self.v_codes, self.v_scale)]
        elif self.fmt == "bf16":
            ks = [bf16_value(c) for c in self.k_codes]
            vs = [bf16_value(c) for c in self.v_codes]
        else:
            deq = dequantize_int8 if self.fmt == "int8" else dequantize_fp8
            ks = [deq(c, s) for c, s in zip(self.k_codes, self.k_scale)]
            vs = [deq(c, s) for c, s in zip(self.v_codes, self.v_scale)]
        K = np.concatenate(ks) if ks else np.zeros((0, d))
        V = np.concatenate(vs) if vs else np.zeros((0, d))
        return K, V


# ---------------------------------------------------------------------------
# Decode attention over the dequantized cache (float64)
# [LLMS / dupenodi: attention reads the low-precision cache; decode attends
#  one new query token to every cached token]
# ---------------------------------------------------------------------------
def attention_one_head(q, K, V, sm_scale) -> np.ndarray:
    """softmax(sm_scale * K q) weighted sum of V rows, in float64.
    q [d], K [n, d], V [n, d]. An empty cache gives zeros."""
    q = np.asarray(q, F64)
    if K.shape[0] == 0:
        return np.zeros(q.shape[-1], F64)
    scores = F64(np.float32(sm_scale)) * (K @ q)
    w = np.exp(scores - scores.max())
    w /= w.sum()
    return w @ V


def decode_attention(seqs_b, q_b, sm_scale) -> np.ndarray:
    """One sequence: seqs_b is the list of Hkv SequenceCache objects, q_b the
    [Hq, d] query. Query head h reads KV head h // (Hq / Hkv).
    Returns float64 [Hq, d]."""
    q_b = np.asarray(q_b, F64)
    hq, d = q_b.shape
    hkv = len(seqs_b)
    g = hq // hkv
    out = np.zeros((hq, d), F64)
    views = [s.dequantized() for s in seqs_b]
    for h in range(hq):
        K, V = views[h // g]
        out[h] = attention_one_head(q_b[h], K, V, sm_scale)
    return out


def default_sm_scale(head_dim: int) -> np.float32:
    return np.float32(1.0 / np.sqrt(head_dim))
