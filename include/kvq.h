/*
 * libkvq — quantized KV cache for AMD MI355X (gfx950): append-time
 * quantization and single-token decode attention over the quantized cache.
 *
 * Sources of the operations (cited by page title and section):
 *   [BEA]  "KV Cache Quantization", infra.bea.ai inference guide — §3 "KIVI:
 *          Asymmetric Key/Value Quantization" (Key per-channel, Value
 *          per-token, "Residual Cache for Streaming"), §4 "FP8 KV Cache"
 *          (per-token scale from the maximum absolute value, stored beside
 *          the data).
 *   [LLMS] "KV Cache Quantization in Production LLM Serving: Comparing FP8,
 *          INT8, INT4, KIVI, and KVQuant", llms.blog — "1. FP8 KV Cache"
 *          (OCP E4M3), "2. INT8 and INT4 Uniform Group-Wise Quantization"
 *          (symmetric INT8 in [-127, 127]), "3. KIVI" (residual window,
 *          quantize and pack tokens leaving it), "Serving Economics"
 *          (decode is bandwidth bound).
 *   [N4N]  "How KV cache quantization reduces GPU memory", n4n.ai blog —
 *          "Step 3: Implement quantization hooks" (append(layer, k, v) with
 *          k, v shaped [batch, heads, seq, head_dim]; get(layer) before the
 *          attention scores), "Step 5" (the dequantize must fuse with the
 *          attention kernel).
 *   [DUP]  "KV cache quantization", guide.dupenodi.dev — "Key takeaways":
 *          the attention kernel must read the quantized cache.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Return value: a kvq_status (0 = KVQ_OK). Argument checks happen on the
 *    host before any HIP call; a failed check launches nothing and changes
 *    nothing. KVQ_ERR_HIP reports a failed kernel launch. No C++ exception
 *    crosses this interface.
 *  - Memory: every buffer is owned by the caller. Pointers named "device"
 *    point to GPU memory of the current device and must be 16-byte aligned.
 *    The library allocates nothing. Its only global state is the fixed
 *    device workspace of kvq_append_decode_noalloc (one array of
 *    KVQ_STATIC_WORKSPACE_BYTES per device, held until the process ends).
 *  - Streams: `stream` is a hipStream_t (NULL = the default stream). Calls
 *    are asynchronous and ordered on that stream; none synchronizes.
 *  - One cache buffer holds one layer (the `layer_idx` of [N4N] Step 3 is
 *    the caller's choice of buffer). A buffer with all seq_lens == 0 is an
 *    empty cache whatever bytes it holds (zero-filling it is customary, not
 *    required): codes, scales and zero-points stored at positions at or
 *    beyond a sequence's length may be loaded with the last, partial tile of
 *    a sequence, but they are masked and never change a result.
 *
 * Numerics
 * --------
 *  Quantization is evaluated in fp32 with IEEE round-to-nearest-even, true
 *  division and no fused multiply-add, so codes, scales and zero-points are
 *  reproducible bit for bit:
 *   FP8 E4M3 per token ([BEA] §4, [LLMS] 1.): a = max|x| over head_dim,
 *     s = a / 448, code = E4M3_rne(clamp(x / s, -448, 448)); s == 0 -> code 0.
 *   INT8 symmetric per token ([LLMS] 2.): s = a / 127,
 *     code = clamp(rint(x / s), -127, 127); s == 0 -> code 0.
 *   KIVI ([BEA] §3, [LLMS] 3.): Key per channel over a group of G tokens,
 *     Value per token over groups of G channels; mn, mx = min, max,
 *     s = (mx - mn) / (2^bits - 1), z = mn, code = clamp(rint((x - mn) / s),
 *     0, 2^bits - 1); s == 0 -> code 0. Signed zeros in s and z become +0.
 *     A sequence of n tokens keeps its first n_q = G * floor(max(n - R, 0) / G)
 *     tokens quantized and tokens [n_q, n) bit-unchanged in a residual ring.
 *  Dequantized value: code * s (FP8, INT8) or code * s + z (KIVI). The
 *  further formats (group-wise INT4, its Hadamard-rotated variant, KIVI with
 *  binary16 metadata, static-scale FP8 and the bf16 baseline) are defined
 *  with kvq_config below.
 *  Attention is fp32 with an online softmax: for query head h of sequence
 *  b, kv = h / (n_q_heads / n_kv_heads),
 *    out[b,h,:] = sum_t softmax_t(sm_scale * <q[b,h,:], K^[b,kv,t,:]>) V^[b,kv,t,:]
 *  over all seq_lens[b] cached tokens. An empty sequence gives zeros.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_INVALID = 1,     /* null pointer, bad size, inconsistent config   */
  KVQ_ERR_UNSUPPORTED = 2, /* well-formed request outside what is built      */
  KVQ_ERR_WORKSPACE = 3,   /* decode workspace smaller than required         */
  KVQ_ERR_HIP = 4          /* HIP reported an error when launching a kernel  */
} kvq_status;

typedef enum kvq_format {
  KVQ_FMT_FP8_E4M3 = 1,    /* per-token OCP FP8 E4M3, fp32 scale per token   */
  KVQ_FMT_INT8 = 2,        /* per-token symmetric INT8, fp32 scale per token */
  KVQ_FMT_KIVI = 3,        /* KIVI asymmetric INT4/INT2 + residual window    */
  KVQ_FMT_BF16 = 4,        /* unquantized bfloat16 cache (the 16-bit baseline) */
  KVQ_FMT_INT4 = 5,        /* group-wise symmetric INT4, per token, fp32 scale per group */
  KVQ_FMT_FP8_STATIC = 6,  /* OCP FP8 E4M3 with the static per-tensor scale 1.0      */
  KVQ_FMT_INT4_HADAMARD = 7, /* KVQ_FMT_INT4 with Walsh-Hadamard rotated Keys         */
  KVQ_FMT_KIVI_F16 = 8     /* KIVI with fp16 scales and zero-points             */
} kvq_format;

typedef enum kvq_dtype {
  KVQ_DT_F32 = 0,          /* IEEE binary32                                  */
  KVQ_DT_BF16 = 1          /* bfloat16                                       */
} kvq_dtype;

/* Shape and format of one layer's cache. Supported: head_dim 64 or 128;
 * n_q_heads = g * n_kv_heads with g in 1..8; bits 8 for FP8/INT8/FP8_STATIC
 * and 16 for BF16 (group and residual must be 0), bits 4 or 2 for KIVI and
 * KIVI_F16 with group 32 or 64 dividing head_dim and 0 <= residual <= 4096,
 * bits 4 for INT4 and INT4_HADAMARD (below); 1 <= max_tokens <= 2^24, and
 * one (sequence, kv head) pair's Key code region, token_capacity *
 * row_bytes bytes, below 2^32 (the kernels address it with 32-bit offsets;
 * this bounds only BF16 at head_dim 128 to max_tokens <= 2^24 - 32);
 * KVQ_ERR_UNSUPPORTED otherwise.
 * KVQ_FMT_INT4 ([LLMS] "2. INT8 and INT4 Uniform Group-Wise Quantization"):
 * bits 4, group 32, 64 or 128 dividing head_dim, residual 0; Key and Value
 * alike, per token and per group of `group` consecutive channels, s = max|x|
 * / 7, code = clamp(rint(x / s), -8, 7) (within [-7, 7]), dequantized code *
 * s, stored as the nibble code + 8.
 * KVQ_FMT_KIVI_F16: KIVI (same bits, group, residual and layout) with its
 * scales and zero-points stored as IEEE binary16: s and z are computed in
 * fp32 as for KIVI, rounded to the nearest binary16 (ties to even), and the
 * codes are taken against the stored values, clamp(rint((x - z16) / s16),
 * 0, 2^bits - 1); dequantized code * s16 + z16. Half the metadata bytes;
 * the values' scales and minima must be within binary16 range (|.| <
 * 65504; a scale below 2^-24 stores 0 and gives code 0).
 * KVQ_FMT_INT4_HADAMARD ([LLMS] "5. QuaRot and RotateKV: Orthogonal
 * Hadamard Dispersal"): KVQ_FMT_INT4 whose Key rows are rotated before
 * they are quantized, by the unnormalized fast Walsh-Hadamard transform over
 * head_dim in fp32 (stages h = 1, 2, 4, ...: pairs (i, i + h) become
 * (a + b, a - b)); decode rotates the query the same way and scales it by
 * 1/head_dim, so scores are unchanged (H H = d I). The rotation spreads a
 * Key outlier channel over all channels, so one group per token (group =
 * head_dim) suffices. Values are not rotated. Same layout as KVQ_FMT_INT4.
 * KVQ_FMT_FP8_STATIC ([LLMS] "1. FP8 KV Cache", per-tensor uncalibrated
 * scaling): bits 8, group and residual 0; code = E4M3_rne(clamp(x, -448,
 * 448)), dequantized as the code's value; no scale arrays.
 * KVQ_FMT_BF16 is the unquantized 16-bit cache of [BEA] §1's table (2 bytes
 * per element): it stores each input rounded to bfloat16 (to nearest, ties
 * to even; bf16 inputs bit-unchanged) with no scales, and decodes through
 * the same attention kernel, as the point of comparison for the formats
 * that store fewer bytes. */
typedef struct kvq_config {
  int32_t format;      /* kvq_format                                         */
  int32_t bits;        /* code width: 8 (FP8, INT8), 4 or 2 (KIVI), 4 (INT4), 16 (BF16) */
  int32_t group;       /* KIVI G: tokens per Key group = channels per Value group; INT4: channels per scale */
  int32_t residual;    /* KIVI R: most recent tokens always kept unquantized */
  int32_t batch;       /* B sequences                                        */
  int32_t n_kv_heads;  /* Hkv                                                */
  int32_t n_q_heads;   /* Hq                                                 */
  int32_t head_dim;    /* d                                                  */
  int32_t max_tokens;  /* capacity per sequence                              */
  int32_t in_dtype;    /* kvq_dtype of K/V inputs, q and the residual ring   */
} kvq_config;

/* Where each array sits inside one layer's cache buffer (byte offsets from
 * the buffer start, each a multiple of 256). Index order is always
 * [b][kv_head][...] with b-major order. cap = token_capacity.
 *
 *  k_codes  [B][Hkv][cap][row_bytes]       token-major; within a row, code of
 *           channel c sits in byte c*bits/8 at bit (c % (8/bits))*bits
 *           (low bits first; one byte per channel for FP8/INT8; BF16: the
 *           bfloat16 of channel c in bytes 2c, 2c+1).
 *  v_codes  [B][Hkv][cap/TB][d][TB*bits/8] tokens in blocks of TB = 8 (BF16,
 *           8-bit codes, INT4) or TB = 16 (INT2); for each block, d
 *           little-endian words of TB*bits bits (16 bytes for BF16, 8 for
 *           8-bit codes, else 4) whose bits [i*bits, (i+1)*bits) hold token
 *           TB*blk+i of one channel (8-bit: byte i; BF16: bytes 2i, 2i+1).
 *           Word slots are permuted within chunks of 16*W channels, W = 16 /
 *           word bytes (1, 2 or 4): slot W*m + x of a chunk holds the word of
 *           channel 16*x + m of that chunk, so a 16-byte load at slot W*m
 *           returns channel m of W consecutive 16-channel tiles (W = 1, BF16:
 *           no permutation).
 *  INT4, INT4_HADAMARD: k_codes rows of d nibbles (code + 8) in chunks of 8 channels:
 *           chunk (kk, r) = channels [32 kk + 8 r, 32 kk + 8 r + 8) sits at
 *           byte (d/8) r + 4 kk, channel 32 kk + 8 r + e in nibble e (low
 *           nibble first); v_codes as KIVI INT4 (TB = 8, 4-byte words);
 *           k_scale, v_scale [B][Hkv][cap][d/group] fp32.
 *  FP8/INT8: k_scale, v_scale [B][Hkv][cap] fp32; k_zero, v_zero unused (0).
 *  BF16, FP8_STATIC: no scale or zero-point arrays (offsets 0); FP8_STATIC
 *           codes are laid out as FP8's.
 *  KIVI:    k_scale, k_zero [B][Hkv][cap/G][d] fp32 (per group, per channel;
 *           KIVI_F16: binary16, here and in v_scale, v_zero);
 *           v_scale, v_zero [B][Hkv][cap][d/G] fp32 (per token, per channel
 *           group); k_resid, v_resid [B][Hkv][resid_slots][d] in in_dtype,
 *           token t of a sequence in slot t % resid_slots.
 *  Unused regions have offset 0. INT8 codes are two's complement bytes. */
typedef struct kvq_layout {
  uint64_t total_bytes;
  uint64_t k_codes_off, v_codes_off;
  uint64_t k_scale_off, v_scale_off;
  uint64_t k_zero_off, v_zero_off;
  uint64_t k_resid_off, v_resid_off;
  int32_t token_capacity;  /* cap: max_tokens rounded up to 32 (FP8/INT8/INT4/BF16) or to G (KIVI) */
  int32_t resid_slots;     /* KIVI ring slots = residual + group; 0 otherwise */
  int32_t row_bytes;       /* head_dim * bits / 8                             */
  int32_t elem_bytes;      /* bytes of one in_dtype element (4 or 2)          */
} kvq_layout;

/* Message for a status code (static storage; never NULL). */
const char* kvq_status_string(int32_t status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t kvq_version(void);

/* Fills *layout for cfg ([N4N] Step 3 constructor arguments: layers are
 * separate buffers; heads, head_dim, dtype and group size set the shape).
 * Host only, no HIP call. Errors: KVQ_ERR_INVALID (null pointer, bad value),
 * KVQ_ERR_UNSUPPORTED (valid but outside the supported shapes above). */
int32_t kvq_get_layout(const kvq_config* cfg, kvq_layout* layout);

/* Appends new tokens to every sequence of one layer's cache and quantizes
 * them ([N4N] Step 3 append; [BEA] §3 and §4; [LLMS] 1.-3.).
 *  cache        device, kvq_layout.total_bytes bytes, modified.
 *  seq_lens     device int32 [B], tokens held per sequence; advanced by the
 *               number of tokens appended to each sequence.
 *  k_new,v_new  device [B][Hkv][t_new][d] in cfg->in_dtype, contiguous,
 *               oldest token first; read only.
 *  t_new        tokens per sequence in k_new/v_new, >= 0 (0 is a no-op).
 *  append_lens  device int32 [B] or NULL: sequence b appends only its first
 *               append_lens[b] tokens (ragged batches); NULL = t_new for all.
 *  skipped      device int32 [B] or NULL (caller-owned, 4-byte aligned): when
 *               given and t_new > 0, the call sets skipped[b] = 1 for every
 *               sequence it leaves unchanged (rule below: capacity overflow
 *               or a malformed length) and 0 for every other, in stream
 *               order with the append; with t_new == 0 it is not written.
 *               A caller sees an overflow here without a host
 *               synchronization or an allocation.
 * The per-token formats (FP8, INT8, INT4, FP8_STATIC, and INT4_HADAMARD
 * after rotating the Key row) quantize each token on arrival; BF16 rounds
 * it. KIVI and KIVI_F16 write new tokens to the residual ring and quantize
 * (and pack) every whole group of G tokens that the flush rule admits, Key
 * per channel and Value per token; a group may mix older residual tokens
 * with new ones. The result depends only on
 * the token sequence, not on how it was split into calls.
 * A sequence with seq_lens[b] < 0, an append length outside [0, t_new], or
 * seq_lens[b] + append length > max_tokens is left entirely unchanged and
 * reported in `skipped`. Calls that overlap in time on the same cache race.
 * Errors: KVQ_ERR_INVALID, KVQ_ERR_UNSUPPORTED, KVQ_ERR_HIP. */
int32_t kvq_quantize_append(const kvq_config* cfg, void* cache, int32_t* seq_lens,
                            const void* k_new, const void* v_new, int32_t t_new,
                            const int32_t* append_lens, int32_t* skipped, void* stream);

/* Workspace bytes that kvq_decode_attention needs for split_tokens (0 =
 * the library's choice for cfg). Host only; the result does not depend on
 * the device. For split_tokens > 0 it holds n = ceil(max_tokens /
 * split_tokens) splits; for 0 it holds n = min(128, max(1, max_tokens /
 * 256)) splits, the most the library's choice can take on any device. The
 * workspace starts with batch * (n_kv_heads + 1) + 1 uint32 counters (see
 * kvq_decode_attention for the zero-fill rule), then per (sequence,
 * query head) n + 1 partial rows of head_dim + 2 fp32, each array 256-byte
 * aligned. kvq_append_decode takes the same workspace. Errors:
 * KVQ_ERR_INVALID, KVQ_ERR_UNSUPPORTED (split_tokens not a positive
 * multiple of 64, or more than 128 splits of max_tokens). */
int32_t kvq_decode_workspace_bytes(const kvq_config* cfg, int32_t split_tokens, uint64_t* bytes);

/* Single-token decode attention that reads the quantized cache directly and
 * dequantizes in registers ([DUP] "Key takeaways"; [N4N] Step 5: no separate
 * dequantize pass). Split-K over the token axis (flash-decoding): the
 * quantized tokens of each sequence are cut into n splits at fixed
 * fractions of its length (whole 32-token tiles, whole groups for KIVI),
 * each producing a partial softmax state (running max, running sum,
 * unnormalized output); the KIVI residual window is one more split. The
 * last split of each (sequence, kv head) to finish merges them with the
 * log-sum-exp rule. One launch.
 *  cache        device, one layer's cache; read only.
 *  seq_lens     device int32 [B]; values are clamped to [0, max_tokens].
 *  q            device [B][Hq][d] in cfg->in_dtype (the new query token).
 *  sm_scale     softmax scale applied to the dot products (1/sqrt(d) is usual).
 *  out          device fp32 [B][Hq][d], written.
 *  workspace    device scratch of at least kvq_decode_workspace_bytes(cfg,
 *               split_tokens) bytes. Its first batch * (n_kv_heads + 1)
 *               + 1 uint32 (the counters) must be zero on entry: zero-fill the
 *               workspace once after allocating it (or when batch or
 *               n_kv_heads change); every call leaves them zero when it
 *               completes. The rest is scratch. Calls that overlap in time
 *               on one workspace race.
 *  split_tokens a positive multiple of 64 giving at most 128 splits of
 *               max_tokens: n = ceil(max_tokens / split_tokens) equal
 *               splits of each sequence. 0 = the library's choice, within
 *               the bound kvq_decode_workspace_bytes gives: for FP8, INT8
 *               and the other per-token formats, equal splits for about two
 *               workgroups per compute unit in one round; for KIVI, about
 *               four rounds of the device's resident workgroups, cut into
 *               large, then medium, then small splits that go out to the
 *               workgroups in that order as they free up.
 * Errors: KVQ_ERR_INVALID, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE,
 * KVQ_ERR_HIP. */
int32_t kvq_decode_attention(const kvq_config* cfg, const void* cache, const int32_t* seq_lens,
                             const void* q, float sm_scale, float* out, void* workspace,
                             uint64_t workspace_bytes, int32_t split_tokens, void* stream);

/* One decode step in one launch: appends one new K/V token to every
 * sequence and then attends over the grown cache. The result equals
 * kvq_quantize_append(cfg, cache, seq_lens, k_new, v_new, 1, NULL, stream)
 * followed by kvq_decode_attention(cfg, cache, seq_lens, q, ...) on the
 * same stream: the same codes, scales, zero-points, residual rows and
 * seq_lens bit for bit, and the same attention up to fp32 rounding order.
 * Sources: [N4N] "Step 5: Integrate with your inference engine" (the
 * attention forward pass appends the step's K, V and then reads the cache);
 * [LLMS] "Serving Economics and Latency Trade-Offs" (scale computation and
 * bit-packing add latency unless fused into a kernel; said there of
 * prefill, applied here to the one-token decode append).
 *  cache        device, one layer's cache; modified (the new token, and for
 *               KIVI a group that it completes, as the append stores them).
 *  seq_lens     device int32 [B]; a sequence with 0 <= seq_lens[b] <
 *               max_tokens takes the token and its length is advanced by
 *               one inside the launch; any other sequence is left unchanged
 *               and attention reads it as kvq_decode_attention does.
 *  k_new,v_new  device [B][Hkv][1][d] in cfg->in_dtype: the new token.
 *  q, sm_scale, out, workspace, workspace_bytes, split_tokens: as in
 *               kvq_decode_attention (the same workspace size and zero-fill
 *               rule). q must not alias cache, k_new or v_new.
 *  skipped      device int32 [B] or NULL (caller-owned, 4-byte aligned): when
 *               given, set to 1 for every sequence that takes no token
 *               (seq_lens[b] < 0 or >= max_tokens) and 0 for every other.
 * Per-token formats (FP8, INT8, INT4, FP8_STATIC, INT4_HADAMARD, BF16):
 * the workgroup of the sequence's first split quantizes the new token,
 * stores it and attends to it. KIVI and KIVI_F16: the residual-window
 * workgroup writes the token to its ring slot (or, with a zero window,
 * straight into the group it completes) and, when a group completes,
 * quantizes and packs it and attends over its dequantized codes. Calls
 * that overlap in time on one cache or one workspace race.
 * Errors: KVQ_ERR_INVALID, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE,
 * KVQ_ERR_HIP. */
int32_t kvq_append_decode(const kvq_config* cfg, void* cache, int32_t* seq_lens, const void* k_new,
                          const void* v_new, const void* q, float sm_scale, float* out, void* workspace,
                          uint64_t workspace_bytes, int32_t split_tokens, int32_t* skipped, void* stream);

/* Bytes of the fixed device workspace behind kvq_append_decode_noalloc. */
#define KVQ_STATIC_WORKSPACE_BYTES (64ull << 20)

/* kvq_append_decode without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. It calls no hipMalloc, hipFree or other
 * allocating routine: the arrival counters and partial states live in a
 * file-scope device array of KVQ_STATIC_WORKSPACE_BYTES (64 MiB), one per
 * device the library runs on, kept until the process ends; its device
 * address is looked up on the entry point's first call on a device, with
 * that device current. Each call first zeroes the counters with a small fill
 * kernel on `stream` (not a memset), then makes the same launch as
 * kvq_append_decode with the same split plan, so the cache, seq_lens,
 * skipped and out are bit for bit those of kvq_append_decode.
 *  Arguments: as kvq_append_decode, without workspace and workspace_bytes.
 *  Limit: the call's workspace (kvq_decode_workspace_bytes' layout for the
 *         planned number of splits: batch * (n_kv_heads + 1) + 1 counters, then
 *         batch * n_q_heads * (splits + 1) partial rows of head_dim + 2
 *         fp32, each array 256-byte aligned) must fit
 *         KVQ_STATIC_WORKSPACE_BYTES; otherwise the call
 *         returns KVQ_ERR_WORKSPACE and launches nothing (with split_tokens
 *         > 0 this is decided before any HIP call).
 *  Concurrency: every call on one device shares that device's array, which
 *         keeps the last call's contents; calls that overlap in time on one
 *         device (two streams, two threads) race, even on different caches.
 * Errors: KVQ_ERR_INVALID, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE,
 * KVQ_ERR_HIP. */
int32_t kvq_append_decode_noalloc(const kvq_config* cfg, void* cache, int32_t* seq_lens, const void* k_new,
                                  const void* v_new, const void* q, float sm_scale, float* out,
                                  int32_t split_tokens, int32_t* skipped, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
