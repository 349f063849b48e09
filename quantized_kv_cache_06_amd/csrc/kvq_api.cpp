// Host side of libkvq: argument validation, the cache layout, split planning
// and kernel dispatch. Every check here runs before any HIP call, so a
// rejected call changes nothing and needs no GPU.
#include <stdint.h>
#include <string.h>

#include "kvq.h"
#include "kvq_internal.h"

// Decode plan constants for KIVI (see plan_for): n = KVQ_PLAN_ROUNDS
// rounds of the resident workgroups; of the n chunks of a pair, n /
// KVQ_PLAN_DIV3 are small (weight KVQ_PLAN_W3), n / KVQ_PLAN_DIV2 medium
// (KVQ_PLAN_W2) and the rest large (KVQ_PLAN_W1). For the long-context INT4
// workload (n = 24) that is 15 chunks of 6.1 % of the pair, 3 of 2.0 % and
// 6 of 0.5 %. Measured on MI355X against equal static splits: 349-351
// against 356-359 us per decode call; the same weights with 5 rounds, with
// 8 small chunks, or with large chunks of weight 16 all measured 350-354.
#ifndef KVQ_PLAN_W1
#define KVQ_PLAN_W1 12
#endif
#ifndef KVQ_PLAN_W2
#define KVQ_PLAN_W2 4
#endif
#ifndef KVQ_PLAN_W3
#define KVQ_PLAN_W3 1
#endif
#ifndef KVQ_PLAN_DIV2
#define KVQ_PLAN_DIV2 8
#endif
#ifndef KVQ_PLAN_DIV3
#define KVQ_PLAN_DIV3 4
#endif
#ifndef KVQ_PLAN_ROUNDS
#define KVQ_PLAN_ROUNDS 4
#endif

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr int64_t kMaxTokens = int64_t(1) << 24;
constexpr int kMaxResidual = 4096;

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

bool kivi_fmt(const kvq_config* c) { return c->format == KVQ_FMT_KIVI || c->format == KVQ_FMT_KIVI_F16; }

int32_t validate(const kvq_config* c) {
  if (!c) return KVQ_ERR_INVALID;
  if (c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1 || c->head_dim < 1 || c->max_tokens < 1)
    return KVQ_ERR_INVALID;
  if (c->n_q_heads % c->n_kv_heads != 0) return KVQ_ERR_INVALID;
  if (c->in_dtype != KVQ_DT_F32 && c->in_dtype != KVQ_DT_BF16) return KVQ_ERR_INVALID;
  if (c->max_tokens > kMaxTokens) return KVQ_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return KVQ_ERR_UNSUPPORTED;
  const int g = c->n_q_heads / c->n_kv_heads;
  if (g > 8) return KVQ_ERR_UNSUPPORTED;
  // Batch and KV heads index grid dimensions y and z of the append kernels
  // (at most 65535 each); the decode numbers its work items (at most 129
  // per (sequence, kv head) pair) in 32 bits.
  if (c->batch > 65535 || c->n_kv_heads > 65535) return KVQ_ERR_UNSUPPORTED;
  if (int64_t(c->batch) * c->n_kv_heads > (int64_t(1) << 24)) return KVQ_ERR_UNSUPPORTED;
  switch (c->format) {
    case KVQ_FMT_FP8_E4M3:
    case KVQ_FMT_FP8_STATIC:
    case KVQ_FMT_INT8:
      if (c->bits != 8 || c->group != 0 || c->residual != 0) return KVQ_ERR_INVALID;
      break;
    case KVQ_FMT_BF16:
      if (c->bits != 16 || c->group != 0 || c->residual != 0) return KVQ_ERR_INVALID;
      break;
    case KVQ_FMT_INT4:
    case KVQ_FMT_INT4_HADAMARD:
      if (c->bits != 4 || c->residual != 0 || c->group <= 0) return KVQ_ERR_INVALID;
      if (c->head_dim % c->group != 0) return KVQ_ERR_INVALID;
      if (c->group != 32 && c->group != 64 && c->group != 128) return KVQ_ERR_UNSUPPORTED;
      break;
    case KVQ_FMT_KIVI:
    case KVQ_FMT_KIVI_F16:
      if (c->bits != 4 && c->bits != 2) return KVQ_ERR_INVALID;
      if (c->group <= 0 || c->residual < 0) return KVQ_ERR_INVALID;
      if (c->head_dim % c->group != 0) return KVQ_ERR_INVALID;
      if (c->group != 32 && c->group != 64) return KVQ_ERR_UNSUPPORTED;
      if (c->residual > kMaxResidual) return KVQ_ERR_UNSUPPORTED;
      break;
    default:
      return KVQ_ERR_INVALID;
  }
  // The kernels address one (sequence, kv head) pair's Key or Value code
  // region (token_capacity * row_bytes bytes) with 32-bit offsets.
  const bool kivi = c->format == KVQ_FMT_KIVI || c->format == KVQ_FMT_KIVI_F16;
  const uint64_t unit = kivi ? uint64_t(c->group) : 32;
  const uint64_t cap = (uint64_t(c->max_tokens) + unit - 1) / unit * unit;
  if (cap * uint64_t(c->head_dim) * uint64_t(c->bits) / 8 >= (uint64_t(1) << 32)) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

void make_layout(const kvq_config* c, kvq_layout* L) {
  memset(L, 0, sizeof(*L));
  const bool kivi = c->format == KVQ_FMT_KIVI || c->format == KVQ_FMT_KIVI_F16;
  const uint64_t meta = c->format == KVQ_FMT_KIVI_F16 ? 2 : 4;  // bytes per scale or zero-point
  const uint64_t pairs = uint64_t(c->batch) * c->n_kv_heads;
  const int D = c->head_dim;
  const int unit = kivi ? c->group : 32;
  const uint64_t cap = (uint64_t(c->max_tokens) + unit - 1) / unit * unit;
  L->token_capacity = int32_t(cap);
  L->row_bytes = D * c->bits / 8;
  L->elem_bytes = c->in_dtype == KVQ_DT_BF16 ? 2 : 4;
  uint64_t off = 0;
  auto region = [&](uint64_t bytes) {
    const uint64_t at = off;
    off = align256(off + bytes);
    return at;
  };
  L->k_codes_off = region(pairs * cap * L->row_bytes);
  L->v_codes_off = region(pairs * cap * L->row_bytes);
  if (c->format == KVQ_FMT_BF16 || c->format == KVQ_FMT_FP8_STATIC) {
    // no scales: the codes are the values
  } else if (c->format == KVQ_FMT_INT4 || c->format == KVQ_FMT_INT4_HADAMARD) {
    L->k_scale_off = region(pairs * cap * (D / c->group) * 4);
    L->v_scale_off = region(pairs * cap * (D / c->group) * 4);
  } else if (!kivi) {
    L->k_scale_off = region(pairs * cap * 4);
    L->v_scale_off = region(pairs * cap * 4);
  } else {
    const uint64_t groups = cap / c->group;
    const uint64_t vgroups = D / c->group;
    L->k_scale_off = region(pairs * groups * D * meta);
    L->k_zero_off = region(pairs * groups * D * meta);
    L->v_scale_off = region(pairs * cap * vgroups * meta);
    L->v_zero_off = region(pairs * cap * vgroups * meta);
    L->resid_slots = c->residual + c->group;
    L->k_resid_off = region(pairs * L->resid_slots * D * L->elem_bytes);
    L->v_resid_off = region(pairs * L->resid_slots * D * L->elem_bytes);
  }
  L->total_bytes = off;
}

kvq::CacheView make_view(const kvq_config* c, const kvq_layout& L, const void* cache) {
  kvq::CacheView v;
  uint8_t* base = static_cast<uint8_t*>(const_cast<void*>(cache));
  const bool kivi = c->format == KVQ_FMT_KIVI || c->format == KVQ_FMT_KIVI_F16;
  v.fmt = c->format;
  v.bits = c->bits;
  v.G = c->group;
  v.R = c->residual;
  v.B = c->batch;
  v.Hkv = c->n_kv_heads;
  v.Hq = c->n_q_heads;
  v.D = c->head_dim;
  v.g = c->n_q_heads / c->n_kv_heads;
  v.max_tokens = c->max_tokens;
  v.bf16 = c->in_dtype == KVQ_DT_BF16;
  v.cap = L.token_capacity;
  v.C = L.resid_slots;
  v.row_bytes = L.row_bytes;
  v.k_codes = base + L.k_codes_off;
  v.v_codes = base + L.v_codes_off;
  const bool scaled = c->format != KVQ_FMT_BF16 && c->format != KVQ_FMT_FP8_STATIC;
  v.k_scale = scaled ? reinterpret_cast<float*>(base + L.k_scale_off) : nullptr;
  v.v_scale = scaled ? reinterpret_cast<float*>(base + L.v_scale_off) : nullptr;
  v.k_zero = kivi ? reinterpret_cast<float*>(base + L.k_zero_off) : nullptr;
  v.v_zero = kivi ? reinterpret_cast<float*>(base + L.v_zero_off) : nullptr;
  v.k_resid = kivi ? base + L.k_resid_off : nullptr;
  v.v_resid = kivi ? base + L.v_resid_off : nullptr;
  return v;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Most quantized splits per sequence the automatic choice may use (the
// workspace for split_tokens == 0 is sized for this many): splits of at
// least 256 tokens of the longest sequence the cache holds, at most
// kMaxDecodeSplits.
int auto_split_bound(const kvq_config* c) {
  int64_t n = c->max_tokens / 256;
  if (n < 1) n = 1;
  if (n > kvq::kMaxDecodeSplits) n = kvq::kMaxDecodeSplits;
  return int(n);
}

// The decode plan: how each (sequence, kv head) pair's quantized tokens are
// cut into chunks, and whether the chunks go out through the item counter.
//  - split_tokens > 0: n = ceil(max_tokens / split_tokens) equal chunks,
//    workgroup x takes item x.
//  - FP8, INT8 and the other per-token formats (split_tokens == 0): n equal
//    chunks for about two workgroups per compute unit in one round. They
//    stream at the memory bound; a third co-resident workgroup gets the
//    least of the unit's memory issue (the oldest waves are served first)
//    and ends the launch late, and each further round adds a prologue and a
//    tail.
//  - KIVI (split_tokens == 0): about four rounds of the device's resident
//    workgroups (workgroups in different phases, loads, group folds and
//    epilogue, share a compute unit), as large chunks, then medium and small
//    ones, handed out in that order through the item counter. Equal static
//    splits end at very different times: co-resident workgroups do not get
//    equal shares of a unit's memory issue, and each XCD runs its own share
//    of the grid. The small chunks at the end fill whichever units finish
//    early.
// n stays within [1, auto_split_bound()] for split_tokens == 0.
struct Plan {
  int n1, w1, n2, w2, n3, w3;  // chunk counts and weights of the three phases
  int dynamic;
};

Plan plan_for(const kvq_config* c, int32_t split_tokens, int64_t resident, int64_t cus) {
  Plan p{0, 1, 0, 1, 0, 1, 0};
  if (split_tokens > 0) {
    p.n1 = int((int64_t(c->max_tokens) + split_tokens - 1) / split_tokens);
    return p;
  }
  const int64_t pairs = int64_t(c->batch) * c->n_kv_heads;
  int64_t n = kivi_fmt(c) ? KVQ_PLAN_ROUNDS * resident / pairs : 2 * cus / pairs;
  const int bound = auto_split_bound(c);
  if (n < 1) n = 1;
  if (n > bound) n = bound;
  if (!kivi_fmt(c)) {
    p.n1 = int(n);
    return p;
  }
  p.n3 = int(n) / KVQ_PLAN_DIV3;
  p.n2 = int(n) / KVQ_PLAN_DIV2;
  p.n1 = int(n) - p.n2 - p.n3;
  p.w1 = KVQ_PLAN_W1;
  p.w2 = KVQ_PLAN_W2;
  p.w3 = KVQ_PLAN_W3;
  p.dynamic = 1;
  return p;
}

// Quantized splits per sequence the workspace must hold: ceil(max_tokens /
// split_tokens) for an explicit split length, auto_split_bound() for 0.
int32_t split_bound(const kvq_config* c, int32_t split_tokens, int* n) {
  if (split_tokens < 0 || (split_tokens > 0 && split_tokens % 64 != 0)) return KVQ_ERR_UNSUPPORTED;
  if (split_tokens > (1 << 24)) return KVQ_ERR_UNSUPPORTED;
  if (split_tokens == 0) {
    *n = auto_split_bound(c);
    return KVQ_OK;
  }
  const int64_t nsplit = (int64_t(c->max_tokens) + split_tokens - 1) / split_tokens;
  if (nsplit > kvq::kMaxDecodeSplits) return KVQ_ERR_UNSUPPORTED;
  *n = int(nsplit);
  return KVQ_OK;
}

// Workspace: [B][Hkv] uint32 arrival counters, [B] per-sequence counters
// (fused calls) and the work-item counter first (they must read zero on
// entry; each call leaves them zero), then the partial states o, m, l.
uint64_t counter_words(const kvq_config* c) {
  return uint64_t(c->batch) * c->n_kv_heads + uint64_t(c->batch) + 1;
}
uint64_t counter_bytes(const kvq_config* c) { return align256(counter_words(c) * 4); }

uint64_t workspace_bytes(const kvq_config* c, int S) {
  const uint64_t rows = uint64_t(c->batch) * c->n_q_heads * S;
  return counter_bytes(c) + align256(rows * c->head_dim * 4) + align256(rows * 4) + align256(rows * 4);
}

}  // namespace

namespace {

// Shared by kvq_decode_attention, kvq_append_decode and
// kvq_append_decode_noalloc: checks the decode arguments, plans the splits,
// lays out the workspace and launches. fixed_ws: the workspace is the
// library's fixed device array (workspace and ws_bytes are ignored); it
// must hold the planned splits, and its arrival counters are zeroed by a
// fill kernel before the decode launch.
int32_t decode_call(const kvq_config* cfg, const void* cache, const int32_t* seq_lens, const void* q, float sm_scale,
                    float* out, void* workspace, uint64_t ws_bytes, int32_t split_tokens, const kvq::AppendIn* app,
                    bool fixed_ws, void* stream) {
  const int32_t st = validate(cfg);
  if (st != KVQ_OK) return st;
  if (!cache || !seq_lens || !q || !out || (!fixed_ws && !workspace)) return KVQ_ERR_INVALID;
  if (!aligned16(cache) || !aligned16(q) || !aligned16(out) || (!fixed_ws && !aligned16(workspace)) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3))
    return KVQ_ERR_INVALID;
  if (app && (!app->k || !app->v || !aligned16(app->k) || !aligned16(app->v))) return KVQ_ERR_INVALID;
  if (!(sm_scale == sm_scale) || sm_scale > 3.0e38f || sm_scale < -3.0e38f) return KVQ_ERR_INVALID;
  int n;
  const int32_t sp = split_bound(cfg, split_tokens, &n);
  if (sp != KVQ_OK) return sp;
  if (!fixed_ws && ws_bytes < workspace_bytes(cfg, n + 1)) return KVQ_ERR_WORKSPACE;
  // an explicit split length fixes the plan: checked before any HIP call
  if (fixed_ws && split_tokens > 0 && workspace_bytes(cfg, n + 1) > kvq::kStaticWorkspaceBytes)
    return KVQ_ERR_WORKSPACE;
  kvq_layout lay;
  make_layout(cfg, &lay);
  const kvq::CacheView v = make_view(cfg, lay, cache);
  const int resident = kvq::decode_resident_workgroups(v);
  const int cus = kvq::decode_compute_units();
  if (resident <= 0 || cus <= 0) return KVQ_ERR_HIP;
  const Plan plan = plan_for(cfg, split_tokens, resident, cus);
  n = plan.n1 + plan.n2 + plan.n3;
  const int S = n + 1;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (fixed_ws) {
    if (workspace_bytes(cfg, S) > kvq::kStaticWorkspaceBytes) return KVQ_ERR_WORKSPACE;
    if (kvq::static_workspace(&workspace) != hipSuccess) return KVQ_ERR_HIP;
    // the array keeps the last call's contents: clear the arrival counters
    const int words = int(counter_words(cfg));
    if (kvq::launch_clear_words(static_cast<uint32_t*>(workspace), words, hs) != hipSuccess) return KVQ_ERR_HIP;
  }
  const uint64_t rows = uint64_t(cfg->batch) * cfg->n_q_heads * S;
  uint8_t* w = static_cast<uint8_t*>(workspace);
  kvq::DecodeWork work;
  work.count = reinterpret_cast<uint32_t*>(w);
  work.bcount = work.count + uint64_t(cfg->batch) * cfg->n_kv_heads;
  work.queue = work.bcount + cfg->batch;
  w += counter_bytes(cfg);
  work.o = reinterpret_cast<float*>(w);
  work.m = reinterpret_cast<float*>(w + align256(rows * cfg->head_dim * 4));
  work.l = reinterpret_cast<float*>(w + align256(rows * cfg->head_dim * 4) + align256(rows * 4));
  work.S = S;
  work.n1 = plan.n1;
  work.w1 = plan.w1;
  work.n2 = plan.n2;
  work.w2 = plan.w2;
  work.n3 = plan.n3;
  work.w3 = plan.w3;
  work.nitems = int(int64_t(cfg->batch) * cfg->n_kv_heads * (n + (kivi_fmt(cfg) ? 1 : 0)));
  // with a dynamic plan, the workgroups of the first round (those the device
  // holds at once) take their items by launch index; only the later ones
  // draw from the counter, so the draws are spread over the call instead of
  // all coming at its start
  work.nstatic = plan.dynamic && resident < work.nitems ? resident : work.nitems;
  const hipError_t e = kvq::launch_decode(v, seq_lens, q, sm_scale, out, work, app, hs);
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace

extern "C" {

const char* kvq_status_string(int32_t s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_WORKSPACE: return "decode workspace too small (the caller's, or the fixed one)";
    case KVQ_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int32_t kvq_version(void) { return kVersion; }

int32_t kvq_get_layout(const kvq_config* cfg, kvq_layout* layout) {
  if (!layout) return KVQ_ERR_INVALID;
  const int32_t st = validate(cfg);
  if (st != KVQ_OK) return st;
  make_layout(cfg, layout);
  return KVQ_OK;
}

int32_t kvq_quantize_append(const kvq_config* cfg, void* cache, int32_t* seq_lens, const void* k_new,
                            const void* v_new, int32_t t_new, const int32_t* append_lens, int32_t* skipped,
                            void* stream) {
  const int32_t st = validate(cfg);
  if (st != KVQ_OK) return st;
  if (!cache || !seq_lens || t_new < 0) return KVQ_ERR_INVALID;
  if (t_new == 0) return KVQ_OK;
  if (!k_new || !v_new) return KVQ_ERR_INVALID;
  if (!aligned16(cache) || !aligned16(k_new) || !aligned16(v_new) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3) || (reinterpret_cast<uintptr_t>(append_lens) & 3) ||
      (reinterpret_cast<uintptr_t>(skipped) & 3))
    return KVQ_ERR_INVALID;
  if (int64_t(t_new) > kMaxTokens) return KVQ_ERR_UNSUPPORTED;
  kvq_layout L;
  make_layout(cfg, &L);
  const kvq::CacheView v = make_view(cfg, L, cache);
  const hipError_t e = kvq::launch_append(v, seq_lens, k_new, v_new, t_new, append_lens, skipped,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

int32_t kvq_decode_workspace_bytes(const kvq_config* cfg, int32_t split_tokens, uint64_t* bytes) {
  if (!bytes) return KVQ_ERR_INVALID;
  const int32_t st = validate(cfg);
  if (st != KVQ_OK) return st;
  int n;
  const int32_t sp = split_bound(cfg, split_tokens, &n);
  if (sp != KVQ_OK) return sp;
  *bytes = workspace_bytes(cfg, n + 1);
  return KVQ_OK;
}

int32_t kvq_decode_attention(const kvq_config* cfg, const void* cache, const int32_t* seq_lens, const void* q,
                             float sm_scale, float* out, void* workspace, uint64_t ws_bytes,
                             int32_t split_tokens, void* stream) {
  return decode_call(cfg, cache, seq_lens, q, sm_scale, out, workspace, ws_bytes, split_tokens, nullptr, false,
                     stream);
}

int32_t kvq_append_decode(const kvq_config* cfg, void* cache, int32_t* seq_lens, const void* k_new,
                          const void* v_new, const void* q, float sm_scale, float* out, void* workspace,
                          uint64_t ws_bytes, int32_t split_tokens, int32_t* skipped, void* stream) {
  if (!k_new || !v_new || !seq_lens) return KVQ_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(skipped) & 3) return KVQ_ERR_INVALID;
  const kvq::AppendIn app{seq_lens, k_new, v_new, skipped};
  return decode_call(cfg, cache, seq_lens, q, sm_scale, out, workspace, ws_bytes, split_tokens, &app, false, stream);
}

int32_t kvq_append_decode_noalloc(const kvq_config* cfg, void* cache, int32_t* seq_lens, const void* k_new,
                                  const void* v_new, const void* q, float sm_scale, float* out,
                                  int32_t split_tokens, int32_t* skipped, void* stream) {
  if (!k_new || !v_new || !seq_lens) return KVQ_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(skipped) & 3) return KVQ_ERR_INVALID;
  const kvq::AppendIn app{seq_lens, k_new, v_new, skipped};
  return decode_call(cfg, cache, seq_lens, q, sm_scale, out, nullptr, 0, split_tokens, &app, true, stream);
}

}  // extern "C"
