// Internal interface between the host entry points (kvq_api.cpp) and the
// HIP kernels (kvq_append.hip, kvq_decode.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// One layer's cache, resolved to device pointers. Built on the host from a
// validated kvq_config and its kvq_layout; passed to kernels by value.
struct CacheView {
  int fmt;         // kvq_format
  int bits;        // 8, 4 or 2
  int G;           // KIVI group (0 for per-token formats)
  int R;           // KIVI residual window
  int B, Hkv, Hq, D, g;
  int max_tokens;
  int bf16;        // in_dtype is bf16 (else fp32)
  int cap;         // token capacity of the code arrays
  int C;           // residual ring slots (KIVI)
  int row_bytes;   // D * bits / 8
  uint8_t* k_codes;
  uint8_t* v_codes;
  float* k_scale;
  float* v_scale;
  float* k_zero;
  float* v_zero;
  uint8_t* k_resid;
  uint8_t* v_resid;
};

// Decode workspace split into its three arrays.
// Most quantized splits per sequence a decode call may use (the merge keeps
// every split's running max and sum of up to 8 heads in LDS).
constexpr int kMaxDecodeSplits = 128;

struct DecodeWork {
  uint32_t* count;  // [B][Hkv] partials finished in this call (zero between calls)
  uint32_t* bcount; // [B] (sequence, kv head) merges finished in a fused call (zero between calls)
  uint32_t* queue;  // [1] work items handed out in this call (zero between calls)
  float* o;         // [B][Hq][S][D] unnormalized partial outputs
  float* m;         // [B][Hq][S] running maxima (log2 domain)
  float* l;         // [B][Hq][S] running sums
  int S;            // partial slots per (b, q head): S - 1 quantized chunks + the KIVI residual
  // chunks of a pair's quantized tokens: n1 of weight w1, n2 of weight w2,
  // n3 of weight w3 (n1 + n2 + n3 = S - 1, n1 >= 1)
  int n1, w1, n2, w2, n3, w3;
  int nitems;       // work items (one workgroup each): B * Hkv * (S - 1), plus B * Hkv for KIVI
  int nstatic;      // workgroup x < nstatic takes item x; the later ones draw items nstatic.. from queue
};

// skipped: NULL, or [B] set to 1 for each sequence the append leaves
// unchanged (malformed or over capacity) and 0 for the others.
hipError_t launch_append(const CacheView& cv, int32_t* seq_lens, const void* k_new,
                         const void* v_new, int T, const int32_t* append_lens, int32_t* skipped,
                         hipStream_t stream);

// The one new token per sequence of a fused append + decode call: K and V
// rows [B][Hkv][1][D] in the input dtype; seq_lens is advanced in place.
struct AppendIn {
  int32_t* seq_lens;
  const void* k;
  const void* v;
  int32_t* skipped;  // NULL, or [B]: 1 for a sequence that takes no token, else 0
};

// Decode attention; with app != nullptr, the fused step that first appends
// app's token to every sequence (as launch_append with T = 1 would) and then
// attends over the grown cache, in one launch.
hipError_t launch_decode(const CacheView& cv, const int32_t* seq_lens, const void* q,
                         float sm_scale, float* out, const DecodeWork& work, const AppendIn* app,
                         hipStream_t stream);

// Decode workgroups the current device holds at once (compute units times
// the kernel's occupancy per unit); 0 when it cannot be queried.
int decode_resident_workgroups(const CacheView& cv);

// Compute units of the current device; 0 when it cannot be queried.
int decode_compute_units();

// Fixed decode workspace of kvq_append_decode_noalloc: a file-scope device
// array of kStaticWorkspaceBytes in kvq_decode.hip, one per device.
constexpr uint64_t kStaticWorkspaceBytes = KVQ_STATIC_WORKSPACE_BYTES;
// Device address of the current device's array (looked up once per device,
// with that device current).
hipError_t static_workspace(void** ptr);
// Zeroes n uint32 words at p with a small fill kernel on `stream` (a kernel,
// not a memset node, so that it can sit in a captured graph).
hipError_t launch_clear_words(uint32_t* p, int n, hipStream_t stream);

}  // namespace kvq
