// Host-only entry points: split-count lookup, status text, version.
#include <stdint.h>

#include "decode_attn.h"

// LightLLM PR #1549, "Covered decode kernels": the KV-cache decode kernel's
// tuned config is num_splits; KV-length run keys are bucketed while the real
// length picks the bucket at run time, and an untuned key falls back to the
// nearest tuned one.  Here: bucket = clamp(ceil(kv_len / bucket_tokens), 1,
// n_buckets); batch key = nearest to `batch`, ties to the smaller key.
extern "C" int32_t decode_attn_pick_splits(const int32_t* table, const int32_t* batch_keys,
                                           int32_t n_batch_keys, int32_t n_buckets,
                                           int32_t bucket_tokens, int32_t batch, int32_t kv_len) {
  if (!table || !batch_keys || n_batch_keys <= 0 || n_buckets <= 0 || bucket_tokens <= 0)
    return -DA_ERR_INVALID_ARG;
  for (int i = 1; i < n_batch_keys; ++i)
    if (batch_keys[i] <= batch_keys[i - 1]) return -DA_ERR_INVALID_ARG;
  long long bucket = kv_len <= 0 ? 1 : ((long long)kv_len + bucket_tokens - 1) / bucket_tokens;
  if (bucket < 1) bucket = 1;
  if (bucket > n_buckets) bucket = n_buckets;
  int best = 0;
  long long best_d = -1;
  for (int i = 0; i < n_batch_keys; ++i) {
    long long d = (long long)batch_keys[i] - batch;
    if (d < 0) d = -d;
    if (best_d < 0 || d < best_d) {  // strict: an equal distance keeps the smaller key
      best = i;
      best_d = d;
    }
  }
  const int32_t s = table[(long long)best * n_buckets + (bucket - 1)];
  if (s < 1 || s > DA_MAX_SPLITS) return -DA_ERR_INVALID_ARG;
  return s;
}

extern "C" const char* decode_attn_strerror(int32_t status) {
  switch (status) {
    case DA_OK: return "ok";
    case DA_ERR_INVALID_ARG: return "invalid argument";
    case DA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case DA_ERR_LAUNCH: return "kernel launch failed";
    case DA_ERR_TOO_LARGE: return "partials exceed the static scratch buffer";
    default: return "unknown status";
  }
}

extern "C" int32_t decode_attn_version(void) { return 300; }
