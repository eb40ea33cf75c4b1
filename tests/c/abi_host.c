/* A plain C99 caller of the decode-attention library: it includes the public
 * header and links the shared library, then calls the host-only entry points
 * and argument-validation paths (they return before any GPU work, so no GPU
 * is needed).  Prints "ok" and exits 0 when every answer is as documented. */
#include <stdio.h>
#include <string.h>

#include "decode_attn.h"

static int fails = 0;
#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++fails;                                                   \
    }                                                            \
  } while (0)

int main(void) {
  /* split counts for batch keys {16, 32, 64} x buckets of 4096 tokens */
  const int32_t table[3][4] = {{1, 2, 4, 8}, {1, 1, 2, 4}, {1, 1, 1, 2}};
  const int32_t keys[3] = {16, 32, 64};
  CHECK(decode_attn_pick_splits(&table[0][0], keys, 3, 4, 4096, 16, 4096) == 1);
  CHECK(decode_attn_pick_splits(&table[0][0], keys, 3, 4, 4096, 16, 4097) == 2);
  CHECK(decode_attn_pick_splits(&table[0][0], keys, 3, 4, 4096, 64, 1 << 20) == 2); /* last bucket */
  CHECK(decode_attn_pick_splits(&table[0][0], keys, 3, 4, 4096, 40, 16384) == 4);  /* 40 -> key 32 */
  /* keys out of order: an error, reported as a negative status */
  const int32_t bad_keys[3] = {32, 16, 64};
  CHECK(decode_attn_pick_splits(&table[0][0], bad_keys, 3, 4, 4096, 16, 100) < 0);

  CHECK(decode_attn_strerror(DA_OK) != NULL);
  CHECK(strlen(decode_attn_strerror(DA_ERR_INVALID_ARG)) > 0);
  CHECK(strlen(decode_attn_strerror(DA_ERR_UNSUPPORTED)) > 0);

  /* null pointers are rejected before anything is enqueued */
  CHECK(decode_attn_merge(NULL, NULL, 1, 1, 8, 128, 4, NULL, NULL, DA_BF16, NULL, NULL) ==
        DA_ERR_INVALID_ARG);
  CHECK(decode_attn_split(NULL, DA_BF16, NULL, NULL, NULL, 16, 16, NULL, NULL, 1, 1, 8, 2, 128,
                          64, 16, DA_KV_HND, 4, NULL, NULL, 0, 0.088f, 0, NULL, NULL, NULL) ==
        DA_ERR_INVALID_ARG);

  if (fails) return 1;
  printf("ok\n");
  return 0;
}
