/* A plain C99 caller of the library: include/pa.h must compile as C, and libpa.so must
 * link and answer its host-only entry points (no GPU, no torch).  Prints one line per
 * check and exits non-zero on the first failure. */
#include <stdint.h>
#include <stdio.h>

#include "pa.h"

#define CHECK(cond, what)                                   \
  do {                                                      \
    if (!(cond)) {                                          \
      printf("FAIL %s\n", what);                            \
      return 1;                                             \
    }                                                       \
    printf("ok %s\n", what);                                \
  } while (0)

int main(void) {
  /* the batch-64 Llama-3-8B shape: J = ceil(3360 / 256) = 14 partitions */
  const size_t rows = (size_t)64 * 32 * 14;
  const size_t want = 2 * ((rows * 4 + 255) / 256 * 256) + (rows * 128 * 4 + 255) / 256 * 256;
  CHECK(pa_decode_workspace_bytes(64, 32, 128, 3360, 0) == want, "workspace bytes");
  CHECK(pa_default_partition_tokens() == 256, "default partition");
  CHECK(pa_partition_tokens_for(4095) == 256 && pa_partition_tokens_for(4096) == 512, "partition for long contexts");
  CHECK(pa_status_str(PA_ERR_SHAPE)[0] == 'P', "status string");

  pa_kv_cache cache = {64, 16, 2, 64, PA_BF16, 1.0f, 1.0f};
  /* host-checkable contract violations return before anything is enqueued */
  CHECK(pa_write_kv(NULL, NULL, PA_BF16, 1, NULL, NULL, NULL, &cache, NULL) == PA_ERR_NULL, "write null");
  cache.head_dim = 96;
  CHECK(pa_decode((void*)16, PA_BF16, 1, 2, (void*)16, (void*)16, &cache, (void*)16, 4, (void*)16, 64, 0.1f,
                  (void*)16, NULL, 0, 0, PA_KERNEL_AUTO, NULL) == PA_ERR_UNSUPPORTED, "decode head_dim");

  /* host-side contract checks on host arrays */
  const int32_t tables[2][3] = {{3, 1, 0}, {2, 5, 4}};
  const int32_t lens[2] = {20, 40};
  int64_t bad = 0;
  CHECK(pa_check_decode_inputs(&tables[0][0], 3, lens, 2, 48, 6, 16, &bad) == PA_OK && bad == -1, "tables pass");
  CHECK(pa_check_decode_inputs(&tables[0][0], 3, lens, 2, 48, 5, 16, &bad) == PA_ERR_SHAPE && bad == 4,
        "block 5 outside a 5-block pool");
  const int32_t slots[5] = {5, 9, -1, 9, 2};
  CHECK(pa_check_slots(slots, 5, 8, 4, &bad) == PA_ERR_SHAPE && bad == 3, "repeated slot");
  return 0;
}
