/*
 * A plain C99 consumer of include/gqa.h: it includes nothing but the header
 * and the C library, calls every declared entry point by name and checks the
 * host-side answers that need no GPU (NULL buffers are rejected with
 * GQA_ERR_INVALID_ARG before anything is enqueued; workspace sizes are
 * positive; version and error strings are set).  Built with
 * `gcc -std=c99 -pedantic -Wall -Wextra -Werror`, linked against libgqa.so
 * and run by tests/test_abi.py.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gqa.h"

static int failures = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    fprintf(stderr, "FAIL: %s (last error: %s)\n", what, gqa_last_error());
    ++failures;
  }
}

#define REJECTS(call) expect((call) == GQA_ERR_INVALID_ARG, #call)

int main(void) {
  const double theta = 1e6;
  const float scale = 0.125f;
  double ms = -1.0;
  int64_t count = -1;
  int64_t start[1] = {0};

  REJECTS(gqa_rope_apply(NULL, GQA_BF16, 1, 1, 1, 128, 0, theta, NULL));
  expect(strlen(gqa_last_error()) > 0, "gqa_last_error after a rejection");

  expect(gqa_prefill_workspace_size(GQA_BF16, 4, 4096, 4, 128) > 0,
         "gqa_prefill_workspace_size");
  REJECTS(gqa_prefill(NULL, NULL, NULL, NULL, GQA_BF16, GQA_F32, 1, 16, 28, 4, 128, theta,
                      scale, 1, NULL, NULL, 0, NULL, 0, NULL));

  expect(gqa_decode_workspace_size(32, 28, 4, 128, 32768) > 0, "gqa_decode_workspace_size");
  REJECTS(gqa_decode(NULL, NULL, NULL, NULL, GQA_BF16, GQA_F32, 1, 28, 4, 128, 16, 16, 16,
                     theta, scale, NULL, 0, NULL));

  REJECTS(gqa_decode_noalloc(NULL, NULL, NULL, NULL, GQA_BF16, GQA_F32, 1, 28, 4, 128, 16, 16,
                             16, theta, scale, NULL));
  {
    /* a step past the static scratch is refused before anything touches the
     * device, so addresses that are never dereferenced serve here */
    void* fake = (void*)(uintptr_t)4096;
    expect(gqa_decode_noalloc(fake, fake, fake, fake, GQA_BF16, GQA_F32, 32, 28, 4, 128,
                              1048576, 1048576, 1048576, theta, scale, NULL) ==
               GQA_ERR_UNSUPPORTED &&
               strstr(gqa_last_error(), "scratch") != NULL,
           "gqa_decode_noalloc past GQA_DECODE_NOALLOC_SCRATCH_BYTES");
  }

  expect(gqa_prefill_chunk_workspace_size(GQA_BF16, 1, 4096, 4, 128) > 0,
         "gqa_prefill_chunk_workspace_size");
  REJECTS(gqa_prefill_chunk(NULL, NULL, NULL, NULL, GQA_BF16, GQA_F32, 1, 16, 28, 4, 128, start,
                            NULL, 16, theta, scale, 0, NULL, NULL, 16, NULL, 0, NULL));
  REJECTS(gqa_decode_ragged(NULL, NULL, NULL, NULL, GQA_BF16, GQA_F32, 1, 28, 4, 128, 16, NULL,
                            NULL, 16, theta, scale, 0, NULL, 0, NULL));
  REJECTS(gqa_decode_append(NULL, NULL, NULL, NULL, NULL, NULL, GQA_BF16, GQA_F32, 1, 28, 4, 128,
                            16, NULL, 0, theta, scale, NULL, 0, NULL));
  REJECTS(gqa_qkv_epilogue(NULL, NULL, NULL, NULL, NULL, GQA_BF16, 1, 16, 28, 4, 128, 16, start,
                           NULL, 16, theta, NULL));

  expect(gqa_decode_paged_workspace_size(32, 28, 4, 128, 32768) > 0,
         "gqa_decode_paged_workspace_size");
  REJECTS(gqa_decode_paged(NULL, NULL, NULL, NULL, NULL, NULL, GQA_BF16, GQA_F32, 1, 28, 4, 128,
                           16, 1, NULL, 1, NULL, NULL, 16, theta, scale, 0, NULL, 0, NULL));

  REJECTS(gqa_set_rope_yarn(0.5, 32768.0, 32.0, 1.0));
  expect(gqa_set_rope_yarn(1.0, 0.0, 32.0, 1.0) == GQA_OK, "gqa_set_rope_yarn(1, ...)");

  expect(strstr(gqa_version(), "gfx950") != NULL, "gqa_version");

  expect(gqa_timing_enable(0) == GQA_OK, "gqa_timing_enable");
  expect(gqa_timing_read(0, &ms, &count) == GQA_OK && count == 0 && ms == 0.0,
         "gqa_timing_read with nothing recorded");
  expect(gqa_timing_read(3, &ms, &count) == GQA_OK && count == 0,
         "gqa_timing_read of whole decode calls");
  REJECTS(gqa_timing_read(4, &ms, &count));

  REJECTS(gqa_stream_read(NULL, 16, NULL, NULL));

  if (failures == 0) printf("c99 consumer ok\n");
  return failures == 0 ? 0 : 1;
}
