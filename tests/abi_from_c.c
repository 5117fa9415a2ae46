/* Calls libstdspec through its C header only (no Python, no GPU): every
 * call below fails a host-side check before any launch, so this runs on a
 * machine without a GPU.  Prints one line per check and exits non-zero on
 * the first unexpected status. */
#include <stdio.h>
#include <string.h>

#include "stdspec.h"

static int failures = 0;

static void expect(const char* what, std_status_t got, std_status_t want) {
  if (got != want) {
    printf("FAIL %s: %s (%s), want %s\n", what, std_status_str(got), std_last_error(),
           std_status_str(want));
    ++failures;
  } else {
    printf("ok   %s: %s\n", what, std_status_str(got));
  }
}

int main(void) {
  const void* fake = (const void*)0x10000;  /* aligned, never dereferenced */
  std_attn_shape_t shape = {28, 4, 128, 0.088f};
  std_kv_t kv = {fake, fake, 1000, 900, STD_DTYPE_BF16};
  std_vis_t vis = {0, 800};

  if (std_abi_version() != STD_ABI_VERSION) {
    printf("FAIL abi version %d != %d\n", std_abi_version(), STD_ABI_VERSION);
    return 1;
  }
  /* the four calls of the hot path, each stopped by a check */
  expect("select: topk 0", std_select_topk(&shape, fake, 800, 64, &kv, vis, 0, NULL, (int32_t*)fake,
                                           NULL, NULL, 0, NULL), STD_ERR_INVALID_ARGUMENT);
  expect("sparse: empty workspace", std_sparse_decode_attn(&shape, fake, &kv, vis, (const int32_t*)fake,
                                                           64, (void*)fake, NULL, 0, NULL),
         STD_ERR_WORKSPACE_TOO_SMALL);
  expect("dense: n_q past len", std_dense_verify_attn(&shape, fake, 901, &kv, (void*)fake, NULL, 0, NULL),
         STD_ERR_INVALID_ARGUMENT);
  expect("accept: vocab 0", std_accept((const int32_t*)fake, 3, fake, 0, STD_DTYPE_F32, (int32_t*)fake,
                                       (int32_t*)fake, NULL, NULL, NULL), STD_ERR_INVALID_ARGUMENT);
  /* a shape the library does not implement */
  std_attn_shape_t d96 = {28, 4, 96, 0.1f};
  expect("dense: head_dim 96", std_dense_verify_attn(&d96, fake, 7, &kv, (void*)fake, NULL, 0, NULL),
         STD_ERR_UNSUPPORTED);
  /* workspace queries agree with their calls */
  size_t ws = std_dense_verify_workspace(&shape, 7, &kv);
  printf("%s dense workspace %zu bytes\n", ws > 0 ? "ok  " : "FAIL", ws);
  if (ws == 0) ++failures;
  if (std_dense_verify_workspace(&shape, 901, &kv) != 0 || strlen(std_last_error()) == 0) {
    printf("FAIL workspace query accepted n_q past len\n");
    ++failures;
  }
  /* the streaming comparator's lists and the no-alloc call check first too */
  expect("static window: sink < 0", std_static_window_idx(4, vis, -1, 64, (int32_t*)fake, NULL),
         STD_ERR_INVALID_ARGUMENT);
  expect("no-alloc: topk past span", std_sparse_decode_attn_noalloc(&shape, fake, &kv, NULL, 0, vis,
                                                                    (const int32_t*)fake, 801,
                                                                    (void*)fake, NULL),
         STD_ERR_INVALID_ARGUMENT);
  printf("%d failure(s)\n", failures);
  return failures ? 1 : 0;
}
