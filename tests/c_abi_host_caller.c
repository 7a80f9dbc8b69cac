/*
 * A plain C11 caller of the host-only part of the library's C ABI (no GPU is
 * touched: every call here returns before any HIP call).  Built and run by
 * tests/test_abi_c_caller.py, which compares what it prints with the Python
 * binding's answers for the same arguments.  Exits non-zero on a failed check.
 */
#include <stdio.h>
#include <string.h>

#include "cosa_osk.h"

static int failures = 0;

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

/* 128K tokens, 32 q heads on 8 KV heads, 64-token pages and blocks, packed
 * [token, head, dim] bfloat16 Q and output, [page, head, token, dim] K and V. */
static cosa_osk_dims_t dims_128k(void) {
  cosa_osk_dims_t d;
  memset(&d, 0, sizeof d);
  d.num_seqs = 1;
  d.num_q_heads = 32;
  d.num_kv_heads = 8;
  d.head_dim = 128;
  d.page_size = 64;
  d.total_q_tokens = 131072;
  d.total_qblocks = 2048;
  d.max_pages_per_seq = 2048;
  d.num_phys_pages = 2048;
  d.max_mask_len = 211;
  d.sm_scale = 0.0f;
  d.block_size = 64;
  d.q_stride_tok = 32 * 128;
  d.q_stride_head = 128;
  d.o_stride_tok = 32 * 128;
  d.o_stride_head = 128;
  d.kv_stride_page = 8 * 64 * 128;
  d.kv_stride_head = 64 * 128;
  d.kv_stride_tok = 128;
  return d;
}

int main(void) {
  CHECK(cosa_abi_version() == COSA_ABI_VERSION);
  CHECK(strcmp(cosa_status_string(COSA_OK), "ok") == 0);
  CHECK(strcmp(cosa_status_string(COSA_ERR_WORKSPACE), cosa_status_string(COSA_ERR_HIP)) != 0);

  cosa_osk_dims_t d = dims_128k();
  const size_t ws = cosa_osk_workspace_bytes(&d);
  CHECK(ws > 0 && ws % 256 == 0);
  CHECK(cosa_osk_workspace_bytes(NULL) == 0);
  CHECK(cosa_osk_check_args(&d, ws) == COSA_OK);
  CHECK(cosa_osk_check_args(&d, ws - 1) == COSA_ERR_WORKSPACE);
  CHECK(cosa_osk_check_args(NULL, ws) == COSA_ERR_INVALID_ARG);
  CHECK(ws <= COSA_OSK_NOALLOC_SCRATCH_BYTES);

  cosa_osk_dims_t bad = d;
  bad.head_dim = 64;
  CHECK(cosa_osk_check_args(&bad, ws) == COSA_ERR_UNSUPPORTED);
  bad = d;
  bad.num_seqs = 0;
  CHECK(cosa_osk_check_args(&bad, ws) == COSA_ERR_INVALID_ARG);
  bad = d;
  bad.num_q_heads = 30; /* not a multiple of the KV heads */
  CHECK(cosa_osk_check_args(&bad, ws) == COSA_ERR_UNSUPPORTED);
  bad = d;
  bad.kv_stride_tok = 100; /* not a multiple of 8 elements */
  CHECK(cosa_osk_check_args(&bad, ws) == COSA_ERR_INVALID_ARG);

  /* null operands are rejected before anything is launched */
  CHECK(cosa_osk_prefill(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 100.0f, NULL, NULL, NULL, NULL,
                         NULL, ws, NULL) == COSA_ERR_INVALID_ARG);

  const int32_t w_proxy = cosa_order_mask_width(2048, 0.1f, COSA_FORCE_FIRST | COSA_FORCE_DIAG);
  const int32_t w_kap = cosa_kap_mask_width(2048, COSA_KAP_FRACTION, 0.1f);
  const int32_t w_union = cosa_union_mask_width(2048, 4, 0.1f, COSA_FORCE_FIRST | COSA_FORCE_DIAG);
  CHECK(w_proxy > 0 && w_kap > 0 && w_union >= w_proxy);
  d.max_mask_len = w_proxy;
  printf("workspace %zu\n", cosa_osk_workspace_bytes(&d));
  printf("builder_workspace %zu\n", cosa_build_order_mask_workspace_bytes(&d));
  printf("order_mask_width %d\n", (int)w_proxy);
  printf("kap_mask_width %d\n", (int)w_kap);
  printf("union_mask_width %d\n", (int)w_union);
  return failures == 0 ? 0 : 1;
}
