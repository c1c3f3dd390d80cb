/* C client of the library's ABI: compiled by gcc as C11 against include/paged_attn.h and
 * linked to libsapaged.so.  It calls only entry points that need no GPU and prints
 * what they return, one "key value..." line each, for tests/test_c_abi_cpu.py. */
#include <stdio.h>
#include <string.h>

#include "paged_attn.h"

int main(void) {
  printf("version %s\n", pa_version());

  /* launch plan of a GQA-4 decode shape: B=64, Hq=32, Hkv=8, D=128, P=16, 512 table columns */
  int32_t plan[6];
  int rc = paged_attn_plan(64, 1, 32, 8, 128, 16, 512, 0, 0, plan);
  printf("plan %d %d %d %d %d %d %d\n", rc, plan[0], plan[1], plan[2], plan[3], plan[4], plan[5]);
  printf("workspace %zu\n", paged_attn_workspace_size(64, 1, 32, 8, 128, 16, 512, 0, 0));
  printf("width %d %d\n", paged_attn_window_width(4096, 16, 16, 2048), paged_attn_window_width(0, 4, 16, 99));

  /* host describe of two requests, window 20, query_len 4, page 16, 2 splits */
  const int32_t table[2 * 7] = {5, 9, 2, 11, 7, 3, 0, 8, 1, 4, 6, 10, 12, 13};
  const int32_t lens[2] = {100, 37};
  int32_t out_lens[2], out_table[2 * 3], ranges[2 * 2 * 4];
  rc = paged_attn_describe_host(table, 7, 7, lens, 2, 4, 4, 1, 64, 16, 20, 2, out_lens, out_table, 3, ranges);
  printf("describe %d lens %d %d table", rc, out_lens[0], out_lens[1]);
  for (int i = 0; i < 6; ++i) printf(" %d", out_table[i]);
  printf(" ranges");
  for (int i = 0; i < 16; ++i) printf(" %d", ranges[i]);
  printf("\n");

  /* argument errors come back as status codes with a message, before anything is enqueued */
  pa_kv_desc kv;
  memset(&kv, 0, sizeof kv);
  kv.page_size = 16;
  kv.num_kv_heads = 1;
  kv.num_pages = 1;
  kv.dtype = PA_BF16;
  kv.k_scale = kv.v_scale = 1.0f;
  kv.page_stride = 16 * 2 * 64;
  kv.head_stride = 16 * 2 * 64;
  kv.token_stride = 2 * 64;
  rc = paged_attn_run(NULL, PA_F32, &kv, NULL, 7, 7, NULL, 1, 1, 4, 64, 0.125f, 0, 1, NULL, PA_BF16,
                      NULL, NULL, 0, NULL);
  printf("bad_dtype %d %s\n", rc, pa_last_error());
  rc = paged_attn_run(NULL, PA_BF16, &kv, NULL, 7, 7, NULL, 0, 1, 4, 64, 0.125f, 0, 1, NULL, PA_BF16,
                      NULL, NULL, 0, NULL);
  printf("empty %d\n", rc);
  return 0;
}
