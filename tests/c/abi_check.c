/* Plain C99 user of include/fd.h: the header compiles as C, the library
 * links from C, and the host-only entry points behave as documented
 * (no GPU needed: nothing here reaches the device). Prints one result per
 * line for tests/test_c_abi.py to check. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "fd.h"

int main(void) {
  int32_t lens[4] = {4096, 4096, 4096, 4096};
  int ns = -1;
  int st = fd_plan_splits(4, 32, 32, 128, FD_F16, lens, 256, 0, &ns);
  printf("plan %d %d\n", st, ns);

  int32_t empty[2] = {5, 0};
  st = fd_plan_splits(2, 8, 1, 128, FD_F16, empty, 256, 0, &ns);
  printf("plan_empty %d\n", st);

  int32_t longs[16];
  for (int i = 0; i < 16; ++i) longs[i] = 131072;
  int planned = -1;
  st = fd_plan_schedule(16, 32, 8, 128, FD_BF16, longs, 256, 0, &planned, &ns);
  printf("plan_sched %d %d %d\n", st, planned, ns);

  printf("ws %zu\n", fd_workspace_bytes(2, 8, 4, 128));
  /* argument order (batch, heads, num_splits, dim): 128 splits of dim 64
   * and 64 splits of dim 128 need different sizes, so a swap shows */
  printf("ws_order %zu %zu\n", fd_workspace_bytes(1, 1, 128, 64), fd_workspace_bytes(1, 1, 64, 128));
  printf("ws_unnorm %zu\n", fd_workspace_bytes_unnorm(2, 8, 4, 128));
  printf("ws_unnorm_order %zu %zu\n", fd_workspace_bytes_unnorm(1, 1, 128, 64),
         fd_workspace_bytes_unnorm(1, 1, 64, 128));
  printf("ws_bad %zu\n", fd_workspace_bytes(1, 8, 4, 100));

  /* argument checks run before anything touches the device */
  st = fd_decode_attention(NULL, NULL, NULL, NULL, 1, 8, 1, 128, 2, 0.1f, NULL, NULL, NULL,
                           FD_F16, NULL);
  printf("null_args %d\n", st);
  st = fd_decode_attention_unnorm((const void*)16, (const void*)16, (const void*)16,
                                  (const int32_t*)16, 1, 8, 1, 96, 2, 0.1f, (void*)16,
                                  (void*)16, NULL, FD_F16, NULL);
  printf("bad_dim %d\n", st);
  st = fd_decode_split((const void*)16, (const void*)16, (const void*)16, (const int32_t*)16,
                       1, 8, 1, 128, 2, NAN, (void*)16, NULL, FD_F16, NULL);
  printf("nan_scale %d\n", st);
  st = fd_decode_combine(NULL, 1, 8, 128, 2, (void*)16, NULL, FD_F16);
  printf("combine_null %d\n", st);

  printf("status %s\n", fd_status_string(FD_ERR_EMPTY_SPLIT));
  int prev = fd_set_kernel_path(FD_PATH_VALU);
  printf("path %d %d %d\n", prev, fd_set_kernel_path(prev), fd_set_kernel_path(42));
  const int sched = fd_set_schedule(FD_SCHED_QUEUE);
  printf("sched %d %d %d\n", sched, fd_set_schedule(sched), fd_set_schedule(42));
  const int comb = fd_set_combine(FD_COMBINE_FUSED);
  printf("combine %d %d %d\n", comb, fd_set_combine(comb), fd_set_combine(42));
  return 0;
}
