/* Deterministic stress of the host-only entry points of include/fd.h, meant
 * to run under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_host_sanitizers.py): random and extreme sequence lengths,
 * batch sizes, head counts, split caps and CU counts go through
 * fd_plan_splits and the workspace-size functions, and every result is
 * checked against what the header documents. No call reaches the device
 * (num_cus is always given). Prints "stress ok <calls>" on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "fd.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void) { /* xorshift64* */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (uint32_t)((state * 0x2545F4914F6CDD1Dull) >> 32);
}

static int pick(const int* v, int n) { return v[next_u32() % (uint32_t)n]; }

#define CHECK(cond, ...)                      \
  do {                                        \
    if (!(cond)) {                            \
      fprintf(stderr, "FAIL line %d: ", __LINE__); \
      fprintf(stderr, __VA_ARGS__);           \
      fprintf(stderr, "\n");                  \
      return 1;                               \
    }                                         \
  } while (0)

int main(void) {
  static int32_t lens[70000];
  const int dims[] = {16, 32, 64, 128};
  const int dtypes[] = {FD_F32, FD_F16, FD_BF16};
  const int groups[] = {1, 2, 3, 4, 7, 8, 9, 16, 64};
  const int cus_list[] = {1, 7, 80, 256, 304, 1024};
  const int caps[] = {0, 1, 2, 16, 128, 1000, FD_MAX_SPLITS, FD_MAX_SPLITS + 5, -3};
  long calls = 0;

  for (int it = 0; it < 4000; ++it) {
    const int batch = (it % 50 == 0) ? 1 + (int)(next_u32() % 70000u) : 1 + (int)(next_u32() % 300u);
    const int kv_heads = 1 + (int)(next_u32() % 8u);
    const int group = pick(groups, (int)(sizeof groups / sizeof *groups));
    const int heads = kv_heads * group;
    const int dim = pick(dims, 4);
    const int dtype = pick(dtypes, 3);
    const int cus = pick(cus_list, (int)(sizeof cus_list / sizeof *cus_list));
    const int cap = pick(caps, (int)(sizeof caps / sizeof *caps));
    const uint32_t mode = next_u32() % 6u;
    int32_t min_len = INT32_MAX;
    int any_empty = 0;
    for (int b = 0; b < batch; ++b) {
      int32_t L;
      switch (mode) {
        case 0: L = 1 + (int32_t)(next_u32() % 64u); break;
        case 1: L = 1 + (int32_t)(next_u32() % 40000u); break;
        case 2: L = (int32_t)(next_u32() % 3u); break;                /* empties */
        case 3: L = INT32_MAX - (int32_t)(next_u32() % 4u); break;    /* extreme */
        case 4: L = 4096; break;                                      /* uniform */
        default: L = 1 + (int32_t)(next_u32() % 2000000u); break;
      }
      lens[b] = L;
      if (L < 1) any_empty = 1;
      if (L < min_len) min_len = L;
    }
    int ns = -7;
    const int st = fd_plan_splits(batch, heads, kv_heads, dim, dtype, lens, cus, cap, &ns);
    ++calls;
    if (group > FD_MAX_GROUP) {
      CHECK(st == FD_ERR_UNSUPPORTED, "group %d st %d", group, st);
      continue;
    }
    if (any_empty) {
      CHECK(st == FD_ERR_EMPTY_SPLIT, "empty length accepted: st %d", st);
      continue;
    }
    CHECK(st == FD_OK, "st %d batch %d heads %d kvh %d dim %d", st, batch, heads, kv_heads, dim);
    const int limit = (cap <= 0 || cap > FD_MAX_SPLITS) ? FD_MAX_SPLITS : cap;
    CHECK(ns >= 1 && ns <= limit, "ns %d outside [1, %d]", ns, limit);
    CHECK(ns <= min_len, "ns %d > shortest sequence %d", ns, (int)min_len);

    /* workspace sizes: zero for bad arguments, monotone in the split count */
    const size_t w1 = fd_workspace_bytes(batch, heads, ns, dim);
    const size_t w2 = fd_workspace_bytes(batch, heads, ns + 1 <= FD_MAX_SPLITS ? ns + 1 : ns, dim);
    const size_t u1 = fd_workspace_bytes_unnorm(batch, heads, ns, dim);
    calls += 3;
    CHECK(w1 > 0 && w2 >= w1 && u1 > 0, "workspace %zu %zu %zu", w1, w2, u1);
    CHECK(w1 >= (size_t)batch * heads * ns * ((size_t)dim + 1) * 4, "workspace too small");

    /* the recommended schedule: a known schedule and a split count within
       bounds; the static recommendation is fd_plan_splits's own count */
    int sched = -1, ns2 = -7;
    const int st2 = fd_plan_schedule(batch, heads, kv_heads, dim, dtype, lens, cus, cap, &sched,
                                     &ns2);
    ++calls;
    CHECK(st2 == FD_OK, "plan_schedule st %d", st2);
    CHECK(sched == FD_SCHED_STATIC || sched == FD_SCHED_STEAL || sched == FD_SCHED_QUEUE,
          "schedule %d", sched);
    CHECK(ns2 >= 1 && ns2 <= limit, "plan_schedule ns %d outside [1, %d]", ns2, limit);
    if (sched == FD_SCHED_QUEUE) CHECK(ns2 <= min_len, "queue ns %d > shortest %d", ns2, (int)min_len);
    if (sched == FD_SCHED_STATIC) CHECK(ns2 == ns, "static ns %d vs %d", ns2, ns);
    if (sched == FD_SCHED_STEAL) CHECK(dim == 128 && ns2 % 4 == 0, "steal ns %d dim %d", ns2, dim);
  }

  /* argument edges */
  int ns = 0;
  lens[0] = 10;
  CHECK(fd_plan_splits(0, 8, 1, 128, FD_F16, lens, 256, 0, &ns) == FD_ERR_INVALID_ARG, "batch 0");
  CHECK(fd_plan_splits(1, 8, 3, 128, FD_F16, lens, 256, 0, &ns) == FD_ERR_INVALID_ARG, "8 heads over 3");
  CHECK(fd_plan_splits(1, 8, 1, 96, FD_F16, lens, 256, 0, &ns) == FD_ERR_UNSUPPORTED, "dim 96");
  CHECK(fd_plan_splits(1, 8, 1, 128, 7, lens, 256, 0, &ns) == FD_ERR_UNSUPPORTED, "dtype 7");
  CHECK(fd_plan_splits(1, 8, 1, 128, FD_F16, NULL, 256, 0, &ns) == FD_ERR_INVALID_ARG, "null");
  CHECK(fd_plan_splits(1, 8, 1, 128, FD_F16, lens, -1, 0, &ns) == FD_ERR_INVALID_ARG, "cus -1");
  {
    int sched = 0;
    CHECK(fd_plan_schedule(1, 8, 1, 128, FD_F16, lens, 256, 0, NULL, &ns) == FD_ERR_INVALID_ARG,
          "null schedule");
    CHECK(fd_plan_schedule(1, 8, 1, 128, FD_F16, lens, 256, 0, &sched, NULL) == FD_ERR_INVALID_ARG,
          "null count");
    CHECK(fd_plan_schedule(1, 8, 1, 128, FD_F16, NULL, 256, 0, &sched, &ns) == FD_ERR_INVALID_ARG,
          "null lengths");
  }
  CHECK(fd_workspace_bytes(INT32_MAX, INT32_MAX, FD_MAX_SPLITS, 128) == 0, "overflow size");
  CHECK(fd_workspace_bytes(1, 1, FD_MAX_SPLITS + 1, 128) == 0, "too many splits");
  CHECK(fd_workspace_bytes_unnorm(1, 1, 2, 100) == 0, "bad dim");
  calls += 9;
  for (int s = -2; s < 8; ++s) CHECK(fd_status_string(s) != NULL, "status string %d", s);

  printf("stress ok %ld\n", calls);
  return 0;
}
