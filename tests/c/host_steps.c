/* A plain C11 client of libpkv's host entry points (no GPU work): a pool, block tables
 * and slot mappings, then a small continuous-batching trace through the scheduler.
 * Prints one line per fact; tests/test_c_client.py compiles it with a C compiler and
 * compares the lines with the oracle's values. */
#include <stdio.h>
#include <string.h>

#include "pkv.h"

#define CHECK(x)                                                                    \
  do {                                                                              \
    int rc_ = (x);                                                                  \
    if (rc_ != PKV_OK) {                                                            \
      printf("error %d at line %d: %s\n", rc_, __LINE__, pkv_last_error());         \
      return 1;                                                                     \
    }                                                                               \
  } while (0)

int main(void) {
  /* pool: 8 blocks of 4 tokens, free list 0..7 popped from its end */
  pkv_pool* pool = NULL;
  int64_t plane = 0;
  CHECK(pkv_alloc_pool(8, 4, 2, 64, PKV_BF16, NULL, &pool, &plane));
  printf("plane_bytes %lld\n", (long long)plane);
  CHECK(pkv_seq_reserve(pool, 1, 9));
  CHECK(pkv_seq_reserve(pool, 2, 4));
  int64_t ids[2] = {1, 2};
  int32_t q[2] = {9, 1}, L[2] = {9, 4}, bt[2 * 3], cu[3];
  int64_t slots[10];
  CHECK(pkv_build_block_table(pool, 2, ids, q, L, 3, bt, cu, slots));
  printf("tables %d %d %d | %d %d %d\n", bt[0], bt[1], bt[2], bt[3], bt[4], bt[5]);
  printf("cu %d %d %d\n", cu[0], cu[1], cu[2]);
  printf("slots");
  for (int i = 0; i < 10; ++i) printf(" %lld", (long long)slots[i]);
  printf("\n");
  int32_t got[8];
  int rc = pkv_pool_alloc(pool, 6, got);          /* 4 free: all-or-nothing failure */
  printf("alloc6 %d %s\n", rc, strlen(pkv_last_error()) > 0 ? "message" : "silent");
  int32_t free_blocks = 0, live = 0;
  CHECK(pkv_pool_stats(pool, &free_blocks, &live));
  printf("stats %d %d\n", free_blocks, live);
  CHECK(pkv_seq_release(pool, 1));
  CHECK(pkv_seq_release(pool, 2));
  pkv_destroy_pool(pool);

  /* scheduler: block 4, pool 6, at most 2 running; A(arrive 0, prompt 5, 3 outputs),
   * B(0, 6, 4), C(1, 2, 2) */
  CHECK(pkv_alloc_pool(6, 4, 2, 64, PKV_BF16, NULL, &pool, NULL));
  pkv_sched* s = NULL;
  CHECK(pkv_sched_create(pool, 2, &s));
  int64_t rid[3] = {0, 1, 2};
  int32_t arr[3] = {0, 0, 1}, prompt[3] = {5, 6, 2}, outs[3] = {3, 4, 2};
  CHECK(pkv_sched_add_requests(s, 3, rid, arr, prompt, outs));
  for (int step = 0; step < 16; ++step) {
    int64_t c[8];
    CHECK(pkv_sched_counters(s, c));
    if (c[5] == 3) break;
    int32_t n = 0, tq = 0, mb = 0;
    CHECK(pkv_sched_schedule(s, &n, &tq, &mb));
    int64_t rids[4];
    int32_t st[4], ql[4], sl[4], tab[4 * 4], cq[5];
    int64_t sm[32];
    CHECK(pkv_sched_plan(s, 4, rids, st, ql, sl, tab, cq, sm));
    printf("step %d", step);
    for (int k = 0; k < n; ++k) printf(" %lld:%d:%d:%d", (long long)rids[k], st[k], ql[k], sl[k]);
    CHECK(pkv_sched_update(s));
    CHECK(pkv_sched_counters(s, c));
    printf(" | free %lld running %lld waiting %lld finished %lld\n", (long long)c[1], (long long)c[2],
           (long long)c[3], (long long)c[5]);
  }
  pkv_sched_destroy(s);
  pkv_destroy_pool(pool);
  return 0;
}
