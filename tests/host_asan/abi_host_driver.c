/* Host-side exercise of the helixdecode C ABI for an AddressSanitizer build
 * of the library (tests/test_host_asan.py builds both).  Only entry points
 * and paths that return before any device work are called: geometry and
 * placement queries, tile offsets, argument checks, and the block-pool
 * allocator under a random sequence of reservations and releases whose
 * tables are checked against the allocator's own free count after every
 * step.  Prints "ok" and exits 0 when every expectation holds. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "helixdecode.h"

static int failures = 0;
#define EXPECT(c)                                                   \
  do {                                                              \
    if (!(c)) {                                                     \
      fprintf(stderr, "line %d: expectation failed: %s\n", __LINE__, #c); \
      ++failures;                                                   \
    }                                                               \
  } while (0)

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void) {   /* xorshift64*: a fixed, seeded sequence */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (uint32_t)((rng * 0x2545f4914f6cdd1dull) >> 32);
}

static void queries(void) {
  const int dtypes[3] = {HX_KV_BF16, HX_KV_FP8_E4M3, HX_KV_MXFP4};
  for (int i = 0; i < 3; ++i) {
    hx_kv_desc d = {8, 3, 2, 128, 128, 0, dtypes[i], 0, 64};
    hx_kv_layout_info lay;
    EXPECT(hx_kv_layout(&d, &lay) == HX_OK);
    for (int which = 0; which < 4; ++which)
      for (int m = 0; m < 16; ++m)
        for (int c = 0; c < 128; ++c) {
          int64_t off2 = -1;
          const hx_status s = hx_kv_tile_offset(&d, which, m, c, &off2);
          EXPECT(s == HX_OK || (which >= 2 && dtypes[i] == HX_KV_BF16));
          if (s == HX_OK) EXPECT(off2 >= 0 && off2 < 2 * (int64_t)lay.k_tile_bytes + 2 * (int64_t)lay.v_tile_bytes);
        }
    int64_t off2;
    EXPECT(hx_kv_tile_offset(&d, 0, 16, 0, &off2) == HX_EINVAL);
    EXPECT(hx_kv_tile_offset(&d, 5, 0, 0, &off2) == HX_EINVAL);
    EXPECT(hx_kv_tile_offset(&d, 0, 0, 0, NULL) == HX_EINVAL);
  }
  hx_kv_desc mla = {4, 1, 1, 576, 512, 1, HX_KV_BF16, 0, 32};
  hx_kv_layout_info lay;
  EXPECT(hx_kv_layout(&mla, &lay) == HX_OK && lay.v_bytes == 0);
  hx_kv_desc bad = {0, 1, 1, 128, 128, 0, HX_KV_BF16, 0, 32};
  EXPECT(hx_kv_layout(&bad, &lay) == HX_EINVAL && strlen(hx_last_error()) > 0);
  bad.P = 4;
  bad.cap = 17;
  EXPECT(hx_kv_layout(&bad, &lay) == HX_EINVAL);
  bad.cap = 32;
  bad.Dk = 64;
  EXPECT(hx_kv_layout(&bad, &lay) == HX_EUNSUPPORTED);
  for (int64_t t = 0; t < 5000; t += 7) {
    int32_t r;
    int64_t j, len, total = 0;
    EXPECT(hx_slot(t, 3, &r, &j) == HX_OK && r >= 0 && r < 3 && j >= 0);
    for (int rr = 0; rr < 3; ++rr) {
      EXPECT(hx_slice_len(t, 3, rr, &len) == HX_OK);
      total += len;
    }
    EXPECT(total == t);
  }
  EXPECT(hx_version() != NULL && strlen(hx_version()) > 0);
}

static void argument_checks(void) {
  /* every call below fails its host-side checks before any launch */
  hx_kv_desc d = {4, 2, 1, 128, 128, 0, HX_KV_BF16, 0, 64};
  hx_kv_cache c = {(void*)0x100000, (void*)0x200000, NULL, NULL};
  hx_kv_cache misaligned = {(void*)0x100004, (void*)0x200000, NULL, NULL};
  int64_t pos[2] = {0, 0}, ctx[2] = {10, 0};
  int32_t cnt[2] = {1, 5};
  EXPECT(hx_kv_append(NULL, &c, (void*)0x300000, (void*)0x400000, NULL, NULL, pos, NULL, 1, NULL) == HX_EINVAL);
  EXPECT(hx_kv_append(&d, &misaligned, (void*)0x300000, (void*)0x400000, NULL, NULL, pos, NULL, 1, NULL) == HX_EINVAL);
  EXPECT(hx_kv_append(&d, &c, (void*)0x300000, (void*)0x400000, NULL, NULL, pos, cnt, 1, NULL) == HX_EINVAL);
  EXPECT(hx_decode_attn_partial(&d, &c, (void*)0x500000, 16, ctx, 0.1f, (float*)0x600000, (float*)0x700000,
                                (void*)0x800000, 1 << 30, NULL) == HX_EINVAL);   /* ctx_len 0 */
  ctx[1] = 10;
  EXPECT(hx_decode_attn_partial(&d, &c, (void*)0x500000, 16, ctx, -1.0f, (float*)0x600000, (float*)0x700000,
                                (void*)0x800000, 1 << 30, NULL) == HX_EINVAL);   /* scale */
  EXPECT(hx_decode_attn(&d, &c, (void*)0x500000, 17, ctx, 0.1f, (float*)0x600000, (float*)0x700000,
                        (void*)0x800000, 1 << 30, NULL) != HX_OK);               /* Hq not a multiple */
  EXPECT(hx_lse_combine(0, 1, 1, 128, (float*)0x600000, (float*)0x700000, (float*)0x800000, (float*)0x900000,
                        NULL) == HX_EINVAL);
  hx_kv_desc fp4 = {4, 2, 1, 128, 128, 0, HX_KV_MXFP4, 0, 64};
  EXPECT(hx_kv_append(&fp4, &c, (void*)0x300000, (void*)0x400000, (void*)0x500000, (void*)0x600000, pos, NULL, 1,
                      NULL) == HX_EINVAL);   /* an MXFP4 cache is one plane: v must be NULL */
  size_t bytes = 0;
  EXPECT(hx_workspace_size(&d, 16, &bytes) == HX_OK && bytes > 0);
  EXPECT(hx_workspace_size(&d, 0, &bytes) != HX_OK);
}

static int count_used(const int32_t* table, int64_t entries) {
  int used = 0;
  for (int64_t i = 0; i < entries; ++i) used += table[i] >= 0;
  return used;
}

static void block_pool(void) {
  const int32_t N = 97;
  hx_kv_desc d = {4, 6, 2, 128, 128, 0, HX_KV_FP8_E4M3, 0, 256};
  const int64_t per_req = (int64_t)d.P * (d.cap / 16), entries = d.B * per_req;
  int32_t* table = (int32_t*)malloc(sizeof(int32_t) * entries);
  int64_t* held = (int64_t*)calloc(d.B, sizeof(int64_t));
  char* seen = (char*)malloc(N);
  for (int64_t i = 0; i < entries; ++i) table[i] = -1;
  hx_block_pool* pool = NULL;
  hx_block_pool* none = NULL;
  EXPECT(hx_block_pool_create(N, &pool) == HX_OK && pool != NULL);
  EXPECT(hx_block_pool_create(0, &none) == HX_EINVAL && none == NULL);
  for (int step = 0; step < 3000; ++step) {
    const int32_t b = (int32_t)(next_u32() % (uint32_t)d.B);
    if (next_u32() % 4 == 0) {
      EXPECT(hx_block_pool_release(pool, &d, table, b) == HX_OK);
      held[b] = 0;
    } else {
      const int64_t n = held[b] + (int64_t)(next_u32() % 200u);
      if (n > (int64_t)d.P * d.cap) continue;
      int32_t taken = -1;
      const hx_status s = hx_block_pool_reserve(pool, &d, table, b, n, &taken);
      EXPECT(s == HX_OK || s == HX_ENOSPC);
      if (s == HX_OK) held[b] = n;
    }
    int32_t n_free = -1;
    EXPECT(hx_block_pool_free_count(pool, &n_free) == HX_OK);
    EXPECT(n_free + count_used(table, entries) == N);
    memset(seen, 0, N);
    for (int64_t i = 0; i < entries; ++i)
      if (table[i] >= 0) {
        EXPECT(table[i] < N && !seen[table[i]]);   /* every block listed once */
        if (table[i] < N) seen[table[i]] = 1;
      }
  }
  /* a foreign block in a request's list is refused and changes nothing */
  for (int32_t b = 0; b < d.B; ++b) EXPECT(hx_block_pool_release(pool, &d, table, b) == HX_OK);
  EXPECT(hx_block_pool_reserve(pool, &d, table, 0, 40, NULL) == HX_OK);
  table[per_req] = table[0];   /* request 1 lists request 0's block */
  EXPECT(hx_block_pool_release(pool, &d, table, 1) == HX_EINVAL);
  table[per_req] = -1;
  EXPECT(hx_block_pool_reserve(pool, &d, table, 0, (int64_t)d.P * d.cap + 1, NULL) == HX_EINVAL);
  hx_block_pool_destroy(pool);
  hx_block_pool_destroy(NULL);
  free(seen);
  free(held);
  free(table);
}

int main(void) {
  queries();
  argument_checks();
  block_pool();
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
