// Host-side block allocator of pool caches (hx_block_pool_*): a free list of
// block ids and the edits of per-(request, slice) block lists.  A slice of a
// request holding n tokens needs one block per 16-row group of its rows,
// ceil(slice_len(n) / 16) of them (Helix summary, paragraph on Helix's two
// layouts: the 16-token group is the unit that rotates over the slices).
// No device work and no device memory here.

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "hx_common.h"

struct hx_block_pool {
  std::mutex mu;
  int32_t n = 0;
  std::vector<int32_t> free_ids;   // stack: back() is handed out next
  std::vector<int32_t> owner;      // request + 1 holding the block, 0 when free
  std::vector<uint32_t> seen;      // duplicate check: seen[id] == epoch once id was met in this scan
  uint32_t epoch = 0;
};

namespace hx {
namespace {

hx_status check_table_args(const hx_block_pool* pool, const hx_kv_desc* desc, const int32_t* table, int32_t b) {
  if (!pool || !desc || !table) return fail(HX_EINVAL, "null argument");
  Geometry g;
  hx_status s = geometry(*desc, &g);
  if (s) return s;
  if (b < 0 || b >= desc->B) return fail(HX_EINVAL, "request %d out of range [0, %d)", b, desc->B);
  return HX_OK;
}

// Whether `id` is a block of this pool handed to request b.
bool held_by(const hx_block_pool& p, int32_t id, int32_t b) { return id >= 0 && id < p.n && p.owner[id] == b + 1; }

// Every entry of request b's lists (rows, m entries) other than -1 must be a
// block handed to request b, listed once.  O(m), no allocation: a block is
// marked with the scan's epoch when first met.  Appends the ids to `ids`
// when given.  Caller holds the pool's lock.
hx_status check_request_entries(hx_block_pool& p, const int32_t* rows, int64_t m, int32_t b,
                                std::vector<int32_t>* ids) {
  if (++p.epoch == 0) {   // wrapped: clear the marks once every 2^32 scans
    std::fill(p.seen.begin(), p.seen.end(), 0u);
    p.epoch = 1;
  }
  for (int64_t i = 0; i < m; ++i) {
    const int32_t id = rows[i];
    if (id == -1) continue;
    if (!held_by(p, id, b))
      return fail(HX_EINVAL, "table entry %lld of request %d = %d is not a block of this pool held by it", (long long)i,
                  b, id);
    if (p.seen[id] == p.epoch) return fail(HX_EINVAL, "request %d lists block %d twice", b, id);
    p.seen[id] = p.epoch;
    if (ids) ids->push_back(id);
  }
  return HX_OK;
}

}  // namespace
}  // namespace hx

using namespace hx;

extern "C" {

hx_status hx_block_pool_create(int32_t num_blocks, hx_block_pool** out) {
  clear_error();
  if (!out) return fail(HX_EINVAL, "null argument");
  *out = nullptr;
  if (num_blocks < 1) return fail(HX_EINVAL, "num_blocks=%d must be >= 1", num_blocks);
  hx_block_pool* p = new (std::nothrow) hx_block_pool;
  if (!p) return fail(HX_ENOSPC, "out of host memory");
  try {
    p->n = num_blocks;
    p->free_ids.resize(num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i) p->free_ids[i] = num_blocks - 1 - i;   // 0 first
    p->owner.assign(num_blocks, 0);
    p->seen.assign(num_blocks, 0u);
  } catch (...) {
    delete p;
    return fail(HX_ENOSPC, "out of host memory");
  }
  *out = p;
  return HX_OK;
}

void hx_block_pool_destroy(hx_block_pool* pool) { delete pool; }

hx_status hx_block_pool_free_count(const hx_block_pool* pool, int32_t* n_free) {
  clear_error();
  if (!pool || !n_free) return fail(HX_EINVAL, "null argument");
  std::lock_guard<std::mutex> lk(const_cast<hx_block_pool*>(pool)->mu);
  *n_free = (int32_t)pool->free_ids.size();
  return HX_OK;
}

hx_status hx_block_pool_reserve(hx_block_pool* pool, const hx_kv_desc* desc, int32_t* table_host, int32_t b,
                                int64_t n, int32_t* n_taken) {
  clear_error();
  hx_status s = check_table_args(pool, desc, table_host, b);
  if (s) return s;
  const hx_kv_desc& d = *desc;
  if (n < 0 || n > (int64_t)d.P * d.cap)
    return fail(HX_EINVAL, "n=%lld must be in [0, P*cap=%lld]", (long long)n, (long long)d.P * d.cap);
  const int64_t capc = d.cap / kChunk;
  std::lock_guard<std::mutex> lk(pool->mu);
  // the request's lists as they stand must be valid (as hx_block_pool_release
  // requires): blocks of this request, none listed twice
  s = check_request_entries(*pool, table_host + (int64_t)b * d.P * capc, (int64_t)d.P * capc, b, nullptr);
  if (s) return s;
  int64_t need = 0;
  for (int r = 0; r < d.P; ++r) {
    const int32_t* row = table_host + ((int64_t)b * d.P + r) * capc;
    const int64_t groups = (slice_len(n, d.P, r) + kChunk - 1) / kChunk;
    for (int64_t c = 0; c < groups; ++c)
      if (row[c] == -1) ++need;
  }
  if (need > (int64_t)pool->free_ids.size())
    return fail(HX_ENOSPC, "request %d needs %lld more blocks, %zu free", b, (long long)need, pool->free_ids.size());
  for (int r = 0; r < d.P; ++r) {
    int32_t* row = table_host + ((int64_t)b * d.P + r) * capc;
    const int64_t groups = (slice_len(n, d.P, r) + kChunk - 1) / kChunk;
    for (int64_t c = 0; c < groups; ++c) {
      if (row[c] != -1) continue;
      const int32_t id = pool->free_ids.back();
      pool->free_ids.pop_back();
      pool->owner[id] = b + 1;
      row[c] = id;
    }
  }
  if (n_taken) *n_taken = (int32_t)need;
  return HX_OK;
}

hx_status hx_block_pool_release(hx_block_pool* pool, const hx_kv_desc* desc, int32_t* table_host, int32_t b) {
  clear_error();
  hx_status s = check_table_args(pool, desc, table_host, b);
  if (s) return s;
  const hx_kv_desc& d = *desc;
  const int64_t capc = d.cap / kChunk;
  int32_t* rows = table_host + (int64_t)b * d.P * capc;
  const int64_t m = (int64_t)d.P * capc;
  std::lock_guard<std::mutex> lk(pool->mu);
  // check every entry first
  std::vector<int32_t> ids;
  s = check_request_entries(*pool, rows, m, b, &ids);
  if (s) return s;
  // free in reverse list order, so the request's first block is handed out first again
  for (auto it = ids.rbegin(); it != ids.rend(); ++it) {
    pool->owner[*it] = 0;
    pool->free_ids.push_back(*it);
  }
  for (int64_t i = 0; i < m; ++i) rows[i] = -1;
  return HX_OK;
}

}  // extern "C"
