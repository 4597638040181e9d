// Host block pool and block-table growth.
//
// "Fast Attention Kernels and Operator Fusion", §Paged Attention Kernels: the
// KV cache is cut into fixed-size blocks, handed out as requests grow, given
// back when a request finishes, and possibly held by several sequences that
// begin with the same tokens; a sequence's block table maps its logical
// blocks to physical ones.  The pool is a LIFO stack of free ids plus one reference count per
// block.  All operations validate completely before changing anything.

#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "mi_attn.h"
#include "status.h"

struct attn_pool {
  int32_t num_blocks;
  int32_t block_size;
  std::vector<int32_t> free_stack;  // top = back()
  std::vector<int32_t> refcount;    // 0 = free
};

extern "C" int attn_pool_create(int32_t num_blocks, int32_t block_size, attn_pool** out) {
  if (!out) return mi_attn::fail(ATTN_E_INVALID, "attn_pool_create: out is NULL");
  *out = nullptr;
  if (num_blocks < 1) return mi_attn::fail(ATTN_E_INVALID, "attn_pool_create: num_blocks must be >= 1");
  if (block_size < 1) return mi_attn::fail(ATTN_E_INVALID, "attn_pool_create: block_size must be >= 1");
  attn_pool* p = new (std::nothrow) attn_pool;
  if (!p) return mi_attn::fail(ATTN_E_NOMEM, "attn_pool_create: host allocation failed");
  try {
    p->num_blocks = num_blocks;
    p->block_size = block_size;
    p->refcount.assign(num_blocks, 0);
    p->free_stack.resize(num_blocks);
    // the first pop returns 0, then 1, ...
    for (int32_t i = 0; i < num_blocks; ++i) p->free_stack[i] = num_blocks - 1 - i;
  } catch (...) {
    delete p;
    return mi_attn::fail(ATTN_E_NOMEM, "attn_pool_create: host allocation failed");
  }
  *out = p;
  return mi_attn::ok();
}

extern "C" void attn_pool_destroy(attn_pool* pool) { delete pool; }

extern "C" int attn_pool_alloc(attn_pool* pool, int32_t n, int32_t* out_ids) {
  if (!pool) return mi_attn::fail(ATTN_E_INVALID, "attn_pool_alloc: pool is NULL");
  if (n < 0) return mi_attn::fail(ATTN_E_INVALID, "attn_pool_alloc: n < 0");
  if (n > 0 && !out_ids) return mi_attn::fail(ATTN_E_INVALID, "attn_pool_alloc: out_ids is NULL");
  if ((size_t)n > pool->free_stack.size())
    return mi_attn::fail(ATTN_E_NOMEM, "attn_pool_alloc: %d blocks requested, %zu free", n,
                         pool->free_stack.size());
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = pool->free_stack.back();
    pool->free_stack.pop_back();
    pool->refcount[id] = 1;
    out_ids[i] = id;
  }
  return mi_attn::ok();
}

// Checks that every id is in range and that the ids (with repetitions) can be
// released or retained.  For release, an id listed r times needs refcount >= r.
static int check_ids(const attn_pool* pool, const int32_t* ids, int32_t n, bool release, const char* fn) {
  if (!pool) return mi_attn::fail(ATTN_E_INVALID, "%s: pool is NULL", fn);
  if (n < 0) return mi_attn::fail(ATTN_E_INVALID, "%s: n < 0", fn);
  if (n > 0 && !ids) return mi_attn::fail(ATTN_E_INVALID, "%s: ids is NULL", fn);
  std::unordered_map<int32_t, int32_t> uses;
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = ids[i];
    if (id < 0 || id >= pool->num_blocks)
      return mi_attn::fail(ATTN_E_INVALID, "%s: id %d out of range [0, %d)", fn, id, pool->num_blocks);
    int32_t r = ++uses[id];
    if (release && r > pool->refcount[id])
      return mi_attn::fail(ATTN_E_STATE, "%s: block %d released more often than referenced", fn, id);
    if (!release && pool->refcount[id] == 0)
      return mi_attn::fail(ATTN_E_STATE, "%s: block %d is free", fn, id);
  }
  return ATTN_OK;
}

extern "C" int attn_pool_free(attn_pool* pool, const int32_t* ids, int32_t n) {
  int st = check_ids(pool, ids, n, true, "attn_pool_free");
  if (st != ATTN_OK) return st;
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = ids[i];
    if (--pool->refcount[id] == 0) pool->free_stack.push_back(id);
  }
  return mi_attn::ok();
}

extern "C" int attn_pool_retain(attn_pool* pool, const int32_t* ids, int32_t n) {
  int st = check_ids(pool, ids, n, false, "attn_pool_retain");
  if (st != ATTN_OK) return st;
  for (int32_t i = 0; i < n; ++i) ++pool->refcount[ids[i]];
  return mi_attn::ok();
}

extern "C" int32_t attn_pool_num_free(const attn_pool* pool) {
  return pool ? (int32_t)pool->free_stack.size() : ATTN_E_INVALID;
}

extern "C" int32_t attn_pool_num_blocks(const attn_pool* pool) {
  return pool ? pool->num_blocks : ATTN_E_INVALID;
}

extern "C" int attn_pool_refcount(const attn_pool* pool, int32_t id) {
  if (!pool) return mi_attn::fail(ATTN_E_INVALID, "attn_pool_refcount: pool is NULL");
  if (id < 0 || id >= pool->num_blocks)
    return mi_attn::fail(ATTN_E_INVALID, "attn_pool_refcount: id %d out of range", id);
  return pool->refcount[id];
}

extern "C" int attn_seq_reserve(attn_pool* pool, int32_t* row, int32_t max_blocks, int32_t cur_len,
                                int32_t n_new, int32_t* slot_mapping_out) {
  if (!pool) return mi_attn::fail(ATTN_E_INVALID, "attn_seq_reserve: pool is NULL");
  if (!row) return mi_attn::fail(ATTN_E_INVALID, "attn_seq_reserve: block_table_row is NULL");
  if (max_blocks < 0 || cur_len < 0 || n_new < 0)
    return mi_attn::fail(ATTN_E_INVALID, "attn_seq_reserve: negative size");
  const int64_t bs = pool->block_size;
  const int64_t have = (cur_len + bs - 1) / bs;
  const int64_t need = ((int64_t)cur_len + n_new + bs - 1) / bs;
  if (need > max_blocks)
    return mi_attn::fail(ATTN_E_INVALID, "attn_seq_reserve: %lld blocks needed, row holds %d",
                         (long long)need, max_blocks);
  for (int64_t b = 0; b < have; ++b)
    if (row[b] < 0 || row[b] >= pool->num_blocks || pool->refcount[row[b]] == 0)
      return mi_attn::fail(ATTN_E_STATE, "attn_seq_reserve: row entry %lld (%d) is not an allocated block",
                           (long long)b, row[b]);
  const int32_t extra = (int32_t)(need - have);
  if (extra > 0) {
    int st = attn_pool_alloc(pool, extra, row + have);
    if (st != ATTN_OK) return st;
  }
  if (slot_mapping_out)
    for (int32_t i = 0; i < n_new; ++i) {
      int64_t t = (int64_t)cur_len + i;
      slot_mapping_out[i] = (int32_t)(row[t / bs] * bs + t % bs);
    }
  return mi_attn::ok();
}

extern "C" int attn_seq_fork(attn_pool* pool, const int32_t* parent_row, int32_t len, int32_t* child_row,
                             int32_t max_blocks) {
  static const char* fn = "attn_seq_fork";
  if (!pool) return mi_attn::fail(ATTN_E_INVALID, "%s: pool is NULL", fn);
  if (!parent_row || !child_row) return mi_attn::fail(ATTN_E_INVALID, "%s: rows must be non-NULL", fn);
  if (len < 0 || max_blocks < 0) return mi_attn::fail(ATTN_E_INVALID, "%s: negative size", fn);
  const int64_t n = ((int64_t)len + pool->block_size - 1) / pool->block_size;
  if (n > max_blocks)
    return mi_attn::fail(ATTN_E_INVALID, "%s: %lld blocks to share, child row holds %d", fn, (long long)n,
                         max_blocks);
  int st = attn_pool_retain(pool, parent_row, (int32_t)n);  // validates every id first
  if (st != ATTN_OK) return st;
  if (child_row != parent_row) std::memmove(child_row, parent_row, (size_t)n * sizeof(int32_t));
  return mi_attn::ok();
}

extern "C" int attn_seq_reserve_cow(attn_pool* pool, int32_t* row, int32_t max_blocks, int32_t cur_len,
                                    int32_t n_new, int32_t* slot_mapping_out, int32_t* copy_pair_out) {
  static const char* fn = "attn_seq_reserve_cow";
  if (!pool) return mi_attn::fail(ATTN_E_INVALID, "%s: pool is NULL", fn);
  if (!row || !copy_pair_out) return mi_attn::fail(ATTN_E_INVALID, "%s: row and copy_pair_out must be non-NULL", fn);
  if (max_blocks < 0 || cur_len < 0 || n_new < 0) return mi_attn::fail(ATTN_E_INVALID, "%s: negative size", fn);
  const int64_t bs = pool->block_size;
  const int64_t have = (cur_len + bs - 1) / bs;
  const int64_t need = ((int64_t)cur_len + n_new + bs - 1) / bs;
  if (need > max_blocks)
    return mi_attn::fail(ATTN_E_INVALID, "%s: %lld blocks needed, row holds %d", fn, (long long)need, max_blocks);
  for (int64_t b = 0; b < have; ++b)
    if (row[b] < 0 || row[b] >= pool->num_blocks || pool->refcount[row[b]] == 0)
      return mi_attn::fail(ATTN_E_STATE, "%s: row entry %lld (%d) is not an allocated block", fn, (long long)b,
                           row[b]);
  // the next token lands in a partly filled block that another sequence
  // still references: this sequence gets its own copy of it
  const bool cow = n_new > 0 && cur_len % bs != 0 && pool->refcount[row[have - 1]] > 1;
  const int64_t fresh = (need - have) + (cow ? 1 : 0);
  if (fresh > (int64_t)pool->free_stack.size())
    return mi_attn::fail(ATTN_E_NOMEM, "%s: %lld blocks needed, %zu free", fn, (long long)fresh,
                         pool->free_stack.size());
  copy_pair_out[0] = copy_pair_out[1] = -1;
  if (cow) {
    int32_t id;
    attn_pool_alloc(pool, 1, &id);
    const int32_t old = row[have - 1];
    --pool->refcount[old];  // still > 0: another sequence holds it
    row[have - 1] = id;
    copy_pair_out[0] = old;
    copy_pair_out[1] = id;
  }
  return attn_seq_reserve(pool, row, max_blocks, cur_len, n_new, slot_mapping_out);
}
