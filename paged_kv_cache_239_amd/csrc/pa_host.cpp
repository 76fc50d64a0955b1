// Pool carving and the host block manager: FIFO free list, per-block
// reference counts, fork / append / free and the copy-on-write decision.
//
// Sources ("vLLM PagedAttention and continuous batching", netleverage.com):
//   section "PagedAttention: fixed blocks, non-contiguous physical memory" --
//     one contiguous device allocation sliced into physical blocks; a block
//     table per sequence filled left to right; a new block only when the
//     previous one is full;
//   section "Sharing with reference counts and copy-on-write" -- refcounts,
//     copy of a shared block on write, release at count zero, the fork /
//     append / free policies.
// Readings where the pages are silent: FIFO free list seeded by a caller
// permutation (release appends at the tail, which keeps a freed address out
// of circulation for as long as possible); batch order decides which of
// several sharers copies (every writer that finds count > 1 copies, the one
// that finds count == 1 writes in place).
//
// Pure host C++ (no HIP), so it also builds with g++ alone for host tests.

#include <cstdio>
#include <cstring>
#include <limits>
#include <new>
#include <string>
#include <vector>

#include "pa_internal.h"

namespace pa_detail {

static thread_local std::string g_last_error;

pa_status fail(pa_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

void clear_error() { g_last_error.clear(); }

}  // namespace pa_detail

using pa_detail::fail;

namespace {

bool mul_ok(size_t a, size_t b, size_t* out) {
  if (a != 0 && b > std::numeric_limits<size_t>::max() / a) return false;
  *out = a * b;
  return true;
}

// Bytes of one layer's K (or V) slab; false on overflow or bad arguments.
bool slab_size(int Hkv, int d, int B, int P, size_t* tile, size_t* slab) {
  if (Hkv <= 0 || d <= 0 || B <= 0 || P <= 0) return false;
  size_t t = 2;
  if (!mul_ok(t, (size_t)Hkv, &t) || !mul_ok(t, (size_t)B, &t) || !mul_ok(t, (size_t)d, &t))
    return false;
  size_t s;
  if (!mul_ok(t, (size_t)P, &s)) return false;
  *tile = t;
  *slab = s;
  return true;
}

pa_status check_pool(const pa_pool* pool) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  return PA_OK;
}

bool in_range(const pa_pool* pool, int32_t blk) { return blk >= 0 && blk < pool->P; }

// --- FIFO free list --------------------------------------------------------
int32_t fifo_pop(pa_pool* pool) {
  int32_t blk = pool->ring[(size_t)pool->head];
  pool->head = (pool->head + 1) % pool->P;
  pool->nfree -= 1;
  return blk;
}

void fifo_push(pa_pool* pool, int32_t blk) {
  int64_t tail = (pool->head + pool->nfree) % pool->P;
  pool->ring[(size_t)tail] = blk;
  pool->nfree += 1;
}

// --- primitives (arguments already validated) --------------------------------
int32_t do_alloc(pa_pool* pool) {
  int32_t blk = fifo_pop(pool);
  pool->ref[(size_t)blk] = 1;
  pool->allocs += 1;
  int32_t live = pool->P - pool->nfree;
  if (live > pool->live_high_water) pool->live_high_water = live;
  return blk;
}

void do_decref(pa_pool* pool, int32_t blk) {
  int32_t& r = pool->ref[(size_t)blk];
  r -= 1;
  if (r == 0) {
    fifo_push(pool, blk);
    pool->releases += 1;
  }
}

// One append; the a1 rule.  Leaves everything unchanged on error.
pa_status do_append(pa_pool* pool, int32_t* table, int32_t maxb, int32_t n_before,
                    int64_t* slot, int32_t* cow_src, int32_t* cow_dst) {
  *cow_src = -1;
  *cow_dst = -1;
  if (n_before < 0) return fail(PA_ERR_INVALID_ARG, "negative sequence length");
  const int32_t idx = n_before / pool->B;
  const int32_t off = n_before % pool->B;
  if (idx >= maxb) return fail(PA_ERR_INVALID_ARG, "block table too short for the new token");
  if (off == 0) {
    if (pool->nfree == 0) return fail(PA_ERR_OUT_OF_BLOCKS, "no free physical block");
    const int32_t blk = do_alloc(pool);
    table[idx] = blk;
    *slot = (int64_t)blk * pool->B;
    return PA_OK;
  }
  const int32_t last = table[idx];
  if (!in_range(pool, last)) return fail(PA_ERR_INVALID_ARG, "table entry outside the pool");
  if (pool->ref[(size_t)last] == 0) return fail(PA_ERR_INVALID_ARG, "table maps a free block");
  if (pool->ref[(size_t)last] > 1) {
    if (pool->nfree == 0) return fail(PA_ERR_OUT_OF_BLOCKS, "no free block for copy-on-write");
    const int32_t fresh = do_alloc(pool);
    do_decref(pool, last);  // count was > 1, so the old block stays live
    table[idx] = fresh;
    pool->cows += 1;
    *cow_src = last;
    *cow_dst = fresh;
    *slot = (int64_t)fresh * pool->B + off;
    return PA_OK;
  }
  *slot = (int64_t)last * pool->B + off;
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_last_error(void) { return pa_detail::g_last_error.c_str(); }

const char* pa_version(void) { return "pa 0.1.0 gfx950"; }

size_t pa_pool_bytes(int L, int Hkv, int d, int B, int P, pa_dtype dtype) {
  if (L <= 0 || (dtype != PA_F16 && dtype != PA_BF16)) return 0;
  size_t tile, slab, total;
  if (!slab_size(Hkv, d, B, P, &tile, &slab)) return 0;
  if (!mul_ok(slab, (size_t)2 * (size_t)L, &total)) return 0;
  return total;
}

pa_status pa_alloc_pool(pa_pool** out, int L, int Hkv, int d, int B, int P, pa_dtype dtype,
                        void* dev_base, size_t dev_bytes, const int32_t* free_order) {
  pa_detail::clear_error();
  if (!out) return fail(PA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (dtype != PA_F16 && dtype != PA_BF16) return fail(PA_ERR_INVALID_ARG, "unknown dtype");
  if (L <= 0) return fail(PA_ERR_INVALID_ARG, "L must be positive");
  size_t tile, slab;
  if (!slab_size(Hkv, d, B, P, &tile, &slab))
    return fail(PA_ERR_INVALID_ARG, "Hkv, d, B and P must be positive and their product must fit");
  const size_t need = pa_pool_bytes(L, Hkv, d, B, P, dtype);
  if (need == 0) return fail(PA_ERR_INVALID_ARG, "pool size overflows");
  if (!dev_base) return fail(PA_ERR_INVALID_ARG, "dev_base is NULL");
  if (reinterpret_cast<uintptr_t>(dev_base) % 256 != 0)
    return fail(PA_ERR_INVALID_ARG, "dev_base must be 256-byte aligned");
  if (dev_bytes < need) return fail(PA_ERR_INVALID_ARG, "device buffer smaller than pa_pool_bytes");

  pa_pool* pool = new (std::nothrow) pa_pool();
  if (!pool) return fail(PA_ERR_INVALID_ARG, "host allocation failed");
  pool->L = L;
  pool->Hkv = Hkv;
  pool->d = d;
  pool->B = B;
  pool->P = P;
  pool->dtype = dtype;
  pool->base = static_cast<char*>(dev_base);
  pool->bytes = dev_bytes;
  pool->tile_bytes = tile;
  pool->slab_bytes = slab;
  try {
    pool->ref.assign((size_t)P, 0);
    pool->ring.assign((size_t)P, 0);
  } catch (...) {
    delete pool;
    return fail(PA_ERR_INVALID_ARG, "host allocation failed");
  }
  if (free_order) {
    std::vector<char> seen((size_t)P, 0);
    for (int i = 0; i < P; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= P || seen[(size_t)b]) {
        delete pool;
        return fail(PA_ERR_INVALID_ARG, "free_order is not a permutation of 0..P-1");
      }
      seen[(size_t)b] = 1;
      pool->ring[(size_t)i] = b;
    }
  } else {
    for (int i = 0; i < P; ++i) pool->ring[(size_t)i] = i;
  }
  pool->head = 0;
  pool->nfree = P;
  *out = pool;
  return PA_OK;
}

void pa_free_pool(pa_pool* pool) { delete pool; }

pa_status pa_pool_layer_ptrs(const pa_pool* pool, int layer, void** k_slab, void** v_slab) {
  pa_detail::clear_error();
  if (pa_status st = check_pool(pool)) return st;
  if (layer < 0 || layer >= pool->L) return fail(PA_ERR_INVALID_ARG, "layer out of range");
  if (k_slab) *k_slab = pool->k_slab(layer);
  if (v_slab) *v_slab = pool->v_slab(layer);
  return PA_OK;
}

pa_status pa_block_alloc(pa_pool* pool, int32_t* blk) {
  pa_detail::clear_error();
  if (pa_status st = check_pool(pool)) return st;
  if (!blk) return fail(PA_ERR_INVALID_ARG, "blk is NULL");
  if (pool->nfree == 0) return fail(PA_ERR_OUT_OF_BLOCKS, "no free physical block");
  *blk = do_alloc(pool);
  return PA_OK;
}

pa_status pa_block_incref(pa_pool* pool, int32_t blk) {
  pa_detail::clear_error();
  if (pa_status st = check_pool(pool)) return st;
  if (!in_range(pool, blk)) return fail(PA_ERR_INVALID_ARG, "block outside the pool");
  if (pool->ref[(size_t)blk] == 0) return fail(PA_ERR_INVALID_ARG, "incref of a free block");
  pool->ref[(size_t)blk] += 1;
  return PA_OK;
}

pa_status pa_block_decref(pa_pool* pool, int32_t blk) {
  pa_detail::clear_error();
  if (pa_status st = check_pool(pool)) return st;
  if (!in_range(pool, blk)) return fail(PA_ERR_INVALID_ARG, "block outside the pool");
  if (pool->ref[(size_t)blk] == 0) return fail(PA_ERR_INVALID_ARG, "decref of a free block (double free)");
  do_decref(pool, blk);
  return PA_OK;
}

int32_t pa_block_refcount(const pa_pool* pool, int32_t blk) {
  if (!pool || !in_range(pool, blk)) return -1;
  return pool->ref[(size_t)blk];
}

int32_t pa_num_free_blocks(const pa_pool* pool) { return pool ? pool->nfree : -1; }

pa_status pa_free_list(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* count) {
  pa_detail::clear_error();
  if (pa_status st = check_pool(pool)) return st;
  if (count) *count = pool->nfree;
  if (!out && cap > 0) return fail(PA_ERR_INVALID_ARG, "out is NULL");
  const int32_t n = pool->nfree < cap ? pool->nfree : cap;
  for (int32_t i = 0; i < n; ++i) out[i] = pool->ring[(size_t)((pool->head + i) % pool->P)];
  return PA_OK;
}

pa_status pa_pool_get_stats(const pa_pool* pool, pa_pool_stats* stats) {
  pa_detail::clear_error();
  if (pa_status st = check_pool(pool)) return st;
  if (!stats) return fail(PA_ERR_INVALID_ARG, "stats is NULL");
  stats->allocs = pool->allocs;
  stats->cows = pool->cows;
  stats->releases = pool->releases;
  stats->live_blocks = pool->P - pool->nfree;
  stats->live_high_water = pool->live_high_water;
  stats->free_blocks = pool->nfree;
  stats->num_blocks = pool->P;
  return PA_OK;
}

pa_status pa_append_slot(pa_pool* pool, int32_t* table, int32_t maxb, int32_t n_before,
                         int64_t* slot, int32_t* cow_src, int32_t* cow_dst) {
  pa_detail::clear_error();
  if (pa_status st = check_pool(pool)) return st;
  if (!table || !slot || !cow_src || !cow_dst) return fail(PA_ERR_INVALID_ARG, "NULL argument");
  if (maxb <= 0) return fail(PA_ERR_INVALID_ARG, "maxb must be positive");
  return do_append(pool, table, maxb, n_before, slot, cow_src, cow_dst);
}

pa_status pa_append_tokens(pa_pool* pool, int32_t* table, int32_t maxb, int32_t n_before,
                           int32_t count, int64_t* slots, int32_t* cow_pairs, int32_t* n_pairs,
                           int32_t* n_done) {
  pa_detail::clear_error();
  if (n_pairs) *n_pairs = 0;
  if (n_done) *n_done = 0;
  if (pa_status st = check_pool(pool)) return st;
  if (!table) return fail(PA_ERR_INVALID_ARG, "table is NULL");
  if (maxb <= 0 || count < 0 || n_before < 0)
    return fail(PA_ERR_INVALID_ARG, "bad maxb, count or n_before");
  if ((int64_t)n_before + count > (int64_t)std::numeric_limits<int32_t>::max())
    return fail(PA_ERR_INVALID_ARG, "length overflows int32");
  int32_t pairs = 0;
  for (int32_t i = 0; i < count; ++i) {
    int64_t slot;
    int32_t src, dst;
    pa_status st = do_append(pool, table, maxb, n_before + i, &slot, &src, &dst);
    if (st != PA_OK) {
      if (n_done) *n_done = i;
      if (n_pairs) *n_pairs = pairs;
      return st;
    }
    if (slots) slots[i] = slot;
    if (src >= 0) {
      if (cow_pairs) {
        cow_pairs[2 * pairs] = src;
        cow_pairs[2 * pairs + 1] = dst;
      }
      pairs += 1;
    }
  }
  if (n_done) *n_done = count;
  if (n_pairs) *n_pairs = pairs;
  return PA_OK;
}

pa_status pa_append_batch(pa_pool* pool, int32_t* tables, int32_t maxb, const int32_t* n_before,
                          int32_t S, int64_t* slots, int32_t* cow_pairs, int32_t* n_pairs,
                          int32_t* n_done) {
  pa_detail::clear_error();
  if (n_pairs) *n_pairs = 0;
  if (n_done) *n_done = 0;
  if (pa_status st = check_pool(pool)) return st;
  if (S < 0 || maxb <= 0) return fail(PA_ERR_INVALID_ARG, "bad S or maxb");
  if (S > 0 && (!tables || !n_before || !slots)) return fail(PA_ERR_INVALID_ARG, "NULL argument");
  int32_t pairs = 0;
  for (int32_t s = 0; s < S; ++s) {
    int32_t src, dst;
    pa_status st = do_append(pool, tables + (size_t)s * maxb, maxb, n_before[s], &slots[s], &src, &dst);
    if (st != PA_OK) {
      if (n_done) *n_done = s;
      if (n_pairs) *n_pairs = pairs;
      return st;
    }
    if (src >= 0) {
      if (cow_pairs) {
        cow_pairs[2 * pairs] = src;
        cow_pairs[2 * pairs + 1] = dst;
      }
      pairs += 1;
    }
  }
  if (n_done) *n_done = S;
  if (n_pairs) *n_pairs = pairs;
  return PA_OK;
}

pa_status pa_seq_fork(pa_pool* pool, const int32_t* parent_table, int32_t n_tokens,
                      int32_t* child_table, int32_t maxb) {
  pa_detail::clear_error();
  if (pa_status st = check_pool(pool)) return st;
  if (n_tokens < 0 || maxb < 0) return fail(PA_ERR_INVALID_ARG, "bad n_tokens or maxb");
  const int32_t nb = (int32_t)(((int64_t)n_tokens + pool->B - 1) / pool->B);
  if (nb > maxb) return fail(PA_ERR_INVALID_ARG, "table too short for the forked length");
  if (nb > 0 && (!parent_table || !child_table)) return fail(PA_ERR_INVALID_ARG, "NULL table");
  for (int32_t j = 0; j < nb; ++j) {
    const int32_t b = parent_table[j];
    if (!in_range(pool, b)) return fail(PA_ERR_INVALID_ARG, "parent entry outside the pool");
    if (pool->ref[(size_t)b] == 0) return fail(PA_ERR_INVALID_ARG, "parent maps a free block");
  }
  for (int32_t j = 0; j < nb; ++j) {
    const int32_t b = parent_table[j];
    pool->ref[(size_t)b] += 1;
    child_table[j] = b;
  }
  return PA_OK;
}

pa_status pa_seq_free(pa_pool* pool, const int32_t* table, int32_t n_tokens) {
  pa_detail::clear_error();
  if (pa_status st = check_pool(pool)) return st;
  if (n_tokens < 0) return fail(PA_ERR_INVALID_ARG, "negative length");
  const int32_t nb = (int32_t)(((int64_t)n_tokens + pool->B - 1) / pool->B);
  if (nb > 0 && !table) return fail(PA_ERR_INVALID_ARG, "table is NULL");
  // validate first so that nothing changes on error (a table may repeat a block)
  std::vector<std::pair<int32_t, int32_t>> need;  // (block, references to drop)
  for (int32_t j = 0; j < nb; ++j) {
    const int32_t b = table[j];
    if (!in_range(pool, b)) return fail(PA_ERR_INVALID_ARG, "table entry outside the pool");
    bool found = false;
    for (auto& e : need)
      if (e.first == b) {
        e.second += 1;
        found = true;
        break;
      }
    if (!found) need.emplace_back(b, 1);
  }
  for (const auto& e : need)
    if (pool->ref[(size_t)e.first] < e.second)
      return fail(PA_ERR_INVALID_ARG, "block has fewer references than the table holds");
  for (int32_t j = 0; j < nb; ++j) do_decref(pool, table[j]);
  return PA_OK;
}

pa_status pa_seq_reorder(pa_pool* pool, const int32_t* tables, const int32_t* lens, int32_t S_old, int32_t maxb,
                         const int32_t* parents, int32_t S_new, int32_t* out_tables, int32_t* out_lens) {
  pa_detail::clear_error();
  if (pa_status st = check_pool(pool)) return st;
  if (S_old < 0 || S_new < 0 || maxb < 0) return fail(PA_ERR_INVALID_ARG, "negative size");
  if (S_new > 0 && S_old == 0) return fail(PA_ERR_INVALID_ARG, "no sequence to continue");
  if (S_old > 0 && (!tables || !lens)) return fail(PA_ERR_INVALID_ARG, "NULL old tables or lengths");
  if (S_new > 0 && (!parents || !out_tables || !out_lens)) return fail(PA_ERR_INVALID_ARG, "NULL new arrays");
  if (S_new > 0 && S_old > 0 && maxb > 0) {
    const char* a0 = reinterpret_cast<const char*>(tables);
    const char* a1 = a0 + (size_t)S_old * maxb * sizeof(int32_t);
    const char* b0 = reinterpret_cast<const char*>(out_tables);
    const char* b1 = b0 + (size_t)S_new * maxb * sizeof(int32_t);
    if (a0 < b1 && b0 < a1) return fail(PA_ERR_INVALID_ARG, "out_tables overlaps tables");
  }
  // validate everything first: parents, lengths, entries, and that the old
  // tables do not hold more references to a block than it has
  std::vector<int32_t> held((size_t)pool->P, 0);
  for (int32_t s = 0; s < S_old; ++s) {
    const int64_t nb = ((int64_t)lens[s] + pool->B - 1) / pool->B;
    if (lens[s] < 0 || nb > maxb) return fail(PA_ERR_INVALID_ARG, "length outside the table");
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t b = tables[(size_t)s * maxb + j];
      if (!in_range(pool, b)) return fail(PA_ERR_INVALID_ARG, "table entry outside the pool");
      held[(size_t)b] += 1;
    }
  }
  for (int32_t b = 0; b < pool->P; ++b)
    if (held[(size_t)b] > pool->ref[(size_t)b])
      return fail(PA_ERR_INVALID_ARG, "block has fewer references than the tables hold");
  for (int32_t i = 0; i < S_new; ++i)
    if (parents[i] < 0 || parents[i] >= S_old) return fail(PA_ERR_INVALID_ARG, "parent out of range");
  // forks, in new-sequence order
  for (int32_t i = 0; i < S_new; ++i) {
    const int32_t par = parents[i];
    const int32_t n = lens[par];
    const int32_t nb = (int32_t)(((int64_t)n + pool->B - 1) / pool->B);
    const int32_t* src = tables + (size_t)par * maxb;
    int32_t* dst = out_tables + (size_t)i * maxb;
    for (int32_t j = 0; j < nb; ++j) {
      pool->ref[(size_t)src[j]] += 1;
      dst[j] = src[j];
    }
    for (int32_t j = nb; j < maxb; ++j) dst[j] = -1;
    out_lens[i] = n;
  }
  // frees, in old-sequence order
  for (int32_t s = 0; s < S_old; ++s) {
    const int32_t nb = (int32_t)(((int64_t)lens[s] + pool->B - 1) / pool->B);
    for (int32_t j = 0; j < nb; ++j) do_decref(pool, tables[(size_t)s * maxb + j]);
  }
  return PA_OK;
}

pa_status pa_move_blocks(pa_pool* from, pa_pool* to, int32_t* tables, const int32_t* lens, int32_t S, int32_t maxb,
                         int32_t* pairs, int32_t cap, int32_t* n_pairs) {
  pa_detail::clear_error();
  if (pa_status st = check_pool(from)) return st;
  if (pa_status st = check_pool(to)) return st;
  if (from == to) return fail(PA_ERR_INVALID_ARG, "from and to are the same pool");
  if (from->L != to->L || from->Hkv != to->Hkv || from->d != to->d || from->B != to->B || from->dtype != to->dtype)
    return fail(PA_ERR_INVALID_ARG, "pools differ in shape");
  if (!n_pairs) return fail(PA_ERR_INVALID_ARG, "n_pairs is NULL");
  if (S < 0 || maxb < 0 || cap < 0) return fail(PA_ERR_INVALID_ARG, "negative size");
  if (S > 0 && (!tables || !lens)) return fail(PA_ERR_INVALID_ARG, "NULL tables or lengths");
  // distinct blocks in order of first appearance, with the group's references
  std::vector<int32_t> held((size_t)from->P, 0);
  std::vector<int32_t> order;
  for (int32_t s = 0; s < S; ++s) {
    const int64_t nb = ((int64_t)lens[s] + from->B - 1) / from->B;
    if (lens[s] < 0 || nb > maxb) return fail(PA_ERR_INVALID_ARG, "length outside the table");
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t b = tables[(size_t)s * maxb + j];
      if (!in_range(from, b)) return fail(PA_ERR_INVALID_ARG, "table entry outside the pool");
      if (held[(size_t)b]++ == 0) order.push_back(b);
    }
  }
  for (int32_t b : order)
    if (from->ref[(size_t)b] != held[(size_t)b])
      return fail(PA_ERR_INVALID_ARG, "a block of the group is also mapped outside it");
  const int32_t n = (int32_t)order.size();
  if (n > cap || (n > 0 && !pairs)) return fail(PA_ERR_INVALID_ARG, "pairs array too small");
  if (to->nfree < n) return fail(PA_ERR_OUT_OF_BLOCKS, "destination pool has too few free blocks");
  // allocate in `to`, in first-appearance order
  std::vector<int32_t> moved((size_t)from->P, -1);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = order[(size_t)i];
    const int32_t nb = do_alloc(to);
    to->ref[(size_t)nb] = held[(size_t)b];
    moved[(size_t)b] = nb;
    pairs[2 * i] = b;
    pairs[2 * i + 1] = nb;
  }
  // drop the group's references in `from` (as pa_seq_free, sequence by sequence)
  for (int32_t s = 0; s < S; ++s) {
    const int32_t nb = (int32_t)(((int64_t)lens[s] + from->B - 1) / from->B);
    for (int32_t j = 0; j < nb; ++j) do_decref(from, tables[(size_t)s * maxb + j]);
  }
  for (int32_t s = 0; s < S; ++s) {
    const int32_t nb = (int32_t)(((int64_t)lens[s] + from->B - 1) / from->B);
    for (int32_t j = 0; j < nb; ++j) {
      int32_t& e = tables[(size_t)s * maxb + j];
      e = moved[(size_t)e];
    }
  }
  *n_pairs = n;
  return PA_OK;
}

pa_status pa_prefix_groups(const pa_pool* pool, const int32_t* tables, const int32_t* lens, int32_t S, int32_t maxb,
                           int32_t* group_start, int32_t* group_len, int32_t* seq_group, int32_t* n_groups,
                           int32_t* max_group, int32_t* max_shared, int32_t* max_suffix) {
  pa_detail::clear_error();
  if (pa_status st = check_pool(pool)) return st;
  if (S < 0 || maxb < 0) return fail(PA_ERR_INVALID_ARG, "negative size");
  if (!n_groups || !max_group || !max_shared || !max_suffix || !group_start)
    return fail(PA_ERR_INVALID_ARG, "NULL output");
  if (S > 0 && (!tables || !lens || !group_len || !seq_group)) return fail(PA_ERR_INVALID_ARG, "NULL array");
  const int B = pool->B;
  for (int32_t s = 0; s < S; ++s)
    if (lens[s] < 0 || ((int64_t)lens[s] + B - 1) / B > maxb) return fail(PA_ERR_INVALID_ARG, "length outside the table");
  // runs of consecutive sequences with the same first block; a run of one,
  // or one whose shared length rounds to 0, shares nothing.  Consecutive
  // runs that share nothing are joined into one.
  int32_t ng = 0, mg = 0, ms = 0, mx = 0;
  int32_t i = 0;
  while (i < S) {
    int32_t j = i + 1;
    if (lens[i] > 0)
      while (j < S && lens[j] > 0 && tables[(size_t)j * maxb] == tables[(size_t)i * maxb]) ++j;
    int32_t L = 0;
    if (j - i >= 2) {
      int32_t nb = maxb, nmin = lens[i];
      for (int32_t m = i; m < j; ++m) {
        nb = std::min<int32_t>(nb, (lens[m] + B - 1) / B);
        nmin = std::min(nmin, lens[m]);
      }
      int32_t k = 0;
      while (k < nb) {
        bool same = true;
        for (int32_t m = i + 1; m < j && same; ++m) same = tables[(size_t)m * maxb + k] == tables[(size_t)i * maxb + k];
        if (!same) break;
        ++k;
      }
      L = (int32_t)std::min<int64_t>((int64_t)k * B, (int64_t)nmin - 1) & ~15;
    }
    if (L == 0 && ng > 0 && group_len[ng - 1] == 0) {
      // extend the previous run that shares nothing
    } else {
      group_start[ng] = i;
      group_len[ng] = L;
      ++ng;
    }
    for (int32_t m = i; m < j; ++m) {
      seq_group[m] = ng - 1;
      mx = std::max(mx, lens[m] - L);   // positions outside the shared prefix
    }
    if (L > 0) {
      mg = std::max(mg, j - i);
      ms = std::max(ms, L);
    }
    i = j;
  }
  group_start[ng] = S;
  *n_groups = ng;
  *max_group = mg;
  *max_shared = ms;
  *max_suffix = mx;
  return PA_OK;
}

pa_status pa_validate_step(const pa_pool* pool, const int32_t* tables, int32_t maxb, const int32_t* lens, int32_t S,
                           const int64_t* slots, int32_t* bad_seq) {
  pa_detail::clear_error();
  if (pa_status st = check_pool(pool)) return st;
  if (bad_seq) *bad_seq = -1;
  if (S < 0 || maxb <= 0) return fail(PA_ERR_INVALID_ARG, "negative S or maxb below 1");
  if (S > 0 && (!tables || !lens)) return fail(PA_ERR_INVALID_ARG, "NULL array");
  const int B = pool->B;
  auto bad = [&](int32_t s, const std::string& what) {
    if (bad_seq) *bad_seq = s;
    return fail(PA_ERR_INVALID_ARG, "sequence " + std::to_string(s) + ": " + what);
  };
  std::vector<int32_t> held((size_t)pool->P, 0);   // references these tables hold
  for (int32_t s = 0; s < S; ++s) {
    const int32_t n = lens[s];
    if (n < 0) return bad(s, "negative length");
    const int64_t nb = ((int64_t)n + B - 1) / B;
    if (nb > maxb) return bad(s, "length " + std::to_string(n) + " needs more than maxb entries");
    const int32_t* t = tables + (size_t)s * maxb;
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t b = t[j];
      if (!in_range(pool, b)) return bad(s, "entry " + std::to_string(j) + " = " + std::to_string(b) + " outside the pool");
      if (pool->ref[(size_t)b] <= 0) return bad(s, "entry " + std::to_string(j) + " maps free block " + std::to_string(b));
      if (++held[(size_t)b] > pool->ref[(size_t)b])
        return bad(s, "block " + std::to_string(b) + " is mapped more often than its reference count");
    }
    if (slots) {
      const int64_t slot = slots[s];
      if (slot < 0) continue;
      if (n < 1) return bad(s, "a slot for an empty sequence");
      const int32_t b = t[(n - 1) / B];
      const int64_t want = (int64_t)b * B + (n - 1) % B;
      if (slot != want)
        return bad(s, "slot " + std::to_string(slot) + " is not position n-1 (" + std::to_string(want) + ")");
      if (pool->ref[(size_t)b] != 1)
        return bad(s, "the written block " + std::to_string(b) + " is shared (copy-on-write missing)");
    }
  }
  return PA_OK;
}

}  // extern "C"
