// C ABI of libpa, host half (declared in include/pa.h): the refcounted block
// pool with copy-on-write, prefix caching and swap bookkeeping, plus the
// status calls every entry point shares.  Plain C++ with no HIP dependency:
// it is linked into libpa.so and also built on its own for the host
// sanitizers (address and undefined behaviour), which run the pool-against-
// model suites on it.  Every entry point checks its arguments and reports
// failures through pa_status plus a thread-local message; nothing throws
// across the ABI.
#include <algorithm>
#include <cstring>
#include <new>
#include <string>

#include "pa.h"
#include "pool.hpp"
#include "status.hpp"

struct pa_pool {
  pa::BlockPool impl;
  pa_pool(int32_t n, int32_t b, uint64_t seed, bool caching, int32_t host)
      : impl(n, b, seed, caching, host) {}
};

namespace pa {

namespace {
thread_local std::string g_err;
}  // namespace

pa_status fail(pa_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

pa_status ok() {
  g_err.clear();
  return PA_OK;
}

}  // namespace pa

using pa::fail;
using pa::ok;

extern "C" {

const char* pa_last_error(void) { return pa::g_err.c_str(); }

const char* pa_version(void) { return "libpa 0.2 gfx950"; }


pa_status pa_pool_create_ex(int32_t num_blocks, int32_t block_size, uint64_t seed, uint32_t flags,
                            int32_t num_host_blocks, pa_pool** out) {
  if (!out) return fail(PA_EINVAL, "pa_pool_create: out is null");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0 || num_host_blocks < 0)
    return fail(PA_EINVAL, "pa_pool_create: num_blocks and block_size must be positive, num_host_blocks >= 0");
  if (flags & ~static_cast<uint32_t>(PA_POOL_PREFIX_CACHING))
    return fail(PA_EINVAL, "pa_pool_create_ex: unknown flags");
  pa_pool* p = new (std::nothrow)
      pa_pool(num_blocks, block_size, seed, (flags & PA_POOL_PREFIX_CACHING) != 0, num_host_blocks);
  if (!p) return fail(PA_ENOMEM, "pa_pool_create: host allocation failed");
  *out = p;
  return ok();
}

pa_status pa_pool_create(int32_t num_blocks, int32_t block_size, uint64_t seed, pa_pool** out) {
  return pa_pool_create_ex(num_blocks, block_size, seed, 0, 0, out);
}

void pa_pool_destroy(pa_pool* pool) { delete pool; }

int32_t pa_pool_num_free(const pa_pool* pool) { return pool ? pool->impl.num_free() : -1; }

int32_t pa_pool_num_blocks(const pa_pool* pool) { return pool ? pool->impl.num_blocks() : -1; }

int32_t pa_pool_num_cached(const pa_pool* pool) { return pool ? pool->impl.num_cached() : -1; }

int32_t pa_pool_num_free_host(const pa_pool* pool) { return pool ? pool->impl.num_free_host() : -1; }

int32_t pa_block_refcount(const pa_pool* pool, int32_t block) {
  return pool ? pool->impl.refcount(block) : -1;
}

pa_status pa_seq_create(pa_pool* pool, int64_t* seq_id) {
  if (!pool || !seq_id) return fail(PA_EINVAL, "pa_seq_create: null pointer");
  *seq_id = pool->impl.create();
  return ok();
}

pa_status pa_seq_fork(pa_pool* pool, int64_t parent, int64_t* child) {
  if (!pool || !child) return fail(PA_EINVAL, "pa_seq_fork: null pointer");
  std::string err;
  if (pool->impl.fork(parent, child, &err) != pa::PoolResult::kOk) return fail(PA_EINVAL, err);
  return ok();
}

namespace {

pa_status seq_append(const char* fn, pa_pool* pool, int64_t seq, const int32_t* tokens, int32_t n_tokens,
                     int32_t max_hit, int64_t* slot_mapping_out, int32_t* cow_pairs_out, int32_t cow_cap,
                     int32_t* n_cow, int32_t* n_hit) {
  if (!pool || !n_cow || !n_hit) return fail(PA_EINVAL, std::string(fn) + ": null pointer");
  if (n_tokens > 0 && !slot_mapping_out) return fail(PA_EINVAL, std::string(fn) + ": slot_mapping_out is null");
  if (cow_cap < 1 || !cow_pairs_out)
    return fail(PA_EINVAL, std::string(fn) + ": cow_pairs_out must hold at least one pair");
  std::string err;
  int32_t src = -1, dst = -1;
  const pa::PoolResult r =
      pool->impl.append(seq, n_tokens, tokens, max_hit, slot_mapping_out, &src, &dst, n_cow, n_hit, &err);
  if (r == pa::PoolResult::kNoMemory) return fail(PA_ENOMEM, err);
  if (r != pa::PoolResult::kOk) return fail(PA_EINVAL, err);
  if (*n_cow) {
    cow_pairs_out[0] = src;
    cow_pairs_out[1] = dst;
  }
  return ok();
}

}  // namespace

pa_status pa_seq_append(pa_pool* pool, int64_t seq, int32_t n_tokens, int64_t* slot_mapping_out,
                        int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow) {
  int32_t n_hit = 0;
  return seq_append("pa_seq_append", pool, seq, nullptr, n_tokens, 0, slot_mapping_out, cow_pairs_out,
                    cow_cap, n_cow, &n_hit);
}

pa_status pa_seq_fork_many(pa_pool* pool, const int64_t* parents, int32_t n, int64_t* children_out,
                           int32_t* n_done) {
  if (!pool || !n_done || (n > 0 && (!parents || !children_out)))
    return fail(PA_EINVAL, "pa_seq_fork_many: null pointer");
  *n_done = 0;
  if (n < 0) return fail(PA_EINVAL, "pa_seq_fork_many: negative count");
  for (int32_t i = 0; i < n; ++i) {
    std::string err;
    if (pool->impl.fork(parents[i], &children_out[i], &err) != pa::PoolResult::kOk) return fail(PA_EINVAL, err);
    *n_done = i + 1;
  }
  return ok();
}

pa_status pa_seq_free_many(pa_pool* pool, const int64_t* seqs, int32_t n, int32_t* n_done) {
  if (!pool || !n_done || (n > 0 && !seqs)) return fail(PA_EINVAL, "pa_seq_free_many: null pointer");
  *n_done = 0;
  if (n < 0) return fail(PA_EINVAL, "pa_seq_free_many: negative count");
  for (int32_t i = 0; i < n; ++i) {
    std::string err;
    if (pool->impl.release(seqs[i], &err) != pa::PoolResult::kOk) return fail(PA_EINVAL, err);
    *n_done = i + 1;
  }
  return ok();
}

pa_status pa_seq_append_many(pa_pool* pool, const int64_t* seqs, const int32_t* n_tokens, int32_t n,
                             int64_t* slot_mapping_out, int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow,
                             int32_t* n_done) {
  if (!pool || !n_cow || !n_done || (n > 0 && (!seqs || !n_tokens)))
    return fail(PA_EINVAL, "pa_seq_append_many: null pointer");
  *n_cow = 0;
  *n_done = 0;
  if (n < 0) return fail(PA_EINVAL, "pa_seq_append_many: negative count");
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) total += n_tokens[i] > 0 ? n_tokens[i] : 0;
  if (total > 0 && !slot_mapping_out) return fail(PA_EINVAL, "pa_seq_append_many: slot_mapping_out is null");
  if (cow_cap < 0 || (cow_cap > 0 && !cow_pairs_out))
    return fail(PA_EINVAL, "pa_seq_append_many: bad cow_pairs_out / cow_cap");
  int64_t at = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (*n_cow >= cow_cap)
      return fail(PA_EINVAL, "pa_seq_append_many: cow_pairs_out full (size it for one pair per sequence)");
    std::string err;
    int32_t src = -1, dst = -1, one = 0, hit = 0;
    const pa::PoolResult r = pool->impl.append(seqs[i], n_tokens[i], nullptr, 0, slot_mapping_out + at, &src,
                                               &dst, &one, &hit, &err);
    if (r == pa::PoolResult::kNoMemory) return fail(PA_ENOMEM, err);
    if (r != pa::PoolResult::kOk) return fail(PA_EINVAL, err);
    if (one) {
      cow_pairs_out[2 * *n_cow] = src;
      cow_pairs_out[2 * *n_cow + 1] = dst;
      ++*n_cow;
    }
    at += n_tokens[i];
    *n_done = i + 1;
  }
  return ok();
}

pa_status pa_seq_append_tokens(pa_pool* pool, int64_t seq, const int32_t* token_ids, int32_t n_tokens,
                               int32_t max_hit_tokens, int64_t* slot_mapping_out, int32_t* cow_pairs_out,
                               int32_t cow_cap, int32_t* n_cow, int32_t* n_hit) {
  if (n_tokens > 0 && !token_ids) return fail(PA_EINVAL, "pa_seq_append_tokens: token_ids is null");
  return seq_append("pa_seq_append_tokens", pool, seq, token_ids, n_tokens, max_hit_tokens, slot_mapping_out,
                    cow_pairs_out, cow_cap, n_cow, n_hit);
}

pa_status pa_seq_swap_out(pa_pool* pool, int64_t seq, int32_t* pairs_out, int32_t cap, int32_t* n_pairs) {
  if (!pool || !n_pairs || (cap > 0 && !pairs_out)) return fail(PA_EINVAL, "pa_seq_swap_out: null pointer");
  std::string err;
  const pa::PoolResult r = pool->impl.swap_out(seq, pairs_out, cap, n_pairs, &err);
  if (r == pa::PoolResult::kNoMemory) return fail(PA_ENOMEM, err);
  if (r != pa::PoolResult::kOk) return fail(PA_EINVAL, err);
  return ok();
}

pa_status pa_seq_swap_in(pa_pool* pool, int64_t seq, int32_t* pairs_out, int32_t cap, int32_t* n_pairs) {
  if (!pool || !n_pairs || (cap > 0 && !pairs_out)) return fail(PA_EINVAL, "pa_seq_swap_in: null pointer");
  std::string err;
  const pa::PoolResult r = pool->impl.swap_in(seq, pairs_out, cap, n_pairs, &err);
  if (r == pa::PoolResult::kNoMemory) return fail(PA_ENOMEM, err);
  if (r != pa::PoolResult::kOk) return fail(PA_EINVAL, err);
  return ok();
}

pa_status pa_seq_free(pa_pool* pool, int64_t seq) {
  if (!pool) return fail(PA_EINVAL, "pa_seq_free: null pool");
  std::string err;
  if (pool->impl.release(seq, &err) != pa::PoolResult::kOk) return fail(PA_EINVAL, err);
  return ok();
}

pa_status pa_seq_block_table(const pa_pool* pool, int64_t seq, int32_t* out, int32_t cap,
                             int32_t* n_blocks, int32_t* n_tokens) {
  if (!pool || !n_blocks || !n_tokens) return fail(PA_EINVAL, "pa_seq_block_table: null pointer");
  const std::vector<int32_t>* t = pool->impl.table(seq);
  if (!t) return fail(PA_EINVAL, "pa_seq_block_table: unknown sequence " + std::to_string(seq));
  *n_blocks = static_cast<int32_t>(t->size());
  *n_tokens = static_cast<int32_t>(pool->impl.num_tokens(seq));
  if (cap > 0 && !out) return fail(PA_EINVAL, "pa_seq_block_table: out is null");
  const int32_t n = std::min<int32_t>(cap, *n_blocks);
  if (n > 0) std::memcpy(out, t->data(), sizeof(int32_t) * n);
  return ok();
}

pa_status pa_seq_block_tables(const pa_pool* pool, const int64_t* seq_ids, int32_t n, int32_t* out,
                              int32_t stride, int32_t pad, int32_t* ctx_out) {
  if (!pool || (n > 0 && (!seq_ids || !out))) return fail(PA_EINVAL, "pa_seq_block_tables: null pointer");
  if (n < 0 || stride <= 0) return fail(PA_EINVAL, "pa_seq_block_tables: bad size");
  for (int32_t i = 0; i < n; ++i) {
    const std::vector<int32_t>* t = pool->impl.table(seq_ids[i]);
    if (!t) return fail(PA_EINVAL, "pa_seq_block_tables: unknown sequence " + std::to_string(seq_ids[i]));
    if (static_cast<int64_t>(t->size()) > stride)
      return fail(PA_EINVAL, "pa_seq_block_tables: table longer than stride");
  }
  for (int32_t i = 0; i < n; ++i) {
    const std::vector<int32_t>* t = pool->impl.table(seq_ids[i]);
    int32_t* row = out + static_cast<int64_t>(i) * stride;
    const int32_t nb = static_cast<int32_t>(t->size());
    if (nb) std::memcpy(row, t->data(), sizeof(int32_t) * nb);
    for (int32_t j = nb; j < stride; ++j) row[j] = pad;
    if (ctx_out) ctx_out[i] = static_cast<int32_t>(pool->impl.num_tokens(seq_ids[i]));
  }
  return ok();
}

}  // extern "C"
