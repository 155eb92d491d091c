// Host-side refcounted KV block pool with copy-on-write.
//
// Blocks are claimed on demand as a sequence grows and released as soon as
// it finishes; forked sequences share blocks by reference count and a shared
// block is copied only when a branch writes into it ("Inside vLLM: How
// PagedAttention Changes Python LLM Inference at the Systems Level", sections
// "PagedAttention: What the OS Figured Out Decades Ago" and "Copy-on-Write
// Makes Beam Search Cheap").  Pure C++, no device code: the pool hands out
// ids; the caller moves data with the copy and write kernels.
//
// Optional prefix caching: the content of each full block is keyed, and a
// request whose leading whole blocks match content already computed reuses
// those physical blocks instead of recomputing them (same page, section
// "PagedAttention in a Python RAG Application" and its question on how prefix
// caching works; "PagedAttention in vLLM: A Throughput Settings Guide",
// section "Tuning Batching, Prefill, and Cache").  A block's key is (content
// id of the block before it, its token ids), compared exactly; each distinct
// key gets a content id the first time it is registered, for good.  Blocks
// released to zero references keep their content on an LRU evictable list
// that allocation drains only when the free stack is empty.
//
// Optional swap space: under memory pressure a whole sequence can move to
// host blocks and come back later at host-link cost (same page, section
// "Python LLM Inference Optimization with vLLM: Parameters That Actually
// Matter").  Host blocks come from their own LIFO stack (identity order).
#pragma once

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

namespace pa {

enum class PoolResult { kOk, kInvalid, kNoMemory };

class BlockPool {
 public:
  BlockPool(int32_t num_blocks, int32_t block_size, uint64_t seed, bool prefix_caching = false,
            int32_t num_host_blocks = 0);

  int32_t num_blocks() const { return num_blocks_; }
  int32_t block_size() const { return block_size_; }
  int32_t num_free() const { return static_cast<int32_t>(free_.size()); }
  int32_t num_cached() const { return ev_size_; }
  int32_t num_free_host() const { return static_cast<int32_t>(host_free_.size()); }
  bool prefix_caching() const { return caching_; }
  int32_t refcount(int32_t block) const;

  int64_t create();
  PoolResult fork(int64_t parent, int64_t* child, std::string* err);
  // Appends n tokens; slots[n] receives storage slots; at most one
  // copy-on-write pair is reported through (*cow_src, *cow_dst, *n_cow).
  // With token ids (tokens != nullptr) and prefix caching on, up to
  // max_hit tokens of leading whole blocks may be served from cached
  // blocks: their slots are -1 and *n_hit counts them.
  PoolResult append(int64_t seq, int32_t n, const int32_t* tokens, int32_t max_hit, int64_t* slots,
                    int32_t* cow_src, int32_t* cow_dst, int32_t* n_cow, int32_t* n_hit,
                    std::string* err);
  PoolResult release(int64_t seq, std::string* err);
  // Moves a resident sequence to host blocks: pairs (device, host) in table
  // order; the device blocks lose one reference each.  cap bounds the pairs.
  PoolResult swap_out(int64_t seq, int32_t* pairs, int32_t cap, int32_t* n_pairs, std::string* err);
  // Brings a swapped sequence back: pairs (host, device) in table order.
  PoolResult swap_in(int64_t seq, int32_t* pairs, int32_t cap, int32_t* n_pairs, std::string* err);
  const std::vector<int32_t>* table(int64_t seq) const;
  int64_t num_tokens(int64_t seq) const;

 private:
  static constexpr int64_t kUnknown = INT64_MIN;   // token appended without an id
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t tokens = 0;
    std::vector<int64_t> ids;   // token ids, kept only with prefix caching
    bool swapped = false;
    std::vector<int32_t> host_blocks;   // while swapped out
  };
  struct Key {
    int64_t prev;                    // content id of the block before, -1 at the start
    std::vector<int64_t> toks;
    bool operator==(const Key& o) const { return prev == o.prev && toks == o.toks; }
  };
  // 64-bit FNV-1a (Fowler, Noll, Vo) over the key's 8-byte words.
  struct KeyHash {
    size_t operator()(const Key& k) const;
  };

  int32_t take();                          // free stack first, then evict
  void drop(int32_t b);                    // one reference less; release at zero
  void ev_push_back(int32_t b);
  void ev_remove(int32_t b);
  void register_block(Seq& s, size_t j);

  int32_t num_blocks_;
  int32_t block_size_;
  bool caching_;
  std::vector<int32_t> free_;      // LIFO: back() is the top
  std::vector<int32_t> host_free_; // host swap blocks, LIFO
  std::vector<int32_t> ref_;
  std::unordered_map<int64_t, Seq> seqs_;
  int64_t next_id_ = 1;
  // Prefix caching state.
  std::vector<int32_t> ev_prev_, ev_next_;   // evictable list, intrusive
  int32_t ev_head_ = -1, ev_tail_ = -1, ev_size_ = 0;
  std::vector<int64_t> content_of_block_;    // -1: not registered
  std::vector<int32_t> block_of_content_;    // by content id, -1: no live block
  std::unordered_map<Key, int64_t, KeyHash> content_ids_;
};

}  // namespace pa
