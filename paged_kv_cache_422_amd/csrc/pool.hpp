// Host-side refcounted KV block pool with copy-on-write.
//
// Blocks are claimed on demand as a sequence grows and released as soon as
// it finishes; forked sequences share blocks by reference count and a shared
// block is copied only when a branch writes into it ("Inside vLLM: How
// PagedAttention Changes Python LLM Inference at the Systems Level", sections
// "PagedAttention: What the OS Figured Out Decades Ago" and "Copy-on-Write
// Makes Beam Search Cheap").  Pure C++, no device code: the pool hands out
// ids; the caller moves data with the copy and write kernels.
#pragma once

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

namespace pa {

enum class PoolResult { kOk, kInvalid, kNoMemory };

class BlockPool {
 public:
  BlockPool(int32_t num_blocks, int32_t block_size, uint64_t seed);

  int32_t num_blocks() const { return num_blocks_; }
  int32_t block_size() const { return block_size_; }
  int32_t num_free() const { return static_cast<int32_t>(free_.size()); }
  int32_t refcount(int32_t block) const;

  int64_t create();
  PoolResult fork(int64_t parent, int64_t* child, std::string* err);
  // Appends n tokens; slots[n] receives storage slots; at most one
  // copy-on-write pair is reported through (*cow_src, *cow_dst, *n_cow).
  PoolResult append(int64_t seq, int32_t n, int64_t* slots, int32_t* cow_src,
                    int32_t* cow_dst, int32_t* n_cow, std::string* err);
  PoolResult release(int64_t seq, std::string* err);
  const std::vector<int32_t>* table(int64_t seq) const;
  int64_t num_tokens(int64_t seq) const;

 private:
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t tokens = 0;
  };
  int32_t pop_free();

  int32_t num_blocks_;
  int32_t block_size_;
  std::vector<int32_t> free_;      // LIFO: back() is the top
  std::vector<int32_t> ref_;
  std::unordered_map<int64_t, Seq> seqs_;
  int64_t next_id_ = 1;
};

}  // namespace pa
