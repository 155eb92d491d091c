// Host-side refcounted KV block pool with copy-on-write (see pool.hpp).
#include "pool.hpp"

#include <utility>

namespace pa {

namespace {

// SplitMix64 (Steele, Lea, Flood, OOPSLA 2014): the state advances by the
// 64-bit golden-ratio increment and each output is the state passed through
// the variant-13 finaliser (xor-shift 30, multiply, xor-shift 27, multiply,
// xor-shift 31).
struct SplitMix64 {
  uint64_t state;
  explicit SplitMix64(uint64_t seed) : state(seed) {}
  uint64_t next() {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

}  // namespace

BlockPool::BlockPool(int32_t num_blocks, int32_t block_size, uint64_t seed)
    : num_blocks_(num_blocks), block_size_(block_size), ref_(num_blocks, 0) {
  // Initial order: Durstenfeld shuffle of [0, N) (seed 0 keeps identity).
  std::vector<int32_t> order(num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) order[i] = i;
  if (seed != 0) {
    SplitMix64 g(seed);
    for (int64_t i = num_blocks - 1; i > 0; --i) {
      const uint64_t j = g.next() % static_cast<uint64_t>(i + 1);
      std::swap(order[i], order[j]);
    }
  }
  // order[0] must come out first, so it sits on top (the back).
  free_.assign(order.rbegin(), order.rend());
}

int32_t BlockPool::refcount(int32_t block) const {
  if (block < 0 || block >= num_blocks_) return -1;
  return ref_[block];
}

int32_t BlockPool::pop_free() {
  const int32_t b = free_.back();
  free_.pop_back();
  ref_[b] = 1;
  return b;
}

int64_t BlockPool::create() {
  const int64_t id = next_id_++;
  seqs_.emplace(id, Seq{});
  return id;
}

PoolResult BlockPool::fork(int64_t parent, int64_t* child, std::string* err) {
  auto it = seqs_.find(parent);
  if (it == seqs_.end()) {
    *err = "pa_seq_fork: unknown sequence " + std::to_string(parent);
    return PoolResult::kInvalid;
  }
  Seq copy = it->second;
  for (int32_t b : copy.blocks) ++ref_[b];
  const int64_t id = next_id_++;
  seqs_.emplace(id, std::move(copy));
  *child = id;
  return PoolResult::kOk;
}

PoolResult BlockPool::append(int64_t seq, int32_t n, int64_t* slots, int32_t* cow_src,
                             int32_t* cow_dst, int32_t* n_cow, std::string* err) {
  *n_cow = 0;
  auto it = seqs_.find(seq);
  if (it == seqs_.end()) {
    *err = "pa_seq_append: unknown sequence " + std::to_string(seq);
    return PoolResult::kInvalid;
  }
  if (n < 0) {
    *err = "pa_seq_append: negative token count";
    return PoolResult::kInvalid;
  }
  Seq& s = it->second;
  const int64_t B = block_size_;
  const bool partial = (s.tokens % B) != 0;
  const bool need_cow = n > 0 && partial && ref_[s.blocks.back()] > 1;
  const int64_t blocks_after = (s.tokens + n + B - 1) / B;
  const int64_t need = blocks_after - static_cast<int64_t>(s.blocks.size()) + (need_cow ? 1 : 0);
  if (need > static_cast<int64_t>(free_.size())) {
    *err = "pa_seq_append: pool exhausted (need " + std::to_string(need) + " blocks, " +
           std::to_string(free_.size()) + " free)";
    return PoolResult::kNoMemory;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int64_t pos = s.tokens;
    if (pos % B == 0) {
      s.blocks.push_back(pop_free());
    } else if (ref_[s.blocks.back()] > 1) {
      const int32_t src = s.blocks.back();
      const int32_t dst = pop_free();
      --ref_[src];
      s.blocks.back() = dst;
      *cow_src = src;
      *cow_dst = dst;
      *n_cow = 1;
    }
    slots[i] = static_cast<int64_t>(s.blocks.back()) * B + pos % B;
    s.tokens = pos + 1;
  }
  return PoolResult::kOk;
}

PoolResult BlockPool::release(int64_t seq, std::string* err) {
  auto it = seqs_.find(seq);
  if (it == seqs_.end()) {
    *err = "pa_seq_free: unknown sequence " + std::to_string(seq);
    return PoolResult::kInvalid;
  }
  for (int32_t b : it->second.blocks) {
    if (--ref_[b] == 0) free_.push_back(b);
  }
  seqs_.erase(it);
  return PoolResult::kOk;
}

const std::vector<int32_t>* BlockPool::table(int64_t seq) const {
  auto it = seqs_.find(seq);
  return it == seqs_.end() ? nullptr : &it->second.blocks;
}

int64_t BlockPool::num_tokens(int64_t seq) const {
  auto it = seqs_.find(seq);
  return it == seqs_.end() ? -1 : it->second.tokens;
}

}  // namespace pa
