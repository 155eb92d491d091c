// Host-side refcounted KV block pool with copy-on-write (see pool.hpp).
#include "pool.hpp"

#include <algorithm>
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

BlockPool::BlockPool(int32_t num_blocks, int32_t block_size, uint64_t seed, bool prefix_caching,
                     int32_t num_host_blocks)
    : num_blocks_(num_blocks), block_size_(block_size), caching_(prefix_caching), ref_(num_blocks, 0) {
  for (int32_t h = num_host_blocks - 1; h >= 0; --h) host_free_.push_back(h);   // host block 0 first
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
  if (caching_) {
    ev_prev_.assign(num_blocks, -1);
    ev_next_.assign(num_blocks, -1);
    content_of_block_.assign(num_blocks, -1);
  }
}

size_t BlockPool::KeyHash::operator()(const Key& k) const {
  uint64_t h = 14695981039346656037ull;     // FNV-1a 64-bit offset basis
  auto mix = [&h](int64_t w) {
    const uint64_t u = static_cast<uint64_t>(w);
    for (int i = 0; i < 8; ++i) {
      h ^= (u >> (8 * i)) & 0xffu;
      h *= 1099511628211ull;                  // FNV 64-bit prime
    }
  };
  mix(k.prev);
  for (int64_t t : k.toks) mix(t);
  return static_cast<size_t>(h);
}

void BlockPool::ev_push_back(int32_t b) {
  ev_prev_[b] = ev_tail_;
  ev_next_[b] = -1;
  if (ev_tail_ >= 0) {
    ev_next_[ev_tail_] = b;
  } else {
    ev_head_ = b;
  }
  ev_tail_ = b;
  ++ev_size_;
}

void BlockPool::ev_remove(int32_t b) {
  const int32_t p = ev_prev_[b], nx = ev_next_[b];
  if (p >= 0) {
    ev_next_[p] = nx;
  } else {
    ev_head_ = nx;
  }
  if (nx >= 0) {
    ev_prev_[nx] = p;
  } else {
    ev_tail_ = p;
  }
  ev_prev_[b] = ev_next_[b] = -1;
  --ev_size_;
}

int32_t BlockPool::take() {
  int32_t b;
  if (!free_.empty()) {
    b = free_.back();
    free_.pop_back();
  } else {
    // Evict the least recently released cached block: its content is gone.
    b = ev_head_;
    ev_remove(b);
    block_of_content_[content_of_block_[b]] = -1;
    content_of_block_[b] = -1;
  }
  ref_[b] = 1;
  return b;
}

// Block j of s has just been filled: register its content if every token id
// is known and the block before it is registered (or it is the first block).
// A content id that already has a live block keeps it; this one stays
// unregistered.
void BlockPool::register_block(Seq& s, size_t j) {
  const int64_t B = block_size_;
  const int64_t prev = j == 0 ? -1 : content_of_block_[s.blocks[j - 1]];
  if (j > 0 && prev < 0) return;
  Key key{prev, std::vector<int64_t>(s.ids.begin() + j * B, s.ids.begin() + (j + 1) * B)};
  if (std::find(key.toks.begin(), key.toks.end(), kUnknown) != key.toks.end()) return;
  auto ins = content_ids_.emplace(std::move(key), static_cast<int64_t>(block_of_content_.size()));
  if (ins.second) block_of_content_.push_back(-1);
  const int64_t cid = ins.first->second;
  if (block_of_content_[cid] >= 0) return;
  block_of_content_[cid] = s.blocks[j];
  content_of_block_[s.blocks[j]] = cid;
}

int32_t BlockPool::refcount(int32_t block) const {
  if (block < 0 || block >= num_blocks_) return -1;
  return ref_[block];
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
  if (it->second.swapped) {
    *err = "pa_seq_fork: sequence " + std::to_string(parent) + " is swapped out";
    return PoolResult::kInvalid;
  }
  Seq copy = it->second;
  for (int32_t b : copy.blocks) ++ref_[b];
  const int64_t id = next_id_++;
  seqs_.emplace(id, std::move(copy));
  *child = id;
  return PoolResult::kOk;
}

PoolResult BlockPool::append(int64_t seq, int32_t n, const int32_t* tokens, int32_t max_hit,
                             int64_t* slots, int32_t* cow_src, int32_t* cow_dst, int32_t* n_cow,
                             int32_t* n_hit, std::string* err) {
  *n_cow = 0;
  *n_hit = 0;
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
  if (s.swapped) {
    *err = "pa_seq_append: sequence " + std::to_string(seq) + " is swapped out";
    return PoolResult::kInvalid;
  }
  const int64_t B = block_size_;

  // Whole leading blocks whose content is cached, along the content chain
  // from the sequence's last block (which must be registered) or the start.
  std::vector<int32_t> hits;
  if (caching_ && tokens && s.tokens % B == 0 &&
      (s.blocks.empty() || content_of_block_[s.blocks.back()] >= 0)) {
    int64_t prev = s.blocks.empty() ? -1 : content_of_block_[s.blocks.back()];
    const int64_t lim = std::min<int64_t>(n, std::max<int32_t>(max_hit, 0));
    Key key{0, std::vector<int64_t>(B)};
    while (static_cast<int64_t>(hits.size() + 1) * B <= lim) {
      key.prev = prev;
      for (int64_t i = 0; i < B; ++i) key.toks[i] = tokens[hits.size() * B + i];
      auto f = content_ids_.find(key);
      if (f == content_ids_.end() || block_of_content_[f->second] < 0) break;
      hits.push_back(block_of_content_[f->second]);
      prev = f->second;
    }
  }
  const int64_t hit_tokens = static_cast<int64_t>(hits.size()) * B;

  const bool partial = (s.tokens % B) != 0;
  const bool need_cow = n - hit_tokens > 0 && partial && ref_[s.blocks.back()] > 1;
  const int64_t blocks_after = (s.tokens + n + B - 1) / B;
  const int64_t need = blocks_after - static_cast<int64_t>(s.blocks.size() + hits.size()) + (need_cow ? 1 : 0);
  int64_t idle_hits = 0;
  for (int32_t b : hits) idle_hits += ref_[b] == 0;
  const int64_t avail = static_cast<int64_t>(free_.size()) + ev_size_ - idle_hits;
  if (need > avail) {
    *err = "pa_seq_append: pool exhausted (need " + std::to_string(need) + " blocks, " +
           std::to_string(avail) + " available)";
    return PoolResult::kNoMemory;
  }

  for (int32_t b : hits) {
    if (ref_[b] == 0) ev_remove(b);
    ++ref_[b];
    s.blocks.push_back(b);
  }
  for (int64_t i = 0; i < hit_tokens; ++i) {
    slots[i] = -1;
    s.ids.push_back(tokens[i]);
  }
  s.tokens += hit_tokens;
  *n_hit = static_cast<int32_t>(hit_tokens);

  for (int64_t i = hit_tokens; i < n; ++i) {
    const int64_t pos = s.tokens;
    if (pos % B == 0) {
      s.blocks.push_back(take());
    } else if (ref_[s.blocks.back()] > 1) {
      const int32_t src = s.blocks.back();
      const int32_t dst = take();
      --ref_[src];
      s.blocks.back() = dst;
      *cow_src = src;
      *cow_dst = dst;
      *n_cow = 1;
    }
    slots[i] = static_cast<int64_t>(s.blocks.back()) * B + pos % B;
    if (caching_) s.ids.push_back(tokens ? tokens[i] : kUnknown);
    s.tokens = pos + 1;
    if (caching_ && s.tokens % B == 0) register_block(s, s.blocks.size() - 1);
  }
  return PoolResult::kOk;
}

PoolResult BlockPool::release(int64_t seq, std::string* err) {
  auto it = seqs_.find(seq);
  if (it == seqs_.end()) {
    *err = "pa_seq_free: unknown sequence " + std::to_string(seq);
    return PoolResult::kInvalid;
  }
  for (int32_t b : it->second.blocks) drop(b);
  for (int32_t h : it->second.host_blocks) host_free_.push_back(h);
  seqs_.erase(it);
  return PoolResult::kOk;
}

void BlockPool::drop(int32_t b) {
  if (--ref_[b] != 0) return;
  if (caching_ && content_of_block_[b] >= 0) {
    ev_push_back(b);          // keeps its content until evicted
  } else {
    free_.push_back(b);
  }
}

PoolResult BlockPool::swap_out(int64_t seq, int32_t* pairs, int32_t cap, int32_t* n_pairs, std::string* err) {
  *n_pairs = 0;
  auto it = seqs_.find(seq);
  if (it == seqs_.end() || it->second.swapped) {
    *err = "pa_seq_swap_out: sequence " + std::to_string(seq) + (it == seqs_.end() ? " unknown" : " already swapped out");
    return PoolResult::kInvalid;
  }
  Seq& s = it->second;
  const int64_t n = static_cast<int64_t>(s.blocks.size());
  if (n > cap) {
    *err = "pa_seq_swap_out: pairs_out holds " + std::to_string(cap) + " pairs, need " + std::to_string(n);
    return PoolResult::kInvalid;
  }
  if (n > static_cast<int64_t>(host_free_.size())) {
    *err = "pa_seq_swap_out: swap space exhausted (need " + std::to_string(n) + " host blocks, " +
           std::to_string(host_free_.size()) + " free)";
    return PoolResult::kNoMemory;
  }
  for (int64_t i = 0; i < n; ++i) {
    const int32_t h = host_free_.back();
    host_free_.pop_back();
    pairs[2 * i] = s.blocks[i];
    pairs[2 * i + 1] = h;
    s.host_blocks.push_back(h);
    drop(s.blocks[i]);
  }
  s.blocks.clear();
  s.swapped = true;
  *n_pairs = static_cast<int32_t>(n);
  return PoolResult::kOk;
}

PoolResult BlockPool::swap_in(int64_t seq, int32_t* pairs, int32_t cap, int32_t* n_pairs, std::string* err) {
  *n_pairs = 0;
  auto it = seqs_.find(seq);
  if (it == seqs_.end() || !it->second.swapped) {
    *err = "pa_seq_swap_in: sequence " + std::to_string(seq) + (it == seqs_.end() ? " unknown" : " is not swapped out");
    return PoolResult::kInvalid;
  }
  Seq& s = it->second;
  const int64_t n = static_cast<int64_t>(s.host_blocks.size());
  if (n > cap) {
    *err = "pa_seq_swap_in: pairs_out holds " + std::to_string(cap) + " pairs, need " + std::to_string(n);
    return PoolResult::kInvalid;
  }
  if (n > static_cast<int64_t>(free_.size()) + ev_size_) {
    *err = "pa_seq_swap_in: pool exhausted (need " + std::to_string(n) + " blocks, " +
           std::to_string(static_cast<int64_t>(free_.size()) + ev_size_) + " available)";
    return PoolResult::kNoMemory;
  }
  for (int64_t i = 0; i < n; ++i) {
    const int32_t d = take();
    pairs[2 * i] = s.host_blocks[i];
    pairs[2 * i + 1] = d;
    s.blocks.push_back(d);
    host_free_.push_back(s.host_blocks[i]);
  }
  s.host_blocks.clear();
  s.swapped = false;
  *n_pairs = static_cast<int32_t>(n);
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
