// C ABI of libpa, device half (declared in include/pa.h): argument
// validation, workspace sizing and kernel dispatch of the device calls.
// Every entry point checks its arguments before launching anything and
// reports failures through pa_status plus a thread-local message (shared
// with the host pool half, capi_pool.cpp); nothing throws across the ABI.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>

#include "launch.hpp"
#include "status.hpp"

using pa::fail;
using pa::ok;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kBlock = 16;
constexpr int kMaxPartitionTokens = 4096;   // 4 block ids per lane of a wave64
constexpr int64_t kTargetItems = 1024;      // work items that fill the GPU (see pa_default_partition_size)

pa_status check_common(const char* fn, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       pa_dtype dtype) {
  if (dtype != PA_FP16 && dtype != PA_BF16)
    return fail(PA_ENOTSUP, std::string(fn) + ": dtype must be PA_FP16 or PA_BF16");
  if (block_size != kBlock)
    return fail(PA_ENOTSUP, std::string(fn) + ": block_size must be 16 (got " +
                                std::to_string(block_size) + ")");
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ENOTSUP, std::string(fn) + ": head_dim must be 64 or 128 (got " +
                                std::to_string(head_dim) + ")");
  if (num_kv_heads <= 0)
    return fail(PA_EINVAL, std::string(fn) + ": num_kv_heads must be positive");
  return PA_OK;
}

pa_status hip_result(const char* fn, hipError_t e) {
  if (e != hipSuccess)
    return fail(PA_EHIP, std::string(fn) + ": " + hipGetErrorString(e));
  return ok();
}

// Waves that interleave the blocks of one decode partition (which fixes the
// reduction order): 8 for partitions of 128 blocks or more (a long partition
// then finishes about as fast as a 64-block one with 4 waves, which keeps the
// end of the launch short), else 4.  A function of the partition size alone,
// so a sequence's result depends only on its own data and the partition
// size.
int32_t decode_waves(int32_t part_blocks) { return part_blocks >= 128 ? 8 : 4; }

// Block buffers per wave of the partition kernel with 8 waves: two (one
// block in flight during the work on another) when no context can exceed
// 2048 tokens, else three.  Short contexts give each wave only a few blocks,
// and a deeper pipeline then spends more of them filling and draining; long
// ones want the bytes in flight.  Measured on MI355X, same box, alternating
// builds: two buffers took the 13B shared-prefix batch (2048-token cap,
// median 400) from 257-258 to 247-249 us with the 7B batch unchanged
// (193.5-193.9 against 193.8-194.1 us), but slowed the mixed step's decode
// (contexts up to 4096 tokens) by up to 6%.  The buffer count changes no
// result bit.
int32_t decode_buffers(int32_t waves, int32_t max_context_len) {
  return waves == 8 && max_context_len <= 2048 ? 2 : 3;
}

// Whether pa_decode may merge a sequence's partitions on chip, in one pass
// (nonzero), or goes through the workspace in two passes (0).  One pass needs
// a batch that fills the GPU without splitting (so one workgroup per sequence
// and head group is enough work), contexts whose block table fits the
// kernel's registers (4096 tokens) and head groups of at most 8 query heads;
// the kernel also checks that the partitions fit its LDS.  Its workgroup is
// one group of 8 waves for partitions of 128 blocks or more and two groups of
// 4 waves taking alternate partitions below: two groups of 4 measured faster
// than one (8B-GQA shape at 512-token partitions: 403 against 418 us; two
// passes took 458).  Either way the result is the same, bit for bit.
int32_t decode_fuse_groups(int64_t items, int32_t group, int32_t max_context_len) {
  if (group > 8 || max_context_len > kMaxPartitionTokens) return 0;
  return items >= kTargetItems ? 2 : 0;
}

int32_t resolve_partition(int32_t requested, int32_t num_seqs, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len) {
  return requested > 0 ? requested
                       : pa_default_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                   max_context_len);
}

}  // namespace

extern "C" {

pa_status pa_write_kv(const void* k, const void* v, int64_t src_token_stride, void* k_cache,
                      void* v_cache, int64_t num_blocks, const int64_t* slot_mapping,
                      int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, pa_dtype dtype, void* stream) {
  const char* fn = "pa_write_kv";
  if (pa_status st = check_common(fn, num_kv_heads, head_dim, block_size, dtype)) return st;
  if (num_tokens < 0 || num_blocks < 0) return fail(PA_EINVAL, "pa_write_kv: negative size");
  if (num_tokens == 0) return ok();
  if (!k || !v || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_EINVAL, "pa_write_kv: null pointer");
  if (src_token_stride < static_cast<int64_t>(num_kv_heads) * head_dim)
    return fail(PA_EINVAL, "pa_write_kv: src_token_stride smaller than num_kv_heads*head_dim");
  if (src_token_stride % 8 != 0 || !aligned16(k) || !aligned16(v) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return fail(PA_ENOTSUP, "pa_write_kv: 16-byte alignment required (pointers, stride % 8)");
  pa::WriteKvArgs a{static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                    src_token_stride, static_cast<uint16_t*>(k_cache),
                    static_cast<uint16_t*>(v_cache), num_blocks, slot_mapping, num_tokens,
                    num_kv_heads, head_dim};
  return hip_result(fn, pa::launch_write_kv(a, dtype, static_cast<hipStream_t>(stream)));
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, int64_t num_blocks, const int32_t* pairs,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, pa_dtype dtype, void* stream) {
  const char* fn = "pa_copy_blocks";
  if (pa_status st = check_common(fn, num_kv_heads, head_dim, block_size, dtype)) return st;
  if (num_pairs < 0 || num_blocks < 0) return fail(PA_EINVAL, "pa_copy_blocks: negative size");
  if (num_pairs == 0) return ok();
  if (!k_cache || !v_cache || !pairs) return fail(PA_EINVAL, "pa_copy_blocks: null pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ENOTSUP, "pa_copy_blocks: caches must be 16-byte aligned");
  pa::CopyBlocksArgs a{static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
                       static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                       num_blocks, num_blocks, pairs, num_pairs,
                       static_cast<int64_t>(num_kv_heads) * block_size * head_dim};
  return hip_result(fn, pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream)));
}

namespace {

// Device address of a pinned (hipHostMalloc) host buffer; nullptr if the
// pointer is not host memory the runtime knows.
void* pinned_device_pointer(const void* host) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, host) != hipSuccess) {
    (void)hipGetLastError();   // clear the sticky error of the query
    return nullptr;
  }
  if (attr.type != hipMemoryTypeHost || !attr.devicePointer) return nullptr;
  return attr.devicePointer;
}

}  // namespace

pa_status pa_swap_blocks(void* k_cache, void* v_cache, int64_t num_blocks, void* host_k, void* host_v,
                         int64_t num_host_blocks, const int32_t* pairs, int32_t num_pairs, int32_t direction,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pa_dtype dtype,
                         void* stream) {
  const char* fn = "pa_swap_blocks";
  if (pa_status st = check_common(fn, num_kv_heads, head_dim, block_size, dtype)) return st;
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN)
    return fail(PA_EINVAL, "pa_swap_blocks: direction must be PA_SWAP_OUT or PA_SWAP_IN");
  if (num_pairs < 0 || num_blocks < 0 || num_host_blocks < 0)
    return fail(PA_EINVAL, "pa_swap_blocks: negative size");
  if (num_pairs == 0) return ok();
  if (!k_cache || !v_cache || !host_k || !host_v || !pairs) return fail(PA_EINVAL, "pa_swap_blocks: null pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(host_k) || !aligned16(host_v))
    return fail(PA_ENOTSUP, "pa_swap_blocks: buffers must be 16-byte aligned");
  void* dk = pinned_device_pointer(host_k);
  void* dv = pinned_device_pointer(host_v);
  if (!dk || !dv)
    return fail(PA_EINVAL, "pa_swap_blocks: host buffers must be pinned host memory (hipHostMalloc)");
  const int64_t elems = static_cast<int64_t>(num_kv_heads) * block_size * head_dim;
  pa::CopyBlocksArgs a{};
  if (direction == PA_SWAP_OUT) {
    a = pa::CopyBlocksArgs{static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
                           static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv),
                           num_blocks, num_host_blocks, pairs, num_pairs, elems};
  } else {
    a = pa::CopyBlocksArgs{static_cast<const uint16_t*>(dk), static_cast<const uint16_t*>(dv),
                           static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                           num_host_blocks, num_blocks, pairs, num_pairs, elems};
  }
  return hip_result(fn, pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream)));
}

// Every partition beyond a sequence's first writes a partial state (head_dim
// + 2 floats per query head) that the second pass reads back, and on MI355X
// those writes cost about ten times their size in lost read bandwidth.  So a
// batch that already offers enough (sequence, KV head) work items to fill
// the GPU many times over (kTargetItems) is not split at all; a smaller batch
// is split just enough to reach that many items.  Partitions are whole
// multiples of 16 tokens between 256 and 4096.  (A partition size the caller
// fixes on such a batch is merged on chip instead: decode_fuse_groups.)
int32_t pa_default_partition_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_context_len) {
  (void)head_dim;
  const int64_t group = num_kv_heads > 0 && num_q_heads > 0 ? num_q_heads / num_kv_heads : 1;
  const int64_t rows = std::max<int64_t>(1, static_cast<int64_t>(num_seqs) * num_kv_heads *
                                                ((group + 15) / 16));
  const int64_t parts = std::max<int64_t>(1, (kTargetItems + rows - 1) / rows);
  int64_t P = (std::max<int64_t>(max_context_len, 1) + parts - 1) / parts;
  P = (P + kBlock - 1) / kBlock * kBlock;
  return static_cast<int32_t>(std::min<int64_t>(kMaxPartitionTokens, std::max<int64_t>(256, P)));
}

pa_status pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                   int32_t max_context_len, int32_t partition_size,
                                   int32_t num_kv_heads, size_t* bytes) {
  if (!bytes) return fail(PA_EINVAL, "pa_decode_workspace_size: bytes is null");
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0 ||
      partition_size < 0 || num_kv_heads <= 0)
    return fail(PA_EINVAL, "pa_decode_workspace_size: bad size");
  const int32_t P = resolve_partition(partition_size, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                      max_context_len);
  const int64_t max_parts = (static_cast<int64_t>(max_context_len) + P - 1) / P;
  if (max_parts <= 1) {
    *bytes = 0;
    return ok();
  }
  const int64_t rows = static_cast<int64_t>(num_seqs) * num_q_heads * max_parts;
  *bytes = static_cast<size_t>(rows) * (head_dim + 2) * sizeof(float);
  return ok();
}

}  // extern "C"

namespace {

// The partitioning fields of a decode call (partition size resolved, waves,
// single pass or two), shared by pa_decode and pa_decode_plan so that the
// plan reported is the one launched.
void fill_decode_plan(pa::DecodeArgs& a, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t P, int32_t max_context_len) {
  const int32_t group = num_q_heads / num_kv_heads;
  const int32_t num_sub = (group + 15) / 16;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.num_sub = num_sub;
  a.part_blocks = P / kBlock;
  a.max_parts = static_cast<int32_t>(std::max<int64_t>(1, (static_cast<int64_t>(max_context_len) + P - 1) / P));
  a.max_context_len = max_context_len;
  a.waves = decode_waves(a.part_blocks);
  a.buffers = decode_buffers(a.waves, max_context_len);
  a.fuse_groups = decode_fuse_groups(static_cast<int64_t>(num_seqs) * num_kv_heads * num_sub, group,
                                     max_context_len);
}

pa_status check_decode_shape(const char* fn, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t max_context_len, int32_t partition_size) {
  if (pa_status st = check_common(fn, num_kv_heads, head_dim, kBlock, PA_FP16)) return st;
  if (num_seqs < 0 || max_context_len < 0)
    return fail(PA_EINVAL, std::string(fn) + ": negative size");
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PA_EINVAL, std::string(fn) + ": num_q_heads must be a positive multiple of num_kv_heads");
  if (partition_size != 0 &&
      (partition_size % kBlock != 0 || partition_size < kBlock || partition_size > kMaxPartitionTokens))
    return fail(PA_ENOTSUP, std::string(fn) + ": partition_size must be 0 or a multiple of 16 in [16, 4096]");
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t max_context_len, int32_t partition_size, int32_t* partition_out,
                         int32_t* merge_out, int32_t* waves_out) {
  const char* fn = "pa_decode_plan";
  if (pa_status st = check_decode_shape(fn, num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                        partition_size))
    return st;
  const int32_t P = resolve_partition(partition_size, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                      max_context_len);
  pa::DecodeArgs a{};
  fill_decode_plan(a, num_seqs, num_q_heads, num_kv_heads, P, max_context_len);
  if (partition_out) *partition_out = P;
  if (merge_out) *merge_out = pa::decode_merge_kind(a, head_dim);
  if (waves_out) *waves_out = a.waves;
  return ok();
}

}  // extern "C"

namespace {

// pa_decode and pa_decode_static: the same checks and kernels; the split-KV
// workspace comes from the caller (pa_decode) or from this device's static
// scratch (from_scratch), which is only needed, and only looked up, when the
// partitions are merged in two passes.
pa_status decode_call(const char* fn, void* out, const void* q, const void* k_cache, const void* v_cache,
                      int64_t num_blocks, const int32_t* block_tables, int32_t bt_stride,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t max_context_len, float scale,
                      int32_t partition_size, void* workspace, size_t workspace_bytes, bool from_scratch,
                      pa_dtype dtype, void* stream) {
  const std::string f(fn);
  if (pa_status st = check_common(fn, num_kv_heads, head_dim, block_size, dtype)) return st;
  if (num_seqs < 0 || num_blocks < 0 || bt_stride <= 0 || max_context_len < 0)
    return fail(PA_EINVAL, f + ": negative size or bt_stride <= 0");
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PA_EINVAL, f + ": num_q_heads must be a positive multiple of num_kv_heads");
  if (partition_size != 0 &&
      (partition_size % kBlock != 0 || partition_size < kBlock || partition_size > kMaxPartitionTokens))
    return fail(PA_ENOTSUP, f + ": partition_size must be 0 or a multiple of 16 in [16, 4096]");
  if (num_seqs == 0) return ok();
  // A bad block id, and a prefetch past a sequence's last block, read block 0.
  if (num_blocks == 0) return fail(PA_EINVAL, f + ": num_blocks must be positive when num_seqs > 0");
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_EINVAL, f + ": null pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ENOTSUP, f + ": 16-byte alignment required");
  if (num_seqs > 65535) return fail(PA_ENOTSUP, f + ": at most 65535 sequences per call");
  const int32_t P = resolve_partition(partition_size, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                      max_context_len);
  const int32_t group = num_q_heads / num_kv_heads;
  const int32_t num_sub = (group + 15) / 16;
  const int64_t max_parts = std::max<int64_t>(1, (static_cast<int64_t>(max_context_len) + P - 1) / P);
  pa::DecodeArgs a{};
  fill_decode_plan(a, num_seqs, num_q_heads, num_kv_heads, P, max_context_len);
  // One workgroup of 64 * waves work-items per (partition, sequence, head
  // group), and one wave per (sequence, query head) in the merge pass; each
  // launch's work-item count must fit the dispatch packet's 32 bits.
  if (max_parts * num_seqs * num_kv_heads * num_sub * 64 * a.waves > static_cast<int64_t>(UINT32_MAX) ||
      static_cast<int64_t>(num_seqs) * num_q_heads * 64 > static_cast<int64_t>(UINT32_MAX))
    return fail(PA_ENOTSUP, f + ": too many (partition, sequence, head) work items");
  const int64_t rows = static_cast<int64_t>(num_seqs) * num_q_heads * max_parts;
  size_t need = 0;
  if (from_scratch) {
    if (pa::decode_merge_kind(a, head_dim) == pa::kMergeTwoPass)
      need = static_cast<size_t>(rows) * (head_dim + 2) * sizeof(float);
    if (need > PA_DECODE_STATIC_SCRATCH_BYTES)
      return fail(PA_ENOTSUP, f + ": the partition states need " + std::to_string(need) +
                                  " bytes, more than the static scratch's " +
                                  std::to_string(PA_DECODE_STATIC_SCRATCH_BYTES) +
                                  " (use pa_decode with a workspace, or larger partitions)");
    if (need > 0) {
      hipError_t e = pa::static_scratch(&workspace);
      if (e != hipSuccess) return fail(PA_EHIP, f + ": static scratch: " + hipGetErrorString(e));
    }
  } else {
    if (pa_status st = pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len, P,
                                                num_kv_heads, &need))
      return st;
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(PA_EINVAL, f + ": workspace too small (need " + std::to_string(need) + " bytes, got " +
                                 std::to_string(workspace_bytes) + ")");
  }
  a.out = static_cast<uint16_t*>(out);
  float* ws = static_cast<float*>(workspace);
  a.ws_acc = need ? ws : nullptr;
  a.ws_ml = need ? ws + rows * head_dim : nullptr;
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_blocks = num_blocks;
  a.bt_stride = bt_stride;
  a.scale_log2 = scale * 1.4426950408889634f;
  return hip_result(fn, pa::launch_decode(a, head_dim, dtype, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    int64_t num_blocks, const int32_t* block_tables, int32_t bt_stride,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t max_context_len, float scale, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, pa_dtype dtype, void* stream) {
  return decode_call("pa_decode", out, q, k_cache, v_cache, num_blocks, block_tables, bt_stride, context_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len, scale,
                     partition_size, workspace, workspace_bytes, false, dtype, stream);
}

pa_status pa_decode_static(void* out, const void* q, const void* k_cache, const void* v_cache,
                           int64_t num_blocks, const int32_t* block_tables, int32_t bt_stride,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t max_context_len, float scale, int32_t partition_size, pa_dtype dtype,
                           void* stream) {
  return decode_call("pa_decode_static", out, q, k_cache, v_cache, num_blocks, block_tables, bt_stride,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
                     scale, partition_size, nullptr, 0, true, dtype, stream);
}

pa_status pa_prefill_chunk(void* out, const void* q, const void* k_cache, const void* v_cache,
                           int64_t num_blocks, const int32_t* block_tables, int32_t bt_stride,
                           const int32_t* q_start_loc, const int32_t* seq_lens, int32_t num_chunks,
                           int32_t max_q_len, int32_t max_seq_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                           pa_dtype dtype, void* stream) {
  const char* fn = "pa_prefill_chunk";
  if (pa_status st = check_common(fn, num_kv_heads, head_dim, block_size, dtype)) return st;
  if (num_chunks < 0 || num_blocks < 0 || bt_stride <= 0 || max_q_len < 0 || max_seq_len < 0)
    return fail(PA_EINVAL, "pa_prefill_chunk: negative size or bt_stride <= 0");
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PA_EINVAL, "pa_prefill_chunk: num_q_heads must be a positive multiple of num_kv_heads");
  if (num_chunks == 0 || max_q_len == 0) return ok();
  // Row blocks of at least 64 rows, one 512-work-item workgroup each: the
  // grid's first dimension must fit the dispatch packet's 32 bits.
  if ((static_cast<int64_t>(max_q_len) + 63) / 64 * 512 > static_cast<int64_t>(UINT32_MAX))
    return fail(PA_ENOTSUP, "pa_prefill_chunk: max_q_len too large for one launch");
  // A bad block id reads block 0 (its tile is then discarded).
  if (num_blocks == 0)
    return fail(PA_EINVAL, "pa_prefill_chunk: num_blocks must be positive when there are chunks");
  if (!out || !q || !k_cache || !v_cache || !block_tables || !q_start_loc || !seq_lens)
    return fail(PA_EINVAL, "pa_prefill_chunk: null pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ENOTSUP, "pa_prefill_chunk: 16-byte alignment required");
  if (num_chunks > 65535) return fail(PA_ENOTSUP, "pa_prefill_chunk: at most 65535 chunks per call");
  pa::PrefillArgs a{};
  a.out = static_cast<uint16_t*>(out);
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.block_tables = block_tables;
  a.q_start_loc = q_start_loc;
  a.seq_lens = seq_lens;
  a.num_blocks = num_blocks;
  a.bt_stride = bt_stride;
  a.num_chunks = num_chunks;
  a.max_q_len = max_q_len;
  a.max_seq_len = max_seq_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  return hip_result(fn, pa::launch_prefill(a, head_dim, dtype, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
