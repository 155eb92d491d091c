// Host-side launchers of the gfx950 kernels.  Called only by capi.cpp after
// every argument has been validated; each returns the launch's hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct WriteKvArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t src_token_stride;   // elements
  uint16_t* k_cache;
  uint16_t* v_cache;
  int64_t num_blocks;
  const int64_t* slot_mapping;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t head_dim;
};

// Whole-block copies from one cache-shaped buffer pair to another (the same
// cache for copy-on-write; the device cache and pinned host swap space for
// swapping).
struct CopyBlocksArgs {
  const uint16_t* src_k;
  const uint16_t* src_v;
  uint16_t* dst_k;
  uint16_t* dst_v;
  int64_t src_blocks;         // ids at or past these are skipped
  int64_t dst_blocks;
  const int32_t* pairs;       // [num_pairs][2] (src, dst), device
  int32_t num_pairs;
  int64_t block_elems;        // num_kv_heads * block_size * head_dim
};

struct DecodeArgs {
  uint16_t* out;              // [S][Hq][D]
  float* ws_acc;              // [S][Hq][max_parts][D]
  float* ws_ml;               // [S][Hq][max_parts][2]  (max in log2 units, sum)
  const uint16_t* q;          // [S][Hq][D]
  const uint16_t* k_cache;    // [N][Hkv][D/32][16][32]
  const uint16_t* v_cache;    // [N][Hkv][4][D][4]
  const int32_t* block_tables;
  const int32_t* context_lens;
  int64_t num_blocks;
  int32_t bt_stride;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;              // num_q_heads / num_kv_heads
  int32_t num_sub;            // ceil(group / 16): head sub-groups per KV head
  int32_t part_blocks;        // partition size in blocks
  int32_t max_parts;
  int32_t max_context_len;
  int32_t waves;              // waves interleaving a partition's blocks (4 or 8): fixes the reduction order
  int32_t buffers;            // block buffers per wave of the two-pass kernel (2 or 3): speed only
  int32_t fuse_groups;        // > 0: single pass allowed, partitions merged on chip (wave groups per workgroup: 1 of 8 waves or 2 of 4, by `waves`)
  float scale_log2;           // scale * log2(e)
};

struct PrefillArgs {
  uint16_t* out;              // [T][Hq][D]
  const uint16_t* q;          // [T][Hq][D]
  const uint16_t* k_cache;    // [N][Hkv][D/32][16][32]
  const uint16_t* v_cache;    // [N][Hkv][4][D][4]
  const int32_t* block_tables;
  const int32_t* q_start_loc;
  const int32_t* seq_lens;
  int64_t num_blocks;
  int32_t bt_stride;
  int32_t num_chunks;
  int32_t max_q_len;
  int32_t max_seq_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  float scale_log2;
};

// dtype: 0 = fp16, 1 = bf16.
hipError_t launch_write_kv(const WriteKvArgs& a, int dtype, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int head_dim, int dtype, hipStream_t stream);
// How launch_decode merges a call's partitions (also reported by pa_decode_plan).
enum { kMergeNone = 0, kMergeOnChip = 1, kMergeTwoPass = 2 };
int decode_merge_kind(const DecodeArgs& a, int head_dim);
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int dtype, hipStream_t stream);
// Device address of the current device's copy of the library's static decode
// scratch (PA_DECODE_STATIC_SCRATCH_BYTES bytes), looked up once per device.
hipError_t static_scratch(void** ptr);

}  // namespace pa
