// Slot-mapped K/V write and whole-block copy kernels (gfx950).
//
// New tokens' keys and values are appended to their sequence's blocks as they
// are generated ("Inside vLLM: How PagedAttention Changes Python LLM Inference
// at the Systems Level", section "PagedAttention: What the OS Figured Out
// Decades Ago"); a shared block is duplicated before a branch writes into it
// (same page, section "Copy-on-Write Makes Beam Search Cheap").  Both kernels
// move raw 16-bit patterns, so they are dtype-agnostic and bit-exact.
//
// Storage: k_cache [N][Hkv][16][D] (slot-major), v_cache [N][Hkv][D][16]
// (dim-major).  HBM-bound: each token moves 2 * Hkv * D * 2 bytes in and the
// same out.
#include "common.hpp"
#include "launch.hpp"

namespace pa {

namespace {

constexpr int kBlock = 16;   // tokens per KV block

// One thread per (token, kv head, 8-element chunk of the head dim): one
// 16-byte load of k and v, one 16-byte store into the K tile row, eight
// 2-byte stores down the V tile's slot column.
__global__ __launch_bounds__(256) void write_kv_kernel(WriteKvArgs a) {
  const int chunks = a.head_dim >> 3;
  const int64_t per_token = static_cast<int64_t>(a.num_kv_heads) * chunks;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= per_token * a.num_tokens) return;
  const int64_t tok = idx / per_token;
  const int rem = static_cast<int>(idx - tok * per_token);
  const int head = rem / chunks;
  const int chunk = rem - head * chunks;

  const int64_t slot = a.slot_mapping[tok];
  if (slot < 0 || slot >= a.num_blocks * kBlock) return;   // skipped token
  const int64_t blk = slot / kBlock;
  const int off = static_cast<int>(slot - blk * kBlock);

  const int64_t src = tok * a.src_token_stride + static_cast<int64_t>(head) * a.head_dim + chunk * 8;
  const u32x4 kk = *reinterpret_cast<const u32x4*>(a.k + src);
  const u32x4 vv = *reinterpret_cast<const u32x4*>(a.v + src);

  const int64_t tile = (blk * a.num_kv_heads + head) * static_cast<int64_t>(kBlock) * a.head_dim;
  *reinterpret_cast<u32x4*>(a.k_cache + tile + static_cast<int64_t>(off) * a.head_dim + chunk * 8) = kk;

  uint16_t* vcol = a.v_cache + tile + static_cast<int64_t>(chunk * 8) * kBlock + off;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    vcol[(2 * e) * kBlock] = static_cast<uint16_t>(vv[e] & 0xffffu);
    vcol[(2 * e + 1) * kBlock] = static_cast<uint16_t>(vv[e] >> 16);
  }
}

// One workgroup per (src, dst) pair, 16-byte copies of the K and V tiles of
// every head.  Out-of-range ids skip the pair.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksArgs a) {
  const int pair = blockIdx.x;
  const int32_t src = a.pairs[2 * pair];
  const int32_t dst = a.pairs[2 * pair + 1];
  if (src < 0 || dst < 0 || src >= a.num_blocks || dst >= a.num_blocks) return;
  const int64_t n16 = a.block_elems / 8;    // 16-byte units per block
  const u32x4* ks = reinterpret_cast<const u32x4*>(a.k_cache + static_cast<int64_t>(src) * a.block_elems);
  const u32x4* vs = reinterpret_cast<const u32x4*>(a.v_cache + static_cast<int64_t>(src) * a.block_elems);
  u32x4* kd = reinterpret_cast<u32x4*>(a.k_cache + static_cast<int64_t>(dst) * a.block_elems);
  u32x4* vd = reinterpret_cast<u32x4*>(a.v_cache + static_cast<int64_t>(dst) * a.block_elems);
  for (int64_t i = threadIdx.x; i < n16; i += blockDim.x) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

}  // namespace

hipError_t launch_write_kv(const WriteKvArgs& a, int /*dtype*/, hipStream_t stream) {
  const int64_t threads = static_cast<int64_t>(a.num_tokens) * a.num_kv_heads * (a.head_dim / 8);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(write_kv_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(a.num_pairs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
