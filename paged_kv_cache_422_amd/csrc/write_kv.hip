// Slot-mapped K/V write and whole-block copy kernels (gfx950).
//
// New tokens' keys and values are appended to their sequence's blocks as they
// are generated ("Inside vLLM: How PagedAttention Changes Python LLM Inference
// at the Systems Level", section "PagedAttention: What the OS Figured Out
// Decades Ago"); a shared block is duplicated before a branch writes into it
// (same page, section "Copy-on-Write Makes Beam Search Cheap").  Both kernels
// move raw 16-bit patterns, so they are dtype-agnostic and bit-exact.
//
// Storage: k_cache [N][Hkv][D/32][16][32] (32-dim chunks, slot-major within
// a chunk), v_cache [N][Hkv][4][D][4] (groups of four slots, dim-major within
// a group: slot s of dim d at [s / 4][d][s % 4]).  HBM-bound: each token
// moves 2 * Hkv * D * 2 bytes in and the same out.
#include "common.hpp"
#include "launch.hpp"

namespace pa {

namespace {

constexpr int kBlock = 16;   // tokens per KV block

// One workgroup per (16 consecutive tokens, kv head), 2 * D threads.
//
// K: thread (chunk c, token i) moves one 16-byte piece of token i's K row:
// dims 8c .. 8c+7, which sit in 32-dim chunk c / 4 at slot i, piece c % 4.
// A wave's 64 threads cover one whole 1 KiB chunk of 16 slots, and a decode
// token (alone in its block) writes four whole 64-byte pieces.
// V: a token's values sit 8 bytes apart (one 2-byte piece per dim in its
// slot group), so a single token only fills a quarter of each 32-byte sector
// it touches: D / 4 sectors per head, where a dim-major [D][16] block would
// touch D of them.  HBM3E has no write mask, so each partly written sector
// costs the memory a read-modify-write; fewer sectors per token is what makes
// the decode tokens' writes cheaper.  The group's values pass through LDS,
// transposed to [dim][token]; thread (key group kg, dim pair d0) then owns
// tokens 4kg .. 4kg+3 of dims d0 and d0 + 1.  When those four tokens go to
// four consecutive slots starting at a multiple of 4 (prefill chunks fill
// their blocks in order) the thread stores them as one 16-byte piece, and the
// 64 threads of a wave complete whole lines.  Any other mapping (decode
// tokens, each alone in its block, or skipped tokens) falls back to one
// 2-byte store per token and dim.
template <int D>
__global__ __launch_bounds__(2 * D) void write_kv_kernel(WriteKvArgs a) {
  __shared__ int64_t slot_s[kBlock];
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * kBlock];   // [dim][token]

  const int tid = threadIdx.x;
  const int head = blockIdx.y;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kBlock;
  const int nt = static_cast<int>(min<int64_t>(kBlock, a.num_tokens - t0));
  const int64_t limit = a.num_blocks * kBlock;
  if (tid < kBlock) {
    int64_t sl = -1;
    if (tid < nt) {
      sl = a.slot_mapping[t0 + tid];
      if (sl < 0 || sl >= limit) sl = -1;                       // skipped token
    }
    slot_s[tid] = sl;
  }

  const int i = tid % kBlock;          // token within the group
  const int c = tid / kBlock;          // 8-element chunk of the head dim
  u32x4 kk{0, 0, 0, 0}, vv{0, 0, 0, 0};
  if (i < nt) {
    const int64_t src = (t0 + i) * a.src_token_stride + static_cast<int64_t>(head) * D + c * 8;
    kk = *reinterpret_cast<const u32x4*>(a.k + src);
    vv = *reinterpret_cast<const u32x4*>(a.v + src);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    vt[(c * 8 + 2 * e) * kBlock + i] = static_cast<uint16_t>(vv[e] & 0xffffu);
    vt[(c * 8 + 2 * e + 1) * kBlock + i] = static_cast<uint16_t>(vv[e] >> 16);
  }
  __syncthreads();

  const int64_t head_tile = static_cast<int64_t>(head) * kBlock * D;
  const int64_t blk_elems = static_cast<int64_t>(a.num_kv_heads) * kBlock * D;
  {
    const int64_t sl = slot_s[i];
    if (sl >= 0) {
      const int64_t blk = sl / kBlock;
      const int off = static_cast<int>(sl - blk * kBlock);
      *reinterpret_cast<u32x4*>(a.k_cache + blk * blk_elems + head_tile + (c >> 2) * (kBlock * 32) + off * 32 +
                                (c & 3) * 8) = kk;
    }
  }

  const int kg = tid / (D / 2);        // group of four tokens
  const int d0 = 2 * (tid % (D / 2));  // first of two dims
  const int64_t s0 = slot_s[4 * kg];
  bool run = s0 >= 0 && (s0 & 3) == 0;
#pragma unroll
  for (int j = 1; j < 4; ++j) run = run && slot_s[4 * kg + j] == s0 + j;
  const uint16_t* const vt0 = &vt[d0 * kBlock + 4 * kg];   // 4 tokens of dim d0
  const uint16_t* const vt1 = vt0 + kBlock;                 // and of dim d0 + 1
  if (run) {
    const int64_t blk = s0 / kBlock;
    const int grp = static_cast<int>(s0 - blk * kBlock) / 4;
    *reinterpret_cast<u32x4*>(a.v_cache + blk * blk_elems + head_tile + (grp * D + d0) * 4) =
        u32x4{pack2(vt0[0], vt0[1]), pack2(vt0[2], vt0[3]), pack2(vt1[0], vt1[1]), pack2(vt1[2], vt1[3])};
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t sl = slot_s[4 * kg + j];
      if (sl < 0) continue;
      const int64_t blk = sl / kBlock;
      const int off = static_cast<int>(sl - blk * kBlock);
      uint16_t* const dst = a.v_cache + blk * blk_elems + head_tile + ((off >> 2) * D + d0) * 4 + (off & 3);
      dst[0] = vt0[j];
      dst[4] = vt1[j];
    }
  }
}

// One workgroup per (src, dst) pair: 16-byte copies of the K and V tiles of
// every head, four of each in flight per thread (the source may sit across
// the host link).  Out-of-range ids skip the pair.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksArgs a) {
  const int pair = blockIdx.x;
  const int32_t src = a.pairs[2 * pair];
  const int32_t dst = a.pairs[2 * pair + 1];
  if (src < 0 || dst < 0 || src >= a.src_blocks || dst >= a.dst_blocks) return;
  const int64_t n16 = a.block_elems / 8;    // 16-byte units per block
  const u32x4* ks = reinterpret_cast<const u32x4*>(a.src_k + static_cast<int64_t>(src) * a.block_elems);
  const u32x4* vs = reinterpret_cast<const u32x4*>(a.src_v + static_cast<int64_t>(src) * a.block_elems);
  u32x4* kd = reinterpret_cast<u32x4*>(a.dst_k + static_cast<int64_t>(dst) * a.block_elems);
  u32x4* vd = reinterpret_cast<u32x4*>(a.dst_v + static_cast<int64_t>(dst) * a.block_elems);
  constexpr int kUnroll = 4;
  int64_t i = threadIdx.x;
  for (; i + (kUnroll - 1) * 256 < n16; i += kUnroll * 256) {
    u32x4 k[kUnroll], v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      k[u] = ks[i + u * 256];
      v[u] = vs[i + u * 256];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      kd[i + u * 256] = k[u];
      vd[i + u * 256] = v[u];
    }
  }
  for (; i < n16; i += 256) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

}  // namespace

hipError_t launch_write_kv(const WriteKvArgs& a, int /*dtype*/, hipStream_t stream) {
  if (a.num_kv_heads > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<uint32_t>((static_cast<int64_t>(a.num_tokens) + kBlock - 1) / kBlock),
                  static_cast<uint32_t>(a.num_kv_heads));
  if (a.head_dim == 64) {
    hipLaunchKernelGGL(write_kv_kernel<64>, grid, dim3(128), 0, stream, a);
  } else {
    hipLaunchKernelGGL(write_kv_kernel<128>, grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(a.num_pairs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
