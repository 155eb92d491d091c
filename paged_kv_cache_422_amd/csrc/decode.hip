// Paged decode attention for gfx950 (MI355X).
//
// One query token per sequence attends to every key of its sequence; the keys
// and values sit in 16-token blocks scattered through the pool and are found
// through the sequence's block table, so the kernel reads the blocks "as if
// contiguous" ("Inside vLLM: How PagedAttention Changes Python LLM Inference
// at the Systems Level", section "PagedAttention: What the OS Figured Out
// Decades Ago").  Decode is bound by memory bandwidth ("PagedAttention in
// vLLM: A Throughput Settings Guide", section "Continuous Batching Keeps the
// GPU Busy"): every K/V byte of the batch is read exactly once per step, so
// the roofline is HBM and the design goal is to keep enough bytes in flight.
//
// Work split (library design, not from the pages): a sequence of nb blocks
// is cut into np = ceil(nb / part_blocks) partitions of nearly equal size
// (partition p covers blocks [p*nb/np, (p+1)*nb/np)), so every work item of a
// sequence is within one block of the others and long sequences do not leave
// a short remainder item for the end of the launch.  One workgroup of W
// wave64s handles one (sequence, KV head, partition) for all query heads of
// that KV head's group, so K/V are read once per group; W is 8 for
// partitions of 128 blocks or more and 4 below, so it depends only on the
// partition size.  Wave w takes blocks w, w+W, ... of the partition; waves
// merge through LDS.  A
// sequence with one partition writes its output directly; otherwise each
// partition writes (max, sum, unnormalised accumulator) and a second kernel
// merges them by log-sum-exp.  When the batch alone fills the GPU, one
// workgroup instead takes all partitions of a sequence and merges them in
// LDS with the same arithmetic (decode_fused_kernel), so partition states
// never go through HBM.  The order of every reduction depends only on the
// sequence's own length and the partition size, so the result for a
// sequence does not depend on the rest of the batch or on where its blocks
// live.
//
// Launch order: the 1-D grid runs KV head (and query-head sub-group)
// fastest, then sequence, then partition.  Workgroups are handed to the
// eight XCDs round-robin by index, so consecutive indices must carry equal
// work: neighbouring heads of one sequence do, neighbouring partitions of
// different lengths do not.  Partition-major order also starts every
// sequence's first partition before any second one.
//
// Per 16-token block a wave does (16 = MFMA tile edge = block size):
//   S^T[16 keys x 16 heads] = K[16 x D] . Q^T[D x 16]    (D/32 MFMA 16x16x32)
//   online softmax in registers (scores in log2 units, fp32)
//   O[16 heads x D] += P[16 x 16 keys] . V[16 keys x D]  (D/16 MFMA 16x16x16)
// The accumulator layout of the first product is exactly the operand layout
// the second needs for P, so probabilities never leave registers.  V is stored
// in groups of four keys per dimension ([key / 4][dim][key % 4] per block),
// which makes the V operand (four consecutive keys of one dimension) an
// 8-byte load per lane.
// Query-head columns beyond the group size are zero padding.
#include <math.h>

#include <mutex>

#include "common.hpp"
#include "launch.hpp"
#include "pa.h"

// Split-KV partition states of pa_decode_static, for callers that cannot
// allocate device memory: a fixed array that every device the library runs
// on holds from the first use until the process ends.  Host code never names
// it as an address; it uses the device address that static_scratch() looks
// up per device.  Every call on one device shares it, so calls that overlap
// on one device race.  Nothing in it needs clearing: each state the merge
// pass reads was written earlier in the same call.
static __device__ __align__(256) unsigned char scratch[PA_DECODE_STATIC_SCRATCH_BYTES];

namespace pa {

namespace {

constexpr int kBlock = 16;   // tokens per KV block == MFMA tile edge
constexpr int kBtRegs = 4;   // block-table registers per lane: partitions up to 256 blocks
// Partitions of at most this many blocks run the 8 interleaved wave states of
// the two-buffer partition kernel on 4 waves (see decode_partition_kernel).
constexpr int kHalfWaveBlocks = 24;

// -1: invalid context length; 0: empty; otherwise number of partitions.
__device__ __forceinline__ int num_partitions(int L, const DecodeArgs& a) {
  if (L < 0 || L > a.max_context_len || L > a.bt_stride * kBlock) return -1;
  const int nb = (L + kBlock - 1) / kBlock;
  return (nb + a.part_blocks - 1) / a.part_blocks;
}

// First block of partition p of a sequence with nb blocks in np partitions.
__device__ __forceinline__ int partition_start(int p, int nb, int np) {
  return static_cast<int>(static_cast<int64_t>(p) * nb / np);
}

template <class T, int D>
struct BlockRegs {
  u32x4 k[D / 32];   // K: key lane%16, dims 32*ks + 8*(lane/16) .. +7 (chunk ks)
  u32x2 v[D / 16];   // V: dim 16*t + lane%16, keys 4*(lane/16) .. +3 (key group lane/16)
};

template <class T, int D>
__device__ __forceinline__ void load_block(BlockRegs<T, D>& r, const uint16_t* kbase,
                                           const uint16_t* vbase, int64_t off) {
  // K and V are read once per step: non-temporal loads.  Each covers whole
  // 128-byte lines: a K load one 1 KiB chunk (16 keys x 32 dims), a V load
  // 16 dims x 4 keys x 2 bytes = one line in each of the four key groups.
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    r.k[ks] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + off + kBlock * 32 * ks));
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    r.v[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vbase + off + 16 * 4 * t));
}

// One 16-token block of one wave: scores, online-softmax update, P.V
// accumulate.  n_valid (>= 1) is the number of the block's keys inside the
// context.  Both decode kernels run exactly this code per block, so a
// partition's state does not depend on which kernel computed it.
template <class T, int D>
__device__ __forceinline__ void process_block(BlockRegs<T, D>& cur, int n_valid, const u32x4 (&qb)[D / 32],
                                              float scale_log2, int quad, float& m_run, float& l_run,
                                              f32x4 (&o)[D / 16]) {
  constexpr int KS = D / 32;
  constexpr int VT = D / 16;
  f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) sacc = mfma16x16x32<T>(cur.k[ks], qb[ks], sacc);

  float sc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    sc[e] = (4 * quad + e < n_valid) ? sacc[e] * scale_log2 : -INFINITY;
  float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  bm = fmaxf(bm, __shfl_xor(bm, 16));
  bm = fmaxf(bm, __shfl_xor(bm, 32));
  const float m_new = fmaxf(m_run, bm);
  const float alpha = fast_exp2(m_run - m_new);
  uint16_t pb[4], pl[4];
  float psum = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float pe = fast_exp2(sc[e] - m_new);
    pb[e] = from_f32<T>(pe);
    float pr = to_f32<T>(pb[e]);
    if constexpr (SplitP<T>::kSplit) {
      pl[e] = from_f32<T>(pe - pr);
      pr += to_f32<T>(pl[e]);
    }
    psum += pr;   // the sum uses the same rounded weights as P.V
  }
  l_run = l_run * alpha + psum;
  m_run = m_new;

  // Output rows are heads 4*quad + e; their rescale factors live in lanes
  // whose column (lane % 16) is that head.
  float ar[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) ar[e] = __shfl(alpha, 4 * quad + e);

  if (n_valid < kBlock) {
    // Keys past the end hold stale data (possibly NaN): zero them.
#pragma unroll
    for (int t = 0; t < VT; ++t) {
      uint32_t lo = cur.v[t][0], hi = cur.v[t][1];
      const int k0 = 4 * quad;
      if (k0 + 0 >= n_valid) lo &= 0xffff0000u;
      if (k0 + 1 >= n_valid) lo &= 0x0000ffffu;
      if (k0 + 2 >= n_valid) hi &= 0xffff0000u;
      if (k0 + 3 >= n_valid) hi &= 0x0000ffffu;
      cur.v[t] = u32x2{lo, hi};
    }
  }
  const u32x2 pa = {pack2(pb[0], pb[1]), pack2(pb[2], pb[3])};
  const u32x2 pal = {pack2(pl[0], pl[1]), pack2(pl[2], pl[3])};
#pragma unroll
  for (int t = 0; t < VT; ++t) {
    f32x4 c = o[t];
    c[0] *= ar[0];
    c[1] *= ar[1];
    c[2] *= ar[2];
    c[3] *= ar[3];
    c = mfma16x16x16<T>(pa, cur.v[t], c);
    if constexpr (SplitP<T>::kSplit) c = mfma16x16x16<T>(pal, cur.v[t], c);
    o[t] = c;
  }
}

// The W (virtual) wave states of one partition merged for head h, dimension
// d, in index order: the partition's max M, sum and unnormalised accumulator
// element.
template <int W, int NH, int D>
__device__ __forceinline__ void merge_waves(const float (*sm_m)[NH], const float (*sm_l)[NH],
                                            const float (*sm_o)[NH][D], int h, int d, float& M,
                                            float& lsum, float& acc) {
  M = -INFINITY;
#pragma unroll
  for (int v = 0; v < W; ++v) M = fmaxf(M, sm_m[v][h]);
  lsum = 0.f;
  acc = 0.f;
#pragma unroll
  for (int v = 0; v < W; ++v) {
    const float f = fast_exp2(sm_m[v][h] - M);
    lsum += sm_l[v][h] * f;
    acc += sm_o[v][h][d] * f;
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// The partitions of one (sequence, query head) merged by log-sum-exp, by one
// wave: m = max_p m_p; l = sum_p l_p 2^(m_p - m); o = sum_p acc_p 2^(m_p - m)
// / l, partitions in index order.  Partition p's (m_p, l_p) is ml[2p],
// ml[2p + 1] and its accumulator row starts at acc + p * acc_stride.  Lane p
// holds partition p's (m_p, l_p) (lanes take partitions p, p + 64, ... when
// there are more than 64), so the state is read once, and the accumulator
// loads of four partitions are in flight together.  Used by the merge pass
// (states in the workspace) and by the single-pass kernel (states in LDS).
template <class T, int D>
__device__ __forceinline__ void merge_partitions(const float* ml, const float* acc, int64_t acc_stride,
                                                 int np, int lane, uint16_t* out_row) {
  const float m0 = lane < np ? ml[2 * lane] : -INFINITY;
  const float l0 = lane < np ? ml[2 * lane + 1] : 0.f;
  float M = m0;
  for (int p = lane + 64; p < np; p += 64) M = fmaxf(M, ml[2 * p]);
  M = wave_max(M);
  const float w0 = fast_exp2(m0 - M);          // weight of partition `lane`
  float lsum = l0 * w0;
  for (int p = lane + 64; p < np; p += 64) lsum += ml[2 * p + 1] * fast_exp2(ml[2 * p] - M);
  lsum = wave_sum(lsum);
  constexpr int PER = D / 64;
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  for (int p0 = 0; p0 < np; p0 += 4) {
    float v[4][PER], f[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = p0 + k;
      f[k] = p >= np ? 0.f : p < 64 ? __shfl(w0, p) : fast_exp2(ml[2 * p] - M);
#pragma unroll
      for (int i = 0; i < PER; ++i)
        v[k][i] = p < np ? acc[static_cast<int64_t>(p) * acc_stride + lane + 64 * i] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int i = 0; i < PER; ++i) o[i] += v[k][i] * f[k];
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) out_row[lane + 64 * i] = from_f32<T>(o[i] / lsum);
}

// Per-wave softmax states of NS segments (a segment is one wave's share of
// one partition): running max (log2 units), running sum and unnormalised
// accumulator, for each of NH query heads.
template <int NH, int D, int NS>
struct WaveStates {
  float m[NS][NH];
  float l[NS][NH];
  float o[NS][NH][D];
};

// The blocks of a partition are interleaved over VW waves: wave v takes
// blocks start + v, start + v + VW, ... and keeps its own softmax state, and
// the partition's state is the merge of its VW wave states in index order
// (merge_waves).  VW depends only on the partition size, so it fixes the
// reduction order.  The walk below also lets pw < VW physical waves run the
// VW interleaved states, each taking several in turn, with results unchanged
// bit for bit.  Measured on MI355X, 4 physical waves for 8 states over a
// whole launch beat 8 only on batches of short contexts and lost elsewhere,
// so the kernels run one physical wave per state except on short partitions
// of the two-buffer kernel (decode_partition_kernel).
//
// A cursor is a position in the list of (partition p, wave state v,
// absolute block j) a physical wave visits: partitions p_first, p_first +
// p_step, ... below p_end (partition p holds blocks [pstart(p), pstart(p +
// 1))), states wl, wl + pw, ... below VW, blocks in steps of VW.  Its state
// goes to segment slot p * VW + v.  p >= p_end once the wave is done.
struct Cursor {
  int p, v, j;
};

template <int VW, class PStart>
struct SegmentWalk {
  int p_step, p_end, wl, pw;
  PStart pstart;

  // Moves c to the first segment at or after (c.p, c.v) that holds a block.
  __device__ __forceinline__ void enter(Cursor& c) const {
    while (c.p < p_end) {
      const int s0 = pstart(c.p);
      if (c.v < VW && c.v < pstart(c.p + 1) - s0) {
        c.j = s0 + c.v;
        return;
      }
      c.p += p_step;
      c.v = wl;
    }
  }
  __device__ __forceinline__ Cursor first(int p_first) const {
    Cursor c{p_first, wl, 0};
    enter(c);
    return c;
  }
  __device__ __forceinline__ void advance(Cursor& c) const {
    if (c.p >= p_end) return;
    c.j += VW;
    if (c.j < pstart(c.p + 1)) return;
    c.v += pw;
    enter(c);
  }
};

// Block ids of the blocks [b0, b0 + nb) of one table row, 64 per register
// with one per lane (nb <= 64 * kBtRegs).  An id outside the pool reads
// block 0 instead and is reported in `bad`.
__device__ __forceinline__ void load_table(int (&bt)[kBtRegs], const int32_t* row, int nb, int lane,
                                           int64_t num_blocks, bool& bad) {
  bad = false;
#pragma unroll
  for (int r = 0; r < kBtRegs; ++r) {
    bt[r] = 0;
    if (64 * r < nb) {                        // wave-uniform
      const int jj = 64 * r + lane;
      if (jj < nb) bt[r] = row[jj];
      const bool b = jj < nb && (bt[r] < 0 || bt[r] >= num_blocks);
      bad |= b;
      if (b) bt[r] = 0;
    }
  }
}

__device__ __forceinline__ int64_t table_entry(const int (&bt)[kBtRegs], int jj) {
  const int r = jj >> 6;                      // wave-uniform
  int id = __builtin_amdgcn_readlane(bt[0], jj & 63);
#pragma unroll
  for (int k = 1; k < kBtRegs; ++k)
    if (r == k) id = __builtin_amdgcn_readlane(bt[k], jj & 63);
  return id;
}

// Everything one physical wave does for one (sequence, head group): walk its
// segments with a register pipeline of NBUF block buffers (the loads of the
// next NBUF - 1 blocks are in flight while it works on the current one) and
// leave the state of every segment it visits in st.  Segments it has no block
// in must hold the empty state beforehand (store_empty).  `tbl_base` is the absolute
// block index of table register lane 0.
template <class T, int D, int NH, int NS, int VW, int NBUF, class Walk>
__device__ __forceinline__ void run_wave(const Walk& walk, int p_first, const int (&bt)[kBtRegs], int tbl_base,
                                         int L, const u32x4 (&qb)[D / 32], float scale_log2,
                                         const uint16_t* kbase, const uint16_t* vbase, int64_t blk_elems,
                                         int lane, WaveStates<NH, D, NS>& st) {
  constexpr int VT = D / 16;
  const int hl = lane & 15;
  const int quad = lane >> 4;
  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x4 o[VT];
#pragma unroll
  for (int t = 0; t < VT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  int slot = -1;
  auto flush = [&]() {
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (lane < NH) {
      st.m[slot][lane] = m_run;
      st.l[slot][lane] = l_run;
    }
#pragma unroll
    for (int t = 0; t < VT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int h = 4 * quad + e;
        if (h < NH) st.o[slot][h][16 * t + hl] = o[t][e];
      }
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int t = 0; t < VT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto process = [&](BlockRegs<T, D>& cur, const Cursor& c) __attribute__((always_inline)) {
    const int sl = c.p * VW + c.v;
    if (sl != slot) {
      if (slot >= 0) flush();
      slot = sl;
    }
    process_block<T, D>(cur, L - c.j * kBlock, qb, scale_log2, quad, m_run, l_run, o);
  };
  auto off = [&](int j) { return table_entry(bt, j - tbl_base) * blk_elems; };
  // Past the end, prefetches read block 0 of the pool (the host rejects an
  // empty pool when there is work): every wave's out-of-range prefetches
  // share those lines, which then stay in L2, where re-reading a wave's own
  // last block would go back to HBM under the non-temporal hint.  Issuing
  // them unconditionally keeps the wait before each block to its own loads.
  auto pf_off = [&](const Cursor& c) -> int64_t { return c.p < walk.p_end ? off(c.j) : int64_t(0); };

  Cursor c0 = walk.first(p_first);
  if (c0.p >= walk.p_end) return;
  Cursor c1 = c0;
  walk.advance(c1);
  if constexpr (NBUF == 2) {
    // One block in flight while the wave works on another.
    BlockRegs<T, D> b0, b1;
    load_block<T, D>(b0, kbase, vbase, off(c0.j));
    auto shift = [&]() {
      c0 = c1;
      walk.advance(c1);
    };
    for (;;) {
      load_block<T, D>(b1, kbase, vbase, pf_off(c1));
      process(b0, c0);
      shift();
      if (c0.p >= walk.p_end) break;
      load_block<T, D>(b0, kbase, vbase, pf_off(c1));
      process(b1, c0);
      shift();
      if (c0.p >= walk.p_end) break;
    }
  } else {
    // Two blocks in flight while the wave works on a third.
    Cursor c2 = c1;
    walk.advance(c2);
    BlockRegs<T, D> b0, b1, b2;
    load_block<T, D>(b0, kbase, vbase, off(c0.j));
    load_block<T, D>(b1, kbase, vbase, pf_off(c1));
    auto shift = [&]() {
      c0 = c1;
      c1 = c2;
      walk.advance(c2);
    };
    for (;;) {
      load_block<T, D>(b2, kbase, vbase, pf_off(c2));
      process(b0, c0);
      shift();
      if (c0.p >= walk.p_end) break;
      load_block<T, D>(b0, kbase, vbase, pf_off(c2));
      process(b1, c0);
      shift();
      if (c0.p >= walk.p_end) break;
      load_block<T, D>(b1, kbase, vbase, pf_off(c2));
      process(b2, c0);
      shift();
      if (c0.p >= walk.p_end) break;
    }
  }
  flush();
}

// The empty state (max -inf, sum 0, accumulator 0) in segment slot sl, as
// left by a virtual wave with no block: it adds nothing to the merge.
template <int NH, int D, int NS>
__device__ __forceinline__ void store_empty(WaveStates<NH, D, NS>& st, int sl, int lane) {
  if (lane < NH) {
    st.m[sl][lane] = -INFINITY;
    st.l[sl][lane] = 0.f;
  }
  for (int i = lane; i < NH * D; i += 64) st.o[sl][i / D][i % D] = 0.f;
}

// Q^T operand of one head group: head column lane % 16, dims 32*ks +
// 8*(lane/16) .. +7; columns beyond the group's nh heads are zero padding.
template <int D>
__device__ __forceinline__ void load_q(u32x4 (&qb)[D / 32], const uint16_t* q_rows, int nh, int lane) {
  const int hl = lane & 15;
  if (hl < nh) {
    const uint16_t* qp = q_rows + hl * D + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qb[ks] = *reinterpret_cast<const u32x4*>(qp + 32 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qb[ks] = u32x4{0, 0, 0, 0};
  }
}

// One partition of one (sequence, head group) per workgroup of W waves
// (W = 4 or 8, the partition's interleave), each with NBUF block buffers
// (2 or 3; either fits two waves per SIMD).
//
// Short partitions on the two-buffer 8-wave kernel (contexts of at most 2048
// tokens): a workgroup's fixed cost (start-up latency, the merge, the idle
// ends of its waves) is a large share of a partition of a few blocks per
// wave.  So a partition of at most kHalfWaveBlocks blocks runs its 8 wave
// states on waves 0-3 (wave w takes states w and w + 4 in turn, each over
// the same blocks in the same order, so the result is unchanged bit for
// bit), and waves 4-7 exit at once.  That kernel is capped at 3 waves per
// SIMD instead of 2 (140 registers fit 3), so the next workgroup can start
// beside the 4 remaining waves instead of after them.  Measured on MI355X,
// same box, three alternating runs: the 13B shared-prefix batch (median 400
// tokens) 247.7-248.4 -> 237.5-238.9 us, the 7B batch 193.3-194.0 -> 193.1-
// 193.2 us; cut-offs of 32-48 blocks took the 7B batch up to 197.5 us, 16
// blocks gained the 13B batch only 242 us.
template <class T, int D, int NH, int W, int NBUF>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, NBUF == 2 ? 3 : 2)))
void decode_partition_kernel(DecodeArgs a) {
  constexpr int kThreads = 64 * W;
  __shared__ WaveStates<NH, D, W> st;

  // blockIdx.x = (part * num_seqs + s) * (num_kv_heads * num_sub) + head group
  const int n_hg = a.num_kv_heads * a.num_sub;
  const int hg = static_cast<int>(blockIdx.x % static_cast<uint32_t>(n_hg));
  const uint32_t rest = blockIdx.x / static_cast<uint32_t>(n_hg);
  const int s = static_cast<int>(rest % static_cast<uint32_t>(a.num_seqs));
  const int part = static_cast<int>(rest / static_cast<uint32_t>(a.num_seqs));
  const int g = hg / a.num_sub;
  const int sub = hg - g * a.num_sub;
  const int hq0 = g * a.group + sub * 16;
  const int nh = min(16, a.group - sub * 16);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int L = a.context_lens[s];
  const int np = num_partitions(L, a);
  if (np <= 0) {
    // Empty context: zero rows.  Invalid length: NaN rows.  Partition 0 only.
    if (part == 0) {
      const uint16_t fill = np == 0 ? uint16_t(0) : from_f32<T>(NAN);
      for (int i = tid; i < nh * D; i += kThreads)
        a.out[(static_cast<int64_t>(s) * a.num_q_heads + hq0 + i / D) * D + i % D] = fill;
    }
    return;
  }
  if (part >= np) return;

  const int nb_seq = (L + kBlock - 1) / kBlock;
  const int blk0 = partition_start(part, nb_seq, np);
  const int nblk = partition_start(part + 1, nb_seq, np) - blk0;   // 1 .. part_blocks
  // Physical waves running the W wave states.  Whole waves leave before any
  // barrier; the barrier below then waits only for the waves that remain.
  const int pw = (W == 8 && NBUF == 2 && nblk <= kHalfWaveBlocks) ? W / 2 : W;
  if (w >= pw) return;

  int bt[kBtRegs];
  bool bad_id;
  load_table(bt, a.block_tables + static_cast<int64_t>(s) * a.bt_stride + blk0, nblk, lane, a.num_blocks,
             bad_id);
  const bool poison = __any(bad_id);

  for (int v = w; v < W; v += pw)
    if (v >= nblk) store_empty(st, v, lane);
  u32x4 qb[D / 32];
  load_q<D>(qb, a.q + (static_cast<int64_t>(s) * a.num_q_heads + hq0) * D, nh, lane);
  const int64_t tile_elems = static_cast<int64_t>(kBlock) * D;
  const int64_t blk_elems = static_cast<int64_t>(a.num_kv_heads) * tile_elems;
  const int hl = lane & 15, quad = lane >> 4;
  const uint16_t* kbase = a.k_cache + g * tile_elems + hl * 32 + 8 * quad;
  const uint16_t* vbase = a.v_cache + g * tile_elems + quad * (4 * D) + hl * 4;
  auto pstart = [=](int p) { return blk0 + (p > 0 ? nblk : 0); };
  const SegmentWalk<W, decltype(pstart)> walk{1, 1, w, pw, pstart};
  run_wave<T, D, NH, W, W, NBUF>(walk, 0, bt, blk0, L, qb, a.scale_log2, kbase, vbase, blk_elems, lane, st);
  __syncthreads();

  for (int i = tid; i < nh * D; i += 64 * pw) {
    const int h = i / D;
    const int d = i - h * D;
    float M, lsum, acc;
    merge_waves<W, NH, D>(st.m, st.l, st.o, h, d, M, lsum, acc);
    if (poison) acc = NAN;
    const int64_t row = static_cast<int64_t>(s) * a.num_q_heads + hq0 + h;
    if (np == 1) {
      a.out[row * D + d] = from_f32<T>(acc / lsum);
    } else {
      const int64_t slot = row * a.max_parts + part;
      a.ws_acc[slot * D + d] = acc;
      if (d == 0) {
        a.ws_ml[slot * 2] = M;
        a.ws_ml[slot * 2 + 1] = lsum;
      }
    }
  }
}

// Single-pass split-KV: one workgroup of NGRP * W waves takes every
// partition of one (sequence, head group) and merges them on chip, so the
// partition states never go through HBM.  Wave group gi = w / W takes
// partitions gi, gi + NGRP, ...; inside a partition its W waves interleave
// the blocks exactly as decode_partition_kernel does, each segment's state
// goes to LDS, and the states are merged with the same code as the two-pass
// path (merge_waves, then merge_partitions).  The result is therefore
// bit-identical to decode_partition_kernel + decode_merge_kernel at the same
// partition size, which keeps it independent of the batch the sequence is
// in.  Each wave's register pipeline runs on across partition boundaries.
// The whole block table of the sequence sits in registers (at most 64 *
// kBtRegs blocks) and at most PMAX partitions fit in LDS; the host only picks
// this kernel when both hold.
//
// Two groups of 4 waves (short partitions) keep one block in flight in two
// buffers and are capped at 3 waves per SIMD (144 registers), and their LDS
// budget is 78 KB whenever that still holds 8 partitions (a 4096-token
// context in 512-token partitions), so two workgroups fit a CU and one can
// start while the other ends.  Measured on MI355X, same box, three
// alternating runs, the 8B-GQA batch at 512-token partitions: 404.1-405.7 ->
// 399.4-400.0 us (two buffers and the cap alone: 403.1-403.5).  The 8-wave
// form (partitions of 2048 tokens and up) needs 2 waves per SIMD per
// workgroup, so a second one never fits; it keeps three buffers and 150 KB.
template <int VW, int NH, int D, int THREADS>
constexpr int fused_max_parts() {
  constexpr int per_part = (VW * NH * (D + 2) + 2 * NH) * 4;
  constexpr int small = 78 * 1024;
  constexpr int budget = (THREADS <= 256 || (VW == 4 && small / per_part >= 8)) ? small : 150 * 1024;
  return budget / per_part < 32 ? budget / per_part : 32;
}

template <class T, int D, int NH, int W, int NGRP>
__global__ __launch_bounds__(64 * W * NGRP) __attribute__((amdgpu_waves_per_eu(2, W == 4 ? 3 : 2)))
void decode_fused_kernel(DecodeArgs a) {
  constexpr int VW = W;
  constexpr int kThreads = 64 * W * NGRP;
  constexpr int PMAX = fused_max_parts<VW, NH, D, kThreads>();
  __shared__ WaveStates<NH, D, PMAX * VW> st;
  __shared__ float sm_ml[NH][PMAX][2];

  // blockIdx.x = s * num_kv_heads + KV head (one head sub-group: the host sends group <= 8)
  const int g = static_cast<int>(blockIdx.x % static_cast<uint32_t>(a.num_kv_heads));
  const int s = static_cast<int>(blockIdx.x / static_cast<uint32_t>(a.num_kv_heads));
  const int hq0 = g * a.group;
  const int nh = a.group;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gi = w / W;
  const int wl = w - gi * W;

  const int L = a.context_lens[s];
  const int np = num_partitions(L, a);
  if (np <= 0) {
    // Empty context: zero rows.  Invalid length: NaN rows.
    const uint16_t fill = np == 0 ? uint16_t(0) : from_f32<T>(NAN);
    for (int i = tid; i < nh * D; i += kThreads)
      a.out[(static_cast<int64_t>(s) * a.num_q_heads + hq0 + i / D) * D + i % D] = fill;
    return;
  }
  const int nb_seq = (L + kBlock - 1) / kBlock;   // <= 64 * kBtRegs, np <= PMAX (host)

  // The sequence's block ids; a bad id anywhere poisons the sequence's row,
  // as it does through the merge of the two-pass path.
  int bt[kBtRegs];
  bool bad_id;
  load_table(bt, a.block_tables + static_cast<int64_t>(s) * a.bt_stride, nb_seq, lane, a.num_blocks, bad_id);
  const bool poison = __any(bad_id);

  // Lane p holds the first block of partition p (p <= np < 64).
  const int start_lane = partition_start(min(lane, np), nb_seq, np);
  auto pstart = [=](int p) { return __builtin_amdgcn_readlane(start_lane, p); };
  for (int p = gi; p < np; p += NGRP)
    for (int v = wl; v < VW; v += W)
      if (v >= pstart(p + 1) - pstart(p)) store_empty(st, p * VW + v, lane);

  u32x4 qb[D / 32];
  load_q<D>(qb, a.q + (static_cast<int64_t>(s) * a.num_q_heads + hq0) * D, nh, lane);
  const int64_t tile_elems = static_cast<int64_t>(kBlock) * D;
  const int64_t blk_elems = static_cast<int64_t>(a.num_kv_heads) * tile_elems;
  const int hl = lane & 15, quad = lane >> 4;
  const uint16_t* kbase = a.k_cache + g * tile_elems + hl * 32 + 8 * quad;
  const uint16_t* vbase = a.v_cache + g * tile_elems + quad * (4 * D) + hl * 4;
  const SegmentWalk<VW, decltype(pstart)> walk{NGRP, np, wl, W, pstart};
  run_wave<T, D, NH, PMAX * VW, VW, W == 4 ? 2 : 3>(walk, gi, bt, 0, L, qb, a.scale_log2, kbase, vbase, blk_elems,
                                                   lane, st);
  __syncthreads();

  // Per partition, the VW wave states merged (same code as the two-pass
  // kernel).  A partition's accumulator replaces its first state in
  // place: the element (p * VW, h, d) is read only by the thread that writes it.
  for (int i = tid; i < np * nh * D; i += kThreads) {
    const int p = i / (nh * D);
    const int r = i - p * (nh * D);
    const int h = r / D;
    const int d = r - h * D;
    float M, lsum, acc;
    merge_waves<VW, NH, D>(st.m + p * VW, st.l + p * VW, st.o + p * VW, h, d, M, lsum, acc);
    if (poison) acc = NAN;
    if (np == 1) {
      a.out[(static_cast<int64_t>(s) * a.num_q_heads + hq0 + h) * D + d] = from_f32<T>(acc / lsum);
    } else {
      st.o[p * VW][h][d] = acc;
      if (d == 0) {
        sm_ml[h][p][0] = M;
        sm_ml[h][p][1] = lsum;
      }
    }
  }
  if (np == 1) return;
  __syncthreads();

  // The partitions merged per query head, one wave per head (the merge
  // pass's code, reading LDS instead of the workspace).
  for (int h = w; h < nh; h += W * NGRP)
    merge_partitions<T, D>(&sm_ml[h][0][0], &st.o[0][h][0], static_cast<int64_t>(VW) * NH * D, np, lane,
                           a.out + (static_cast<int64_t>(s) * a.num_q_heads + hq0 + h) * D);
}

// Second pass: one wave per (sequence, query head) with more than one
// partition, merging the partition states of the workspace.
template <class T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= static_cast<int64_t>(a.num_seqs) * a.num_q_heads) return;
  const int s = static_cast<int>(row / a.num_q_heads);
  const int np = num_partitions(a.context_lens[s], a);
  if (np <= 1) return;
  merge_partitions<T, D>(a.ws_ml + row * a.max_parts * 2, a.ws_acc + row * a.max_parts * D, D, np, lane,
                         a.out + row * D);
}

// How one call merges partitions, for query-head groups of NH (template
// bucket) and head_dim D: kMergeOnChip when the host chose the single pass
// (fuse_groups > 0: the batch fills the GPU without splitting, a sequence's
// table fits the registers and a head group is at most 8 query heads) and the
// partitions fit the kernel's LDS; kMergeTwoPass otherwise.
template <int D, int NH>
int merge_kind_nh(const DecodeArgs& a) {
  if (a.max_parts <= 1) return kMergeNone;
  if constexpr (NH > 8) {
    return kMergeTwoPass;
  } else {
    if (a.fuse_groups <= 0 || a.num_sub != 1) return kMergeTwoPass;
    const int cap = a.waves == 8 ? fused_max_parts<8, NH, D, 512>() : fused_max_parts<4, NH, D, 512>();
    return a.max_parts <= cap ? kMergeOnChip : kMergeTwoPass;
  }
}

template <class T, int D, int NH>
hipError_t launch_nh(const DecodeArgs& a, hipStream_t stream) {
  if constexpr (NH <= 8) {
    if (merge_kind_nh<D, NH>(a) == kMergeOnChip) {
      // One workgroup per (sequence, KV head): 8 waves on long partitions, or
      // two groups of 4 waves taking alternate short partitions.
      const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.num_seqs) * a.num_kv_heads));
      if (a.waves == 8)
        hipLaunchKernelGGL((decode_fused_kernel<T, D, NH, 8, 1>), grid, dim3(512), 0, stream, a);
      else
        hipLaunchKernelGGL((decode_fused_kernel<T, D, NH, 4, 2>), grid, dim3(512), 0, stream, a);
      return hipGetLastError();
    }
  }
  const int64_t n_wg = static_cast<int64_t>(a.max_parts) * a.num_seqs * a.num_kv_heads * a.num_sub;
  const dim3 grid(static_cast<uint32_t>(n_wg));
  if (a.waves == 8 && a.buffers == 2)
    hipLaunchKernelGGL((decode_partition_kernel<T, D, NH, 8, 2>), grid, dim3(512), 0, stream, a);
  else if (a.waves == 8)
    hipLaunchKernelGGL((decode_partition_kernel<T, D, NH, 8, 3>), grid, dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_partition_kernel<T, D, NH, 4, 3>), grid, dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;
  const int64_t rows = static_cast<int64_t>(a.num_seqs) * a.num_q_heads;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(static_cast<uint32_t>((rows + 3) / 4)),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Query heads per work item, rounded up to the template bucket 1, 2, 4, 8, 16.
int nh_bucket(int group) {
  const int nh = group < 16 ? group : 16;
  return nh <= 1 ? 1 : nh <= 2 ? 2 : nh <= 4 ? 4 : nh <= 8 ? 8 : 16;
}

template <class T, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  switch (nh_bucket(a.group)) {
    case 1: return launch_nh<T, D, 1>(a, stream);
    case 2: return launch_nh<T, D, 2>(a, stream);
    case 4: return launch_nh<T, D, 4>(a, stream);
    case 8: return launch_nh<T, D, 8>(a, stream);
    default: return launch_nh<T, D, 16>(a, stream);
  }
}

template <int D>
int merge_kind_d(const DecodeArgs& a) {
  switch (nh_bucket(a.group)) {
    case 1: return merge_kind_nh<D, 1>(a);
    case 2: return merge_kind_nh<D, 2>(a);
    case 4: return merge_kind_nh<D, 4>(a);
    case 8: return merge_kind_nh<D, 8>(a);
    default: return merge_kind_nh<D, 16>(a);
  }
}

}  // namespace

hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // The symbol resolves to the copy on the current device, which is dev.
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

int decode_merge_kind(const DecodeArgs& a, int head_dim) {
  return head_dim == 64 ? merge_kind_d<64>(a) : merge_kind_d<128>(a);
}

hipError_t launch_decode(const DecodeArgs& a, int head_dim, int dtype, hipStream_t stream) {
  if (dtype == 0) return head_dim == 64 ? launch_d<F16, 64>(a, stream) : launch_d<F16, 128>(a, stream);
  return head_dim == 64 ? launch_d<BF16, 64>(a, stream) : launch_d<BF16, 128>(a, stream);
}

}  // namespace pa
