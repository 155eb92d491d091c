// Chunked-prefill attention over the paged KV cache for gfx950 (MI355X).
//
// The scheduler serves decode first and fills the rest of a step's token
// budget with prefill chunks ("PagedAttention in vLLM: A Throughput Settings
// Guide", section "Tuning Batching, Prefill, and Cache").  A chunk continues
// its own sequence: its n query rows are the sequence's newest tokens (their
// K/V already written to the cache), so row j sits at position
// n_cached + j and attends keys 0 .. n_cached + j, read through the
// sequence's block table like any other paged read ("Inside vLLM: How
// PagedAttention Changes Python LLM Inference at the Systems Level", section
// "PagedAttention: What the OS Figured Out Decades Ago").
//
// This is a dense contraction, so it runs on the matrix cores (MFMA
// 32x32x16, fp32 accumulate).  Flash-style tiling:
//   one wave64  = 32 query rows of one query head,
//   one 256-thread workgroup = 4 waves over (heads of one KV group) x (row
//   tiles), so the 4 waves read the same K/V tiles (L1/L2 reuse),
//   key tiles of 32 = two 16-token blocks.
// Per key tile a wave computes S^T[32 keys x 32 rows] = K . Q^T (D/16 MFMAs),
// masks the causal diagonal and the sequence end, updates an online softmax
// per row in registers, and accumulates O^T[D x 32 rows] += V^T . P^T
// (2 * D/32 MFMAs).  The accumulator layout of S^T is the operand layout P^T
// needs (keys permuted consistently in V^T), and O^T's columns are the same
// rows as S^T's, so neither probabilities nor rescale factors move between
// lanes.  V is stored dim-major per block, so V^T operands are 8-byte loads.
// Row tiles are dispatched heaviest (longest causal range) first.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace pa {

namespace {

constexpr int kBlock = 16;

template <class T, int D>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  constexpr int KS = D / 16;   // QK k-steps
  constexpr int DT = D / 32;   // 32-dim output tiles
  const int c = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;          // 0 / 1: which 8-element k slice / key group
  const int r32 = lane & 31;

  // Waves split over heads of the group first, then over row tiles.
  const int G = a.group;
  const int hpw = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const int tiles_per_wg = 4 / hpw;
  const int nhsub = G / hpw;
  const int g = blockIdx.z / nhsub;
  const int hsub = blockIdx.z - g * nhsub;
  const int hq = g * G + hsub * hpw + (w % hpw);
  const int rt = w / hpw;
  const int wg_rows = 32 * tiles_per_wg;
  const int n_rb = (a.max_q_len + wg_rows - 1) / wg_rows;
  const int rb = n_rb - 1 - static_cast<int>(blockIdx.x);

  const int r_start = a.q_start_loc[c];
  const int n = a.q_start_loc[c + 1] - r_start;
  const int L = a.seq_lens[c];
  const int n_cached = L - n;
  if (n <= 0 || n > a.max_q_len) return;   // nothing addressable to write
  const int row0 = rb * wg_rows + rt * 32;
  if (row0 >= n) return;
  const int my_row = row0 + r32;
  const bool row_ok = my_row < n;
  const int64_t out_row = (static_cast<int64_t>(r_start) + my_row) * a.num_q_heads + hq;

  const bool bad_len = n_cached < 0 || L > a.max_seq_len || L > a.bt_stride * kBlock;
  if (bad_len) {
    if (row_ok) {
      const uint16_t nanv = from_f32<T>(NAN);
      for (int d = half; d < D; d += 2) a.out[out_row * D + d] = nanv;
    }
    return;
  }

  // Q^T operand: row my_row, dims 16*ks + 8*half .. +7.
  u32x4 qb[KS];
  if (row_ok) {
    const uint16_t* qp = a.q + out_row * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = u32x4{0, 0, 0, 0};
  }

  const int last_row = min(row0 + 31, n - 1);
  const int key_end = n_cached + last_row + 1;       // keys this wave needs
  const int n_tiles = (key_end + 31) / 32;
  const int nb_seq = (L + kBlock - 1) / kBlock;
  const int lim = min(n_cached + my_row, L - 1);      // last visible key of my row
  const int32_t* bt = a.block_tables + static_cast<int64_t>(c) * a.bt_stride;
  const int64_t tile_elems = static_cast<int64_t>(kBlock) * D;
  const int64_t blk_elems = static_cast<int64_t>(a.num_kv_heads) * tile_elems;
  const int64_t head_off = static_cast<int64_t>(g) * tile_elems;

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  bool poison = false;

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int k0 = kt * 32;
    const int lb0 = k0 / kBlock;
    int p0 = bt[lb0];
    int p1 = (lb0 + 1 < nb_seq) ? bt[lb0 + 1] : -1;
    if (p0 < 0 || p0 >= a.num_blocks) { poison = true; p0 = 0; }
    if (lb0 + 1 < nb_seq && (p1 < 0 || p1 >= a.num_blocks)) { poison = true; p1 = 0; }

    // K operand: key r32 of the tile (block r32/16, slot r32%16), dims
    // 16*ks + 8*half .. +7.
    const int pk = (r32 < kBlock) ? p0 : p1;
    u32x4 kr[KS];
    if (pk >= 0) {
      const uint16_t* kp = a.k_cache + pk * blk_elems + head_off + (r32 & 15) * D + 8 * half;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kr[ks] = *reinterpret_cast<const u32x4*>(kp + 16 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kr[ks] = u32x4{0, 0, 0, 0};
    }
    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sacc = mfma32x32x16<T>(kr[ks], qb[ks], sacc);

    // Element i of this lane is key k0 + 8*(i/4) + 4*half + i%4 of row my_row.
    float sc[16];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = k0 + 8 * (i / 4) + 4 * half + (i % 4);
      sc[i] = (key <= lim) ? sacc[i] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sc[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    uint16_t pbits[16], plo[16];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pe = fast_exp2(sc[i] - m_new);
      pbits[i] = from_f32<T>(pe);
      float pr = to_f32<T>(pbits[i]);
      if constexpr (SplitP<T>::kSplit) {
        plo[i] = from_f32<T>(pe - pr);
        pr += to_f32<T>(plo[i]);
      }
      psum += pr;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[t][i] *= alpha;

    // P^T operand for k-step ks: this lane's elements 8*ks .. 8*ks+7.
    u32x4 pB[2], pBl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      pB[ks] = u32x4{pack2(pbits[8 * ks + 0], pbits[8 * ks + 1]), pack2(pbits[8 * ks + 2], pbits[8 * ks + 3]),
                     pack2(pbits[8 * ks + 4], pbits[8 * ks + 5]), pack2(pbits[8 * ks + 6], pbits[8 * ks + 7])};
      pBl[ks] = u32x4{pack2(plo[8 * ks + 0], plo[8 * ks + 1]), pack2(plo[8 * ks + 2], plo[8 * ks + 3]),
                      pack2(plo[8 * ks + 4], plo[8 * ks + 5]), pack2(plo[8 * ks + 6], plo[8 * ks + 7])};
    }

    // V^T operand for k-step ks (= block ks of the tile): dim 32*t + r32,
    // slots 4*half .. +3 and 8 + 4*half .. +3 (the same key order as P^T).
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int pv = ks ? p1 : p0;
      if (pv < 0) continue;                              // whole block past the end
      const int kbase = k0 + 16 * ks;
      const int valid = L - kbase;                       // keys of this block in range
      const uint16_t* vp = a.v_cache + pv * blk_elems + head_off + r32 * kBlock + 4 * half;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const uint16_t* vt = vp + static_cast<int64_t>(32 * t) * kBlock;
        u32x2 lo = *reinterpret_cast<const u32x2*>(vt);
        u32x2 hi = *reinterpret_cast<const u32x2*>(vt + 8);
        if (valid < kBlock) {
          // Slots past the sequence end hold stale data (possibly NaN).
          const int s0 = 4 * half;
          uint32_t w0 = lo[0], w1 = lo[1], w2 = hi[0], w3 = hi[1];
          if (s0 + 0 >= valid) w0 &= 0xffff0000u;
          if (s0 + 1 >= valid) w0 &= 0x0000ffffu;
          if (s0 + 2 >= valid) w1 &= 0xffff0000u;
          if (s0 + 3 >= valid) w1 &= 0x0000ffffu;
          if (s0 + 8 >= valid) w2 &= 0xffff0000u;
          if (s0 + 9 >= valid) w2 &= 0x0000ffffu;
          if (s0 + 10 >= valid) w3 &= 0xffff0000u;
          if (s0 + 11 >= valid) w3 &= 0x0000ffffu;
          lo = u32x2{w0, w1};
          hi = u32x2{w2, w3};
        }
        const u32x4 vA = {lo[0], lo[1], hi[0], hi[1]};
        o[t] = mfma32x32x16<T>(vA, pB[ks], o[t]);
        if constexpr (SplitP<T>::kSplit) o[t] = mfma32x32x16<T>(vA, pBl[ks], o[t]);
      }
    }
  }

  l_run += __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const float inv_nan = poison ? NAN : 0.f;
  uint16_t* op = a.out + out_row * D;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      // elements 4*q4 .. 4*q4+3: dims 32*t + 8*q4 + 4*half + 0..3
      uint16_t r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = from_f32<T>(o[t][4 * q4 + e] / l_run + inv_nan);
      *reinterpret_cast<u32x2*>(op + 32 * t + 8 * q4 + 4 * half) = u32x2{pack2(r[0], r[1]), pack2(r[2], r[3])};
    }
}

template <class T, int D>
hipError_t launch_td(const PrefillArgs& a, hipStream_t stream) {
  const int G = a.group;
  const int hpw = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const int wg_rows = 32 * (4 / hpw);
  const int n_rb = (a.max_q_len + wg_rows - 1) / wg_rows;
  const dim3 grid(n_rb, a.num_chunks, a.num_kv_heads * (G / hpw));
  hipLaunchKernelGGL((prefill_kernel<T, D>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int dtype, hipStream_t stream) {
  if (dtype == 0) return head_dim == 64 ? launch_td<F16, 64>(a, stream) : launch_td<F16, 128>(a, stream);
  return head_dim == 64 ? launch_td<BF16, 64>(a, stream) : launch_td<BF16, 128>(a, stream);
}

}  // namespace pa
