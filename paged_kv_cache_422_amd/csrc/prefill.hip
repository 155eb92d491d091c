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
//   one wave64 = 32 query rows of one query head;
//   one 512-thread workgroup = 8 waves over (heads of one KV group) x (row
//   tiles), all reading the same keys;
//   key tiles of 64 keys (four 16-token blocks) are staged in LDS once per
//   workgroup: the K/V of the next two tiles are in flight in registers
//   while the current tile is computed, then written to LDS between two
//   barriers.
// Per key tile a wave computes S^T[64 keys x 32 rows] = K . Q^T (two 32-key
// halves, D/16 MFMAs each), masks the causal diagonal and the sequence end,
// updates an online softmax per row in registers, and accumulates
// O^T[D x 32 rows] += V^T . P^T (D/32 x 4 MFMAs).
//
// Precision of P.V.  fp16 data: weights in fp16, one product each (good to
// 2^-12).  bf16 data: Q.K^T stays in bf16, but V is converted to fp16 while
// it is staged (exact up to 65504: bf16's 8 significant bits fit in fp16's
// 11) and P.V runs in fp16 with one product per weight.  bf16 weights alone
// (8 significant bits) would break the tolerance when a few keys carry the
// softmax, so a workgroup whose fp16 pass read a V value beyond fp16's range
// (it converts to inf, and the accumulators end non-finite) starts over with
// bf16 weights split into hi + lo halves (two products).
//
// Operand layouts.  In LDS the K rows of each 32-key half are stored with
// bits 2 and 3 of the key index swapped, so the accumulator element i of
// lane l (half h = l / 32) holds key 16 * (i / 8) + 8 * h + i % 8: the eight
// probabilities a lane feeds to the P.V step for 16 keys are its own eight
// consecutive accumulator elements, and the matching V^T operand is eight
// consecutive keys of one dimension, i.e. 16 contiguous bytes of that
// dimension's LDS row (V is staged as one row of 16 keys per dimension; the
// cache holds it in groups of four keys, [key / 4][dim][key % 4]).  LDS rows
// are padded by 16 bytes so that the 16-byte operand reads of a wave hit
// distinct banks.  Each XCD takes a contiguous
// run of row blocks of one chunk and head group (so they share its L2), and
// within it row blocks are dispatched heaviest (longest causal range) first.
#include <float.h>
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace pa {

namespace {

constexpr int kBlock = 16;
constexpr int kTileKeys = 64;                      // keys per LDS stage
constexpr int kTileBlocks = kTileKeys / kBlock;

template <class T, int D>
struct PrefillLds {
  static constexpr int kRow = D * 2 + 16;          // bytes per K row (one key)
  static constexpr int kVRow = kBlock * 2 + 16;    // bytes per V row (one dim of a block)
  static constexpr int kBytesK = kTileKeys * kRow;
  static constexpr int kBytesVBlock = D * kVRow;
  static constexpr int kBytesStage = kBytesK + kTileBlocks * kBytesVBlock;
  static constexpr int kBytes = kBytesStage;
};

template <class X> struct TypeTag { using type = X; };
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Position of key r (0..31) of a 32-key half in LDS: bits 2 and 3 swapped.
__device__ __forceinline__ int swap_bits23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

constexpr int kPrefillWaves = 8;
constexpr int kXcds = 8;              // MI355X: 8 XCDs, 32 CUs and one L2 each
constexpr float kLazyLog2 = 8.f;      // running-maximum slack, log2 units
constexpr int kPrefetch = 4;          // LDS operand reads in flight ahead of the MFMAs
constexpr int kPrefillThreads = 64 * kPrefillWaves;

template <class T, int D>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillArgs a) {
  using Lds = PrefillLds<T, D>;
  constexpr int KS = D / 16;                 // QK^T k-steps
  constexpr int DT = D / 32;                 // 32-dim output tiles
  constexpr int UPB = 2 * D;                 // 16-byte units per block per tensor
  constexpr int UPT = kTileBlocks * UPB / kPrefillThreads;   // units per thread per tensor per tile
  __shared__ __attribute__((aligned(16))) unsigned char lds[Lds::kBytes];

  // Workgroups are dealt to the 8 XCDs round-robin by linear index, and each
  // XCD has its own L2.  Renumber them so that XCD x takes a contiguous run
  // of the (row block, chunk, head group) order: the row blocks of one chunk
  // and head group, which read the same keys, then share one L2 instead of
  // streaming those keys through all eight.  The renumbering is a bijection
  // for any workgroup count (XCD x owns ceil((n - x) / 8) of them).
  int bx, by, bz;
  {
    const int nx = gridDim.x, ny = gridDim.y;
    const int n = nx * ny * static_cast<int>(gridDim.z);
    const int lin = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
    const int q8 = n / kXcds, r8 = n % kXcds, x = lin % kXcds;
    const int v = x * q8 + min(x, r8) + lin / kXcds;
    bx = v % nx;
    by = (v / nx) % ny;
    bz = v / (nx * ny);
  }
  const int c = by;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int r32 = lane & 31;

  // Waves split over heads of the group first, then over row tiles.
  const int G = a.group;
  const int hpw = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const int tiles_per_wg = kPrefillWaves / hpw;
  const int nhsub = G / hpw;
  const int g = bz / nhsub;
  const int hsub = bz - g * nhsub;
  const int hq = g * G + hsub * hpw + (w % hpw);
  const int rt = w / hpw;
  const int wg_rows = 32 * tiles_per_wg;
  const int n_rb = (a.max_q_len + wg_rows - 1) / wg_rows;
  const int rb = n_rb - 1 - bx;

  const int r_start = a.q_start_loc[c];
  const int n = a.q_start_loc[c + 1] - r_start;
  const int L = a.seq_lens[c];
  const int n_cached = L - n;
  if (n <= 0) return;                        // empty chunk
  const int wg_row0 = rb * wg_rows;
  if (wg_row0 >= n) return;                  // whole workgroup past the chunk
  const int row0 = wg_row0 + rt * 32;
  const bool wave_on = row0 < n;
  const int my_row = row0 + r32;
  const bool row_ok = my_row < n;
  const int64_t out_row = (static_cast<int64_t>(r_start) + my_row) * a.num_q_heads + hq;

  // A chunk longer than max_q_len (the grid covers only that many rows per
  // chunk) or a length outside the host's bounds gets NaN in every row the
  // grid covers.
  const bool bad_len = n > a.max_q_len || n_cached < 0 || L > a.max_seq_len || L > a.bt_stride * kBlock;
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
  // Logits enter the exponent as fma(s, c, -m) with c = |scale * log2(e)|,
  // so the tile maximum can be taken on the raw products.  A negative scale
  // is carried by Q instead: flipping its sign bits is exact, and the
  // products come out exactly negated.  A zero scale becomes the smallest
  // normal float, which leaves every weight at exactly 1 and keeps masked
  // keys (-inf) at -inf rather than NaN.
  const float c_log2 = a.scale_log2 == 0.f ? FLT_MIN : fabsf(a.scale_log2);
  if (a.scale_log2 < 0.f) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) qb[ks][e] ^= 0x80008000u;
  }

  const int wg_last_row = min(wg_row0 + wg_rows - 1, n - 1);
  const int key_end = n_cached + wg_last_row + 1;            // keys the workgroup needs
  const int n_tiles = __builtin_amdgcn_readfirstlane((key_end + kTileKeys - 1) / kTileKeys);
  const int nb_seq = (L + kBlock - 1) / kBlock;
  const int lim = min(n_cached + my_row, L - 1);              // last visible key of my row
  const int wave_lim = min(n_cached + min(row0 + 31, n - 1), L - 1);    // last key any row of the wave sees
  const int wave_lim_lo = min(n_cached + row0, L - 1);                  // last key every row of the wave sees
  // The table is read through the constant address space: it is not written
  // while the kernel runs, and a wave-uniform index then becomes a scalar
  // load, which keeps off the vector-load counter the K/V waits use.
  typedef const int32_t __attribute__((address_space(4)))* TableRow;
  const TableRow bt = (TableRow)(a.block_tables + static_cast<int64_t>(c) * a.bt_stride);
  const int64_t tile_elems = static_cast<int64_t>(kBlock) * D;
  const int64_t blk_elems = static_cast<int64_t>(a.num_kv_heads) * tile_elems;
  const int64_t head_off = static_cast<int64_t>(g) * tile_elems;
  // Block ids are int32, so the pool bound can be too: the id check below
  // then stays a 32-bit scalar compare (there is no 64-bit scalar compare).
  const uint32_t nb_bound = static_cast<uint32_t>(min<int64_t>(a.num_blocks, INT32_MAX));

  // Cooperative loads of one key tile: unit u = r * threads + tid of each
  // tensor is 16 bytes of block u / UPB of the tile.  Two register sets hold
  // the next two tiles; a tile index past the end re-reads the last tile so
  // that the loads are unconditional and each wait covers only its own set.
  u32x4 pk0[UPT], pv0[UPT], pk1[UPT], pv1[UPT];
  bool bad_id = false;
  auto fetch = [&](u32x4 (&pk)[UPT], u32x4 (&pv)[UPT], int t) __attribute__((always_inline)) {
    t = min(t, n_tiles - 1);
#pragma unroll
    for (int r = 0; r < UPT; ++r) {
      const int u = r * kPrefillThreads + tid;
      // The block of a unit is the same for the whole wave (UPB is a multiple
      // of 64), so its table entry is one scalar load.
      const int lb = t * kTileBlocks + (r * kPrefillThreads + w * 64) / UPB;
      const int wu = u % UPB;
      // Blocks past the sequence end read its last block (always valid); the
      // stash zeroes their V, and their keys are masked.
      int id = bt[min(lb, nb_seq - 1)];
      if (static_cast<uint32_t>(id) >= nb_bound) {   // negative ids wrap to large
        bad_id |= lb < nb_seq;
        id = 0;
      }
      const int64_t base = static_cast<int64_t>(id) * blk_elems + head_off;
      pk[r] = *reinterpret_cast<const u32x4*>(a.k_cache + base + static_cast<int64_t>(wu) * 8);
      pv[r] = *reinterpret_cast<const u32x4*>(a.v_cache + base + static_cast<int64_t>(wu) * 8);
    }
  };
  // Registers -> LDS.  V slots past the sequence end are zeroed (they may
  // hold stale data, and 0 * NaN would leak into P.V).  With kHalf the V
  // tile is stored as fp16, rounded to nearest: bf16 -> fp16 is exact for
  // magnitudes up to 65504 (8 significant bits fit in 11) and loses at most
  // 2^-25 in absolute terms below fp16's normal range; every larger bf16
  // magnitude (65536 and up) becomes inf, and NaN stays NaN.
  auto stash = [&](auto half_tag, const u32x4 (&pk)[UPT], const u32x4 (&pv)[UPT],
                   int t) __attribute__((always_inline)) {
    constexpr bool kHalf = decltype(half_tag)::value;
#pragma unroll
    for (int r = 0; r < UPT; ++r) {
      const int u = r * kPrefillThreads + tid;
      const int b = u / UPB;
      const int wu = u % UPB;
      // K unit wu is 16 bytes of 32-dim chunk wu / 64: key (wu / 4) % 16,
      // dims 32 * (wu / 64) + 8 * (wu % 4) .. +7.
      // Keys past the sequence end are stored as read (the last block's
      // stale slots, or the last block again): every tile that reaches past a
      // row's last visible key replaces those scores by -inf with a select,
      // so whatever they hold, NaN included, never reaches the softmax.
      const int kt = b * kBlock + ((wu >> 2) & (kBlock - 1));   // key within the tile
      const int row = (kt & 32) | swap_bits23(kt & 31);
      *reinterpret_cast<u32x4*>(lds + row * Lds::kRow + ((wu >> 6) * 4 + (wu & 3)) * 16) = pk[r];
      // V unit wu is 16 bytes of key group kg = wu / (D/2): dims d0 and
      // d0 + 1 (d0 = 2 * (wu % (D/2))), keys 4*kg .. +3 of each; dword e holds
      // dim d0 + e/2, keys 4*kg + 2*(e%2) and the next.
      // A wave's 64 units start at a multiple of 64; with D/2 = 64 units per
      // key group (D = 128) they lie in one group, so kg is wave-uniform and
      // the end-of-sequence test below is a scalar branch.  With D = 64 a
      // wave covers two groups.
      int kg = wu / (D / 2);
      if constexpr ((D / 2) % 64 == 0) kg = __builtin_amdgcn_readfirstlane(kg);
      const int d0 = 2 * (wu % (D / 2));
      // Keys of this group past the sequence end (all four when n_ok <= 0)
      // are zeroed half by half.
      u32x4 v = pv[r];
      const int n_ok = L - ((t * kTileBlocks + b) * kBlock + 4 * kg);   // keys of this group in range
      if (n_ok < 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 2 * (e & 1);
          uint32_t x = v[e];
          if (k >= n_ok) x &= 0xffff0000u;
          if (k + 1 >= n_ok) x &= 0x0000ffffu;
          v[e] = x;
        }
      }
      if constexpr (kHalf) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x = v[e];
          const f32x2 f = {__builtin_bit_cast(float, x << 16), __builtin_bit_cast(float, x & 0xffff0000u)};
          v[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
        }
      }
      unsigned char* const vrow = lds + Lds::kBytesK + b * Lds::kBytesVBlock + d0 * Lds::kVRow + kg * 8;
      *reinterpret_cast<u32x2*>(vrow) = u32x2{v[0], v[1]};
      *reinterpret_cast<u32x2*>(vrow + Lds::kVRow) = u32x2{v[2], v[3]};
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;

  // One key tile: S^T, online softmax, P.V, all from LDS.
  // The first kPrefetch K operands of a tile, read right after the barrier
  // that publishes it, ahead of the fetch: the fetch's wait for its table
  // entries then covers their LDS latency too.
  const unsigned char* const kr = lds + r32 * Lds::kRow + 16 * half;
  auto kop = [&](int j) __attribute__((always_inline)) {
    return *reinterpret_cast<const u32x4*>(kr + (j & 1) * 32 * Lds::kRow + 32 * (j >> 1));
  };
  u32x4 kb[kPrefetch];
  auto preload_k = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) kb[j] = kop(j);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto compute = [&](auto half_tag, int t) __attribute__((always_inline)) {
    const int k0 = t * kTileKeys;
    if (!wave_on || k0 > wave_lim) return;

    // S^T for the two 32-key halves of the tile, their k-steps alternating
    // (two independent accumulation chains).  Operand j is read from LDS
    // kPrefetch products ahead of its use, and the scheduling fences keep
    // the compiler from sinking the reads next to their uses.
    f32x16 s[2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[c2][i] = 0.f;
    {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2 * KS; ++j) {
        s[j & 1] = mfma32x32x16<T>(kb[j % kPrefetch], qb[j >> 1], s[j & 1]);
        if (j + kPrefetch < 2 * KS) kb[j % kPrefetch] = kop(j + kPrefetch);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // Element i of half c2 in this lane is key k0 + 32*c2 + 16*(i/8) + 8*half + i%8.
    // Only tiles that cross some row's last visible key need the mask.
    const bool need_mask = k0 + kTileKeys - 1 > wave_lim_lo;
    float mx = -INFINITY;
    if (need_mask) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 32 * c2 + 16 * (i / 8) + 8 * half + (i % 8);
          s[c2][i] = (key <= lim) ? s[c2][i] : -INFINITY;
          mx = fmaxf(mx, s[c2][i]);
        }
    } else {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[c2][i]);
    }
    mx = max_xor32(mx);
    // Lazy rescaling: the running maximum moves only when the tile's exceeds
    // it by more than kLazyLog2, so weights stay below 2^kLazyLog2 (the
    // arithmetic is unchanged and fp32 has the range) and the accumulators
    // are rescaled only when some row of the wave moves.  A row with no
    // visible key in the tile has mx = -inf, which never moves.
    const float mt = mx * c_log2;
    const bool move = mt > m_run + kLazyLog2;
    if (__ballot(move)) {
      const float m_new = move ? mt : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
    }
    const float neg_m = -m_run;
    // One P.V pass in element type P from the V copy at vbase.  kPart 0
    // enters each weight whole, 1 its leading half (its type's rounding of
    // it), 2 the remainder; passes 0 and 1 add the unrounded weights to the
    // row sum.  fp16 weights alone are good to 2^-12 and bf16 hi + lo to
    // about 2^-17, so either way the normalisation stays consistent with P.V
    // to far below the output's own rounding.  Splitting into two passes
    // (recomputing the exponentials) keeps one set of P operands live.
    auto pv_pass = [&](auto ptag, auto part, const unsigned char* vbase) __attribute__((always_inline)) {
      using P = typename decltype(ptag)::type;
      constexpr int kPart = decltype(part)::value;
      float psum = 0.f;
      const unsigned char* vr = vbase + r32 * Lds::kVRow + 16 * half;
      auto vop = [&](int j) __attribute__((always_inline)) {
        return *reinterpret_cast<const u32x4*>(vr + (j / DT) * Lds::kBytesVBlock + 32 * (j % DT) * Lds::kVRow);
      };
      u32x4 vb[kPrefetch];
#pragma unroll
      for (int j = 0; j < kPrefetch; ++j) vb[j] = vop(j);
      __builtin_amdgcn_sched_barrier(0);
      u32x4 pB[4];                     // P^T operands of the four 16-key k-steps
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          uint16_t w16[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float pe = fast_exp2(fmaf(s[c2][8 * cc + j], c_log2, neg_m));   // masked: -inf
            const uint16_t h = from_f32<P>(pe);
            w16[j] = kPart == 2 ? from_f32<P>(pe - to_f32<P>(h)) : h;
            if constexpr (kPart != 2) psum += pe;
          }
          pB[2 * c2 + cc] = u32x4{pack2(w16[0], w16[1]), pack2(w16[2], w16[3]), pack2(w16[4], w16[5]), pack2(w16[6], w16[7])};
        }
      if constexpr (kPart != 2) l_run += psum;

      // O^T += V^T . P^T; k-step kk covers block kk of the tile, keys
      // 8*half .. +7.  Product j = (kk, dt) = (j / DT, j % DT); operands are
      // read kPrefetch products ahead, as for S^T, the first ones before the
      // exponentials above (they do not depend on P).
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4 * DT; ++j) {
        o[j % DT] = mfma32x32x16<P>(vb[j % kPrefetch], pB[j / DT], o[j % DT]);
        if (j + kPrefetch < 4 * DT) vb[j % kPrefetch] = vop(j + kPrefetch);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    using Part0 = std::integral_constant<int, 0>;
    using Part1 = std::integral_constant<int, 1>;
    using Part2 = std::integral_constant<int, 2>;
    if constexpr (decltype(half_tag)::value) {
      pv_pass(TypeTag<F16>{}, Part0{}, lds + Lds::kBytesK);
    } else if constexpr (SplitP<T>::kSplit) {
      pv_pass(TypeTag<T>{}, Part1{}, lds + Lds::kBytesK);
      pv_pass(TypeTag<T>{}, Part2{}, lds + Lds::kBytesK);
    } else {
      pv_pass(TypeTag<T>{}, Part0{}, lds + Lds::kBytesK);
    }
  };

  // Tiles go in pairs, one per register set, with a single exit test at the
  // bottom (an odd count gets one more, fully masked tile whose compute
  // returns at once): a break between the two halves would merge a path on
  // which set 1 was never loaded into the loop header and force every wait
  // there to drain all loads.
  auto run = [&](auto half_tag) __attribute__((always_inline)) {
    fetch(pk0, pv0, 0);
    __builtin_amdgcn_sched_barrier(0);   // keep set 0's loads older than set 1's
    fetch(pk1, pv1, 1);
    int t = 0;
    do {
      __syncthreads();                 // every wave is done with the previous tile
      stash(half_tag, pk0, pv0, t);
      __syncthreads();                 // tile t is in LDS
      preload_k();
      fetch(pk0, pv0, t + 2);
      compute(half_tag, t);
      __syncthreads();
      stash(half_tag, pk1, pv1, t + 1);
      __syncthreads();
      preload_k();
      fetch(pk1, pv1, t + 3);
      compute(half_tag, t + 1);
      t += 2;
    } while (t < n_tiles);
  };
  // bf16 data first tries the fp16 P.V (one product per weight).  A V value
  // the fp16 copy could not hold (inf, NaN, or 65536 and up) makes the
  // accumulators of every wave that read its tile non-finite: its weight is
  // finite and >= 0, and 0 * inf is NaN in the matrix product.  A workgroup
  // where any accumulator ended non-finite starts over with split bf16
  // weights (two products per weight).  Waves that never read such a tile
  // do not depend on it, so a finite fp16 pass is exact to its own rounding.
  bool done = false;
  if constexpr (std::is_same<T, BF16>::value) {
    run(std::true_type{});
    bool bad = false;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) bad |= !__builtin_isfinite(o[dt][i]);
    done = !__syncthreads_or(bad);
  }
  if (!done) {
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    run(std::false_type{});
  }

  const bool poison = __syncthreads_or(bad_id);
  l_run = add_xor32(l_run);
  if (!row_ok) return;
  const float inv_nan = poison ? NAN : 0.f;
  uint16_t* op = a.out + out_row * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      // elements 4*q4 .. 4*q4+3: dims 32*dt + 8*q4 + 4*half + 0..3
      uint16_t r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = from_f32<T>(o[dt][4 * q4 + e] / l_run + inv_nan);
      *reinterpret_cast<u32x2*>(op + 32 * dt + 8 * q4 + 4 * half) = u32x2{pack2(r[0], r[1]), pack2(r[2], r[3])};
    }
}

template <class T, int D>
hipError_t launch_td(const PrefillArgs& a, hipStream_t stream) {
  const int G = a.group;
  const int hpw = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const int wg_rows = 32 * (kPrefillWaves / hpw);
  const int n_rb = (a.max_q_len + wg_rows - 1) / wg_rows;
  const dim3 grid(n_rb, a.num_chunks, a.num_kv_heads * (G / hpw));
  hipLaunchKernelGGL((prefill_kernel<T, D>), grid, dim3(kPrefillThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int dtype, hipStream_t stream) {
  if (dtype == 0) return head_dim == 64 ? launch_td<F16, 64>(a, stream) : launch_td<F16, 128>(a, stream);
  return head_dim == 64 ? launch_td<BF16, 64>(a, stream) : launch_td<BF16, 128>(a, stream);
}

}  // namespace pa
