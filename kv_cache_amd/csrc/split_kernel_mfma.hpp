// Split kernel for bf16 K/V with D = 128: QK^T on the matrix cores; PV on
// the vector ALUs for up to 4 (virtual) heads, on the matrix cores for 8 or
// more.
//
// Same ownership and output as split_kernel (workgroup (b, h_kv, s), G query
// heads, one exact (m, l, u) state per head, "M4.5 - Decode Attention Kernels,
// Mask Programs, and Backend Boundaries", sections 0x02A and 0x03A).  Each wave
// consumes tiles of 16 visible rows:
//
//  * Scores.  v_mfma_f32_16x16x32_bf16 with A = the 16 K rows of the tile
//    (M = rows, K = 32 channels per instruction, 4 instructions for D = 128)
//    and B = the q rows of the group (N = 16 columns, the first G used, the
//    rest zero).  Lane l loads 16 bytes of row l%16 for channel group l/16 of
//    each 32-channel slice, i.e. exactly the A operand; q is loaded once in
//    the B operand layout.  The result gives lane l the scores of rows
//    4*(l/16) .. 4*(l/16)+3 for head l%16.  The products of the bf16 inputs
//    are exact and accumulate in fp32, so this is a small dense tile of the
//    GQA group rather than a reshaped memory-bound product.
//  * Softmax.  Per head: tile maximum across the 4 lanes that hold the head,
//    online rescale of the running state, p = 2^(s - m) (scores in base 2).
//  * PV.  Row slot r = l/16 owns rows 4r .. 4r+3 of the tile; lane l holds
//    channels 8*(l%16) .. +7 of those V rows and accumulates u for the G heads.
//    The weight p(row 4r+j, head i) sits in lane 16r+i of the same 16-lane
//    DPP row, so it is fetched with row_newbcast:i.
//  * PV with 8 or more heads.  v_mfma_f32_16x16x16_bf16 per 16-row tile:
//    A = the weights (heads x rows of the tile) as bf16 hi + lo, two
//    instructions per block, B = V (rows x channels).  Block c takes channel
//    8n + c of the tile's rows, i.e. element c of the 8 channels lane n
//    already holds, so the V registers feed the matrix cores without moving
//    between lanes.
#pragma once

#include <type_traits>

#include "split_common.hpp"

namespace da {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Broadcast lane I of each 16-lane row to the whole row.
template <int I>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + I, 0xF, 0xF, false));
}

template <int G, int I = 0>
struct HeadLoop {
  // u[i][:] = u[i][:] * row_bcast<i>(scale)
  __device__ __forceinline__ static void rescale(float (&u)[G][8], float scale) {
    const float a = row_bcast<I>(scale);
#pragma unroll
    for (int e = 0; e < 8; ++e) u[I][e] *= a;
    HeadLoop<G, I + 1>::rescale(u, scale);
  }
  // u[i][:] += row_bcast<i>(w) * v[:]
  __device__ __forceinline__ static void accumulate(float (&u)[G][8], float w, const float (&v)[8]) {
    const float a = row_bcast<I>(w);
#pragma unroll
    for (int e = 0; e < 8; ++e) u[I][e] = fmaf(a, v[e], u[I][e]);
    HeadLoop<G, I + 1>::accumulate(u, w, v);
  }
};
template <int G>
struct HeadLoop<G, G> {
  __device__ __forceinline__ static void rescale(float (&)[G][8], float) {}
  __device__ __forceinline__ static void accumulate(float (&)[G][8], float, const float (&)[8]) {}
};

struct MfmaTile {
  uint4 k[4];   // A operand, one per 32-channel slice
  uint4 v[4];   // V rows 4r + j, channels 8*(l%16) .. +7
};

// Waves per SIMD the register budget must allow: 4 (<= 128 VGPRs) for up to
// 4 heads per group, so that four 4-wave workgroups are resident on every CU
// and a grid of 4 x CU workgroups runs in one round; 8 heads need 64
// accumulators per lane and get 3.
template <int G> struct MfmaOccupancy { static constexpr int value = G <= 4 ? 4 : 3; };
// A partitioned run is sized for one round of workgroups at this many per CU
// (the host's default item count uses the same figure).
constexpr int kPartitionWgPerCu = 3;

// FlashMask tile numbering ("M4.5 ...", sections 0x06C-0x06F: SKIP blocks
// are never visited, and the work a split does should follow the blocks that
// are not skipped, not the positions they cover).  The workgroup classifies
// all of the request's 16-key tiles for the decode row from the block
// summaries and numbers the non-SKIP ones in position order; split s takes
// numbers [s*ct, (s+1)*ct) with ct = ceil(count / S), so the splits share the
// tiles to load evenly whatever the mask hides, as the sink+window mask is
// compiled into visible ordinals.  Every workgroup of the request derives the
// same numbering, so the splits stay a disjoint exact cover of the non-SKIP
// tiles.
struct Empty {};
template <int NWAVES>
struct FmCompact {
  static constexpr int kEntries = kFmMaxTiles / 64;   // 64 tiles per entry
  uint64_t ns[kEntries];    // entry e: non-SKIP bits of tiles 64e .. 64e+63
  uint64_t pa[kEntries];    // PARTIAL bits of the same tiles
  int pre[kEntries];        // non-SKIP tiles before entry e
  uint32_t list[64];        // the split's tiles in order: tile | PARTIAL << 31
  int count;                // non-SKIP tiles of the request
};

// The summaries of tiles 64*wave + lane (this wave's entry of the first
// pass), requested before the request length is known.
struct FmFirst {
  int4 u, l;
};
template <int NWAVES>
__device__ __forceinline__ FmFirst fm_prefetch(const SplitParams& p, int b, int wave, int lane) {
  if (p.n_mask_blocks <= 0) return FmFirst{};
  const int t = min(64 * wave + lane, p.n_mask_blocks - 1);
  const int4* sm = p.mask_sum + ((int64_t)b * p.n_mask_blocks + t) * 2;
  return FmFirst{sm[0], sm[1]};
}

// Fills f.list with split s's tiles and returns how many there are (<= 64:
// ct <= ceil(ceil(T/16) / S) <= plan chunk / 16).  Contains three workgroup
// barriers: every wave calls it.
template <int NWAVES>
__device__ __forceinline__ int fm_compact(const SplitParams& p, int b, int q_row, int n_vis, int s,
                                          const FmFirst& first, FmCompact<NWAVES>& f, int wave, int lane) {
  const int nblk = min((n_vis + 15) / 16, kFmMaxTiles);   // the plan admits n_vis <= 16 * kFmMaxTiles
  const int ne = (nblk + 63) / 64;
  for (int e = wave; e < ne; e += NWAVES) {
    const int t = 64 * e + lane;
    int cls = kTileSkip;
    if (t < nblk) cls = e == wave ? fm_class(q_row, first.u, first.l) : fm_tile_class(p, b, q_row, 16 * t);
    const uint64_t ns = __ballot(cls != kTileSkip);
    const uint64_t pa = __ballot(cls == kTilePartial);
    if (lane == 0) {
      f.ns[e] = ns;
      f.pa[e] = pa;
    }
  }
  __syncthreads();
  if (wave == 0) {
    // Exclusive prefix of the entries' counts, 64 entries per pass, by bit
    // planes: a count c <= 64 is the sum of its bits (c >> k & 1) << k, and
    // the lanes below this one holding bit k number mbcnt(ballot of bit k).
    // No cross-lane data movement, so no LDS round trips.
    int run = 0;
    for (int e0 = 0; e0 < ne; e0 += 64) {
      const int e = e0 + lane;
      const int c = e < ne ? __popcll(f.ns[e]) : 0;
      int x = 0, sum = 0;
#pragma unroll
      for (int k = 0; k < 7; ++k) {
        const uint64_t bk = __ballot((c >> k) & 1);
        x += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bk, 0u)) << k;
        sum += __popcll(bk) << k;
      }
      if (e < ne) f.pre[e] = run + x;
      run += sum;
    }
    if (lane == 0) f.count = run;
  }
  __syncthreads();
  const int total = f.count;
  const int ct = (total + p.num_splits - 1) / p.num_splits;
  const int j0 = min(s * ct, total), j1 = min(j0 + ct, total);
  for (int e = wave; e < ne; e += NWAVES) {
    const uint64_t ns = f.ns[e];
    const int idx = f.pre[e] + __popcll(ns & ((1ull << lane) - 1));
    if (((ns >> lane) & 1) && idx >= j0 && idx < j1 && idx - j0 < 64)
      f.list[idx - j0] = (uint32_t)(64 * e + lane) | ((uint32_t)((f.pa[e] >> lane) & 1) << 31);
  }
  __syncthreads();
  return min(j1 - j0, 64);
}

// INSTR: kInstrRows is the index-trace instance, which also records each row
// load where it is issued (trace_k / trace_v); kInstrStamps records
// per-workgroup timestamps; otherwise identical.
template <int G, bool PAGED, int NWAVES, bool FUSED, bool FM, bool PART = false, int INSTR = 0>
__global__ __launch_bounds__(NWAVES * 64, PART ? kPartitionWgPerCu : MfmaOccupancy<G>::value) void split_kernel_mfma(SplitParams p) {
  constexpr int D = 128;
  constexpr int TW = 16;
  constexpr int kStep = NWAVES * TW;   // rows of one step of the workgroup's waves
  static_assert(G >= 1 && G <= 16, "");

  WgStamps<INSTR> stamps(p);
  const PartitionHeaderAtExit header_at_exit{p};
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
  const int n = lane & 15;     // K row of the tile / score column (head)
  const int kg = lane >> 4;    // channel group of the MFMA slice / V row slot
  __shared__ WaveStates<G, D, NWAVES> sh;
  __shared__ std::conditional_t<FM, FmCompact<NWAVES>, Empty> fmc;

  // One piece of work: visible ordinals [pbeg, pend) of request b for K/V
  // head h, stored as split slot s.  pend < 0: the plan's split s.
  auto piece = [&](int b, int h, int s, int pbeg, int pend) {
  // B operand: q[head n][32c + 8kg .. +7], zero for columns n >= G; requested
  // before the request length is known.
  uint4 qop[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    qop[c] = make_uint4(0u, 0u, 0u, 0u);
    if (n < G)
      qop[c] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) +
                                               out_row(p, b, h, n) * D + 32 * c + 8 * kg);
  }

  // Row addresses: lane (n, kg) loads 16 bytes of K row n at channel 8kg of
  // each 32-channel slice, and 16 bytes of V row 4kg + j at channel 8n.
  const RowAddr ra = row_addr<PAGED>(p, b, h, D);
  const int64_t hb = ra.base;
  const uint16_t* kb = static_cast<const uint16_t*>(p.k) + hb + 8 * kg;
  const uint16_t* vb = static_cast<const uint16_t*>(p.v) + hb + 8 * n;
  const uint32_t row_stride = p.row_stride;
  // Speculative first tile: with a plain contiguous cache and the causal mask
  // the first tile's rows (ordinals s*chunk + wave*16 + r, positions equal to
  // ordinals) do not depend on the request length, so they are requested
  // before it arrives, clamped to the capacity (in bounds); once the split end
  // is known, rows at or past it get zero V, and their scores are masked like
  // those of any row past the end.
  MfmaTile t;
  bool spec = false;
  int spec_t0 = 0;
  if constexpr (!PAGED && !FM && !PART) {
    spec = p.mask_kind == DA_MASK_CAUSAL && p.layout == DA_LAYOUT_CONTIG_NHD && !p.cache_batch_idx &&
           p.kv_capacity > 0;
    if (spec) {
      // the first tile of a full split under the sweep rotation below
      const int t0 = s * p.chunk + kStep * sweep_start(b, s, (p.chunk + kStep - 1) / kStep) + wave * TW;
      spec_t0 = t0;
      const int cap = p.kv_capacity;
      const uint16_t* row = kb + (uint64_t)(uint32_t)min(t0 + n, cap - 1) * row_stride;
#pragma unroll
      for (int c = 0; c < 4; ++c) t.k[c] = stream_load<kHalfLineNT>(reinterpret_cast<const uint4*>(row + 32 * c));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t rj = (uint32_t)min(t0 + 4 * kg + j, cap - 1);
        t.v[j] = stream_load(reinterpret_cast<const uint4*>(vb + (uint64_t)rj * row_stride));
      }
    }
  }

  FmFirst fm_first{};
  if constexpr (FM) fm_first = fm_prefetch<NWAVES>(p, b, wave, lane);
  const int T = request_len(p, b);
  const VisProgram vis = make_vis(T, p.mask_kind, p.n_sink, p.window);
  int begin, end;
  if (FM) {
    begin = 0;            // the split's share is its tile list (below)
    end = vis.n_vis;
  } else if (pend < 0) {
    split_range(vis.n_vis, s, p.chunk, &begin, &end);
  } else {
    begin = min(pbeg, vis.n_vis);
    end = min(pend, vis.n_vis);
  }

  // K rows of tile tl: lane (n, kg) loads row tl + n, whose row index is ri.
  // The trace instance records the rows inside the split (loads past its end
  // repeat a visible row and are weighted 0).
  auto issue_k = [&](int tl, uint32_t ri, uint4 (&k)[4]) {
    const uint16_t* row = kb + (uint64_t)ri * row_stride;
#pragma unroll
    for (int c = 0; c < 4; ++c) k[c] = stream_load<kHalfLineNT>(reinterpret_cast<const uint4*>(row + 32 * c));
    if constexpr (INSTR == kInstrRows) {
      if (kg == 0 && tl + n >= begin && tl + n < end)
        trace_k(p, b, h, tl + n, vis_pos(vis, tl + n), hb + (int64_t)((uint64_t)ri * row_stride));
    }
  };
  // V rows of tile tl: lane (n, kg) loads rows tl + 4kg + j, whose row
  // indices lanes 4kg + j hold.
  auto issue_v = [&](int tl, uint32_t ri, uint4 (&v)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t rj = (uint32_t)__shfl((int)ri, 4 * kg + j);
      v[j] = stream_load(reinterpret_cast<const uint4*>(vb + (uint64_t)rj * row_stride));
      if constexpr (INSTR == kInstrRows) {
        const int o = tl + 4 * kg + j;
        if (n == 0 && o >= begin && o < end) trace_v(p, b, h, o, hb + (int64_t)((uint64_t)rj * row_stride));
      }
    }
  };
  // Score column n is virtual head n, with its own visible end (C > 1 rows).
  // An empty split (begin == end) runs no tile and stores the empty state
  // (m = -inf, l = 0, u = 0) through the same merge as any other.
  const int end_n = min(end, row_limit(p, vis.n_vis, n));

  // Row r of the tile is ordinal tile + r; rows past the split end are
  // clamped to its last row, which is visible and finite, and then get weight
  // 0 (score -inf), so the loads need no branches.  Lane l resolves the row
  // index of tile row l%16 (one page-table lookup per row); the V rows 4kg+j
  // take theirs from lane 4kg+j.
  auto row_index = [&](int tile) {
    return kv_row_index<PAGED>(p, ra, vis_pos(vis, min(tile + n, end - 1)));
  };

  float m_run = -INFINITY;   // running max of head n (base 2), equal in the 4 lanes of the head
  float l_run = 0.f;         // partial denominator over rows 4kg .. 4kg+3 of every tile
  float u[G][8];
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) u[i][e] = 0.f;
  // Eight or more (virtual) heads: PV on the matrix cores, o[c] of lane (n, kg)
  // accumulating heads 4kg .. 4kg+3 at channel 8n + c (the VALU form would
  // need 8 FMAs per head, row and channel group: issue-bound at G = 8).
  constexpr bool kMfmaPV = G >= 8;
  f32x4_t o[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) o[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // One tile of registers: the next tile's K rows are requested as soon as
  // the score instructions have read the current ones, its V rows once the
  // current ones have arrived (PV then reads them from a copy) or, where
  // registers are short, once PV has read them.  The requests after the last tile repeat
  // row end-1 (already cached) and keep the loop free of branches.
  // FlashMask: the split's non-SKIP tiles come from fm_compact in position
  // order; the wave walks entries wave, wave + NWAVES, ... of that list, its
  // k-th tile held by lane k (read with v_readlane).  PARTIAL tiles bring the
  // interval vectors of their rows with their K rows.
  const int q_row = vis.n_vis - 1;
  const int past = end + NWAVES * TW * 2;     // any ordinal >= end: row_index clamps it
  int n_mine = 0, kc = 0;                     // FlashMask: the wave's tiles, index of the current one
  uint32_t mine = 0;                          // lane k: the wave's k-th list entry
  if constexpr (FM) {
    const int n_list = fm_compact<NWAVES>(p, b, q_row, vis.n_vis, s, fm_first, fmc, wave, lane);
    n_mine = n_list > wave ? (n_list - wave + NWAVES - 1) / NWAVES : 0;   // <= 16
    if (lane < n_mine) mine = fmc.list[wave + NWAVES * lane];
  }
  auto entry_at = [&](int k) -> uint32_t { return (uint32_t)__builtin_amdgcn_readlane((int)mine, k & 63); };
  // Sweep order (no FlashMask): the split's steps of NWAVES tiles are visited
  // from step j0 on and wrap around, wave w taking tile w of each step that
  // has one (only the last step can lack it).  j0 staggers the splits' starts
  // (sweep_start), or is 0 where the wave has fewer steps than the staggered
  // start.
  const int n_steps = (end - begin + kStep - 1) / kStep;
  int j0 = 0;
  if constexpr (!FM && !PAGED) {
    // (contiguous NHD: the request and split strides are the large powers of
    // two; paged and HND caches are read in step order)
    const int ref = (pend < 0 && !PART) ? (p.chunk + kStep - 1) / kStep : n_steps;
    j0 = p.layout == DA_LAYOUT_CONTIG_NHD ? sweep_start(b, s, ref) : 0;
    if (j0 >= n_steps) j0 = 0;
  }
  auto tile_at = [&](int k) -> int {          // first position of the wave's tile k
    if constexpr (FM) {
      return k < n_mine ? TW * (int)(entry_at(k) & 0x7fffffffu) : past;
    } else {
      if (k >= n_steps) return past;
      const int j = j0 + k;
      return begin + kStep * (j >= n_steps ? j - n_steps : j) + wave * TW;
    }
  };
  auto partial_at = [&](int k) -> bool {
    if constexpr (FM) return k < n_mine && (entry_at(k) >> 31) != 0u;
    else return false;
  };
  auto first_tile = [&]() -> int { return tile_at(0); };
  // The wave's tile d steps after the current one (d = 1, 2).
  auto ahead = [&](int, int d) -> int { return tile_at(kc + d); };
  // whether the wave has a tile at step k (FlashMask: a listed tile)
  auto has_step = [&](int tile, int k) -> bool {
    if constexpr (FM) return tile < end;
    else return k < n_steps;
  };
  int4 ivt = make_int4(0, 0, 0, 0);   // FlashMask intervals of row tile + n (PARTIAL tiles)
  auto issue_iv = [&](int tile, bool part) {
    if constexpr (FM) {
      if (tile < end && part) ivt = p.mask_iv[(int64_t)b * p.max_seq_len + min(tile + n, end - 1)];
    }
  };

  int tile = first_tile();
  // Row indices run one tile ahead of the loads that use them, so a paged
  // cache's block-table lookup is off the load path.
  uint32_t ri = 0, ri_ahead = 0;
  if (has_step(tile, 0)) {
    if (spec && tile == spec_t0) {
      // the first tile (t0) was requested above; trace its rows now that the
      // split end is known, with the row indices those loads used
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (tile + 4 * kg + j >= end) t.v[j] = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (INSTR == kInstrRows) {
          // tile == t0 here, the first row of the loads above
          const int o = tile + 4 * kg + j;
          const uint32_t rj = (uint32_t)min(o, p.kv_capacity - 1);
          if (n == 0 && o < end) trace_v(p, b, h, o, hb + (int64_t)((uint64_t)rj * row_stride));
        }
      }
      if constexpr (INSTR == kInstrRows) {
        const uint32_t rk = (uint32_t)min(tile + n, p.kv_capacity - 1);
        if (kg == 0 && tile + n < end)
          trace_k(p, b, h, tile + n, vis_pos(vis, tile + n), hb + (int64_t)((uint64_t)rk * row_stride));
      }
    } else {
      ri = row_index(tile);
      issue_k(tile, ri, t.k);
      issue_iv(tile, partial_at(kc));
      issue_v(tile, ri, t.v);
    }
    ri_ahead = row_index(ahead(tile, 1));
  }
  while (has_step(tile, kc)) {
    const int next_tile = ahead(tile, 1);
    uint32_t hidden = 0;                  // rows of this tile hidden by FlashMask (bit r)
    if constexpr (FM) {
      if (partial_at(kc)) hidden = (uint32_t)__ballot(fm_hidden(ivt, q_row)) & 0xFFFFu;
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, t.k[c]),
                                                    __builtin_bit_cast(bf16x8_t, qop[c]), acc, 0, 0, 0);
    ri = ri_ahead;
    ri_ahead = row_index(ahead(tile, 2));
    issue_k(next_tile, ri, t.k);
    issue_iv(next_tile, partial_at(kc + 1));
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sc[i] = (tile + 4 * kg + i < end_n && !((hidden >> (4 * kg + i)) & 1u)) ? acc[i] * p.qscale
                                                                             : -INFINITY;
    float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mt = xor32_max(xor16_max(mt));
    const float mn = fmaxf(m_run, mt);
    const float mz = mn == -INFINITY ? 0.f : mn;     // no -inf - -inf
    const float alpha = fast_exp2(m_run - mz);
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(sc[i] - mz);
    l_run = fmaf(l_run, alpha, (pr[0] + pr[1]) + (pr[2] + pr[3]));
    m_run = mn;

    // The next tile's V rows are requested before PV reads this tile's (kept
    // in a second set of registers), so they are in flight during PV -- where
    // the registers allow it: not with a paged cache's table lookups at four
    // waves per SIMD, nor with eight heads.
    constexpr bool kEarlyV = (!PAGED || PART) && G <= 4;
    uint4 vcur[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vcur[j] = t.v[j];
    if constexpr (kEarlyV) issue_v(next_tile, ri, t.v);
    if constexpr (kMfmaPV) {
      // O (heads x channels) += P (heads x the tile's 16 rows) V: A = P of
      // head n, rows 4kg .. 4kg+3, as bf16 hi + lo (together exact to about
      // 2^-17); B block c = channel 8n + c of rows 4kg .. 4kg+3, taken from
      // the V registers (v_mfma_f32_16x16x16_bf16: lane (n, kg) holds k rows
      // 4kg .. 4kg+3 of column n), so no value moves between lanes.
      if (__any(alpha != 1.f)) {      // skipped while no head max moved
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = __shfl(alpha, 4 * kg + i);
#pragma unroll
          for (int c = 0; c < 8; ++c) o[c][i] *= a;
        }
      }
      uint32_t ah[2], al[2];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const float x0 = pr[2 * q2], x1 = pr[2 * q2 + 1];
        const uint32_t hw = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1) << 16);
        const float r0 = x0 - bf16_lo(hw), r1 = x1 - bf16_hi(hw);
        ah[q2] = hw;
        al[q2] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)r0) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)r1) << 16);
      }
      const s16x4_t a_hi = __builtin_bit_cast(s16x4_t, make_uint2(ah[0], ah[1]));
      const s16x4_t a_lo = __builtin_bit_cast(s16x4_t, make_uint2(al[0], al[1]));
      auto word = [](const uint4& v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; };
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;   // high or low half of each word
        const uint32_t b01 = __builtin_amdgcn_perm(word(vcur[1], c >> 1), word(vcur[0], c >> 1), sel);
        const uint32_t b23 = __builtin_amdgcn_perm(word(vcur[3], c >> 1), word(vcur[2], c >> 1), sel);
        const s16x4_t bv = __builtin_bit_cast(s16x4_t, make_uint2(b01, b23));
        o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_hi, bv, o[c], 0, 0, 0);
        o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_lo, bv, o[c], 0, 0, 0);
      }
    } else {
      if (__any(alpha != 1.f)) HeadLoop<G>::rescale(u, alpha);   // skipped while no head max moved
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w[4] = {vcur[j].x, vcur[j].y, vcur[j].z, vcur[j].w};
        float vx[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) { vx[2 * e] = bf16_lo(w[e]); vx[2 * e + 1] = bf16_hi(w[e]); }
        HeadLoop<G>::accumulate(u, pr[j], vx);
      }
    }
    if constexpr (!kEarlyV) issue_v(next_tile, ri, t.v);
    tile = next_tile;
    ++kc;
  }

  if constexpr (kMfmaPV) {
    // o in the layout of u: lane (n, kg) keeps head i at channels 8n .. 8n+7
    // where kg = i / 4 (the sums over kg below complete it), zero elsewhere
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) u[i][e] = kg == (i >> 2) ? o[e][i & 3] : 0.f;
  }
  // ---- wave state: all rows of a head share m, so l and u just add ---------
  l_run = xor32_sum(xor16_sum(l_run));
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u[i][e] = xor32_sum(xor16_sum(u[i][e]));
    }

  if (kg == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) sh.u[wave][i][8 * n + e] = u[i][e];
    if (n < G) {
      sh.m[wave][n] = m_run;
      sh.l[wave][n] = l_run;
    }
  }
  __syncthreads();
  merge_waves_and_store<G, D, NWAVES, FUSED>(p, b, h, s, sh);
  stamps.states_stored();
  stamps.folded = finish_split<G, D, NWAVES, FUSED>(p, b, h);
  };

  if constexpr (!PART) {
    int b, h, s;
    decode_workgroup(p, &b, &h, &s);
    piece(b, h, s, 0, -1);
  } else {
    // Balanced partition: workgroup (item, h) takes ordinals [item*L,
    // (item+1)*L) of the requests' visible ordinals laid end to end, one piece
    // per request it meets, stored as split slot (items since the request's
    // first).  Descriptor values are checked against the plan, so a corrupt
    // descriptor skips work instead of addressing memory outside the buffers.
    static_assert(!FUSED && !FM, "partitions fold in the combine kernel; FlashMask walks <= 64 tiles");
    const int32_t* part = p.partition;
    const int h = (int)(blockIdx.x % (unsigned)p.num_kv_heads);
    const int item = (int)(blockIdx.x / (unsigned)p.num_kv_heads);
    const int L = part[1];
    if (part[2] != p.batch || L <= 0 || item >= part[0]) return;
    int x = item * L;
    const int xe = min(x + L, part[4 + p.batch]);
    for (int b = part[5 + p.batch + item]; x < xe && b >= 0 && b < p.batch; ++b) {
      const int pb = part[4 + b], pb1 = part[5 + b];
      if (pb1 <= x) continue;                     // empty request
      const int j = item - pb / L;
      if (j < 0 || j >= p.num_splits || x < pb) return;
      if (x != item * L) __syncthreads();          // the previous piece has read sh
      piece(b, h, j, x - pb, min(xe, pb1) - pb);
      x = min(xe, pb1);
    }
  }
}

}  // namespace da
