// Device-side address and mask code shared by the split kernels and their
// index-trace instances (one source of truth for which K/V rows a workgroup
// reads).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_attn.h"

namespace da {

// Instrumentation instances of a split kernel (a template parameter): the
// product code, the index trace (every row load recorded where it is
// issued), or per-workgroup timestamps.
constexpr int kInstrNone = 0, kInstrRows = 1, kInstrStamps = 2;

// Index trace outputs of a split kernel's trace instance, one slot per
// (b, h_kv, visible ordinal), `stride` ordinals per (b, h_kv).
struct TraceOut {
  int64_t* k_off;    // element offset of the K row's first element
  int64_t* v_off;    // element offset of the V row's first element
  int32_t* pos;      // logical key position
  int32_t* count;    // +1 per K row load, +(1 << 16) per V row load
  int64_t* ks_off;   // int8 codes: element offset of the K scale row used (else unused)
  int64_t* vs_off;   // int8 codes: element offset of the V scale used (else unused)
  int32_t stride;
};

// Kernel arguments of the split kernels (passed by value).
struct SplitParams {
  const void* q;
  const void* k;
  const void* v;
  const uint16_t* k_scale;   // fp16 bits
  const uint16_t* v_scale;   // fp16 bits
  const void* k_resid;
  const void* v_resid;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* work_order;
  const int32_t* indptr;           // ragged rows / CSR table entries, [B + 1]
  const int32_t* cache_batch_idx;  // contiguous: cache row of each request, or null
  const int4* mask_iv;             // FlashMask: [B, max_seq_len] (UTS, UTE, LTS, LTE)
  const int4* mask_sum;            // FlashMask: [B, n_mask_blocks, 2] block min/max pairs
  const int32_t* partition;        // balanced partition [W, L, B, 0, P_0..P_B, first request of item i], or null
  int32_t* ws_part;                // workspace partition header [W, L, B, 0, P_0..P_B] for the combine
  float* ws_u;
  float* ws_m;
  float* ws_l;
  uint32_t* counters;        // one arrival counter per (b, h_kv) (single-launch mode)
  float* out;                // single-launch mode: O [B, H_q, D]
  float* lse;                // single-launch mode: LSE [B, H_q] or null
  int32_t num_q_heads;
  int32_t num_queries;       // C query rows per request (bottom-right causal)
  int32_t q_group_shift;     // log2(H_q / H_kv)
  int32_t num_kv_heads;
  int32_t batch;
  int32_t num_splits;
  int32_t chunk;
  int32_t kv_capacity;
  int32_t page_size;
  int32_t page_shift;        // log2(page_size) when a power of two, else -1
  int32_t max_pages;
  int32_t mask_kind;
  int32_t n_sink;
  int32_t window;
  int32_t k_group_shift;     // log2(k_group)
  int32_t residual_len;
  int32_t residual_policy;   // DA_RESIDUAL_*
  int32_t max_seq_len;       // plan bound: seq_lens are clamped to [0, max_seq_len]
  int32_t num_pages;
  int32_t layout;            // DA_LAYOUT_*
  int32_t page_csr;          // paged: 1 for DA_PAGE_TABLE_CSR
  int32_t cache_rows;        // contiguous: B_c (0: B); ragged: packed rows
  int32_t num_page_entries;  // CSR table entries
  uint32_t row_stride;       // elements between consecutive row indices
  uint32_t page_rows;        // paged: row indices per page (P for NHD, H_kv*P for HND)
  int32_t n_mask_blocks;     // FlashMask: ceil(max_seq_len / 16)
  float qscale;              // softmax_scale * log2(e): scores are kept in base-2 units
  int32_t num_cus;           // the plan's CU count (host-side launch choices only)
  TraceOut tr;               // trace instances only
  uint64_t* stamps;          // timestamp instances only: [grid, 4]
};

// ---------------------------------------------------------------------------
// Mask program.  The visible set of the decode row of a request with visible
// length T is at most two intervals ("M5.4 - Long-Context KV Policies:
// Retention, Compression, and Budget Allocation", sections 0x04-0x05):
// causal [0, T); sink+window [0, min(n_sink, T)) U [max(0, T - W), T).  It is
// compiled into (ns, gap): the o-th visible row (o = 0, 1, ...) sits at
// position o for o < ns and o + gap after, and N = T - gap rows are visible.
// Splits partition the ordinals [0, N), so a workgroup never enumerates a
// hidden row: every SKIP tile of "M4.5 - Decode Attention Kernels, Mask
// Programs, and Backend Boundaries" section 0x05C is dropped before any
// address work (section 0x05D), and the only PARTIAL tiles are ragged tails,
// whose out-of-range rows get score -inf before the max (section 0x05C).
// ---------------------------------------------------------------------------
struct VisProgram {
  int n_vis;
  int ns;
  int gap;
};

__device__ __forceinline__ VisProgram make_vis(int T, int kind, int n_sink, int window) {
  VisProgram v;
  if (kind == DA_MASK_SINK_WINDOW) {
    const int ns = min(n_sink, T);
    const int ws = max(0, T - window);
    v.ns = ns;
    v.gap = max(0, ws - ns);
    v.n_vis = T - v.gap;
  } else {
    v.ns = T;
    v.gap = 0;
    v.n_vis = T;
  }
  return v;
}

// ---------------------------------------------------------------------------
// FlashMask ("M4.5 ...", sections 0x06A-0x06D): key t is hidden from query
// row q when q lies in [UTS_t, UTE_t) or [LTS_t, LTE_t).  A block of 16 keys
// is classified for the rows [q, q+1) from its eight min/max values.
// ---------------------------------------------------------------------------
constexpr int kMaskBlock = 16;
enum { kTileSkip = 0, kTileFull = 1, kTilePartial = 2 };
constexpr int kFmMaxTiles = DA_FLASHMASK_MAX_SEQ / kMaskBlock;   // tiles a request may have under FlashMask

__device__ __forceinline__ bool fm_hidden(const int4& iv, int q) {
  return (iv.x <= q && q < iv.y) || (iv.z <= q && q < iv.w);
}
// relation of rows [q, q+1) to one interval family: 0 covers, 1 overlaps, 2 disjoint
__device__ __forceinline__ int fm_family(int q, int s_min, int s_max, int e_min, int e_max) {
  if (q >= s_max && q + 1 <= e_min) return 0;
  if (q + 1 > s_min && q < e_max) return 1;
  return 2;
}
// class of a tile from its block summary (u, l) = (UTS min, max, UTE min, max),
// (LTS ..., LTE ...) for decode row q
__device__ __forceinline__ int fm_class(int q, const int4& u, const int4& l) {
  const int fu = fm_family(q, u.x, u.y, u.z, u.w);
  const int fl = fm_family(q, l.x, l.y, l.z, l.w);
  if (fu == 0 || fl == 0) return kTileSkip;
  if (fu == 2 && fl == 2) return kTileFull;
  return kTilePartial;
}
__device__ __forceinline__ int fm_tile_class(const SplitParams& p, int b, int q, int tile) {
  const int4* sm = p.mask_sum + ((int64_t)b * p.n_mask_blocks + tile / kMaskBlock) * 2;
  return fm_class(q, sm[0], sm[1]);
}

__device__ __forceinline__ int vis_pos(const VisProgram& v, int o) {
  return o < v.ns ? o : o + v.gap;
}

// Every run records in the workspace how its states are laid out, so that
// the combine (which gets no run arguments) folds the right slots: W = 0 for
// the plan's fixed splits, else the partition header [W, L, B, 0, P_0..P_B].
// Written by workgroup 0.
__device__ __forceinline__ void write_partition_header(const SplitParams& p) {
  if (blockIdx.x != 0 || !p.ws_part) return;
  for (int i = threadIdx.x; i < p.batch + 5; i += blockDim.x)
    p.ws_part[i] = (p.partition && i != 3) ? p.partition[i] : 0;
}

// Writes the header when a split kernel returns, on every path.  A store at
// the start of the kernel would keep the compiler from proving the request
// metadata (lengths, work order) unchanged when it is read, so those reads
// could not go through the scalar unit and their waits would also wait for
// every vector load issued before them.
struct PartitionHeaderAtExit {
  const SplitParams& p;
  __device__ ~PartitionHeaderAtExit() { write_partition_header(p); }
};

// Visible length of request b, clamped to the plan's bound so that no load
// can leave the buffers the plan was sized for.
__device__ __forceinline__ int request_len(const SplitParams& p, int b) {
  return min(max(p.seq_lens[b], 0), p.max_seq_len);
}

// Split s of a request with N visible rows owns ordinals [s*chunk, min(.., N)):
// a fixed-width chunk policy ("M4.5 ...", section 0x03B) whose width is a
// multiple of 16 rows; splits past the tail own nothing and write the empty
// identity (section 0x03G).
// Workgroup -> (b, h_kv, s).  Workgroups are dealt to the 8 XCDs round-robin
// by index, so with s = index mod S every split s of every (b, h_kv) would land
// on XCD s mod 8 whenever S is a multiple of 8, and a ragged batch (short
// requests own only their low splits) would load the XCDs unevenly.  Rotating
// the split index by the (b, h_kv) index sends split 0 of consecutive
// (b, h_kv) to different XCDs, which evens the per-XCD rows for any length mix.
// A caller-supplied work order (a permutation of the work items, largest
// first for ragged batches) replaces this mapping.
__device__ __forceinline__ void decode_workgroup(const SplitParams& p, int* b, int* h, int* s) {
  const int wg = blockIdx.x;
  int bh;
  if (p.work_order) {
    int item = __builtin_amdgcn_readfirstlane(p.work_order[wg]);   // one entry per workgroup
    if ((unsigned)item >= gridDim.x) item = wg;   // never index outside the grid's work

    bh = item / p.num_splits;
    *s = item - bh * p.num_splits;
  } else {
    bh = wg / p.num_splits;
    const int r = wg - bh * p.num_splits;
    *s = (int)(((long long)r + bh) % p.num_splits);
  }
  *h = bh % p.num_kv_heads;
  *b = bh / p.num_kv_heads;
}

// First step (of `steps` equal steps) at which the split (b, s) starts its
// sweep, wrapping around to cover every step.  Equal splits of a contiguous
// cache start at byte offsets that differ by multiples of large powers of two
// (the request and split strides), so sweeps that all start at their first
// row request, at any moment, addresses that agree in their low bits; starting
// at staggered eighths of the split ((2b + s) mod 8) spreads the concurrent
// requests over those bits.  Any order visits the same rows, so results
// change only in the order of the fp32 sums.
__device__ __forceinline__ int sweep_start(int b, int s, int steps) {
  return ((2 * b + s) & 7) * (steps >> 3);
}

// A workgroup of K/V head h serves "virtual heads" j = 0 .. C*g-1: query row
// i = j / g of request b, query head h*g + j % g (g = H_q/H_kv).  Its row of
// q, of the split states and of O/LSE, ordered (b, i, h_q):
__device__ __forceinline__ int64_t out_row(const SplitParams& p, int b, int h, int j) {
  const int i = j >> p.q_group_shift;
  const int gi = j - (i << p.q_group_shift);
  return ((int64_t)b * p.num_queries + i) * p.num_q_heads + ((int64_t)h << p.q_group_shift) + gi;
}
// Visible ordinals of virtual head j: query row i sits C-1-i positions before
// the last one and sees keys up to its own (bottom-right causal alignment,
// "M4.5 ...", section 0x08B).  Multi-row calls use the causal mask only, where
// ordinals are positions.
__device__ __forceinline__ int row_limit(const SplitParams& p, int n_vis, int j) {
  return n_vis - (p.num_queries - 1 - (j >> p.q_group_shift));
}

// Tokens of a request of length T held as int8 codes (the oldest n_q); the
// rest are bf16 residual rows t - n_q (DA_RESIDUAL_* in the header).
__device__ __forceinline__ int quantized_len(const SplitParams& p, int T) {
  const int R = p.residual_len;
  if (p.residual_policy == DA_RESIDUAL_GROUPS) {
    const int excess = T - R;
    const int G = 1 << p.k_group_shift;
    return excess > 0 ? ((excess + G - 1) >> p.k_group_shift) << p.k_group_shift : 0;
  }
  return T - min(T, R);
}

// First visible ordinal whose position is >= n_q (positions grow with the
// ordinal, so [o_res, n_vis) are the visible residual rows).
__device__ __forceinline__ int residual_ordinal(const VisProgram& vis, int n_q) {
  return n_q <= vis.ns ? n_q : max(vis.ns, n_q - vis.gap);
}

__device__ __forceinline__ void split_range(int n_vis, int s, int chunk, int* begin, int* end) {
  const long long b = (long long)s * chunk;
  const long long e = b + chunk;
  *begin = (int)min<long long>(b, n_vis);
  *end = (int)min<long long>(e, n_vis);
}

// int8 caches: the residual ordinals [o_res, n_vis) are bf16 K and V rows,
// twice the bytes of an int8 row, so the plan's chunk counts them twice:
// split s owns the ordinals whose weighted offsets (int8 rows 1, residual
// rows 2) fall in [s*chunk, (s+1)*chunk) -- still a disjoint exact cover of
// [0, n_vis), with the residual rows' cost spread over the splits.
__device__ __forceinline__ void split_range_weighted(int n_vis, int o_res, int s, int chunk, int* begin,
                                                     int* end) {
  const long long n_w = (long long)n_vis + (n_vis - o_res);
  auto ord = [&](long long x) { return (int)(x <= o_res ? x : o_res + (x - o_res + 1) / 2); };
  const long long xb = min((long long)s * chunk, n_w);
  const long long xe = min(xb + chunk, n_w);
  *begin = ord(xb);
  *end = ord(xe);
}

// ---------------------------------------------------------------------------
// Address translation ("M4.5 ...", sections 0x04B, 0x04D): element offset of
// the first element of row (b, t, h) in the buffer it lives in.
// ---------------------------------------------------------------------------
// Split into a part that is uniform over a workgroup (RowAddr: the element
// offset of head h's first row, and what the row lookup needs) and a row index
// per token; the element offset of row (b, t, h) is base + row_index *
// row_stride:
//   contiguous NHD  base ((c*T_cap)*H + h)*D,  row t,              stride H*D
//   contiguous HND  base ((c*H + h)*T_cap)*D,  row t,              stride D
//   ring NHD        as contiguous NHD (T_cap = n_sink + W), row t < n_sink ? t : n_sink + t mod W
//   ragged NHD      base ((indptr[b])*H + h)*D, row t,             stride H*D
//   paged NHD       base h*D,                  row pi*P + t%P,     stride H*D
//   paged HND       base h*P*D,                row pi*H*P + t%P,   stride D
// with c = cache_batch_idx[b] (or b) and pi the table's page for block t/P.
// Metadata read from memory is clamped into the buffers it indexes.
struct RowAddr {
  int64_t base;
  int32_t row_cap;    // non-paged: rows addressable from base
  int32_t tbase;      // paged: index of the request's first table entry
};

template <bool PAGED>
__device__ __forceinline__ RowAddr row_addr(const SplitParams& p, int b, int h, int D) {
  RowAddr a;
  const int64_t H = p.num_kv_heads;
  if (PAGED) {
    a.base = p.layout == DA_LAYOUT_PAGED_HND ? (int64_t)h * p.page_size * D : (int64_t)h * D;
    a.tbase = p.page_csr ? min(max(p.indptr[b], 0), p.num_page_entries - 1) : b * p.max_pages;
    a.row_cap = 0;
  } else if (p.layout == DA_LAYOUT_RAGGED_NHD) {
    const int r0 = min(max(p.indptr[b], 0), p.cache_rows - 1);
    a.base = ((int64_t)r0 * H + h) * D;
    a.row_cap = p.cache_rows - r0;
    a.tbase = 0;
  } else {
    const int c = p.cache_batch_idx ? min(max(p.cache_batch_idx[b], 0), p.cache_rows - 1) : b;
    a.base = p.layout == DA_LAYOUT_CONTIG_HND ? (((int64_t)c * H + h) * p.kv_capacity) * D
                                              : (((int64_t)c * p.kv_capacity) * H + h) * D;
    a.row_cap = p.kv_capacity;
    a.tbase = 0;
  }
  return a;
}

template <bool PAGED>
__device__ __forceinline__ uint32_t kv_row_index(const SplitParams& p, const RowAddr& a, int t) {
  if (PAGED) {
    int j, r;
    if (p.page_shift >= 0) {
      j = t >> p.page_shift;
      r = t & (p.page_size - 1);
    } else {
      j = t / p.page_size;
      r = t - j * p.page_size;
    }
    int e = a.tbase + j;
    if (p.page_csr) e = min(e, p.num_page_entries - 1);
    // A visible block must map to a pool page; clamping keeps a corrupt table
    // from addressing memory outside the pool.
    const int page = min(max(p.block_table[e], 0), p.num_pages - 1);
    return (uint32_t)page * p.page_rows + (uint32_t)r;
  }
  if (p.layout == DA_LAYOUT_RING_NHD)   // sinks in their own slots, the rest in a ring of W slots
    return (uint32_t)(t < p.n_sink ? t : p.n_sink + t % p.window);
  return (uint32_t)min(t, a.row_cap - 1);
}

template <bool PAGED>
__device__ __forceinline__ int64_t kv_row_offset(const SplitParams& p, const RowAddr& a, int t) {
  return a.base + (int64_t)((uint64_t)kv_row_index<PAGED>(p, a, t) * p.row_stride);
}

// int8 format: tokens t < n_q come from the code buffers, the newest
// min(T, R) tokens from the bf16 residual, row t - n_q ("M8.6 - Live-Data
// Quantization: Activations and KV Cache", section 0x06B).
__device__ __forceinline__ int64_t resid_row_offset(const SplitParams& p, int b, int tr, int h, int D) {
  return (((int64_t)b * p.residual_len + tr) * p.num_kv_heads + h) * (int64_t)D;
}

// ---------------------------------------------------------------------------
// Index trace ("M4.5 ...", sections 0x04F and 0x04H: the rows a kernel reads
// must be exactly the visible rows, each once, at their translated
// addresses).  A split kernel's trace instance calls these where it issues
// each K and V row load, with the offset that load used; the product
// instances compile them out.  Slots outside the trace buffer are dropped.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t trace_slot(const SplitParams& p, int b, int h, int o) {
  return o >= 0 && o < p.tr.stride ? ((int64_t)b * p.num_kv_heads + h) * p.tr.stride + o : -1;
}
__device__ __forceinline__ void trace_k(const SplitParams& p, int b, int h, int o, int t, int64_t k_off,
                                        int64_t ks_off = -1) {
  const int64_t i = trace_slot(p, b, h, o);
  if (i < 0) return;
  p.tr.k_off[i] = k_off;
  p.tr.pos[i] = t;
  if (ks_off >= 0) p.tr.ks_off[i] = ks_off;
  atomicAdd(p.tr.count + i, 1);
}
__device__ __forceinline__ void trace_v(const SplitParams& p, int b, int h, int o, int64_t v_off,
                                        int64_t vs_off = -1) {
  const int64_t i = trace_slot(p, b, h, o);
  if (i < 0) return;
  p.tr.v_off[i] = v_off;
  if (vs_off >= 0) p.tr.vs_off[i] = vs_off;
  atomicAdd(p.tr.count + i, 1 << 16);
}

// ---------------------------------------------------------------------------
// Cross-lane helpers (64-wide wavefronts)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over groups of LANES adjacent lanes (LANES in {4, 8, 16, 32, 64}); every
// lane of a group receives the group total.  Within a 16-lane DPP row:
// quad_perm [1,0,3,2] and [2,3,0,1] give the quad sum, row_half_mirror pairs
// each quad with the other quad of its half row, row_mirror pairs the two
// halves.  Wider groups use ds_swizzle-free xor shuffles.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES == 4 || LANES == 8 || LANES == 16 || LANES == 32 || LANES == 64, "");
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  if (LANES >= 8) x += dpp_f32<0x141>(x);   // row_half_mirror
  if (LANES >= 16) x += dpp_f32<0x140>(x);  // row_mirror
  if (LANES >= 32) x += __shfl_xor(x, 16);
  if (LANES >= 64) x += __shfl_xor(x, 32);
  return x;
}

// x combined with the lane 16 (32) apart in the same 32 (64) lanes, as
// x + (or max with) __shfl_xor(x, 16 or 32) gives it, without LDS and without
// lane-index registers: v_permlane16_swap / v_permlane32_swap exchange rows
// between two copies of x, so each lane holds its own value and its partner's
// in the two results, whichever copy took which (the sum and the max are
// symmetric in the two).  The second copy is an identity DPP move, which the
// compiler does not see as equal to x, so it does not take the swap of two
// equal operands for two equal results.
__device__ __forceinline__ uint32_t opaque_copy(uint32_t b) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)b, 0xE4, 0xF, 0xF, false);   // quad_perm [0,1,2,3]
}
template <bool MAX, int ROWS>
__device__ __forceinline__ float xor_rows(float x) {
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  uint32_t r0, r1;
  if constexpr (ROWS == 1) {
    const auto r = __builtin_amdgcn_permlane16_swap(b, opaque_copy(b), false, false);
    r0 = r[0];
    r1 = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(b, opaque_copy(b), false, false);
    r0 = r[0];
    r1 = r[1];
  }
  const float a = __builtin_bit_cast(float, r0), c = __builtin_bit_cast(float, r1);
  return MAX ? fmaxf(a, c) : a + c;
}
__device__ __forceinline__ float xor16_sum(float x) { return xor_rows<false, 1>(x); }
__device__ __forceinline__ float xor32_sum(float x) { return xor_rows<false, 2>(x); }
__device__ __forceinline__ float xor16_max(float x) { return xor_rows<true, 1>(x); }
__device__ __forceinline__ float xor32_max(float x) { return xor_rows<true, 2>(x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float i8_at(uint32_t w, int byte) {
  return (float)(int32_t)((int32_t)(w << (24 - 8 * byte)) >> 24);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
}

}  // namespace da
