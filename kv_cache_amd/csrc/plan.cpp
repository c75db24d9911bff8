// decode_attn_plan: validation, admission reasons, split choice, workspace
// sizing and the frozen plan key.  Host code only.
//
// Follows "M4.5 - Decode Attention Kernels, Mask Programs, and Backend
// Boundaries": semantic checks before capability checks (section 0x07A),
// admission as a conjunction whose failures are all reported (0x07B), a plan
// whose static projection is frozen and re-checked at run (0x07F), split count
// as a tuning decision that trades producer parallelism against workspace
// round trip and reducer fan-in (0x03I, 0x03F).
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <vector>
#include <algorithm>

#include "plan_internal.hpp"

namespace da {

bool current_device_info(int* device, int* num_cus, bool* is_gfx950) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
  if (device) *device = dev;
  if (num_cus) *num_cus = prop.multiProcessorCount;
  if (is_gfx950) *is_gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  return true;
}

bool current_device_is_gfx950() {
  static std::atomic<int8_t> cache[64];   // 0 unknown, 1 gfx950, 2 other
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (dev >= 0 && dev < 64) {
    int8_t c = cache[dev].load(std::memory_order_relaxed);
    if (c) return c == 1;
  }
  bool ok = false;
  if (!current_device_info(nullptr, nullptr, &ok)) return false;
  if (dev >= 0 && dev < 64) cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok;
}

}  // namespace da

namespace {

// Automatic split choice.  A K/V head of one request is an independent
// stream of rows, and the plan knows only the longest request.
//  * When B*H_kv is below the CU count, the rows are cut into splits until
//    about one workgroup per CU exists (kWgPerCu): the split kernels run 4
//    waves per workgroup with two tiles in flight per wave, which keeps
//    enough bytes in flight per CU, and every extra split adds one (m, l, u)
//    state per query head to the workspace round trip and to the reducer's
//    fan-in (measured on the 8 x 4096 GQA shape: 4 splits 27.0 us per
//    single-launch call, 12 splits 28.0 us; int8 sink+window shape: 2 splits
//    31.4 us, 6 splits 32.7 us; 128k context: 32 splits 88.9 us, 128 splits
//    90.9 us).  Splits are at most kMaxChunk rows long.
//  * When B*H_kv alone fills the CUs, splits only balance ragged lengths:
//    about kBalanceWgPerCu workgroups per CU and never more than
//    kBalanceChunk rows, so that the hardware dispatcher can even out the
//    work (splits past a short request's end exit at once; measured on the
//    32-request ragged paged batch: 1024-row splits 383 us, 4096-row splits
//    456 us per call).
// Splits are never shorter than kMinChunk rows.
constexpr int kWgPerCu = 1;
constexpr int kMaxChunk = 4096;
constexpr int kBalanceWgPerCu = 3;
constexpr int kBalanceChunk = 1024;
constexpr int kMinChunk = 256;
constexpr int kRowAlign = 16;
constexpr int kStepRows = 64;
// Workgroups per CU a balanced partition targets by default: one round of the
// partitioned split kernel (its launch bound allows this many per CU).
constexpr int kPartitionWgPerCu = 3;
constexpr int kI8PartitionWgPerCu = 2;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
// ceil(a / b) for b > 0 and any sign of a
int64_t ceil_div_i64(int64_t a, int64_t b) { return a >= 0 ? (a + b - 1) / b : -((-a) / b); }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

}  // namespace

extern "C" da_status decode_attn_plan(const da_problem* problem, da_plan* plan_out,
                                      uint64_t* workspace_bytes, uint64_t* reasons_out) {
  uint64_t reasons = 0;
  if (reasons_out) *reasons_out = 0;
  if (!problem) return DA_ERR_INVALID;
  da_problem p = *problem;

  // ---- semantic checks: malformed calls are not "unsupported" -------------
  if (p.batch < 0 || p.num_q_heads < 1 || p.num_kv_heads < 1) return DA_ERR_INVALID;
  if (p.num_q_heads % p.num_kv_heads != 0) return DA_ERR_INVALID;
  if (p.head_dim_qk < 1 || p.head_dim_v < 1) return DA_ERR_INVALID;
  if (p.max_seq_len < 0 || p.num_splits < 0 || p.num_cus < 0) return DA_ERR_INVALID;
  if (!std::isfinite(p.softmax_scale) || p.softmax_scale < 0.f) return DA_ERR_INVALID;
  if (p.reserved1 != 0) return DA_ERR_INVALID;
  const bool paged = p.layout == DA_LAYOUT_PAGED_NHD || p.layout == DA_LAYOUT_PAGED_HND;
  const bool contig = p.layout == DA_LAYOUT_CONTIG_NHD || p.layout == DA_LAYOUT_CONTIG_HND ||
                      p.layout == DA_LAYOUT_RING_NHD;
  if (p.layout == DA_LAYOUT_RING_NHD &&
      (p.mask_kind != DA_MASK_SINK_WINDOW || (int64_t)p.kv_capacity != (int64_t)p.n_sink + p.window))
    return DA_ERR_INVALID;
  if (paged) {
    if (p.page_size <= 0 || p.num_pages < 1) return DA_ERR_INVALID;
    if (p.kv_capacity != 0 || p.cache_rows != 0) return DA_ERR_INVALID;
    if (p.page_table == DA_PAGE_TABLE_DENSE) {
      if (p.max_pages_per_seq < 1 || p.num_page_entries != 0) return DA_ERR_INVALID;
      if (ceil_div(p.max_seq_len, p.page_size) > p.max_pages_per_seq) return DA_ERR_INVALID;
    } else if (p.page_table == DA_PAGE_TABLE_CSR) {
      if (p.max_pages_per_seq != 0 || p.num_page_entries < 1) return DA_ERR_INVALID;
    } else {
      return DA_ERR_INVALID;
    }
  } else if (contig) {
    if (p.page_size != 0 || p.max_pages_per_seq != 0 || p.num_pages != 0) return DA_ERR_INVALID;
    if (p.kv_capacity < 0 || p.cache_rows < 0 || p.page_table != 0 || p.num_page_entries != 0)
      return DA_ERR_INVALID;
  } else if (p.layout == DA_LAYOUT_RAGGED_NHD) {
    if (p.page_size != 0 || p.max_pages_per_seq != 0 || p.num_pages != 0 || p.kv_capacity != 0 ||
        p.page_table != 0 || p.num_page_entries != 0)
      return DA_ERR_INVALID;
    if (p.cache_rows < 1 && p.batch > 0 && p.max_seq_len > 0) return DA_ERR_INVALID;
  }
  if (p.mask_kind == DA_MASK_SINK_WINDOW) {
    if (p.window <= 0 || p.n_sink < 0) return DA_ERR_INVALID;
  } else if (p.mask_kind == DA_MASK_CAUSAL || p.mask_kind == DA_MASK_FLASHMASK) {
    if (p.window != 0 || p.n_sink != 0) return DA_ERR_INVALID;
  }
  if (p.num_queries < 0) return DA_ERR_INVALID;
  if (p.num_queries == 0) p.num_queries = 1;
  if (p.kv_format == DA_KV_I8) {
    if (p.k_group <= 0 || p.residual_len < 0) return DA_ERR_INVALID;
    if (p.residual_policy != DA_RESIDUAL_WINDOW && p.residual_policy != DA_RESIDUAL_GROUPS)
      return DA_ERR_INVALID;
    // closing G rows must leave a row in the residual
    if (p.residual_policy == DA_RESIDUAL_GROUPS && p.k_group > p.residual_len) return DA_ERR_INVALID;
    if (p.layout == DA_LAYOUT_CONTIG_NHD) {
      // n_q grows with T, so its largest value is at T = max_seq_len
      const int64_t excess = (int64_t)p.max_seq_len - p.residual_len;
      const int64_t nq_max = p.residual_policy == DA_RESIDUAL_GROUPS
                                 ? p.k_group * std::max<int64_t>(0, ceil_div_i64(excess, p.k_group))
                                 : std::max<int64_t>(0, excess);
      if (p.kv_capacity < nq_max) return DA_ERR_INVALID;
    }
  } else {
    if (p.k_group != 0 || p.residual_len != 0 || p.residual_policy != 0) return DA_ERR_INVALID;
    if (contig && p.layout != DA_LAYOUT_RING_NHD && p.kv_capacity < p.max_seq_len) return DA_ERR_INVALID;
  }

  // ---- capability predicates: collect every failure ------------------------
  const int g = p.num_q_heads / p.num_kv_heads;
  if (p.head_dim_qk != 64 && p.head_dim_qk != 128) reasons |= DA_R_HEAD_DIM;
  if (p.head_dim_v != p.head_dim_qk) reasons |= DA_R_HEAD_DIM_V;
  if (g != 1 && g != 2 && g != 4 && g != 8) reasons |= DA_R_GQA_GROUP;
  {
    const int64_t gc = (int64_t)g * p.num_queries;
    if ((gc != 1 && gc != 2 && gc != 4 && gc != 8) ||
        (p.num_queries > 1 && p.mask_kind != DA_MASK_CAUSAL))
      reasons |= DA_R_QUERY_ROWS;
  }
  const bool fmt_ok = p.kv_format == DA_KV_F32 || p.kv_format == DA_KV_BF16 || p.kv_format == DA_KV_I8;
  if (!fmt_ok) reasons |= DA_R_KV_FORMAT;
  if (fmt_ok) {
    const bool q_ok = (p.kv_format == DA_KV_F32) ? p.q_dtype == DA_F32 : p.q_dtype == DA_BF16;
    if (!q_ok) reasons |= DA_R_Q_DTYPE;
  }
  if (p.out_dtype != DA_F32) reasons |= DA_R_OUT_DTYPE;
  if (!paged && !contig && p.layout != DA_LAYOUT_RAGGED_NHD) reasons |= DA_R_LAYOUT;
  if (p.kv_format == DA_KV_I8 && (p.layout != DA_LAYOUT_CONTIG_NHD || p.cache_rows != 0))
    reasons |= DA_R_LAYOUT;
  if (p.kv_format == DA_KV_I8 &&
      !(p.k_group >= 16 && p.k_group <= 1024 && (p.k_group & (p.k_group - 1)) == 0))
    reasons |= DA_R_INT8_PARAMS;
  // the int8 kernel forms row offsets inside a phase as 24-bit products
  // r * (num_kv_heads * head_dim) with r < 2048, kept below 2^31
  if (p.kv_format == DA_KV_I8 && (int64_t)p.num_kv_heads * p.head_dim_qk > (1 << 20))
    reasons |= DA_R_INDEX_RANGE;
  if (p.mask_kind != DA_MASK_CAUSAL && p.mask_kind != DA_MASK_SINK_WINDOW &&
      p.mask_kind != DA_MASK_FLASHMASK)
    reasons |= DA_R_MASK_KIND;
  if (p.mask_kind == DA_MASK_FLASHMASK &&
      (p.kv_format != DA_KV_BF16 || p.head_dim_qk != 128 || p.num_queries != 1 ||
       p.max_seq_len > DA_FLASHMASK_MAX_SEQ))
    reasons |= DA_R_MASK_KIND;
  if (p.num_splits > DA_MAX_SPLITS) reasons |= DA_R_SPLITS;

  int num_cus = p.num_cus;
  if (num_cus == 0) {
    int dev = 0, cus = 0;
    bool gfx950 = false;
    if (!da::current_device_info(&dev, &cus, &gfx950) || !gfx950 || cus <= 0) {
      reasons |= DA_R_DEVICE;
      cus = 256;
    }
    num_cus = cus;
  }

  // ---- split plan ----------------------------------------------------------
  int64_t max_vis = p.max_seq_len;
  if (p.mask_kind == DA_MASK_SINK_WINDOW)
    max_vis = std::min<int64_t>(max_vis, (int64_t)p.n_sink + (int64_t)p.window);
  // Splits cut the visible ordinals into chunks of equal length (for int8
  // caches by weight, a residual row (bf16 K and V) counting as two int8
  // rows).  Tiles start at the split, so chunks need no tile alignment, except
  // under FlashMask, whose tiles are the 16-key blocks of the summaries.
  const bool i8 = p.kv_format == DA_KV_I8;
  const int64_t split_len = max_vis + (i8 ? std::min<int64_t>(std::max(p.residual_len, 0), max_vis) : 0);
  const int64_t align = p.mask_kind == DA_MASK_FLASHMASK ? kRowAlign : 1;
  int64_t chunk;
  if (max_vis == 0) {
    chunk = kRowAlign;
  } else if (p.num_splits > 0) {
    chunk = round_up(ceil_div(split_len, p.num_splits), align);
  } else {
    const int64_t units = std::max<int64_t>(1, (int64_t)p.batch * p.num_kv_heads);
    const bool fills = units >= num_cus;
    const int64_t s0 = std::max<int64_t>(1, ceil_div((int64_t)(fills ? kBalanceWgPerCu : kWgPerCu) * num_cus, units));
    chunk = round_up(ceil_div(split_len, s0), align);
    chunk = std::min<int64_t>(chunk, fills ? kBalanceChunk : kMaxChunk);
    // FlashMask splits hold at most 64 tiles of 16 keys
    if (p.mask_kind == DA_MASK_FLASHMASK) chunk = std::min<int64_t>(chunk, 64 * kRowAlign);
    chunk = std::max<int64_t>(chunk, std::min<int64_t>(kMinChunk, round_up(split_len, align)));
    // bf16 and fp32 splits of whole steps (the split kernels' 4 waves x 16-row
    // tiles) where that keeps the split count: a split ending inside a step
    // leaves some waves a tile without rows
    if (!i8 && p.mask_kind != DA_MASK_FLASHMASK) {
      const int64_t whole = round_up(chunk, kStepRows);
      if (ceil_div(split_len, whole) == ceil_div(split_len, chunk)) chunk = whole;
    }
  }
  int64_t S = max_vis == 0 ? 1 : ceil_div(split_len, chunk);
  if (S > DA_MAX_SPLITS) reasons |= DA_R_SPLITS;
  // FlashMask classifies at most 64 tiles of 16 keys per split
  if (p.mask_kind == DA_MASK_FLASHMASK && chunk > 64 * 16) reasons |= DA_R_MASK_KIND;

  const int64_t grid = (int64_t)p.batch * p.num_kv_heads * S;
  if (grid > 0x7fffffffLL) reasons |= DA_R_INDEX_RANGE;
  if ((int64_t)p.batch * p.num_kv_heads * S * chunk > (1LL << 40)) reasons |= DA_R_INDEX_RANGE;

  if (reasons_out) *reasons_out = reasons;
  if (reasons) return DA_ERR_UNSUPPORTED;

  if (p.softmax_scale == 0.f) p.softmax_scale = 1.0f / std::sqrt((float)p.head_dim_qk);
  const uint64_t ws = da::workspace_bytes_for((int64_t)p.batch * p.num_queries * p.num_q_heads,
                                              (int64_t)p.batch * p.num_kv_heads, p.batch, S, p.head_dim_v);

  da_plan plan;
  std::memset(&plan, 0, sizeof(plan));
  plan.problem = p;
  plan.num_splits = (int32_t)S;
  plan.chunk = (int32_t)chunk;
  plan.max_visible = (int32_t)max_vis;
  plan.num_cus = num_cus;
  plan.workspace_bytes = ws;
  plan.key = da::plan_hash(plan);
  if (plan_out) *plan_out = plan;
  if (workspace_bytes) *workspace_bytes = ws;
  return DA_OK;
}

extern "C" const char* decode_attn_reason(int bit) {
  static const char* const text[DA_NUM_REASONS] = {
      "head_dim_qk must be 64 or 128",
      "head_dim_v must equal head_dim_qk",
      "query heads per K/V head must be 1, 2, 4 or 8",
      "q dtype must be f32 with f32 K/V and bf16 with bf16 or int8 K/V",
      "output dtype must be f32",
      "unknown K/V storage format",
      "layout not available for this K/V format (int8 is contiguous NHD without a batch index)",
      "int8 k_group must be a power of two in [16, 1024]",
      "split count above the library maximum",
      "grid or trace size exceeds the index range, or int8 with num_kv_heads * head_dim > 2^20",
      "current device is not gfx950 or cannot be queried",
      "mask program unknown, or FlashMask outside bf16 / head_dim 128 / one query row / "
      "splits of at most 1024 keys",
      "(H_q/H_kv) * num_queries must be 1, 2, 4 or 8, and num_queries > 1 needs the causal mask",
  };
  if (bit < 0 || bit >= DA_NUM_REASONS) return "unknown reason bit";
  return text[bit];
}

extern "C" const char* decode_attn_status_string(da_status s) {
  switch (s) {
    case DA_OK: return "ok";
    case DA_ERR_INVALID: return "invalid call";
    case DA_ERR_UNSUPPORTED: return "unsupported (see reason bits)";
    case DA_ERR_WORKSPACE: return "workspace missing or too small";
    case DA_ERR_PLAN_MISMATCH: return "plan changed after planning";
    case DA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

extern "C" da_status decode_attn_schedule(const da_plan* plan, const int32_t* seq_lens_host,
                                          int32_t* order, uint64_t order_len) {
  if (!plan || !seq_lens_host || !order) return DA_ERR_INVALID;
  if (!da::plan_intact(plan)) return DA_ERR_PLAN_MISMATCH;
  const da_problem& p = plan->problem;
  const int64_t S = plan->num_splits, H = p.num_kv_heads, B = p.batch, chunk = plan->chunk;
  if (order_len < (uint64_t)(B * H * S)) return DA_ERR_INVALID;
  std::vector<int64_t> full(B), part(B);
  for (int64_t b = 0; b < B; ++b) {
    const int64_t T = seq_lens_host[b];
    if (T < 0 || T > p.max_seq_len) return DA_ERR_INVALID;
    int64_t n_vis = T, ns = T, gap = 0;
    if (p.mask_kind == DA_MASK_SINK_WINDOW) {
      ns = std::min<int64_t>(p.n_sink, T);
      gap = std::max<int64_t>(0, std::max<int64_t>(0, T - p.window) - ns);
      n_vis = T - gap;
    }
    int64_t len = n_vis;   // split length: int8 residual rows count twice
    if (p.kv_format == DA_KV_I8) {
      int64_t n_q = T - std::min<int64_t>(T, p.residual_len);
      if (p.residual_policy == DA_RESIDUAL_GROUPS)
        n_q = T > p.residual_len ? ceil_div(T - p.residual_len, p.k_group) * p.k_group : 0;
      const int64_t o_res = n_q <= ns ? n_q : std::max<int64_t>(ns, n_q - gap);
      len += n_vis - o_res;
    }
    full[b] = std::min<int64_t>(S, len / chunk);
    part[b] = full[b] < S ? len - full[b] * chunk : 0;   // length of split full[b] (0: empty)
  }
  int64_t pos = 0;
  auto put = [&](int64_t b, int64_t h, int64_t s) { order[pos++] = (int32_t)((b * H + h) * S + s); };
  // full splits: split-major, then request, then head
  for (int64_t s = 0; s < S; ++s)
    for (int64_t b = 0; b < B; ++b)
      if (s < full[b])
        for (int64_t h = 0; h < H; ++h) put(b, h, s);
  // partial last splits, largest first (ties by request index)
  std::vector<int64_t> idx;
  for (int64_t b = 0; b < B; ++b)
    if (part[b] > 0) idx.push_back(b);
  std::stable_sort(idx.begin(), idx.end(), [&](int64_t x, int64_t y) { return part[x] > part[y]; });
  for (int64_t b : idx)
    for (int64_t h = 0; h < H; ++h) put(b, h, full[b]);
  // empty splits
  for (int64_t s = 0; s < S; ++s)
    for (int64_t b = 0; b < B; ++b)
      if (s > full[b] || (s == full[b] && part[b] == 0))
        for (int64_t h = 0; h < H; ++h) put(b, h, s);
  return DA_OK;
}

// Balanced partition of a ragged batch: equal runs of L visible ordinals over
// the requests concatenated in order ("M4.5 ...", sections 0x09E and 0x09G).
extern "C" da_status decode_attn_partition(const da_plan* plan, const int32_t* seq_lens_host,
                                           int32_t items_per_head, int32_t* part, uint64_t part_len,
                                           int32_t* items_out) {
  if (!plan || !seq_lens_host || !part || !items_out) return DA_ERR_INVALID;
  if (!da::plan_intact(plan)) return DA_ERR_PLAN_MISMATCH;
  const da_problem& p = plan->problem;
  const int64_t B = p.batch, H = p.num_kv_heads, S = plan->num_splits;
  if (items_per_head < 0) return DA_ERR_INVALID;
  int64_t target = items_per_head;
  // default: one dispatch round of the partition instance (bf16: 3 workgroups
  // per CU; int8: 2, the register budget of its partition instance)
  const int64_t per_cu = p.kv_format == DA_KV_I8 ? kI8PartitionWgPerCu : kPartitionWgPerCu;
  if (target == 0) target = std::max<int64_t>(1, (per_cu * (int64_t)plan->num_cus) / std::max<int64_t>(H, 1));
  if (part_len < (uint64_t)(5 + B + target)) return DA_ERR_INVALID;
  if (S < 2) return DA_ERR_UNSUPPORTED;
  std::vector<int64_t> n(B);
  int64_t N = 0, nmax = 0;
  for (int64_t b = 0; b < B; ++b) {
    const int64_t T = seq_lens_host[b];
    if (T < 0 || T > p.max_seq_len) return DA_ERR_INVALID;
    int64_t v = T;
    if (p.mask_kind == DA_MASK_SINK_WINDOW) v = std::min<int64_t>(T, (int64_t)p.n_sink + (int64_t)p.window);
    n[b] = v;
    N += v;
    nmax = std::max(nmax, v);
  }
  if (N >= (1LL << 31)) return DA_ERR_INVALID;
  // L: equal work per item, and long enough that no request has more than S
  // pieces (a request of n rows spans at most ceil(n / L) + 1 items).
  int64_t L = std::max<int64_t>(ceil_div(std::max<int64_t>(N, 1), target), ceil_div(nmax, S - 1));
  L = std::max<int64_t>(round_up(L, kRowAlign), kRowAlign);
  const int64_t W = N == 0 ? 0 : ceil_div(N, L);
  part[0] = (int32_t)W;
  part[1] = (int32_t)L;
  part[2] = (int32_t)B;
  part[3] = 0;
  int64_t P = 0;
  for (int64_t b = 0; b < B; ++b) {
    part[4 + b] = (int32_t)P;
    P += n[b];
  }
  part[4 + B] = (int32_t)P;
  // first request of each item: the request holding ordinal i*L (empty
  // requests are skipped: P_b == P_{b+1})
  int64_t b = 0;
  for (int64_t i = 0; i < W; ++i) {
    const int64_t x = i * L;
    while (b + 1 <= B && (int64_t)part[4 + b + 1] <= x) ++b;
    part[5 + B + i] = (int32_t)b;
  }
  *items_out = (int32_t)W;
  return DA_OK;
}
