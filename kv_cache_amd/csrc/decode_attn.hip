// C-ABI launch entry points: decode_attn_run, decode_attn_combine,
// decode_attn_forward and its allocation-free form, decode_attn_append,
// decode_attn_trace_indices.  Argument and plan checks happen on the host
// before any launch; the launches are asynchronous on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "combine_kernel.hpp"
#include "append_kernel.hpp"
#include "device_common.hpp"
#include "plan_internal.hpp"
#include "split_kernel.hpp"
#include "split_kernel_mfma.hpp"
#include "split_kernel_mfma_i8.hpp"

namespace {

// Launch shape of the split kernel: waves per workgroup and rows per row slot
// per tile (see split_kernel.hpp).
#ifndef DA_WAVES
#define DA_WAVES 4
#endif
#ifndef DA_UNROLL
#define DA_UNROLL 4
#endif
#ifndef DA_UNROLL_I8
#define DA_UNROLL_I8 2
#endif
// bf16 and int8 K/V with D = 128 take the matrix-core score kernels.
#ifndef DA_MFMA_QK
#define DA_MFMA_QK 1
#endif
constexpr int kWaves = DA_WAVES;

template <int FMT> struct Unroll { static constexpr int value = DA_UNROLL; };
template <> struct Unroll<DA_KV_I8> { static constexpr int value = DA_UNROLL_I8; };

template <int FMT, int D>
constexpr bool use_mfma() { return DA_MFMA_QK && (FMT == DA_KV_BF16 || FMT == DA_KV_I8) && D == 128; }

int log2_exact(int x) {
  if (x <= 0 || (x & (x - 1))) return -1;
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

da_status check_args(const da_plan* plan, const da_args* a) {
  if (!plan || !a) return DA_ERR_INVALID;
  if (!da::plan_intact(plan)) return DA_ERR_PLAN_MISMATCH;
  const da_problem& p = plan->problem;
  if (p.batch == 0) return DA_OK;
  if (!a->q || !a->k || !a->v || !a->seq_lens) return DA_ERR_INVALID;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v)) return DA_ERR_INVALID;
  const bool paged = p.layout == DA_LAYOUT_PAGED_NHD || p.layout == DA_LAYOUT_PAGED_HND;
  if (paged && !a->block_table) return DA_ERR_INVALID;
  if (p.mask_kind == DA_MASK_FLASHMASK) {
    if (!a->mask_intervals || !a->mask_summary) return DA_ERR_INVALID;
    if ((reinterpret_cast<uintptr_t>(a->mask_intervals) & 15u) != 0 ||
        (reinterpret_cast<uintptr_t>(a->mask_summary) & 15u) != 0)
      return DA_ERR_INVALID;
  }
  if (((paged && p.page_table == DA_PAGE_TABLE_CSR) || p.layout == DA_LAYOUT_RAGGED_NHD) && !a->indptr)
    return DA_ERR_INVALID;
  if (p.cache_rows > 0 &&
      (p.layout == DA_LAYOUT_CONTIG_NHD || p.layout == DA_LAYOUT_CONTIG_HND || p.layout == DA_LAYOUT_RING_NHD) &&
      !a->cache_batch_idx)
    return DA_ERR_INVALID;
  if (a->partition) {
    if (a->partition_items < 0) return DA_ERR_INVALID;
    // balanced partitions run on the bf16 and int8 D = 128 matrix-core kernels, without FlashMask
    if ((p.kv_format != DA_KV_BF16 && p.kv_format != DA_KV_I8) || p.head_dim_qk != 128 ||
        p.mask_kind == DA_MASK_FLASHMASK || plan->num_splits < 2 || !DA_MFMA_QK)
      return DA_ERR_UNSUPPORTED;
  } else if (a->partition_items != 0) {
    return DA_ERR_INVALID;
  }
  if (p.kv_format == DA_KV_I8) {
    if (!a->k_scale || !a->v_scale) return DA_ERR_INVALID;
    if (p.residual_len > 0 && (!a->k_resid || !a->v_resid)) return DA_ERR_INVALID;
    if ((a->k_resid && !aligned16(a->k_resid)) || (a->v_resid && !aligned16(a->v_resid)))
      return DA_ERR_INVALID;
    if ((reinterpret_cast<uintptr_t>(a->k_scale) & 15u) != 0 || (reinterpret_cast<uintptr_t>(a->v_scale) & 1u) != 0)
      return DA_ERR_INVALID;
  }
  return DA_OK;
}

da::SplitParams make_params(const da_plan* plan, const da_args* a) {
  const da_problem& p = plan->problem;
  da::SplitParams sp;
  sp.q = a->q;
  sp.k = a->k;
  sp.v = a->v;
  sp.k_scale = static_cast<const uint16_t*>(a->k_scale);
  sp.v_scale = static_cast<const uint16_t*>(a->v_scale);
  sp.k_resid = a->k_resid;
  sp.v_resid = a->v_resid;
  sp.block_table = a->block_table;
  sp.seq_lens = a->seq_lens;
  sp.work_order = a->work_order;
  sp.indptr = a->indptr;
  const bool contig = p.layout == DA_LAYOUT_CONTIG_NHD || p.layout == DA_LAYOUT_CONTIG_HND ||
                      p.layout == DA_LAYOUT_RING_NHD;
  sp.cache_batch_idx = contig && p.cache_rows > 0 ? a->cache_batch_idx : nullptr;
  sp.layout = p.layout;
  sp.page_csr = p.page_table == DA_PAGE_TABLE_CSR;
  sp.cache_rows = p.cache_rows;
  sp.num_page_entries = p.num_page_entries;
  const bool hnd = p.layout == DA_LAYOUT_CONTIG_HND || p.layout == DA_LAYOUT_PAGED_HND;
  sp.row_stride = (uint32_t)(hnd ? p.head_dim_qk : p.num_kv_heads * p.head_dim_qk);
  sp.page_rows = (uint32_t)(p.layout == DA_LAYOUT_PAGED_HND ? p.num_kv_heads * p.page_size : p.page_size);
  const bool fm = p.mask_kind == DA_MASK_FLASHMASK;
  sp.mask_iv = fm ? reinterpret_cast<const int4*>(a->mask_intervals) : nullptr;
  sp.mask_sum = fm ? reinterpret_cast<const int4*>(a->mask_summary) : nullptr;
  sp.n_mask_blocks = (p.max_seq_len + da::kMaskBlock - 1) / da::kMaskBlock;
  const uint64_t n_states = (uint64_t)da::output_rows(p) * plan->num_splits;
  float* ws = static_cast<float*>(a->workspace);
  sp.ws_u = ws;
  sp.ws_m = ws ? ws + n_states * p.head_dim_v : nullptr;
  sp.ws_l = ws ? sp.ws_m + n_states : nullptr;
  sp.counters = ws ? reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws) + da::states_bytes(*plan))
                   : nullptr;
  sp.out = nullptr;
  sp.lse = nullptr;
  sp.tr = da::TraceOut{};
  sp.stamps = nullptr;
  sp.num_q_heads = p.num_q_heads;
  sp.num_kv_heads = p.num_kv_heads;
  sp.batch = p.batch;
  sp.partition = a->partition;
  sp.ws_part = ws ? reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + da::partition_header_offset(*plan))
                  : nullptr;
  sp.num_queries = p.num_queries;
  sp.q_group_shift = log2_exact(p.num_q_heads / p.num_kv_heads);
  sp.num_splits = plan->num_splits;
  sp.chunk = plan->chunk;
  sp.kv_capacity = p.kv_capacity;
  sp.page_size = p.page_size;
  sp.page_shift = log2_exact(p.page_size);
  sp.max_pages = p.max_pages_per_seq;
  sp.mask_kind = p.mask_kind;
  sp.n_sink = p.n_sink;
  sp.window = p.window;
  sp.k_group_shift = p.kv_format == DA_KV_I8 ? log2_exact(p.k_group) : 0;
  sp.residual_len = p.residual_len;
  sp.residual_policy = p.residual_policy;
  sp.max_seq_len = p.max_seq_len;
  sp.num_pages = p.num_pages;
  sp.qscale = p.softmax_scale * 1.4426950408889634f;
  sp.num_cus = plan->num_cus;
  return sp;
}

// INSTR selects an instrumentation instance of the same kernel (debug entry
// points only): da::kInstrRows the index trace, da::kInstrStamps per-workgroup
// timestamps (matrix-core kernels without a partition or FlashMask only).
// Returns false when no such instance exists.
template <int FMT, int D, int G, bool PAGED, bool FUSED, bool FM, int INSTR>
bool launch_split(const da::SplitParams& sp, unsigned grid, hipStream_t st) {
  constexpr bool kStamps = INSTR == da::kInstrStamps;
  if constexpr (use_mfma<FMT, D>() && FMT == DA_KV_I8) {
    static_assert(!FM, "FlashMask runs on the bf16 matrix-core kernel only");
    if constexpr (!FUSED && !kStamps) {
      if (sp.partition) {
        hipLaunchKernelGGL((da::split_kernel_mfma_i8<G, kWaves, false, INSTR, true>), dim3(grid),
                           dim3(kWaves * 64), 0, st, sp);
        return true;
      }
    }
    if (kStamps && sp.partition) return false;
    // At most 2 workgroups per CU: the instance with the larger register
    // budget (it folds the sinks into the first window phase).
    if constexpr (G <= 4) {
      if ((uint64_t)grid <= 2ull * (uint64_t)std::max(sp.num_cus, 1)) {
        hipLaunchKernelGGL((da::split_kernel_mfma_i8<G, kWaves, FUSED, INSTR, false, true>), dim3(grid),
                           dim3(kWaves * 64), 0, st, sp);
        return true;
      }
    }
    hipLaunchKernelGGL((da::split_kernel_mfma_i8<G, kWaves, FUSED, INSTR>), dim3(grid), dim3(kWaves * 64), 0,
                       st, sp);
    return true;
  } else if constexpr (use_mfma<FMT, D>()) {
    if constexpr (!FUSED && !FM && !kStamps) {
      if (sp.partition) {
        hipLaunchKernelGGL((da::split_kernel_mfma<G, PAGED, kWaves, false, false, true, INSTR>), dim3(grid),
                           dim3(kWaves * 64), 0, st, sp);
        return true;
      }
    }
    if constexpr (kStamps && FM) {
      return false;
    } else {
      if (kStamps && sp.partition) return false;
      hipLaunchKernelGGL((da::split_kernel_mfma<G, PAGED, kWaves, FUSED, FM, false, INSTR>), dim3(grid),
                         dim3(kWaves * 64), 0, st, sp);
      return true;
    }
  } else {
    if constexpr (kStamps || FM) {   // FlashMask runs on the bf16 matrix-core kernel only
      return false;
    } else {
      hipLaunchKernelGGL((da::split_kernel<FMT, D, G, PAGED, kWaves, Unroll<FMT>::value, FUSED, INSTR>),
                         dim3(grid), dim3(kWaves * 64), 0, st, sp);
      return true;
    }
  }
}

template <int FMT, int D, bool PAGED, bool FUSED, bool FM, int INSTR>
bool dispatch_g(int g, const da::SplitParams& sp, unsigned grid, hipStream_t st) {
  switch (g) {
    case 1: return launch_split<FMT, D, 1, PAGED, FUSED, FM, INSTR>(sp, grid, st);
    case 2: return launch_split<FMT, D, 2, PAGED, FUSED, FM, INSTR>(sp, grid, st);
    case 4: return launch_split<FMT, D, 4, PAGED, FUSED, FM, INSTR>(sp, grid, st);
    case 8: return launch_split<FMT, D, 8, PAGED, FUSED, FM, INSTR>(sp, grid, st);
    default: return false;
  }
}

template <int FMT, bool PAGED, bool FUSED, bool FM, int INSTR>
bool dispatch_d(int d, int g, const da::SplitParams& sp, unsigned grid, hipStream_t st) {
  if constexpr (FM) {
    return d == 128 && dispatch_g<FMT, 128, PAGED, FUSED, true, INSTR>(g, sp, grid, st);
  } else {
    if (d == 64) return dispatch_g<FMT, 64, PAGED, FUSED, false, INSTR>(g, sp, grid, st);
    if (d == 128) return dispatch_g<FMT, 128, PAGED, FUSED, false, INSTR>(g, sp, grid, st);
    return false;
  }
}

template <bool FUSED, int INSTR = da::kInstrNone>
bool dispatch_split(const da_problem& p, const da::SplitParams& sp, unsigned grid, hipStream_t st) {
  // A workgroup serves the C query rows of each of its H_q/H_kv heads: C*g
  // "virtual heads" sharing one K/V head.
  const int g = p.num_q_heads / p.num_kv_heads * p.num_queries;
  const bool paged = p.layout == DA_LAYOUT_PAGED_NHD || p.layout == DA_LAYOUT_PAGED_HND;
  switch (p.kv_format) {
    case DA_KV_F32:
      if (p.mask_kind == DA_MASK_FLASHMASK) return false;
      return paged ? dispatch_d<DA_KV_F32, true, FUSED, false, INSTR>(p.head_dim_qk, g, sp, grid, st)
                   : dispatch_d<DA_KV_F32, false, FUSED, false, INSTR>(p.head_dim_qk, g, sp, grid, st);
    case DA_KV_BF16:
      if (p.mask_kind == DA_MASK_FLASHMASK)
        return paged ? dispatch_d<DA_KV_BF16, true, FUSED, true, INSTR>(p.head_dim_qk, g, sp, grid, st)
                     : dispatch_d<DA_KV_BF16, false, FUSED, true, INSTR>(p.head_dim_qk, g, sp, grid, st);
      return paged ? dispatch_d<DA_KV_BF16, true, FUSED, false, INSTR>(p.head_dim_qk, g, sp, grid, st)
                   : dispatch_d<DA_KV_BF16, false, FUSED, false, INSTR>(p.head_dim_qk, g, sp, grid, st);
    case DA_KV_I8:
      if (p.mask_kind == DA_MASK_FLASHMASK) return false;
      return !paged && dispatch_d<DA_KV_I8, false, FUSED, false, INSTR>(p.head_dim_qk, g, sp, grid, st);
    default:
      return false;
  }
}

// Largest split count for which decode_attn_forward folds inside the split
// kernel (measured: at S = 12 on the 8 x 4096 GQA shape the single launch is
// slightly faster than split + combine, at S = 32 and S = 128 slower).  Must
// not exceed da::kFoldMaxSplits, the fold's own limit.
constexpr int kFusedMaxSplits = 16;
static_assert(kFusedMaxSplits <= da::kFoldMaxSplits, "fold handles at most 64 states per row");

__global__ void zero_words(uint32_t* w, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) w[i] = 0u;
}

// ---------------------------------------------------------------------------
// Allocation-free forward: the workspace is this library's own device array.
// Each GPU the library runs on holds one copy from the module's load until
// the process ends; its device address differs per GPU and is looked up once
// per device (with that device current) and kept.  The array's name denotes a
// host-side stand-in in host code, so only the looked-up address is ever
// passed to a kernel.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[DA_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's array (nullptr if it cannot be
// resolved).
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" da_status decode_attn_run(const da_plan* plan, const da_args* args, void* stream) {
  const da_status chk = check_args(plan, args);
  if (chk != DA_OK) return chk;
  const da_problem& p = plan->problem;
  if (p.batch == 0) return DA_OK;
  if (!args->workspace || args->workspace_bytes < plan->workspace_bytes) return DA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(args->workspace) & 15u) != 0) return DA_ERR_WORKSPACE;
  if (!da::current_device_is_gfx950()) return DA_ERR_UNSUPPORTED;
  const da::SplitParams sp = make_params(plan, args);
  // With a partition, W*H_kv workgroups (at least one: workgroup 0 writes the
  // workspace's partition header even when every request is empty).
  const uint64_t grid64 = args->partition
                              ? (uint64_t)std::max(args->partition_items, 1) * p.num_kv_heads
                              : (uint64_t)p.batch * p.num_kv_heads * plan->num_splits;
  if (grid64 > 0x7fffffffull) return DA_ERR_INVALID;
  (void)hipGetLastError();
  if (!dispatch_split<false>(p, sp, (unsigned)grid64, static_cast<hipStream_t>(stream))) return DA_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_HIP;
}

extern "C" da_status decode_attn_forward(const da_plan* plan, const da_args* args, float* out,
                                         float* lse, void* stream) {
  const da_status chk = check_args(plan, args);
  if (chk != DA_OK) return chk;
  const da_problem& p = plan->problem;
  if (p.batch == 0) return DA_OK;
  if (!out || (reinterpret_cast<uintptr_t>(out) & 15u) != 0) return DA_ERR_INVALID;
  if (!args->workspace || args->workspace_bytes < plan->workspace_bytes) return DA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(args->workspace) & 15u) != 0) return DA_ERR_WORKSPACE;
  if (!da::current_device_is_gfx950()) return DA_ERR_UNSUPPORTED;
  const unsigned grid = (unsigned)((uint64_t)p.batch * p.num_kv_heads * plan->num_splits);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (plan->num_splits > kFusedMaxSplits || args->partition) {
    // Many splits per row: the separate combine kernel folds them with far
    // more threads than the last-arriving workgroup has, and the arrival
    // round trip of every extra workgroup costs more than the launch it saves.
    // A partitioned run always folds in the combine kernel.
    const da_status st_run = decode_attn_run(plan, args, stream);
    if (st_run != DA_OK) return st_run;
    return decode_attn_combine(plan, args->workspace, args->workspace_bytes, out, lse, stream);
  }
  da::SplitParams sp = make_params(plan, args);
  sp.out = out;
  sp.lse = lse;
  if (!dispatch_split<true>(p, sp, grid, st)) return DA_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_HIP;
}

extern "C" da_status decode_attn_append(const da_plan* plan, const da_append_args* a, void* stream) {
  if (!plan || !a) return DA_ERR_INVALID;
  if (!da::plan_intact(plan)) return DA_ERR_PLAN_MISMATCH;
  const da_problem& p = plan->problem;
  if (p.kv_format != DA_KV_I8 || p.layout != DA_LAYOUT_CONTIG_NHD || p.cache_rows != 0 ||
      p.residual_policy != DA_RESIDUAL_GROUPS || p.residual_len < p.k_group ||
      p.k_group > da::kAppendThreads || (p.head_dim_qk != 64 && p.head_dim_qk != 128))
    return DA_ERR_UNSUPPORTED;
  if (p.batch == 0) return DA_OK;
  if (!a->k_new || !a->v_new || !a->k || !a->v || !a->k_scale || !a->v_scale || !a->k_resid ||
      !a->v_resid || !a->seq_lens)
    return DA_ERR_INVALID;
  if (!da::current_device_is_gfx950()) return DA_ERR_UNSUPPORTED;
  da::AppendParams ap;
  ap.k_new = static_cast<const uint16_t*>(a->k_new);
  ap.v_new = static_cast<const uint16_t*>(a->v_new);
  ap.k = static_cast<int8_t*>(a->k);
  ap.v = static_cast<int8_t*>(a->v);
  ap.k_scale = static_cast<uint16_t*>(a->k_scale);
  ap.v_scale = static_cast<uint16_t*>(a->v_scale);
  ap.k_resid = static_cast<uint16_t*>(a->k_resid);
  ap.v_resid = static_cast<uint16_t*>(a->v_resid);
  ap.seq_lens = a->seq_lens;
  ap.status = a->status;
  ap.num_kv_heads = p.num_kv_heads;
  ap.kv_capacity = p.kv_capacity;
  ap.max_seq_len = p.max_seq_len;
  ap.group = p.k_group;
  ap.resid_len = p.residual_len;
  ap.n_groups = (p.kv_capacity + p.k_group - 1) / p.k_group;
  const dim3 grid((unsigned)(p.batch * p.num_kv_heads));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // closure rows per thread: G / (threads / (D / 8)), i.e. G / 16 (D = 128) or G / 32 (D = 64)
  if (p.head_dim_qk == 128 && p.k_group <= 128)
    hipLaunchKernelGGL((da::append_kernel<128, 8>), grid, dim3(da::kAppendThreads), 0, st, ap);
  else if (p.head_dim_qk == 128)
    hipLaunchKernelGGL((da::append_kernel<128, 16>), grid, dim3(da::kAppendThreads), 0, st, ap);
  else
    hipLaunchKernelGGL((da::append_kernel<64, 8>), grid, dim3(da::kAppendThreads), 0, st, ap);
  return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_HIP;
}

__global__ void flashmask_summary_kernel(const int4* __restrict__ iv, int4* __restrict__ sum, int B,
                                         int L, int nblk) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * nblk) return;
  const int b = i / nblk, J = i - b * nblk;
  const int j0 = J * da::kMaskBlock, j1 = min(L, j0 + da::kMaskBlock);
  int4 mn = make_int4(INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX);
  int4 mx = make_int4(INT32_MIN, INT32_MIN, INT32_MIN, INT32_MIN);
  for (int j = j0; j < j1; ++j) {
    const int4 v = iv[(int64_t)b * L + j];
    mn = make_int4(min(mn.x, v.x), min(mn.y, v.y), min(mn.z, v.z), min(mn.w, v.w));
    mx = make_int4(max(mx.x, v.x), max(mx.y, v.y), max(mx.z, v.z), max(mx.w, v.w));
  }
  // (UTS min, UTS max, UTE min, UTE max), (LTS min, LTS max, LTE min, LTE max)
  sum[(int64_t)i * 2] = make_int4(mn.x, mx.x, mn.y, mx.y);
  sum[(int64_t)i * 2 + 1] = make_int4(mn.z, mx.z, mn.w, mx.w);
}

extern "C" da_status decode_attn_flashmask_summarize(const da_plan* plan, const int32_t* intervals,
                                                     int32_t* summary, void* stream) {
  if (!plan) return DA_ERR_INVALID;
  if (!da::plan_intact(plan)) return DA_ERR_PLAN_MISMATCH;
  const da_problem& p = plan->problem;
  if (p.mask_kind != DA_MASK_FLASHMASK) return DA_ERR_INVALID;
  if (p.batch == 0 || p.max_seq_len == 0) return DA_OK;
  if (!intervals || !summary) return DA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(intervals) & 15u) != 0 || (reinterpret_cast<uintptr_t>(summary) & 15u) != 0)
    return DA_ERR_INVALID;
  if (!da::current_device_is_gfx950()) return DA_ERR_UNSUPPORTED;
  const int nblk = (p.max_seq_len + da::kMaskBlock - 1) / da::kMaskBlock;
  const int n = p.batch * nblk;
  (void)hipGetLastError();
  hipLaunchKernelGGL(flashmask_summary_kernel, dim3((n + 255) / 256), dim3(256), 0,
                     static_cast<hipStream_t>(stream), reinterpret_cast<const int4*>(intervals),
                     reinterpret_cast<int4*>(summary), p.batch, p.max_seq_len, nblk);
  return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_HIP;
}

extern "C" da_status decode_attn_workspace_init(const da_plan* plan, void* workspace,
                                                uint64_t workspace_bytes, void* stream) {
  if (!plan) return DA_ERR_INVALID;
  if (!da::plan_intact(plan)) return DA_ERR_PLAN_MISMATCH;
  const da_problem& p = plan->problem;
  if (p.batch == 0) return DA_OK;
  if (!workspace || workspace_bytes < plan->workspace_bytes) return DA_ERR_WORKSPACE;
  if (!da::current_device_is_gfx950()) return DA_ERR_UNSUPPORTED;
  const int n = p.batch * p.num_kv_heads;
  uint32_t* counters = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) +
                                                   da::states_bytes(*plan));
  (void)hipGetLastError();
  hipLaunchKernelGGL(zero_words, dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                     counters, n);
  return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_HIP;
}

extern "C" da_status decode_attn_combine(const da_plan* plan, const void* workspace,
                                         uint64_t workspace_bytes, float* out, float* lse,
                                         void* stream) {
  if (!plan) return DA_ERR_INVALID;
  if (!da::plan_intact(plan)) return DA_ERR_PLAN_MISMATCH;
  const da_problem& p = plan->problem;
  if (p.batch == 0) return DA_OK;
  if (!out) return DA_ERR_INVALID;
  if (!workspace || workspace_bytes < plan->workspace_bytes) return DA_ERR_WORKSPACE;
  if (!da::current_device_is_gfx950()) return DA_ERR_UNSUPPORTED;
  const uint64_t n_states = (uint64_t)da::output_rows(p) * plan->num_splits;
  const float* ws_u = static_cast<const float*>(workspace);
  const float* ws_m = ws_u + n_states * p.head_dim_v;
  const float* ws_l = ws_m + n_states;
  const unsigned rows = (unsigned)da::output_rows(p);
  const size_t lds = (size_t)plan->num_splits * sizeof(float);
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int32_t* part = reinterpret_cast<const int32_t*>(static_cast<const char*>(workspace) +
                                                        da::partition_header_offset(*plan));
  const int rows_per_request = p.num_queries * p.num_q_heads;
  const int S = plan->num_splits;
  const bool small = S <= da::kCombineSmallS;
  const bool sliced = rows < (unsigned)da::kCombineSliceRows;
  constexpr int NS = da::kCombineThreadsSmall, NL = da::kCombineThreads, DS = da::kCombineSlice;
  if (p.head_dim_v == 64 && sliced)
    hipLaunchKernelGGL((da::combine_kernel<64, NS, DS>), dim3(rows * (64 / DS)), dim3(NS), lds, st, ws_u,
                       ws_m, ws_l, out, lse, S, part, rows_per_request);
  else if (p.head_dim_v == 64 && small)
    hipLaunchKernelGGL((da::combine_kernel<64, NS>), dim3(rows), dim3(NS), lds, st, ws_u, ws_m, ws_l, out,
                       lse, S, part, rows_per_request);
  else if (p.head_dim_v == 64)
    hipLaunchKernelGGL((da::combine_kernel<64, NL>), dim3(rows), dim3(NL), lds, st, ws_u, ws_m, ws_l, out,
                       lse, S, part, rows_per_request);
  else if (p.head_dim_v == 128 && sliced)
    hipLaunchKernelGGL((da::combine_kernel<128, NS, DS>), dim3(rows * (128 / DS)), dim3(NS), lds, st, ws_u,
                       ws_m, ws_l, out, lse, S, part, rows_per_request);
  else if (p.head_dim_v == 128 && small)
    hipLaunchKernelGGL((da::combine_kernel<128, NS>), dim3(rows), dim3(NS), lds, st, ws_u, ws_m, ws_l, out,
                       lse, S, part, rows_per_request);
  else if (p.head_dim_v == 128)
    hipLaunchKernelGGL((da::combine_kernel<128, NL>), dim3(rows), dim3(NL), lds, st, ws_u, ws_m, ws_l, out,
                       lse, S, part, rows_per_request);
  else
    return DA_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_HIP;
}

extern "C" da_status decode_attn_trace_indices(const da_plan* plan, const da_args* args,
                                               const da_trace* trace, float* out, float* lse,
                                               void* stream) {
  const da_status chk = check_args(plan, args);
  if (chk != DA_OK) return chk;
  const da_problem& p = plan->problem;
  if (p.batch == 0) return DA_OK;
  if (!trace || !trace->k_offset || !trace->v_offset || !trace->position || !trace->count)
    return DA_ERR_INVALID;
  if (p.kv_format == DA_KV_I8 && (!trace->k_scale_offset || !trace->v_scale_offset)) return DA_ERR_INVALID;
  if (out && (reinterpret_cast<uintptr_t>(out) & 15u) != 0) return DA_ERR_INVALID;
  if (!args->workspace || args->workspace_bytes < plan->workspace_bytes) return DA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(args->workspace) & 15u) != 0) return DA_ERR_WORKSPACE;
  if (!da::current_device_is_gfx950()) return DA_ERR_UNSUPPORTED;
  da::SplitParams sp = make_params(plan, args);
  sp.tr.k_off = trace->k_offset;
  sp.tr.v_off = trace->v_offset;
  sp.tr.pos = trace->position;
  sp.tr.count = trace->count;
  sp.tr.ks_off = trace->k_scale_offset;
  sp.tr.vs_off = trace->v_scale_offset;
  sp.tr.stride = plan->max_visible;
  const uint64_t grid64 = args->partition
                              ? (uint64_t)std::max(args->partition_items, 1) * p.num_kv_heads
                              : (uint64_t)p.batch * p.num_kv_heads * plan->num_splits;
  if (grid64 > 0x7fffffffull) return DA_ERR_INVALID;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // The launches of decode_attn_forward (out given) or of decode_attn_run,
  // each with the trace instance of the same kernel.
  if (out && plan->num_splits <= kFusedMaxSplits && !args->partition) {
    sp.out = out;
    sp.lse = lse;
    if (!dispatch_split<true, da::kInstrRows>(p, sp, (unsigned)grid64, st)) return DA_ERR_UNSUPPORTED;
    return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_HIP;
  }
  if (!dispatch_split<false, da::kInstrRows>(p, sp, (unsigned)grid64, st)) return DA_ERR_UNSUPPORTED;
  if (hipGetLastError() != hipSuccess) return DA_ERR_HIP;
  return out ? decode_attn_combine(plan, args->workspace, args->workspace_bytes, out, lse, stream) : DA_OK;
}

extern "C" da_status decode_attn_timestamps(const da_plan* plan, const da_args* args, float* out,
                                            float* lse, uint64_t* stamps, uint64_t* clock_hz,
                                            void* stream) {
  const da_status chk = check_args(plan, args);
  if (chk != DA_OK) return chk;
  const da_problem& p = plan->problem;
  if (p.batch == 0) return DA_OK;
  if (!out || !stamps || !clock_hz || (reinterpret_cast<uintptr_t>(out) & 15u) != 0) return DA_ERR_INVALID;
  if (args->partition || p.mask_kind == DA_MASK_FLASHMASK) return DA_ERR_UNSUPPORTED;
  if (!args->workspace || args->workspace_bytes < plan->workspace_bytes) return DA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(args->workspace) & 15u) != 0) return DA_ERR_WORKSPACE;
  if (!da::current_device_is_gfx950()) return DA_ERR_UNSUPPORTED;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return DA_ERR_HIP;
  *clock_hz = (uint64_t)khz * 1000u;
  da::SplitParams sp = make_params(plan, args);
  sp.stamps = stamps;
  const uint64_t grid64 = (uint64_t)p.batch * p.num_kv_heads * plan->num_splits;
  if (grid64 > 0x7fffffffull) return DA_ERR_INVALID;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (plan->num_splits <= kFusedMaxSplits) {
    sp.out = out;
    sp.lse = lse;
    if (!dispatch_split<true, da::kInstrStamps>(p, sp, (unsigned)grid64, st)) return DA_ERR_UNSUPPORTED;
    return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_HIP;
  }
  if (!dispatch_split<false, da::kInstrStamps>(p, sp, (unsigned)grid64, st)) return DA_ERR_UNSUPPORTED;
  if (hipGetLastError() != hipSuccess) return DA_ERR_HIP;
  return decode_attn_combine(plan, args->workspace, args->workspace_bytes, out, lse, stream);
}

extern "C" da_status decode_attn_forward_static(const da_plan* plan, const da_args* args, float* out,
                                                float* lse, void* stream) {
  if (!plan || !args) return DA_ERR_INVALID;
  if (!da::plan_intact(plan)) return DA_ERR_PLAN_MISMATCH;
  if (plan->workspace_bytes > (uint64_t)DA_STATIC_WORKSPACE_BYTES) return DA_ERR_WORKSPACE;
  if (args->workspace || args->workspace_bytes) return DA_ERR_INVALID;
  const da_status chk = check_args(plan, args);
  if (chk != DA_OK) return chk;
  const da_problem& p = plan->problem;
  if (p.batch == 0) return DA_OK;
  if (!out || (reinterpret_cast<uintptr_t>(out) & 15u) != 0) return DA_ERR_INVALID;
  if (!da::current_device_is_gfx950()) return DA_ERR_UNSUPPORTED;
  void* ws = scratch_for_current_device();
  if (!ws) return DA_ERR_HIP;
  da_args a = *args;
  a.workspace = ws;
  a.workspace_bytes = DA_STATIC_WORKSPACE_BYTES;
  // The array keeps whatever the previous call on this GPU left in it: the
  // arrival counters of the single-launch fold are cleared on every call, with
  // a fill kernel on the caller's stream.
  if (plan->num_splits <= kFusedMaxSplits && !args->partition) {
    const da_status st_init = decode_attn_workspace_init(plan, ws, DA_STATIC_WORKSPACE_BYTES, stream);
    if (st_init != DA_OK) return st_init;
  }
  return decode_attn_forward(plan, &a, out, lse, stream);
}

