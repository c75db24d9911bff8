/*
 * decode_attn.h - C ABI of the MI355X (gfx950) Flash-Decoding decode-attention
 * library (libdecode_attn.so).
 *
 * One call computes, for every query row (b, h_q) of a one-token decode step,
 *
 *     O[b, h_q, :] = softmax(q . K^T * scale over the visible keys) @ V
 *     LSE[b, h_q]  = natural log of the softmax denominator (scaled scores)
 *
 * ("M4.5 - Decode Attention Kernels, Mask Programs, and Backend Boundaries",
 * section 0x01), with the Flash-Decoding schedule of sections 0x02-0x03:
 * decode_attn_run streams disjoint slices ("splits") of each request's
 * visible keys and writes one exact partial softmax state (m, l, u) per
 * (b, h_q, split) into a caller-owned workspace (section 0x02A, structure of
 * arrays of section 0x03D); decode_attn_combine merges those states into the
 * final row (sections 0x02B, 0x02C) and applies the all-masked policy
 * O = +0.0, LSE = -inf.
 *
 * Conventions (all calls):
 *  - Every pointer inside da_args, and the out/lse/workspace/offsets/positions
 *    arguments, is a DEVICE pointer; problem, plan, reasons and
 *    workspace_bytes pointers are HOST pointers.  The caller owns every
 *    buffer; the library allocates no device memory and keeps no state
 *    beyond a per-device cache of the architecture check, except the one
 *    workspace array per GPU of decode_attn_forward_static.
 *  - Calls return a da_status; nothing throws across the ABI and nothing is
 *    printed.  decode_attn_run and decode_attn_combine are asynchronous on the
 *    given HIP stream (hipStream_t passed as void*, NULL = default stream) and
 *    never synchronize; run must precede combine on that stream.
 *  - Semantic errors (DA_ERR_INVALID) are checked before capability checks and
 *    before any metadata is dereferenced (section 0x07A).  Capability
 *    failures (DA_ERR_UNSUPPORTED) report EVERY failed predicate as a bit in
 *    *reasons (section 0x07B, admission as a conjunction with a complete
 *    reason vector); there is no fallback path (section 0x07C, forced backend
 *    fails closed).
 */
#ifndef DECODE_ATTN_H_
#define DECODE_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t da_status;
#define DA_OK                 0
#define DA_ERR_INVALID       (-1)  /* malformed call (bad GQA ratio, layout/page_size mismatch, W <= 0, ...) */
#define DA_ERR_UNSUPPORTED   (-2)  /* well-formed but outside this library: see *reasons */
#define DA_ERR_WORKSPACE     (-3)  /* workspace pointer missing or smaller than the plan needs */
#define DA_ERR_PLAN_MISMATCH (-4)  /* plan fields changed after decode_attn_plan froze them */
#define DA_ERR_HIP           (-5)  /* a HIP runtime call or kernel launch failed */

/* element types */
#define DA_F32  0
#define DA_BF16 1
#define DA_F16  2

/* K/V storage formats */
#define DA_KV_F32  0   /* fp32 rows */
#define DA_KV_BF16 1   /* bf16 rows */
#define DA_KV_I8   2   /* int8 codes + fp16 scales + bf16 residual, see da_args */

/* DA_KV_I8 residual policies: which of a request's T tokens are int8 codes
 * (the oldest n_q) and which are bf16 residual rows (row t - n_q holds token t)
 * ("M8.6 - Live-Data Quantization: Activations and KV Cache", section 0x06B) */
#define DA_RESIDUAL_WINDOW 0  /* n_q = T - min(T, R): the newest min(T, R) tokens are bf16     */
#define DA_RESIDUAL_GROUPS 1  /* n_q = G * max(0, ceil((T - R) / G)): whole K groups close as
                                 soon as more than R tokens are unclosed (the streaming rule
                                 decode_attn_append maintains; requires G <= R)             */

/* cache layouts ("M4.5 ...", sections 0x04B and 0x04D) */
#define DA_LAYOUT_CONTIG_NHD 0  /* [B_c, T_cap, H_kv, D]; element ((c*T_cap + t)*H_kv + h)*D + x  */
#define DA_LAYOUT_PAGED_NHD  1  /* pool [N_pages, P, H_kv, D]; element ((pi*P + t%P)*H_kv + h)*D + x */
#define DA_LAYOUT_CONTIG_HND 2  /* [B_c, H_kv, T_cap, D]; element ((c*H_kv + h)*T_cap + t)*D + x  */
#define DA_LAYOUT_PAGED_HND  3  /* pool [N_pages, H_kv, P, D]; element ((pi*H_kv + h)*P + t%P)*D + x */
#define DA_LAYOUT_RAGGED_NHD 4  /* packed [N_rows, H_kv, D]; request b's token t is packed row
                                   indptr[b] + t: element ((indptr[b] + t)*H_kv + h)*D + x
                                   ("M4.5 ...", section 0x04C)                             */
#define DA_LAYOUT_RING_NHD   5  /* fixed-capacity sink + window cache [B_c, n_sink + W, H_kv, D]
                                   with DA_MASK_SINK_WINDOW: position t < n_sink lives in slot t,
                                   any other position in ring slot n_sink + t mod W ("M5.4 ...",
                                   section 0x04: the slot is an address, the position stays t);
                                   kv_capacity must equal n_sink + W                       */
/* Contiguous layouts: cache row c = cache_batch_idx[b] when given, else b
 * (section 0x04B).  Paged layouts: the physical page pi of logical block
 * j = t / P of request b comes from the page table (section 0x04D): */
#define DA_PAGE_TABLE_DENSE 0   /* pi = block_table[b * max_pages_per_seq + j]              */
#define DA_PAGE_TABLE_CSR   1   /* pi = block_table[indptr[b] + j]  (kv_page_indices with
                                   kv_page_indptr; num_page_entries entries)               */

/* mask programs: visibility of logical key t for the decode row of request b,
 * whose visible length is T = seq_lens[b] (the row sits at position T-1) */
#define DA_MASK_CAUSAL      0  /* every t in [0, T)                                  */
#define DA_MASK_SINK_WINDOW 1  /* t < min(n_sink, T)  or  t >= T - window  (window > 0)
                                  ("M5.4 - Long-Context KV Policies: Retention,
                                  Compression, and Budget Allocation", sections
                                  0x04-0x05: sink and recent sets as a union)       */
#define DA_MASK_FLASHMASK   2  /* FlashMask ("M4.5 ...", sections 0x06A-0x06D): key t < T is
                                  hidden when q = T-1 lies in [UTS_t, UTE_t) or [LTS_t, LTE_t)
                                  (da_args mask_intervals); 16-key tiles are classified SKIP /
                                  FULL / PARTIAL from mask_summary and SKIP tiles are never
                                  loaded; splits share the non-SKIP tiles evenly.  bf16 K/V,
                                  head_dim 128, one query row, max_seq_len <=
                                  DA_FLASHMASK_MAX_SEQ.                                       */
#define DA_FLASHMASK_MAX_SEQ 131072

/* admission reason bits (DA_ERR_UNSUPPORTED) */
#define DA_R_HEAD_DIM    (1ull << 0)   /* head_dim_qk not in {64, 128}                 */
#define DA_R_HEAD_DIM_V  (1ull << 1)   /* head_dim_v != head_dim_qk                    */
#define DA_R_GQA_GROUP   (1ull << 2)   /* H_q / H_kv not in {1, 2, 4, 8}              */
#define DA_R_Q_DTYPE     (1ull << 3)   /* q dtype not paired with the K/V format      */
#define DA_R_OUT_DTYPE   (1ull << 4)   /* output must be DA_F32                       */
#define DA_R_KV_FORMAT   (1ull << 5)   /* unknown K/V format                          */
#define DA_R_LAYOUT      (1ull << 6)   /* layout not available for this K/V format    */
#define DA_R_INT8_PARAMS (1ull << 7)   /* int8: k_group not a power of two in [16, 1024] */
#define DA_R_SPLITS      (1ull << 8)   /* num_splits above DA_MAX_SPLITS              */
#define DA_R_INDEX_RANGE (1ull << 9)   /* an index exceeds its range: grid >= 2^31
                                          workgroups, or int8 with H_kv * d > 2^20 bytes
                                          per position                               */
#define DA_R_DEVICE      (1ull << 10)  /* current device is not gfx950 or cannot be queried */
#define DA_R_MASK_KIND   (1ull << 11)  /* unknown mask program, or FlashMask outside its
                                          domain (bf16, d=128, C=1, splits <= 1024 keys) */
#define DA_R_QUERY_ROWS  (1ull << 12)  /* num_queries C: (H_q/H_kv)*C not in {1,2,4,8}, or
                                          C > 1 with a mask other than causal        */
#define DA_NUM_REASONS   13

#define DA_MAX_SPLITS 4096

/* The decode coordinate of one call ("M4.5 ...", sections 0x00B and 0x07A). */
typedef struct da_problem {
  int32_t batch;             /* B >= 0                                              */
  int32_t num_q_heads;       /* H_q >= 1                                            */
  int32_t num_kv_heads;      /* H_kv >= 1, H_q % H_kv == 0; head h_q reads h_q / (H_q/H_kv) */
  int32_t head_dim_qk;       /* D                                                   */
  int32_t head_dim_v;        /* must equal head_dim_qk                              */
  int32_t q_dtype;           /* DA_F32 with DA_KV_F32; DA_BF16 with DA_KV_BF16 / DA_KV_I8 */
  int32_t out_dtype;         /* DA_F32                                              */
  int32_t kv_format;         /* DA_KV_*                                             */
  int32_t layout;            /* DA_LAYOUT_*                                         */
  int32_t kv_capacity;       /* contiguous: token capacity T_cap of each batch row; paged: 0 */
  int32_t page_size;         /* paged: P > 0; contiguous: must be 0                */
  int32_t max_pages_per_seq; /* paged: columns of block_table                       */
  int32_t num_pages;         /* paged: N_pages of the pool                          */
  int32_t max_seq_len;       /* upper bound on every seq_lens[b]; sizes the splits  */
  int32_t mask_kind;         /* DA_MASK_*                                           */
  int32_t n_sink;            /* DA_MASK_SINK_WINDOW: sink positions >= 0            */
  int32_t window;            /* DA_MASK_SINK_WINDOW: recent window W > 0            */
  float   softmax_scale;     /* 0 -> 1/sqrt(head_dim_qk); must be finite and >= 0   */
  int32_t num_splits;        /* 0 -> automatic (B*H_kv below the CU count: about one
                                 workgroup per CU, splits of 256..4096 rows; otherwise
                                 about 3 per CU, splits of 256..1024 rows); otherwise
                                 the requested split count */
  int32_t k_group;           /* DA_KV_I8: tokens per K-scale group (128); else 0   */
  int32_t residual_len;      /* DA_KV_I8: bf16 residual rows R >= 0; else 0        */
  int32_t num_cus;           /* 0 -> query the current device; > 0: plan for this many CUs */
  int32_t residual_policy;   /* DA_KV_I8: DA_RESIDUAL_*; else 0                     */
  int32_t num_queries;       /* C query rows per request (0 -> 1); see da_args q     */
  int32_t page_table;        /* paged: DA_PAGE_TABLE_*; else 0                      */
  int32_t cache_rows;        /* contiguous: rows B_c of the cache (0 -> B; > 0 needs
                                cache_batch_idx); ragged: packed rows N_rows           */
  int32_t num_page_entries;  /* DA_PAGE_TABLE_CSR: entries of block_table; else 0  */
  int32_t reserved1;         /* must be 0                                           */
} da_problem;

/* A frozen plan: a plain value the caller owns and may copy; nothing to free.
 * Run and combine recompute `key` from the other fields and refuse a plan
 * whose fields changed after planning (section 0x07F). */
typedef struct da_plan {
  uint64_t   key;              /* hash of every field below                         */
  da_problem problem;          /* normalized copy (softmax_scale resolved)          */
  int32_t    num_splits;       /* S launched: producer grid is B*H_kv*S workgroups  */
  int32_t    chunk;            /* visible rows per split; int8: weighted rows (a    */
                               /* residual row counts 2); FlashMask: multiple of 16 */
  int32_t    max_visible;      /* bound on visible rows of one request              */
  int32_t    num_cus;          /* CU count the split heuristic used                 */
  uint64_t   workspace_bytes;  /* states round_up(B*H_q*S*(D + 2)*4, 256), then     */
                               /* counters round_up(B*H_kv*4, 256), then the        */
                               /* partition header round_up((B+5)*4, 256)           */
  uint64_t   reserved[2];
} da_plan;

/* Per-call device buffers.  Layouts (row-major, no padding):
 *   q           [B, C, H_q, D]             q_dtype; C = num_queries (C = 1: the decode row).
 *               Query row i of request b sits at position T_b - C + i and sees keys
 *               [0, T_b - C + i + 1): bottom-right causal alignment ("M4.5 ...",
 *               sections 0x08B-0x08C: the C new rows are already in the cache, so
 *               T_b counts them and a one-token decode is C = 1)
 *   k, v        per DA_LAYOUT_* (B_c = cache_rows or B): contiguous NHD [B_c, T_cap, H_kv, D],
 *               contiguous HND [B_c, H_kv, T_cap, D], paged NHD [N_pages, P, H_kv, D],
 *               paged HND [N_pages, H_kv, P, D], ragged NHD [N_rows, H_kv, D]
 *               DA_KV_I8: int8 codes [B, T_cap, H_kv, D] of tokens t < n_q(b) (contiguous NHD)
 *   k_scale     DA_KV_I8: fp16 [B, ceil(T_cap/k_group), H_kv, D]; group j scales
 *               tokens [j*k_group, (j+1)*k_group), one scale per channel
 *   v_scale     DA_KV_I8: fp16 [B, T_cap, H_kv]; one scale per token.
 *               Domain: any finite normal fp16 scales (the writer rule of "M8.6 ...",
 *               section 0x02A) with any finite bf16 q; the matrix-core int8 kernel
 *               scales q (per head) and the K and V scales (per run of at most 2048
 *               rows) by powers of two into fp16's range and undoes them exactly, so
 *               K values up to 127 * 65504 and |q| beyond 65504 stay finite.  Scores
 *               must be finite in fp32.
 *   k_resid,
 *   v_resid     DA_KV_I8: bf16 [B, R, H_kv, D]; row t - n_q(b) holds token t for
 *               t >= n_q(b) = seq_lens[b] - min(seq_lens[b], R)
 *   block_table paged, dense: int32 [B, max_pages_per_seq]; CSR: int32 [num_page_entries];
 *               only the entries of blocks < ceil(T_b/P) are read
 *   indptr      int32 [B + 1]: ragged layout: packed row of each request's token 0;
 *               CSR page table: first table entry of each request.  Else NULL.
 *   cache_batch_idx optional int32 [B] (contiguous layouts): cache row of request b
 *               (cache_rows > 0).  Out-of-range entries and table values are clamped into
 *               the buffers they index, so corrupt metadata can never address memory
 *               outside them.
 *   seq_lens    int32 [B]; visible length T_b of each request, 0 <= T_b <= max_seq_len
 *   work_order  optional int32 [B*H_kv*S]: workgroup i runs work item work_order[i] =
 *               (b*H_kv + h_kv)*S + s.  It must be a permutation of 0 .. B*H_kv*S-1 (as
 *               written by decode_attn_schedule); any permutation gives the same result
 *               bit for bit, only the schedule changes.  NULL: the built-in order.
 *   workspace   >= plan.workspace_bytes, 256-byte aligned.  The state region
 *               (first round_up(B*H_q*S*(D+2)*4, 256) bytes) is ignored on
 *               entry.  The B*H_kv uint32 arrival counters after it are used
 *               only by decode_attn_forward: they must be zero when it starts
 *               (decode_attn_workspace_init) and it leaves them zero.  The
 *               last round_up((B+5)*4, 256) bytes receive, from every run, the
 *               partition header the combine needs (ignored on entry).
 *   partition   optional int32 descriptor from decode_attn_partition (device copy);
 *               NULL: the plan's fixed splits.  With a partition the producer grid is
 *               partition_items*H_kv workgroups of equal work (see decode_attn_partition).
 *   partition_items  the descriptor's item count W (host value; 0 without partition)
 * q, k, v, k_resid, v_resid and k_scale must be 16-byte aligned, v_scale 2-byte
 * aligned (DA_ERR_INVALID otherwise). */
typedef struct da_args {
  const void*    q;
  const void*    k;
  const void*    v;
  const void*    k_scale;
  const void*    v_scale;
  const void*    k_resid;
  const void*    v_resid;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void*          workspace;
  uint64_t       workspace_bytes;
  const int32_t* work_order;   /* NULL, or B*H_kv*S work items from decode_attn_schedule */
  const int32_t* indptr;       /* ragged layout / CSR page table: [B + 1]; else NULL     */
  const int32_t* cache_batch_idx; /* contiguous layouts with cache_rows > 0: [B]; else NULL */
  const int32_t* mask_intervals;  /* DA_MASK_FLASHMASK: [B, max_seq_len, 4] (UTS, UTE, LTS, LTE) */
  const int32_t* mask_summary;    /* DA_MASK_FLASHMASK: [B, ceil(max_seq_len/16), 8]           */
  const int32_t* partition;       /* NULL, or a descriptor from decode_attn_partition          */
  int32_t        partition_items; /* W of that descriptor (0 without one)                      */
  int32_t        reserved0;
} da_args;

/* Validate the problem (semantic checks first, then every capability
 * predicate), choose the split count, size the workspace and freeze the plan
 * ("M4.5 ...", sections 0x07A-0x07B: the dispatch key is frozen before
 * selection, admission is a conjunction and a rejection reports every failed
 * predicate; 0x07F: the plan is a second immutable key; 0x03B and 0x03D-0x03E:
 * split bounds and the workspace follow from the problem).
 * Host only: touches the device only to read its CU count and architecture
 * when problem->num_cus == 0.  plan, workspace_bytes and reasons may each be
 * NULL; *reasons receives the complete bit vector of failed predicates. */
da_status decode_attn_plan(const da_problem* problem, da_plan* plan,
                           uint64_t* workspace_bytes, uint64_t* reasons);

/* Host-side work ordering for ragged batches ("M4.5 ...", sections 0x09E and
 * 0x09G: a plan built on the host from the batch's lengths balances uneven
 * requests).  Only the order in which workgroups take work items changes; the
 * split boundaries, and so the arithmetic, stay those of the plan.  Given the
 * requests' lengths on the host, writes into order[0 .. B*H_kv*S) the work
 * items largest first: every full split (chunk visible rows), then each
 * request's partial last split by decreasing size, then the empty splits;
 * within a class the items of one request are spread over consecutive
 * positions so that they reach different XCDs.  Copy the result to the device
 * and pass it as da_args.work_order.  Errors: DA_ERR_INVALID for a NULL
 * pointer, order_len < B*H_kv*S, or a length outside [0, max_seq_len];
 * DA_ERR_PLAN_MISMATCH for an altered plan. */
da_status decode_attn_schedule(const da_plan* plan, const int32_t* seq_lens_host, int32_t* order,
                               uint64_t order_len);

/* Host-side balanced partition of a ragged batch ("M4.5 ...", sections 0x09E
 * and 0x09G: a plan built from the lengths gives every workgroup the same
 * amount of work, as LeanAttention and FlashInfer's planner do, instead of
 * fixed splits whose last round runs part-empty).  The visible ordinals of
 * the requests, concatenated in request order (N = sum of N_b), are cut into W
 * items of L consecutive ordinals (the last may be shorter); workgroup
 * (i, h_kv) processes item i for K/V head h_kv.  Where an item crosses request
 * boundaries it produces one state per request piece: piece j of request b
 * is item floor(P_b / L) + j with P_b = N_0 + ... + N_{b-1}, stored in split
 * slot j, and request b has last_item(b) - first_item(b) + 1 <= S pieces
 * (L >= max_b N_b / (S - 1) guarantees it; S >= 2 is required).  The combine
 * folds exactly those pieces, in ascending order; the arithmetic is the same
 * split/merge, so the result matches the oracle to the same tolerance (but is
 * not bitwise equal to the fixed-split result).
 *   items_per_head  target W (0: one dispatch round, 3 workgroups per CU of the plan / H_kv
 *                   for bf16, 2 for int8)
 *   part            host int32 [5 + B + W_max] with W_max = the target W:
 *                   [W, L, B, 0, P_0 .. P_B, first request of item 0 .. W-1]
 *   *items_out      W (may be 0 when every request is empty)
 * Copy part to the device and pass it with W as da_args.partition /
 * partition_items.  Supported by the bf16 (any layout) and int8 D = 128
 * matrix-core kernels with the causal or sink+window mask; items count visible
 * rows (an int8 cache's bf16 residual rows, at most R per request, count as one
 * row each although they carry twice the bytes).  Errors: DA_ERR_INVALID for a NULL
 * pointer, a length outside [0, max_seq_len], part_len too small, or N >= 2^31;
 * DA_ERR_UNSUPPORTED for S < 2; DA_ERR_PLAN_MISMATCH for an altered plan. */
da_status decode_attn_partition(const da_plan* plan, const int32_t* seq_lens_host, int32_t items_per_head,
                                int32_t* part, uint64_t part_len, int32_t* items_out);

/* Launch the split kernel ("M4.5 ...", sections 0x02A, 0x02C, 0x03C and
 * 0x03D: the producer grid, one state per split and query head, the empty
 * identity, the workspace shapes): grid B*H_kv*S workgroups; workgroup (b, h_kv, s)
 * owns visible rows [s*chunk, min((s+1)*chunk, N_b)) of request b (int8:
 * the rows whose weighted offsets fall there, a residual row weighing 2) and the
 * H_q/H_kv query heads sharing h_kv, reads each of its K/V rows once, and
 * writes one (m, l, u) state per query head into the workspace: u fp32
 * [B, H_q, S, D], then m fp32 [B, H_q, S] (natural-log units of the scaled
 * scores), then l fp32 [B, H_q, S].  An empty split writes the identity
 * (m = -inf, l = 0, u = 0); l > 0 marks a valid state.  With a partition
 * (da_args.partition) the grid is W*H_kv workgroups and only the pieces of the
 * partition are written (slots j >= the request's piece count are left as
 * they were).  Every run also writes the partition header of the workspace
 * (W = 0 without a partition), which the combine reads. */
da_status decode_attn_run(const da_plan* plan, const da_args* args, void* stream);

/* Launch the combine kernel ("M4.5 ...", sections 0x02B-0x02C, 0x03C and
 * 0x03I: the reducer grid, the binary merge, the empty-aware fold): for each
 * (b, i, h_q), fold its S states (with
 * a partition: its pieces, as the workspace's partition header written by
 * the preceding run says) in ascending split order and write out fp32
 * [B, C, H_q, D] = u/l and, when lse
 * is not NULL, lse fp32 [B, C, H_q] = m + ln(l); an all-masked row gets
 * O = +0.0 and LSE = -inf.  (State rows, out and lse rows are ordered
 * (b, i, h_q); with C = 1 this is [B, H_q].) */
da_status decode_attn_combine(const da_plan* plan, const void* workspace,
                              uint64_t workspace_bytes, float* out, float* lse,
                              void* stream);

/* Single-launch form of run + combine ("M4.5 ...", sections 0x02B, 0x03F and
 * 0x09B: Flash-Decoding's second reduction level, here without the second
 * launch): the same split kernel, with the reduction of section 0x02B folded
 * into it.  Each workgroup stores its
 * states, makes them visible device-wide, and increments the arrival counter
 * of its (b, h_kv); the workgroup that arrives last (the S-th) reads the S
 * states of its H_q/H_kv rows, folds them in ascending split order exactly as
 * the combine kernel defines, writes out fp32 [B, H_q, D] and (when lse is not
 * NULL) lse fp32 [B, H_q], and resets the counter to zero.  No workgroup waits
 * for another, so the launch completes whatever the scheduling order.
 * Requirements: the workspace counters are zero on entry (see
 * decode_attn_workspace_init; every completed forward leaves them zero), and
 * calls that share a workspace are ordered on one stream.  out must be
 * 16-byte aligned (DA_ERR_INVALID otherwise).  Results match run + combine up
 * to the order of the final fp32 sums.  With a partition, or when S exceeds
 * the in-kernel fold's limit, it launches run then combine. */
da_status decode_attn_forward(const da_plan* plan, const da_args* args, float* out, float* lse,
                              void* stream);

/* ---- allocation-free forward ------------------------------------------------ */

/* Size of the library's own workspace array (one per GPU, see below). */
#define DA_STATIC_WORKSPACE_BYTES (32u << 20)

/* decode_attn_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, and harnesses that forbid
 * hipMalloc.  Instead of a caller-owned workspace it uses a device array of
 * DA_STATIC_WORKSPACE_BYTES that the library holds on each GPU it runs on
 * from the first call there until the process ends; it calls no allocating
 * routine.  The caller still owns q, K/V, metadata, out and lse; args->workspace
 * must be NULL and args->workspace_bytes 0 (DA_ERR_INVALID otherwise).  Every
 * call on one GPU shares that GPU's array and finds it as the previous call
 * left it: the call clears what must start at zero (the arrival counters, by
 * a fill kernel on `stream`), so consecutive calls are independent, but calls
 * that overlap on one GPU (different streams, or different host threads,
 * without ordering between them) race on the array and must not be issued.
 * Errors: those of decode_attn_forward, and DA_ERR_WORKSPACE when the plan's
 * workspace_bytes exceeds DA_STATIC_WORKSPACE_BYTES (checked before anything
 * else is read).  Results are those of decode_attn_forward for the same plan
 * and inputs, bit for bit. */
da_status decode_attn_forward_static(const da_plan* plan, const da_args* args, float* out, float* lse,
                                     void* stream);

/* FlashMask block summaries ("M4.5 ...", section 0x06C): for each request b
 * and block J of 16 key columns [16J, min(16J+16, max_seq_len)), write
 * summary[b][J] = (UTS min, UTS max, UTE min, UTE max, LTS min, LTS max,
 * LTE min, LTE max) over the block's columns of intervals [B, max_seq_len, 4].
 * Both pointers are device pointers, 16-byte aligned.  Run it whenever the
 * intervals change, before decode_attn_run / decode_attn_forward. */
da_status decode_attn_flashmask_summarize(const da_plan* plan, const int32_t* intervals,
                                          int32_t* summary, void* stream);

/* Zero the arrival counters ("M4.5 ...", section 0x03E: temporary storage
 * derived from the ABI) of a workspace sized for `plan` (a fill kernel on
 * `stream`, so it may be captured into a graph).  Needed once per workspace
 * before its first decode_attn_forward. */
da_status decode_attn_workspace_init(const da_plan* plan, void* workspace,
                                     uint64_t workspace_bytes, void* stream);

/* Index trace ("M4.5 ...", sections 0x04F and 0x04H: a kernel must read
 * exactly the visible rows, each once, at the addresses the translation
 * gives, and never a page tail or a table slot past the request).  Debug
 * only, never on the timed path.  Each split kernel has a trace instance:
 * the same code, which in addition records every K and V row load at the
 * point where it is issued, with the address that load used.  Slots are per
 * (b, h_kv, visible ordinal o), o < plan.max_visible; ordinal o of request b
 * is its o-th visible key in position order (FlashMask: o = position).
 * Arrays of B * H_kv * plan.max_visible entries, all device pointers: */
typedef struct da_trace {
  int64_t* k_offset;        /* element offset of the K row's first element in the buffer it was read
                               from: k (int8: the codes) or, for DA_KV_I8 positions >= n_q(b), k_resid */
  int64_t* v_offset;        /* the same for the V row (v or v_resid)                                  */
  int32_t* position;        /* logical key position t of the row                                      */
  int32_t* count;           /* caller zeroes; +1 per K row load, +(1 << 16) per V row load            */
  int64_t* k_scale_offset;  /* DA_KV_I8 codes: element offset of the k_scale row (its channel 0) the
                               row's dequantization used; else may be NULL                           */
  int64_t* v_scale_offset;  /* DA_KV_I8 codes: element offset into v_scale; else may be NULL         */
} da_trace;

/* Runs the trace instance of the kernels the timed calls launch: with out ==
 * NULL those of decode_attn_run (states into args->workspace), with out given
 * those of decode_attn_forward (the single launch with its fold for S <= 16
 * without a partition -- workspace counters zero on entry, as for
 * decode_attn_forward -- else run then combine), writing out/lse as they do.
 * A balanced partition (args->partition) runs the partition instance.  Only
 * rows a workgroup consumes are recorded (loads issued past a split's end
 * repeat a visible row and are weighted 0); under FlashMask the rows of
 * PARTIAL tiles are loaded and recorded whether or not they are hidden, SKIP
 * tiles never.  Entries never written keep their prior values (callers fill
 * them with -1).  Errors: those of decode_attn_run / decode_attn_forward, and
 * DA_ERR_INVALID for a NULL trace array (the scale arrays only for DA_KV_I8). */
da_status decode_attn_trace_indices(const da_plan* plan, const da_args* args, const da_trace* trace,
                                    float* out, float* lse, void* stream);

/* Per-workgroup timestamps of the launches decode_attn_forward makes, for
 * schedule analysis ("M4.5 ...", sections 0x0BF and 0x0BH: a trace shows
 * what ran; raw synchronized samples close the measurement).  Debug only,
 * never on the timed path: a timestamp
 * instance of the same kernels, in which thread 0 of each workgroup reads the
 * device's constant-rate clock (s_memrealtime) at its start, when its states
 * are stored, and at its end.  stamps: device uint64 [B*H_kv*S, 4] per
 * workgroup index: start, states stored, end, and the XCC_ID register (bits
 * 0..3) | the HW_ID register << 8 (CU, shader engine) | 1 << 63 when the
 * workgroup folded the states of its (b, h_kv).  *clock_hz (host) receives
 * the clock's rate.  With S above the single-launch limit the split kernel is
 * stamped and the combine follows.  Matrix-core kernels (bf16 / int8,
 * head_dim 128) without a partition or FlashMask; else DA_ERR_UNSUPPORTED.
 * Other errors as decode_attn_forward. */
da_status decode_attn_timestamps(const da_plan* plan, const da_args* args, float* out, float* lse,
                                 uint64_t* stamps, uint64_t* clock_hz, void* stream);

/* ---- streaming append for DA_KV_I8 with DA_RESIDUAL_GROUPS ------------------ */

/* per-request error bits written (OR-ed) into da_append_args.status[b] */
#define DA_APPEND_NO_ROOM   1  /* seq_lens[b] < 0 or seq_lens[b] + 1 > max_seq_len: nothing written */
#define DA_APPEND_BAD_SCALE 2  /* a closing group had a non-finite value or a non-finite or
                                  subnormal fp16 scale: nothing written for that (b, h_kv)      */

typedef struct da_append_args {
  const void*    k_new;     /* bf16 [B, H_kv, D]: K row of the token appended to request b      */
  const void*    v_new;     /* bf16 [B, H_kv, D]                                                 */
  void*          k;         /* int8 codes [B, T_cap, H_kv, D] (the da_args k of the same cache)   */
  void*          v;
  void*          k_scale;   /* fp16 [B, ceil(T_cap/G), H_kv, D]                                  */
  void*          v_scale;   /* fp16 [B, T_cap, H_kv]                                             */
  void*          k_resid;   /* bf16 [B, R, H_kv, D]                                              */
  void*          v_resid;
  const int32_t* seq_lens;  /* int32 [B]: lengths before the append; the caller adds 1 after    */
  int32_t*       status;    /* int32 [B] or NULL: error bits are OR-ed in (caller zeroes it)     */
} da_append_args;

/* Append one token to every request of an int8 cache that follows
 * DA_RESIDUAL_GROUPS with k_group <= residual_len ("M8.6 ...", sections 0x05B
 * and 0x06B).  For request b of length T = seq_lens[b]: if its residual holds
 * R rows, its oldest G are closed first -- K quantized per channel over the G
 * rows into scale group n_q/G, V quantized per row (scale per token), codes at
 * positions n_q .. n_q+G-1 -- and the other R - G rows move down to residual
 * rows 0 .. R-G-1 (residual row i always holds token n_q + i); then the new
 * rows go to residual row T - n_q(T+1).
 * The quantizer is that of the int8 format (section 0x02A).  One workgroup per
 * (b, h_kv), asynchronous on `stream`; nothing is written for a request whose
 * status gets an error bit (the heads of one request may then disagree, so
 * the request must be dropped).  The same plan serves attention over the
 * cache after seq_lens has been advanced.  Errors: DA_ERR_INVALID (NULL
 * buffer, altered key -> DA_ERR_PLAN_MISMATCH), DA_ERR_UNSUPPORTED (not
 * int8 + contiguous + DA_RESIDUAL_GROUPS with k_group <= residual_len and k_group <= 256,
 * or head_dim not 64/128), DA_ERR_HIP. */
da_status decode_attn_append(const da_plan* plan, const da_append_args* args, void* stream);

/* Static text for one reason bit index (0 .. DA_NUM_REASONS-1) or status
 * ("M4.5 ...", section 0x07B: a rejection is a vector of named predicates). */
const char* decode_attn_reason(int bit);
const char* decode_attn_status_string(da_status status);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_H_ */
