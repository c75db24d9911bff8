// Combine (reduction) kernel of the Flash-Decoding schedule.
//
// One workgroup per output row (b, h_q) folds that row's S split states.  It
// is the log-sum-exp-weighted reduction of "M4.5 - Decode Attention Kernels,
// Mask Programs, and Backend Boundaries", sections 0x02B and 0x09B written in
// two passes: the global maximum M over the valid states first, then
// l = sum_s e^(m_s - M) l_s and u = sum_s e^(m_s - M) u_s, which in exact
// arithmetic equals the sequential binary merge of section 0x02B (sections
// 0x02D-0x02E).  A state is valid iff l_s > 0 (a non-empty state has l >= 1
// because its maximum contributes e^0); an invalid state gets weight 0 and its
// u is never used, so no exponential or product ever sees it (section 0x02C).
// Finalize: O = u / l and LSE = M + ln l, or O = +0.0 and LSE = -inf when no
// state is valid.
//
// Work split: a workgroup owns DS columns of a row (all D, or a slice when
// the rows are too few to spread the state reads over the chip); thread t
// owns column t % DS of the split class t / DS (mod NG = threads / DS).  Every
// slice derives the same weights from the row's (m, l) values.  The u values
// of the first 16 states of each class are requested before the weights are
// known, so the state loads and the weight computation overlap; the NG
// partial sums are then added in fixed order.
// Every reduction has a fixed shape, so the result is bitwise repeatable for a
// fixed plan (section 0x02H, determinism contract).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

// Threads per row: 1024 for many states, 256 when a row has at most
// kCombineSmallS of them (two split classes of D = 128 columns, 16 states each
// in flight), so short rows do not hold a full 1024-thread workgroup.  With
// fewer rows than kCombineSliceRows, 256-thread workgroups of kCombineSlice
// columns each.
constexpr int kCombineThreads = 1024;
constexpr int kCombineThreadsSmall = 256;
constexpr int kCombineSmallS = 32;
constexpr int kCombineSlice = 32;
constexpr int kCombineSliceRows = 256;

template <int D, int NT, int DS = D>
__global__ __launch_bounds__(NT) void combine_kernel(const float* __restrict__ ws_u,
                                                                  const float* __restrict__ ws_m,
                                                                  const float* __restrict__ ws_l,
                                                                  float* __restrict__ out,
                                                                  float* __restrict__ lse, int S_plan,
                                                                  const int32_t* __restrict__ part_hdr,
                                                                  int rows_per_request) {
  static_assert(D % DS == 0 && NT % DS == 0, "");
  constexpr int NG = NT / DS;
  constexpr int NW = NT / 64;
  constexpr int U = 16;
  const int row = blockIdx.x / (D / DS);
  const int col0 = (blockIdx.x % (D / DS)) * DS;
  const int tid = threadIdx.x;
  // States of this row: the plan's S splits, or with a balanced partition
  // (header W > 0, written by the run) the request's pieces: items
  // floor(P_b / L) .. floor((P_{b+1} - 1) / L), stored as slots 0, 1, ...
  int S = S_plan;
  if (part_hdr[0] > 0) {
    const int b = row / rows_per_request;
    const int L = part_hdr[1], pb = part_hdr[4 + b], pb1 = part_hdr[5 + b];
    S = (pb1 > pb && L > 0) ? min((pb1 - 1) / L - pb / L + 1, S_plan) : 0;
  }
  if (S == 0) {                     // no state: all-masked row (O = +0.0, LSE = -inf)
    if (tid < DS) out[(int64_t)row * D + col0 + tid] = 0.f;
    if (lse && col0 == 0 && tid == 0) lse[row] = -INFINITY;
    return;
  }
  const int lane = tid & 63, wave = tid >> 6;
  const int c = col0 + tid % DS, g = tid / DS;
  const float* m = ws_m + (int64_t)row * S_plan;
  const float* l = ws_l + (int64_t)row * S_plan;
  const float* u = ws_u + (int64_t)row * S_plan * D;

  __shared__ float red_m[NW];
  __shared__ float red_l[NW];
  __shared__ float part[NG][DS];
  extern __shared__ float w_s[];   // S weights

  float x[U];
#pragma unroll
  for (int j = 0; j < U; ++j) x[j] = u[(int64_t)min(g + j * NG, S - 1) * D + c];

  float ms = -INFINITY, ls = 0.f;
  if (tid < S) {
    ms = m[tid];
    ls = l[tid];
  }
  float M = -INFINITY;
  for (int s = tid; s < S; s += NT) {
    const float mv = s == tid ? ms : m[s];
    const float lv = s == tid ? ls : l[s];
    if (lv > 0.f) M = fmaxf(M, mv);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) red_m[wave] = M;
  __syncthreads();
  M = red_m[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, red_m[w]);

  float Lp = 0.f;
  for (int s = tid; s < S; s += NT) {
    const float mv = s == tid ? ms : m[s];
    const float lv = s == tid ? ls : l[s];
    float w = 0.f;
    if (lv > 0.f) {
      w = __expf(mv - M);
      Lp = fmaf(w, lv, Lp);
    }
    w_s[s] = w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) Lp += __shfl_xor(Lp, off);
  if (lane == 0) red_l[wave] = Lp;
  __syncthreads();
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) L += red_l[w];

  float acc = 0.f;
  for (int s0 = g;; s0 += U * NG) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int s = s0 + j * NG;
      const float w = s < S ? w_s[s] : 0.f;
      acc = fmaf(w, w > 0.f ? x[j] : 0.f, acc);
    }
    if (s0 + U * NG >= S) break;
#pragma unroll
    for (int j = 0; j < U; ++j) x[j] = u[(int64_t)min(s0 + U * NG + j * NG, S - 1) * D + c];
  }
  part[g][c - col0] = acc;
  __syncthreads();
  if (tid < DS) {
    float a = part[0][tid];
#pragma unroll
    for (int k = 1; k < NG; ++k) a += part[k][tid];
    const bool valid = L > 0.f;
    out[(int64_t)row * D + col0 + tid] = valid ? a / L : 0.f;
    if (lse && col0 == 0 && tid == 0) lse[row] = valid ? M + logf(L) : -INFINITY;
  }
}

}  // namespace da
