// Pieces shared by the split kernels and the index trace kernel: streaming
// loads, the empty-split identity, the cross-wave merge of partial states and
// their store into the workspace, and the trace walk.
#pragma once

#include "device_common.hpp"

namespace da {

// K/V rows are read exactly once per call: the loads carry the non-temporal
// hint so they do not displace lines that are reused (q, block table, scales).
#ifndef DA_NT_LOADS
#define DA_NT_LOADS 1
#endif
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 stream_load(const uint4* p) {
#if DA_NT_LOADS
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *p;
#endif
}

__device__ __forceinline__ uint2 stream_load(const uint2* p) {
#if DA_NT_LOADS
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
#else
  return *p;
#endif
}

// The empty identity (m = -inf, l = 0, u = 0) for the G query heads of an
// empty split ("M4.5 - Decode Attention Kernels, Mask Programs, and Backend
// Boundaries", section 0x02C): every slot the reducer reads is defined
// (section 0x03G).
template <int G, int D, int NWAVES>
__device__ __forceinline__ void write_identity(const SplitParams& p, int64_t st0) {
  for (int idx = threadIdx.x; idx < G * D; idx += NWAVES * 64) {
    const int i = idx / D, c = idx % D;
    p.ws_u[(st0 + (int64_t)i * p.num_splits) * D + c] = 0.f;
  }
  if (threadIdx.x < G) {
    p.ws_m[st0 + (int64_t)threadIdx.x * p.num_splits] = -INFINITY;
    p.ws_l[st0 + (int64_t)threadIdx.x * p.num_splits] = 0.f;
  }
}

// One partial state per (wave, query head); m in base-2 units.
template <int G, int D, int NWAVES>
struct WaveStates {
  float u[NWAVES][G][D];
  float m[NWAVES][G];
  float l[NWAVES][G];
};

// Merge the NWAVES wave states of each head (binary merge of section 0x02B
// folded over the waves, with the empty branch taken by weight 0) and store
// (m, l, u) of the split; m is converted to natural-log units.
template <int G, int D, int NWAVES>
__device__ __forceinline__ void merge_waves_and_store(const SplitParams& p, int64_t st0,
                                                      const WaveStates<G, D, NWAVES>& sh) {
  constexpr float kLn2 = 0.69314718055994530942f;
  for (int idx = threadIdx.x; idx < G * D; idx += NWAVES * 64) {
    const int i = idx / D, c = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) M = fmaxf(M, sh.m[w][i]);
    const float Mz = M == -INFINITY ? 0.f : M;
    float acc = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) {
      const float f = fast_exp2(sh.m[w][i] - Mz);
      acc = fmaf(f, sh.u[w][i][c], acc);
      L = fmaf(f, sh.l[w][i], L);
    }
    const int64_t st = st0 + (int64_t)i * p.num_splits;
    p.ws_u[st * D + c] = acc;
    if (c == 0) {
      p.ws_m[st] = M == -INFINITY ? -INFINITY : M * kLn2;
      p.ws_l[st] = L;
    }
  }
}

// Index trace: the workgroup decomposition, tile walk (TW rows per wave tile,
// tiles dealt round-robin to NWAVES waves) and address code of the split
// kernels, recording each row instead of consuming it.
template <bool I8, int D, bool PAGED, int NWAVES, int TW>
__global__ __launch_bounds__(NWAVES * 64) void trace_kernel(SplitParams p, int64_t* offsets,
                                                            int32_t* positions) {
  const int wg = blockIdx.x;
  const int s = wg % p.num_splits;
  const int bh = wg / p.num_splits;
  const int h = bh % p.num_kv_heads;
  const int b = bh / p.num_kv_heads;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int T = request_len(p, b);
  const VisProgram vis = make_vis(T, p.mask_kind, p.n_sink, p.window);
  int begin, end;
  split_range(vis.n_vis, s, p.chunk, &begin, &end);
  const int n_q = I8 ? T - min(T, p.residual_len) : T;
  const int64_t base = (int64_t)wg * p.chunk;
  for (int tile = begin + wave * TW; tile < end; tile += NWAVES * TW) {
    for (int j = lane; j < TW; j += 64) {
      const int o = tile + j;
      if (o < end) {
        const int t = vis_pos(vis, o);
        int64_t off;
        if (I8)
          off = t < n_q ? kv_row_offset<false>(p, b, t, h, D) : resid_row_offset(p, b, t - n_q, h, D);
        else
          off = kv_row_offset<PAGED>(p, b, t, h, D);
        offsets[base + (o - begin)] = off;
        positions[base + (o - begin)] = t;
      }
    }
  }
}

}  // namespace da
