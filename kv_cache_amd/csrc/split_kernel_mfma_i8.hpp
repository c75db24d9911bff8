// Split kernel for the int8 K/V format with D = 128: QK^T on the matrix
// cores, PV on the vector ALUs.
//
// Format ("M8.6 - Live-Data Quantization: Activations and KV Cache",
// sections 0x06-0x06C): K codes with one fp16 scale per (128-token group,
// channel), V codes with one fp16 scale per token, and the newest min(T, R)
// tokens as bf16 rows; quantized history and residual share one softmax.
//
// A workgroup's visible ordinals [begin, end) split into an int8 part
// [begin, mid) and a residual part [mid, end) (positions grow with the
// ordinal and the residual holds the newest positions).  Both parts run the
// tile loop of split_kernel_mfma with the same running state:
//
//  * int8 part.  A per-channel K scale cannot leave the dot product (section
//    0x03B), so it is folded into q once per 128-token group:
//    q'_d = q_d * sigma_K[group, d], split into bf16 hi + lo parts (hi =
//    bf16(q'), lo = bf16(q' - hi)); the codes are exact in bf16.  Scores are
//    two MFMA chains, A = codes, B = hi and lo.  A tile whose rows span
//    several groups is scored once per group and each row keeps its own
//    group's result.  The V scale of a row multiplies that row's softmax
//    weight (section 0x03C) before PV; the denominator uses the unscaled
//    weight.
//  * residual part: exactly the bf16 kernel's tile (A = bf16 K rows, B = q).
#pragma once

#include "split_kernel_mfma.hpp"

namespace da {

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Round two floats to bf16 (nearest even) and pack them, first in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Eight int8 codes (two dwords) -> eight bf16 values (exact: |code| <= 127).
__device__ __forceinline__ uint4 codes_to_bf16(uint2 c) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = i < 2 ? c.x : c.y;
    const int sh = 16 * (i & 1);
    const float a = (float)(int32_t)((int32_t)(w << (24 - sh)) >> 24);
    const float b = (float)(int32_t)((int32_t)(w << (16 - sh)) >> 24);
    o[i] = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// 3 waves per SIMD (<= 168 VGPRs) up to 4 heads per group, 2 for 8 heads.
template <int G, int NWAVES>
__global__ __launch_bounds__(NWAVES * 64, G <= 4 ? 3 : 2) void split_kernel_mfma_i8(SplitParams p) {
  constexpr int D = 128;
  constexpr int TW = 16;
  constexpr int STEP = NWAVES * TW;
  static_assert(G >= 1 && G <= 16, "");

  const int wg = blockIdx.x;
  const int s = wg % p.num_splits;
  const int bh = wg / p.num_splits;
  const int h = bh % p.num_kv_heads;
  const int b = bh / p.num_kv_heads;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;     // K row of the tile / score column (head)
  const int kg = lane >> 4;    // channel group of the MFMA slice / V row slot

  // q rows in the B operand layout, q[head n][32c + 8kg .. +7] (zero for
  // n >= G), staged in LDS: the int8 part derives its group operands from
  // them and the residual part uses them directly.
  __shared__ uint4 q_lds[4][64];
  if (wave == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (n < G)
        x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) +
                                            ((int64_t)b * p.num_q_heads + h * G + n) * D + 32 * c + 8 * kg);
      q_lds[c][lane] = x;
    }
  }
  __syncthreads();

  const int T = request_len(p, b);
  const VisProgram vis = make_vis(T, p.mask_kind, p.n_sink, p.window);
  int begin, end;
  split_range(vis.n_vis, s, p.chunk, &begin, &end);
  const int64_t st0 = ((int64_t)b * p.num_q_heads + (int64_t)h * G) * p.num_splits + s;
  if (begin >= end) {
    write_identity<G, D, NWAVES>(p, st0);
    return;
  }
  const int n_q = T - min(T, p.residual_len);
  // first ordinal whose position is >= n_q
  const int o_res = n_q <= vis.ns ? n_q : max(vis.ns, n_q - vis.gap);
  const int mid = min(max(o_res, begin), end);

  const uint32_t row_stride = (uint32_t)(p.num_kv_heads * D);
  const int64_t code_base = ((int64_t)b * p.kv_capacity * p.num_kv_heads + h) * D;
  const int8_t* kc = static_cast<const int8_t*>(p.k) + code_base + 8 * kg;
  const int8_t* vc = static_cast<const int8_t*>(p.v) + code_base + 8 * n;
  const int64_t res_base = ((int64_t)b * p.residual_len * p.num_kv_heads + h) * D;
  const uint16_t* kr = static_cast<const uint16_t*>(p.k_resid) + res_base + 8 * kg;
  const uint16_t* vr = static_cast<const uint16_t*>(p.v_resid) + res_base + 8 * n;
  const int n_groups = (p.kv_capacity + (1 << p.k_group_shift) - 1) >> p.k_group_shift;
  const uint16_t* ks = p.k_scale + ((int64_t)b * n_groups * p.num_kv_heads + h) * D + 8 * kg;
  const uint16_t* vs = p.v_scale + (int64_t)b * p.kv_capacity * p.num_kv_heads + h;

  float m_run = -INFINITY;   // running max of head n (base 2)
  float l_run = 0.f;         // partial denominator over rows 4kg .. 4kg+3 of every tile
  float u[G][8];
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) u[i][e] = 0.f;

  // Online softmax over the 4 scores of this lane (rows 4kg+i, head n);
  // returns the weights and rescales l and u.
  auto softmax = [&](const f32x4_t& acc, int tile, int lim, float (&pr)[4]) {
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = (tile + 4 * kg + i < lim) ? acc[i] * p.qscale : -INFINITY;
    float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m_run, mt);
    const float mz = mn == -INFINITY ? 0.f : mn;
    const float alpha = fast_exp2(m_run - mz);
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(sc[i] - mz);
    l_run = fmaf(l_run, alpha, (pr[0] + pr[1]) + (pr[2] + pr[3]));
    m_run = mn;
    HeadLoop<G>::rescale(u, alpha);
  };

  // ================= int8 part: ordinals [begin, mid) =================
  if (begin < mid) {
    auto pos = [&](int o) { return vis_pos(vis, min(o, mid - 1)); };
    auto group_of = [&](int o) { return pos(o) >> p.k_group_shift; };
    // B operand (hi, lo) of q' = q * sigma_K[group], kept per wave in LDS,
    // and the group it holds
    __shared__ uint4 b_lds[NWAVES][2][4][64];
    int cur_group = -1;
    auto load_sigma = [&](int grp, uint4 (&sg)[4]) {
      const uint16_t* row = ks + (int64_t)grp * row_stride;
#pragma unroll
      for (int c = 0; c < 4; ++c) sg[c] = *reinterpret_cast<const uint4*>(row + 32 * c);
    };
    auto make_b = [&](const uint4 (&sg)[4]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 qv = q_lds[c][lane];
        const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
        const uint32_t sw[4] = {sg[c].x, sg[c].y, sg[c].z, sg[c].w};
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float q0 = bf16_lo(qw[e]) * f16_bits_to_f32(sw[e] & 0xffffu);
          const float q1 = bf16_hi(qw[e]) * f16_bits_to_f32(sw[e] >> 16);
          hw[e] = pack_bf16(q0, q1);
          lw[e] = pack_bf16(q0 - bf16_lo(hw[e]), q1 - bf16_hi(hw[e]));
        }
        b_lds[wave][0][c][lane] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        b_lds[wave][1][c][lane] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      }
    };
    auto score = [&](const uint2 (&k)[4]) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, codes_to_bf16(k[c]));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, b_lds[wave][0][c][lane]),
                                                      acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, b_lds[wave][1][c][lane]),
                                                      acc, 0, 0, 0);
      }
      return acc;
    };
    auto issue_k = [&](int tile, uint2 (&k)[4]) {
      const int8_t* row = kc + (uint64_t)(uint32_t)pos(tile + n) * row_stride;
#pragma unroll
      for (int c = 0; c < 4; ++c) k[c] = stream_load(reinterpret_cast<const uint2*>(row + 32 * c));
    };
    auto issue_v = [&](int tile, uint2 (&v)[4], uint32_t (&sv)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t t = (uint32_t)pos(tile + 4 * kg + j);
        v[j] = stream_load(reinterpret_cast<const uint2*>(vc + (uint64_t)t * row_stride));
        sv[j] = vs[(int64_t)t * p.num_kv_heads];
      }
    };

    uint2 kt[4], vt[4];
    uint32_t svt[4];
    uint4 sig[4];
    int sig_group = -1;
    int tile = begin + wave * TW;
    if (tile < mid) {
      issue_k(tile, kt);
      issue_v(tile, vt, svt);
      sig_group = group_of(tile);
      load_sigma(sig_group, sig);
    }
    for (; tile < mid; tile += STEP) {
      const int next_tile = tile + STEP;
      const int g0 = group_of(tile), g1 = group_of(tile + TW - 1);
      f32x4_t acc;
      if (g0 == g1) {
        if (g0 != cur_group) {
          if (g0 != sig_group) { sig_group = g0; load_sigma(g0, sig); }
          make_b(sig);
          cur_group = g0;
        }
        acc = score(kt);
      } else {
        // rows of several 128-token groups: score once per group
        int rg[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) rg[i] = group_of(tile + 4 * kg + i);
        const int my = group_of(tile + n);
        acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        int grp = g0;
        while (true) {
          if (grp != cur_group) {
            if (grp != sig_group) { sig_group = grp; load_sigma(grp, sig); }
            make_b(sig);
            cur_group = grp;
          }
          const f32x4_t a = score(kt);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = rg[i] == grp ? a[i] : acc[i];
          if (grp == g1) break;
          int cand = my > grp ? my : 0x7fffffff;     // smallest group above grp in the tile
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) cand = min(cand, __shfl_xor(cand, off));
          grp = cand;
        }
      }
      issue_k(next_tile, kt);
      const int ng = group_of(next_tile);
      if (next_tile < mid && ng != cur_group && ng != sig_group) {   // prefetch the next group's scales
        sig_group = ng;
        load_sigma(ng, sig);
      }
      float pr[4];
      softmax(acc, tile, mid, pr);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float vx[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vx[e] = i8_at(e < 4 ? vt[j].x : vt[j].y, e & 3);
        HeadLoop<G>::accumulate(u, pr[j] * f16_bits_to_f32(svt[j]), vx);
      }
      issue_v(next_tile, vt, svt);
    }
  }

  // ============ residual part: ordinals [mid, end), bf16 rows ============
  if (mid < end) {
    auto rrow = [&](int o) { return (uint32_t)(vis_pos(vis, min(o, end - 1)) - n_q); };
    auto issue_k = [&](int tile, uint4 (&k)[4]) {
      const uint16_t* row = kr + (uint64_t)rrow(tile + n) * row_stride;
#pragma unroll
      for (int c = 0; c < 4; ++c) k[c] = stream_load(reinterpret_cast<const uint4*>(row + 32 * c));
    };
    auto issue_v = [&](int tile, uint4 (&v)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = stream_load(reinterpret_cast<const uint4*>(vr + (uint64_t)rrow(tile + 4 * kg + j) * row_stride));
    };
    MfmaTile t;
    int tile = mid + wave * TW;
    if (tile < end) {
      issue_k(tile, t.k);
      issue_v(tile, t.v);
    }
    for (; tile < end; tile += STEP) {
      const int next_tile = tile + STEP;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, t.k[c]),
                                                      __builtin_bit_cast(bf16x8_t, q_lds[c][lane]), acc, 0, 0, 0);
      issue_k(next_tile, t.k);
      float pr[4];
      softmax(acc, tile, end, pr);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w[4] = {t.v[j].x, t.v[j].y, t.v[j].z, t.v[j].w};
        float vx[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) { vx[2 * e] = bf16_lo(w[e]); vx[2 * e + 1] = bf16_hi(w[e]); }
        HeadLoop<G>::accumulate(u, pr[j], vx);
      }
      issue_v(next_tile, t.v);
    }
  }

  // ---- wave state: all rows of a head share m, so l and u just add ---------
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u[i][e] += __shfl_xor(u[i][e], 16);
      u[i][e] += __shfl_xor(u[i][e], 32);
    }
  __shared__ WaveStates<G, D, NWAVES> sh;
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
  merge_waves_and_store<G, D, NWAVES>(p, st0, sh);
}

}  // namespace da
