// Split (partial-attention) kernel of the Flash-Decoding schedule.
//
// Workgroup (b, h_kv, s) owns the ordinals [begin, end) of request b's
// visible rows (device_common.hpp) and the G = H_q/H_kv query heads that share
// K/V head h_kv, so each K/V byte of the split is read once for the whole GQA
// group ("M4.5 - Decode Attention Kernels, Mask Programs, and Backend
// Boundaries", sections 0x03A and 0x03F: unique payload versus per-query-head
// demand).  It writes one exact partial state per query head (section 0x02A):
//   m = max score, l = sum e^(s - m), u = sum e^(s - m) v   (u not normalized)
// or the empty identity (m = -inf, l = 0, u = 0) when it owns no row (0x02C).
//
// Data mapping (64-wide wavefronts).  A K or V row of D elements is LPR lanes
// x 16 bytes; a wave covers RPW = 64/LPR rows per load instruction ("row
// slots").  Lane (slot r, column group c) holds elements [c*EPL, c*EPL+EPL)
// of its slot's rows.  Each slot keeps its own online-softmax state over the
// rows it sees (ordinals tile + j*RPW + r, j < U, for successive tiles of
// RPW*U rows, tiles dealt round-robin to the waves); scores are completed by a
// DPP butterfly over the slot's LPR lanes, so no LDS is touched in the loop.
// The next tile's rows are loaded before the current tile is consumed.  At
// the end the RPW slot states of a wave and then the wave states of the
// workgroup are merged with the binary merge of section 0x02B.  Scores are
// kept in base 2 (q pre-multiplied by scale*log2 e) and converted back to
// natural-log units when m is stored.
#pragma once

#include "split_common.hpp"

namespace da {

template <int FMT> struct KvTraits;
template <> struct KvTraits<DA_KV_F32> { static constexpr int EPL = 4; };
template <> struct KvTraits<DA_KV_BF16> { static constexpr int EPL = 8; };
template <> struct KvTraits<DA_KV_I8> { static constexpr int EPL = 8; };

// Raw (still encoded) data of one K or V row slice held by one lane.
struct RawRow {
  uint4 k;        // f32: 4 floats; bf16: 8 bf16; int8 codes: .x,.y = 8 codes; residual: 8 bf16
  uint4 v;
  uint4 ks;       // int8: 8 fp16 channel scales of the token's K group
  uint32_t vs;    // int8: fp16 token scale of V
  int region;     // 0 main / int8 codes, 1 bf16 residual
  bool valid;
};

// Loads this lane's slice of the K and V rows of visible ordinal o (position
// t).  kInstrRows: lane `rec` also records the row loads (trace instances only).
template <int FMT, int D, bool PAGED, int INSTR>
__device__ __forceinline__ void load_row(const SplitParams& p, const RowAddr& ra, int b, int h, int o, int t,
                                         int n_q, int col0, bool rec, RawRow& raw) {
  constexpr int EB = FMT == DA_KV_F32 ? 4 : FMT == DA_KV_BF16 ? 2 : 1;
  if (FMT != DA_KV_I8) {
    const int64_t off = kv_row_offset<PAGED>(p, ra, t) + col0;
    raw.k = stream_load(reinterpret_cast<const uint4*>(static_cast<const char*>(p.k) + off * EB));
    raw.v = stream_load(reinterpret_cast<const uint4*>(static_cast<const char*>(p.v) + off * EB));
    raw.region = 0;
    if (INSTR == kInstrRows && rec) {
      trace_k(p, b, h, o, t, off - col0);
      trace_v(p, b, h, o, off - col0);
    }
  } else {
    if (t < n_q) {
      const int64_t off = kv_row_offset<false>(p, ra, t) + col0;
      const uint2 kc = stream_load(reinterpret_cast<const uint2*>(static_cast<const int8_t*>(p.k) + off));
      const uint2 vc = stream_load(reinterpret_cast<const uint2*>(static_cast<const int8_t*>(p.v) + off));
      raw.k = make_uint4(kc.x, kc.y, 0u, 0u);
      raw.v = make_uint4(vc.x, vc.y, 0u, 0u);
      const int grp = t >> p.k_group_shift;
      const int64_t soff = (((int64_t)b * ((p.kv_capacity + (1 << p.k_group_shift) - 1) >> p.k_group_shift) + grp)
                                * p.num_kv_heads + h) * (int64_t)D + col0;
      const int64_t vsoff = ((int64_t)b * p.kv_capacity + t) * p.num_kv_heads + h;
      raw.ks = *reinterpret_cast<const uint4*>(p.k_scale + soff);
      raw.vs = p.v_scale[vsoff];
      raw.region = 0;
      if (INSTR == kInstrRows && rec) {
        trace_k(p, b, h, o, t, off - col0, soff - col0);
        trace_v(p, b, h, o, off - col0, vsoff);
      }
    } else {
      const int64_t off = resid_row_offset(p, b, t - n_q, h, D) + col0;
      raw.k = stream_load(reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.k_resid) + off));
      raw.v = stream_load(reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.v_resid) + off));
      raw.region = 1;
      if (INSTR == kInstrRows && rec) {
        trace_k(p, b, h, o, t, off - col0);
        trace_v(p, b, h, o, off - col0);
      }
    }
  }
}

// Decode one lane's EPL elements of a row to fp32.
template <int FMT>
__device__ __forceinline__ void decode_k(const RawRow& raw, float* x) {
  if (FMT == DA_KV_F32) {
    x[0] = __uint_as_float(raw.k.x); x[1] = __uint_as_float(raw.k.y);
    x[2] = __uint_as_float(raw.k.z); x[3] = __uint_as_float(raw.k.w);
  } else if (FMT == DA_KV_BF16 || raw.region == 1) {
    const uint32_t w[4] = {raw.k.x, raw.k.y, raw.k.z, raw.k.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[2 * i] = bf16_lo(w[i]); x[2 * i + 1] = bf16_hi(w[i]); }
  } else {
    const uint32_t sc[4] = {raw.ks.x, raw.ks.y, raw.ks.z, raw.ks.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float code = i8_at(e < 4 ? raw.k.x : raw.k.y, e & 3);
      const float s = f16_bits_to_f32((sc[e >> 1] >> (16 * (e & 1))) & 0xffffu);
      x[e] = code * s;
    }
  }
}

// V elements; for int8 the per-token scale is returned separately so that it
// is folded into the softmax weight ("M8.6 - Live-Data Quantization:
// Activations and KV Cache", section 0x03C).
template <int FMT>
__device__ __forceinline__ float decode_v(const RawRow& raw, float* x) {
  if (FMT == DA_KV_F32) {
    x[0] = __uint_as_float(raw.v.x); x[1] = __uint_as_float(raw.v.y);
    x[2] = __uint_as_float(raw.v.z); x[3] = __uint_as_float(raw.v.w);
    return 1.f;
  } else if (FMT == DA_KV_BF16 || raw.region == 1) {
    const uint32_t w[4] = {raw.v.x, raw.v.y, raw.v.z, raw.v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[2 * i] = bf16_lo(w[i]); x[2 * i + 1] = bf16_hi(w[i]); }
    return 1.f;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = i8_at(e < 4 ? raw.v.x : raw.v.y, e & 3);
    return f16_bits_to_f32(raw.vs);
  }
}

// INSTR: kInstrRows is the index-trace instance, which also records each row
// load where it is issued; otherwise identical (no timestamp instance).
template <int FMT, int D, int G, bool PAGED, int NWAVES, int U, bool FUSED, int INSTR = 0>
__global__ __launch_bounds__(NWAVES * 64) void split_kernel(SplitParams p) {
  constexpr int EPL = KvTraits<FMT>::EPL;
  constexpr int LPR = D / EPL;           // lanes per row
  constexpr int RPW = 64 / LPR;          // rows per wave load
  constexpr int TW = RPW * U;            // rows per wave tile
  static_assert(LPR >= 4 && LPR <= 64 && (64 % LPR) == 0, "row must span 4..64 lanes");

  int b, h, s;
  const PartitionHeaderAtExit header_at_exit{p};
  decode_workgroup(p, &b, &h, &s);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane / LPR;              // row slot
  const int cg = lane % LPR;             // column group
  const int col0 = cg * EPL;

  const int T = request_len(p, b);
  const VisProgram vis = make_vis(T, p.mask_kind, p.n_sink, p.window);
  const int n_q = FMT == DA_KV_I8 ? quantized_len(p, T) : T;
  int begin, end;
  if (FMT == DA_KV_I8)
    split_range_weighted(vis.n_vis, residual_ordinal(vis, n_q), s, p.chunk, &begin, &end);
  else
    split_range(vis.n_vis, s, p.chunk, &begin, &end);

  if (begin >= end) {   // empty split: the identity state, written before any arithmetic
    write_identity<G, D, NWAVES, FUSED>(p, b, h, s);
    finish_split<G, D, NWAVES, FUSED>(p, b, h);
    return;
  }

  // q rows of the G heads, this lane's columns, pre-scaled into base 2.
  float qf[G][EPL];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int64_t qoff = out_row(p, b, h, i) * D + col0;
    if (FMT == DA_KV_F32) {
      const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(p.q) + qoff);
      qf[i][0] = x.x * p.qscale; qf[i][1] = x.y * p.qscale;
      qf[i][2] = x.z * p.qscale; qf[i][3] = x.w * p.qscale;
    } else {
      const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + qoff);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[i][2 * e] = bf16_lo(w[e]) * p.qscale;
        qf[i][2 * e + 1] = bf16_hi(w[e]) * p.qscale;
      }
    }
  }

  int lim[G];
#pragma unroll
  for (int i = 0; i < G; ++i) lim[i] = row_limit(p, vis.n_vis, i);

  float m[G], l[G], u[G][EPL];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) u[i][e] = 0.f;
  }

  const RowAddr ra = row_addr<PAGED>(p, b, h, D);
  RawRow nxt[U];
  auto issue = [&](int tile, RawRow* rr) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int o = tile + j * RPW + r;
      rr[j].valid = o < end;
      rr[j].k = make_uint4(0u, 0u, 0u, 0u);
      rr[j].v = make_uint4(0u, 0u, 0u, 0u);
      rr[j].ks = make_uint4(0u, 0u, 0u, 0u);
      rr[j].vs = 0u;
      rr[j].region = 0;
      if (rr[j].valid) load_row<FMT, D, PAGED, INSTR>(p, ra, b, h, o, vis_pos(vis, o), n_q, col0, cg == 0, rr[j]);
    }
  };

  int tile = begin + wave * TW;
  if (tile < end) issue(tile, nxt);
  for (; tile < end; tile += NWAVES * TW) {
    RawRow cur[U];
#pragma unroll
    for (int j = 0; j < U; ++j) cur[j] = nxt[j];
    const int next_tile = tile + NWAVES * TW;
    if (next_tile < end) issue(next_tile, nxt);

    float sc[U][G];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      float kx[EPL];
      decode_k<FMT>(cur[j], kx);
#pragma unroll
      for (int i = 0; i < G; ++i) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) part = fmaf(qf[i][e], kx[e], part);
        part = group_sum<LPR>(part);
        // virtual head i sees ordinals below its own limit (C > 1 rows)
        sc[j][i] = (cur[j].valid && tile + j * RPW + r < lim[i]) ? part : -INFINITY;
      }
    }
    float pw[U][G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float mt = sc[0][i];
#pragma unroll
      for (int j = 1; j < U; ++j) mt = fmaxf(mt, sc[j][i]);
      const float mn = fmaxf(m[i], mt);
      const float mz = mn == -INFINITY ? 0.f : mn;    // no -inf - -inf
      const float alpha = fast_exp2(m[i] - mz);
      l[i] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) u[i][e] *= alpha;
#pragma unroll
      for (int j = 0; j < U; ++j) {
        pw[j][i] = fast_exp2(sc[j][i] - mz);
        l[i] += pw[j][i];
      }
      m[i] = mn;
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      float vx[EPL];
      const float vscale = decode_v<FMT>(cur[j], vx);
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float pv = pw[j][i] * vscale;
#pragma unroll
        for (int e = 0; e < EPL; ++e) u[i][e] = fmaf(pv, vx[e], u[i][e]);
      }
    }
  }

  // ---- merge the RPW slot states of this wave (binary merge, 0x02B) -------
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float mo = __shfl_xor(m[i], off);
      const float lo = __shfl_xor(l[i], off);
      const float mn = fmaxf(m[i], mo);
      const float mz = mn == -INFINITY ? 0.f : mn;
      const float a = fast_exp2(m[i] - mz);
      const float c = fast_exp2(mo - mz);
      l[i] = a * l[i] + c * lo;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float uo = __shfl_xor(u[i][e], off);
        u[i][e] = a * u[i][e] + c * uo;
      }
      m[i] = mn;
    }
  }

  // ---- merge the wave states through LDS and store ------------------------
  __shared__ WaveStates<G, D, NWAVES> sh;
  if (r == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sh.u[wave][i][col0 + e] = u[i][e];
    }
    if (cg == 0) {
#pragma unroll
      for (int i = 0; i < G; ++i) { sh.m[wave][i] = m[i]; sh.l[wave][i] = l[i]; }
    }
  }
  __syncthreads();
  merge_waves_and_store<G, D, NWAVES, FUSED>(p, b, h, s, sh);
  finish_split<G, D, NWAVES, FUSED>(p, b, h);
}

}  // namespace da
