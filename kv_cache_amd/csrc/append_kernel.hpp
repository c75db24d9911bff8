// Streaming append for the int8 K/V format under the group-closing residual
// policy ("M8.6 - Live-Data Quantization: Activations and KV Cache",
// sections 0x05B, 0x06B): the new token's bf16 K and V rows enter the
// residual; when the residual already holds R rows (G <= R), its oldest G
// rows are closed first -- K quantized per channel over the G rows into one
// new scale group, V quantized per row -- the other R - G rows move down by G
// (residual row i holds token n_q + i), and the new row takes slot R - G.
// Quantizer rule (section 0x02A): scale = fp16(amax / 127) re-read as the
// effective scale (1 for an all-zero vector), code = clip(rint(x / scale),
// -127, 127) with ties to even; a non-finite input or a non-finite or
// subnormal stored scale fails the closure.  A failed closure writes nothing
// for that (b, h_kv) and sets DA_APPEND_BAD_SCALE in status[b] (section
// 0x00C: a failed quantizer must not expose half an append).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_attn.h"

namespace da {

struct AppendParams {
  const uint16_t* k_new;   // [B, H, D] bf16
  const uint16_t* v_new;
  int8_t* k;               // [B, T_cap, H, D] codes
  int8_t* v;
  uint16_t* k_scale;       // [B, n_groups, H, D] fp16
  uint16_t* v_scale;       // [B, T_cap, H] fp16
  uint16_t* k_resid;       // [B, R, H, D] bf16
  uint16_t* v_resid;
  const int32_t* seq_lens; // [B], lengths before the append
  int32_t* status;         // [B] or null
  int32_t num_kv_heads;
  int32_t kv_capacity;
  int32_t max_seq_len;
  int32_t group;           // G
  int32_t resid_len;       // R >= G
  int32_t n_groups;        // ceil(T_cap / G)
};

constexpr int kAppendThreads = 256;

__device__ __forceinline__ float bf16_value(uint16_t bits) { return __uint_as_float((uint32_t)bits << 16); }
// the two bf16 values packed in a 32-bit word (element 2j in the low half)
__device__ __forceinline__ float bf16_word_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_word_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Stored fp16 scale of a vector with largest magnitude amax; clears ok when it
// is not a finite normal fp16 value.
__device__ __forceinline__ uint16_t stored_scale(float amax, bool& ok) {
  if (amax == 0.f) return 0x3C00u;                        // 1.0
  const _Float16 s = (_Float16)(amax / 127.0f);            // fp32 quotient, then nearest-even fp16
  const float sf = (float)s;
  ok = ok && __builtin_isfinite(sf) && sf >= 6.103515625e-05f;   // 2^-14: smallest normal fp16
  return __builtin_bit_cast(uint16_t, s);
}

__device__ __forceinline__ int8_t code_of(float x, uint16_t scale_bits) {
  const double s = (double)(float)__builtin_bit_cast(_Float16, scale_bits);
  const double q = __builtin_rint((double)x / s);
  return (int8_t)fmin(fmax(q, -127.0), 127.0);
}

// MR: sweeps of the closure layout the instance holds, at least G / RS.
template <int D, int MR>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendParams p) {
  static_assert(D % 64 == 0 && D <= kAppendThreads, "");
  // Closure layout: thread t holds the 16-byte channel group cg = t % CG of
  // rows t / CG, t / CG + RS, ... of the G closed rows (K and V), loaded once
  // and all at the start; K scales reduce over the threads of one channel
  // group, V scales over the CG consecutive lanes of one row.
  constexpr int CG = D / 8;                       // channel groups per row
  constexpr int RS = kAppendThreads / CG;         // rows per sweep of all threads
  const int H = p.num_kv_heads;
  const int b = blockIdx.x / H;
  const int h = blockIdx.x - b * H;
  const int tid = threadIdx.x;
  const int G = p.group;
  const int R = p.resid_len;
  const int T = p.seq_lens[b];
  if (T < 0 || T >= p.max_seq_len) {
    if (tid == 0 && p.status) atomicOr(p.status + b, (int)DA_APPEND_NO_ROOM);
    return;
  }
  const int n_q = T > R ? (T - R + G - 1) / G * G : 0;  // closed rows
  const int r = T - n_q;                                  // residual rows, 0 .. R
  const int64_t row_stride = (int64_t)H * D;
  uint16_t* kres = p.k_resid + ((int64_t)b * R * H + h) * D;
  uint16_t* vres = p.v_resid + ((int64_t)b * R * H + h) * D;
  int slot = r;

  if (r == R) {
    __shared__ uint32_t kmax[D];                 // per-channel amax bits (non-negative floats order as integers)
    __shared__ uint16_t ks[D];
    const int cg = tid % CG, r0 = tid / CG;
    if (tid < D) kmax[tid] = 0u;
    uint4 kx[MR], vx[MR];
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      const int row = r0 + i * RS;
      kx[i] = vx[i] = make_uint4(0u, 0u, 0u, 0u);
      if (row < G) {
        kx[i] = *reinterpret_cast<const uint4*>(kres + row * row_stride + 8 * cg);
        vx[i] = *reinterpret_cast<const uint4*>(vres + row * row_stride + 8 * cg);
      }
    }
    auto elem = [](const uint4& w, int j) { return j < 2 ? (j == 0 ? w.x : w.y) : (j == 2 ? w.z : w.w); };
    bool ok = true;
    // K: partial amax of my 8 channels over my rows, folded into kmax
    float kam[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) kam[e] = 0.f;
#pragma unroll
    for (int i = 0; i < MR; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = elem(kx[i], e >> 1);
        const float x = (e & 1) ? bf16_word_hi(w) : bf16_word_lo(w);
        ok = ok && __builtin_isfinite(x);
        kam[e] = fmaxf(kam[e], fabsf(x));
      }
    }
    __syncthreads();                             // kmax cleared
#pragma unroll
    for (int e = 0; e < 8; ++e) atomicMax(&kmax[8 * cg + e], __float_as_uint(kam[e]));
    // V: amax of each of my rows over the row's CG lanes, then its scale
    uint16_t vsc[MR];
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = elem(vx[i], e >> 1);
        const float x = (e & 1) ? bf16_word_hi(w) : bf16_word_lo(w);
        ok = ok && __builtin_isfinite(x);
        a = fmaxf(a, fabsf(x));
      }
#pragma unroll
      for (int off = 1; off < CG; off <<= 1) a = fmaxf(a, __shfl_xor(a, off));
      bool row_ok = true;
      vsc[i] = stored_scale(a, row_ok);
      if (r0 + i * RS < G) ok = ok && row_ok;
    }
    __syncthreads();                             // kmax complete
    if (tid < D) ks[tid] = stored_scale(__uint_as_float(kmax[tid]), ok);
    if (!__syncthreads_and(ok)) {
      if (tid == 0 && p.status) atomicOr(p.status + b, (int)DA_APPEND_BAD_SCALE);
      return;
    }
    // codes of the closed rows from the registers, then the scales
    int8_t* kc = p.k + ((int64_t)b * p.kv_capacity + n_q) * row_stride + (int64_t)h * D;
    int8_t* vc = p.v + ((int64_t)b * p.kv_capacity + n_q) * row_stride + (int64_t)h * D;
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      const int row = r0 + i * RS;
      if (row >= G) continue;
      uint32_t kw[2] = {0u, 0u}, vw[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = elem(kx[i], e >> 1), u = elem(vx[i], e >> 1);
        const float xk = (e & 1) ? bf16_word_hi(w) : bf16_word_lo(w);
        const float xv = (e & 1) ? bf16_word_hi(u) : bf16_word_lo(u);
        kw[e >> 2] |= (uint32_t)(uint8_t)code_of(xk, ks[8 * cg + e]) << (8 * (e & 3));
        vw[e >> 2] |= (uint32_t)(uint8_t)code_of(xv, vsc[i]) << (8 * (e & 3));
      }
      *reinterpret_cast<uint2*>(kc + row * row_stride + 8 * cg) = make_uint2(kw[0], kw[1]);
      *reinterpret_cast<uint2*>(vc + row * row_stride + 8 * cg) = make_uint2(vw[0], vw[1]);
      if (cg == 0) p.v_scale[((int64_t)b * p.kv_capacity + n_q + row) * H + h] = vsc[i];
    }
    if (tid < D) p.k_scale[(((int64_t)b * p.n_groups + n_q / G) * H + h) * D + tid] = ks[tid];
    __syncthreads();      // every read of the closed rows precedes their overwrite
    // rows G .. R-1 move to 0 .. R-G-1, RS rows per pass in ascending order: a
    // pass writes rows below every row a later pass reads, and its barrier
    // keeps its writes after every thread's reads of the previous pass
    for (int base = 0; base < R - G; base += RS) {
      const int row = base + r0;
      uint4 kw4 = make_uint4(0u, 0u, 0u, 0u), vw4 = kw4;
      if (row < R - G) {
        kw4 = *reinterpret_cast<const uint4*>(kres + (row + G) * row_stride + 8 * cg);
        vw4 = *reinterpret_cast<const uint4*>(vres + (row + G) * row_stride + 8 * cg);
      }
      __syncthreads();
      if (row < R - G) {
        *reinterpret_cast<uint4*>(kres + row * row_stride + 8 * cg) = kw4;
        *reinterpret_cast<uint4*>(vres + row * row_stride + 8 * cg) = vw4;
      }
    }
    __syncthreads();      // every read of residual row R - G precedes its overwrite
    slot = R - G;
  }
  if (tid < D) {
    kres[slot * row_stride + tid] = p.k_new[((int64_t)b * H + h) * D + tid];
    vres[slot * row_stride + tid] = p.v_new[((int64_t)b * H + h) * D + tid];
  }
}

}  // namespace da
