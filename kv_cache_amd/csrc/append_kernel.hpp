// Streaming append for the int8 K/V format under the group-closing residual
// policy ("M8.6 - Live-Data Quantization: Activations and KV Cache",
// sections 0x05B, 0x06B): the new token's bf16 K and V rows enter the
// residual; when the residual already holds R rows (R == G), those G rows are
// closed first -- K quantized per channel over the G rows into one new scale
// group, V quantized per row -- and the new row takes residual slot 0.
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
  int32_t group;           // G == R
  int32_t n_groups;        // ceil(T_cap / G)
};

constexpr int kAppendThreads = 256;

__device__ __forceinline__ float bf16_value(uint16_t bits) { return __uint_as_float((uint32_t)bits << 16); }

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

template <int D>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendParams p) {
  static_assert(D % 64 == 0 && D <= kAppendThreads, "");
  constexpr int CPL = D / 64;                      // channels per lane in the V row pass
  constexpr int NW = kAppendThreads / 64;
  const int H = p.num_kv_heads;
  const int b = blockIdx.x / H;
  const int h = blockIdx.x - b * H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.group;
  const int T = p.seq_lens[b];
  if (T < 0 || T >= p.max_seq_len) {
    if (tid == 0 && p.status) atomicOr(p.status + b, (int)DA_APPEND_NO_ROOM);
    return;
  }
  const int n_q = T > G ? (T - G + G - 1) / G * G : 0;  // closed rows (R == G)
  const int r = T - n_q;                                  // residual rows, 0 .. G
  const int64_t row_stride = (int64_t)H * D;
  uint16_t* kres = p.k_resid + ((int64_t)b * G * H + h) * D;
  uint16_t* vres = p.v_resid + ((int64_t)b * G * H + h) * D;
  int slot = r;

  if (r == G) {
    __shared__ uint16_t ks[D];
    __shared__ uint16_t vs[kAppendThreads];              // G <= 256 rows
    bool ok = true;
    // K: thread c owns channel c over the G rows
    if (tid < D) {
      float amax = 0.f;
      for (int i = 0; i < G; ++i) {
        const float x = bf16_value(kres[i * row_stride + tid]);
        ok = ok && __builtin_isfinite(x);
        amax = fmaxf(amax, fabsf(x));
      }
      ks[tid] = stored_scale(amax, ok);
    }
    // V: wave w owns rows w, w + NW, ...; lane holds CPL channels of the row
    for (int i = wave; i < G; i += NW) {
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const float x = bf16_value(vres[i * row_stride + lane + 64 * j]);
        ok = ok && __builtin_isfinite(x);
        amax = fmaxf(amax, fabsf(x));
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
      bool row_ok = true;
      const uint16_t s = stored_scale(amax, row_ok);
      ok = ok && row_ok;
      if (lane == 0) vs[i] = s;
    }
    if (!__syncthreads_and(ok)) {
      if (tid == 0 && p.status) atomicOr(p.status + b, (int)DA_APPEND_BAD_SCALE);
      return;
    }
    // codes of the closed rows, then their scales
    int8_t* kc = p.k + ((int64_t)b * p.kv_capacity + n_q) * row_stride + (int64_t)h * D;
    int8_t* vc = p.v + ((int64_t)b * p.kv_capacity + n_q) * row_stride + (int64_t)h * D;
    if (tid < D) {
      const uint16_t s = ks[tid];
      for (int i = 0; i < G; ++i) kc[i * row_stride + tid] = code_of(bf16_value(kres[i * row_stride + tid]), s);
      p.k_scale[(((int64_t)b * p.n_groups + n_q / G) * H + h) * D + tid] = s;
    }
    for (int i = wave; i < G; i += NW) {
      const uint16_t s = vs[i];
#pragma unroll
      for (int j = 0; j < CPL; ++j)
        vc[i * row_stride + lane + 64 * j] = code_of(bf16_value(vres[i * row_stride + lane + 64 * j]), s);
      if (lane == 0) p.v_scale[((int64_t)b * p.kv_capacity + n_q + i) * H + h] = s;
    }
    __syncthreads();      // every read of residual row 0 precedes its overwrite
    slot = 0;
  }
  if (tid < D) {
    kres[slot * row_stride + tid] = p.k_new[((int64_t)b * H + h) * D + tid];
    vres[slot * row_stride + tid] = p.v_new[((int64_t)b * H + h) * D + tid];
  }
}

}  // namespace da
