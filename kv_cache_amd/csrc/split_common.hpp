// Pieces shared by the split kernels: streaming loads, the empty-split
// identity, the cross-wave merge of partial states and their store into the
// workspace, and the single-launch fold.
#pragma once

#include "device_common.hpp"

namespace da {

// K/V rows are read exactly once per call.  Loads whose lanes cover whole
// 128-byte lines carry the non-temporal hint (they stream past the caches);
// loads that take half lines (a tile's 16 rows at 64 bytes each, the other
// half following in the next instruction) are plain, so the second half
// finds the line the first one brought in.
#ifndef DA_NT_LOADS
#define DA_NT_LOADS 1
#endif
#ifndef DA_K_NT
#define DA_K_NT 0
#endif
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <bool NT = true>
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  if constexpr (NT && DA_NT_LOADS) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *p;
  }
}

template <bool NT = true>
__device__ __forceinline__ uint2 stream_load(const uint2* p) {
  if constexpr (NT && DA_NT_LOADS) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(v.x, v.y);
  } else {
    return *p;
  }
}
// the half-line K loads of the matrix-core kernels
constexpr bool kHalfLineNT = DA_K_NT != 0;

// The empty identity (m = -inf, l = 0, u = 0) for the G query heads of an
// empty split ("M4.5 - Decode Attention Kernels, Mask Programs, and Backend
// Boundaries", section 0x02C): every slot the reducer reads is defined
// (section 0x03G).
// State stores and loads.  In single-launch mode a split's states are read by
// another workgroup, possibly on another XCD, whose L2 is not coherent with
// ours for ordinary accesses.  There the states are written and read as
// device-scope relaxed atomics (plain stores and loads with the device
// coherence bit): each such access is performed at the device coherence point,
// so no L2 write-back or invalidate is needed to publish or observe them.
template <bool SHARED>
__device__ __forceinline__ void put_state(float* a, float v) {
  if constexpr (SHARED)
    __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *a = v;
}
__device__ __forceinline__ float get_shared_state(const float* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int G, int D, int NWAVES, bool SHARED>
__device__ __forceinline__ void write_identity(const SplitParams& p, int b, int h, int s) {
  for (int idx = threadIdx.x; idx < G * D; idx += NWAVES * 64) {
    const int i = idx / D, c = idx % D;
    put_state<SHARED>(p.ws_u + (out_row(p, b, h, i) * p.num_splits + s) * D + c, 0.f);
  }
  if (threadIdx.x < G) {
    const int64_t st = out_row(p, b, h, threadIdx.x) * p.num_splits + s;
    put_state<SHARED>(p.ws_m + st, -INFINITY);
    put_state<SHARED>(p.ws_l + st, 0.f);
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
template <int G, int D, int NWAVES, bool SHARED>
__device__ __forceinline__ void merge_waves_and_store(const SplitParams& p, int b, int h, int s,
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
    const int64_t st = out_row(p, b, h, i) * p.num_splits + s;
    put_state<SHARED>(p.ws_u + st * D + c, acc);
    if (c == 0) {
      put_state<SHARED>(p.ws_m + st, M == -INFINITY ? -INFINITY : M * kLn2);
      put_state<SHARED>(p.ws_l + st, L);
    }
  }
}

// ---------------------------------------------------------------------------
// Single-launch mode: the last of the S workgroups of a (b, h_kv) to store its
// states folds the S states of each of its G query-head rows, with the same
// two-pass arithmetic as the combine kernel (maximum over valid states, then
// weights e^(m_s - M) summed in ascending split order, O = u / l, LSE = M +
// ln l, all-masked rows O = +0.0 and LSE = -inf; "M4.5 - Decode Attention
// Kernels, Mask Programs, and Backend Boundaries", sections 0x02B-0x02C and
// 0x03C, which lists a fused reduction among the legal launch shapes).
//
// Arrival protocol.  Every wave waits until its device-coherent state stores
// have completed (s_waitcnt 0), the workgroup synchronises, and one thread
// increments the (b, h_kv) counter (a device-scope atomic).  The workgroup that
// reads S-1 is the last: every other workgroup's stores completed before its
// increment, which precedes ours in the counter's order, and our state loads
// are issued after the increment returned and are themselves device-coherent,
// so they observe those stores.  The last workgroup resets the counter to 0 for
// the next call.  No workgroup ever waits for another.
//
// The fold runs after the streaming is over, so it is pure latency: it issues
// the u loads of a batch of states (16-byte column quads, several states per
// wave-wide load) together with the m and l loads, keeps its code short (it
// runs once per (b, h_kv), from a cold instruction cache), and reduces across
// lanes with DPP instead of LDS shuffles where it can.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float lane_read(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}
// Wave-wide max / sum: DPP inside each 16-lane row, then the four row results.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));
  x = fmaxf(x, dpp_f32<0x4E>(x));
  x = fmaxf(x, dpp_f32<0x141>(x));
  x = fmaxf(x, dpp_f32<0x140>(x));
  return fmaxf(fmaxf(lane_read(x, 0), lane_read(x, 16)), fmaxf(lane_read(x, 32), lane_read(x, 48)));
}
__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  return (lane_read(x, 0) + lane_read(x, 16)) + (lane_read(x, 32) + lane_read(x, 48));
}
// Four consecutive device-coherent floats (two 8-byte relaxed atomic loads).
__device__ __forceinline__ float4 get_shared_state4(const float* a) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(a);
  const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float4(__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                     __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32)));
}

// Single-launch mode is used for S <= kFoldMaxSplits: lane s holds the m and
// l of state s.
constexpr int kFoldMaxSplits = 64;

template <int D>
__device__ __forceinline__ void fold_row(const SplitParams& p, int64_t row) {
  constexpr int QPS = D / 4;               // column quads per state row
  constexpr int SPI = 64 / QPS;            // states per wave-wide quad load
  constexpr int NI = 8;                    // quad loads in flight per lane
  constexpr int NB = NI * SPI;             // states per batch (divides 64)
  const int lane = threadIdx.x & 63;
  const int sub = lane / QPS;
  const int S = p.num_splits;
  const float* u = p.ws_u + row * S * D + (lane % QPS) * 4;
  // m and l are requested first, so waiting for them does not wait for the
  // u loads queued behind them.
  const int sl = min(lane, S - 1);
  float ls = get_shared_state(p.ws_l + row * S + sl);
  const float ms = get_shared_state(p.ws_m + row * S + sl);
  // only the quad loads that hold states are issued (wave-uniform guard);
  // the others stay zero and get weight 0 below
  float4 x[NI];
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    x[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (k * SPI < S) x[k] = get_shared_state4(u + (int64_t)min(k * SPI + sub, S - 1) * D);
  }
  if (lane >= S) ls = 0.f;
  const float M = wave_max(ls > 0.f ? ms : -INFINITY);
  const float w = ls > 0.f ? __expf(ms - M) : 0.f;        // 0 for invalid and absent states
  const float L = wave_sum(w * ls);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0;;) {
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const float wj = __shfl(w, j0 + k * SPI + sub);
      const bool on = wj > 0.f;            // invalid or absent states never touch acc
      acc.x = fmaf(wj, on ? x[k].x : 0.f, acc.x);
      acc.y = fmaf(wj, on ? x[k].y : 0.f, acc.y);
      acc.z = fmaf(wj, on ? x[k].z : 0.f, acc.z);
      acc.w = fmaf(wj, on ? x[k].w : 0.f, acc.w);
    }
    j0 += NB;
    if (j0 >= S) break;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      x[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j0 + k * SPI < S) x[k] = get_shared_state4(u + (int64_t)min(j0 + k * SPI + sub, S - 1) * D);
    }
  }
#pragma unroll
  for (int off = QPS; off < 64; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off);
    acc.y += __shfl_xor(acc.y, off);
    acc.z += __shfl_xor(acc.z, off);
    acc.w += __shfl_xor(acc.w, off);
  }
  const bool valid = L > 0.f;
  const float r = valid ? __builtin_amdgcn_rcpf(L) : 0.f;
  if (sub == 0)
    reinterpret_cast<float4*>(p.out + row * D)[lane] =
        make_float4(acc.x * r, acc.y * r, acc.z * r, acc.w * r);
  if (p.lse && lane == 0) p.lse[row] = valid ? M + __logf(L) : -INFINITY;
}

// Returns whether this workgroup folded (single-launch mode).
template <int G, int D, int NWAVES, bool FUSED>
__device__ __forceinline__ bool finish_split(const SplitParams& p, int b, int h) {
  if constexpr (FUSED) {
    __shared__ int is_last;
    uint32_t* cnt = p.counters + (int64_t)b * p.num_kv_heads + h;
    __builtin_amdgcn_s_waitcnt(0);       // this wave's state stores have completed
    __syncthreads();
    if (threadIdx.x == 0)
      is_last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (uint32_t)(p.num_splits - 1);
    __syncthreads();
    if (!is_last) return false;
    const int wave = threadIdx.x >> 6;
    for (int i = wave; i < G; i += NWAVES) fold_row<D>(p, out_row(p, b, h, i));
    if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  return false;
}

// Per-workgroup timestamps (timestamp instances only).  Thread 0 writes
// stamps[4 * workgroup + k]: k = 0 the kernel's start, 1 the split's states
// stored (just before the arrival protocol), 2 the end (after any fold), from
// the constant-rate counter read by s_memrealtime; k = 3 the XCC_ID register
// (bits 0..3), the HW_ID register (bits 8..39) and bit 63 set when the
// workgroup folded.  Product instances compile all of it out.
template <int INSTR>
struct WgStamps {
  const SplitParams& p;
  bool folded = false;
  // The start and states-stored times wait in LDS, so no register holds them
  // through the kernel (and no global store precedes the metadata reads).
  __device__ static uint64_t* slots() {
    __shared__ uint64_t t[2];
    return t;
  }
  __device__ explicit WgStamps(const SplitParams& pp) : p(pp) {
    if constexpr (INSTR == kInstrStamps) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      if (threadIdx.x == 0) slots()[0] = t0;
    }
  }
  __device__ void states_stored() {
    if constexpr (INSTR == kInstrStamps) {
      const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
      if (threadIdx.x == 0) slots()[1] = t1;
    }
  }
  __device__ ~WgStamps() {
    if constexpr (INSTR == kInstrStamps) {
      const uint64_t t2 = __builtin_amdgcn_s_memrealtime();
      if (threadIdx.x == 0) {
        // s_getreg operands: (size - 1) << 11 | offset << 6 | register id
        const uint32_t xcc = (uint32_t)__builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xfu;   // XCC_ID
        const uint32_t hw = (uint32_t)__builtin_amdgcn_s_getreg((31 << 11) | 4);          // HW_ID
        uint64_t* st = p.stamps + 4 * (uint64_t)blockIdx.x;
        st[0] = slots()[0];
        st[1] = slots()[1];
        st[2] = t2;
        st[3] = (uint64_t)xcc | ((uint64_t)hw << 8) | ((uint64_t)folded << 63);
      }
    }
  }
};

}  // namespace da
