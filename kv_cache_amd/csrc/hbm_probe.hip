// Measurement aid (not on the decode path): plain streaming kernels that give
// the box's practical HBM ceiling and a copy of known size against which the
// profiler's FETCH_SIZE / WRITE_SIZE counters are calibrated.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Each thread streams 16-byte words with a grid stride, folding them into a
// checksum that is stored once per thread block so the loads cannot be
// removed.
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, size_t n16,
                                                   uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 x = src[i];
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int i = 0; i < 256; ++i) t ^= red[i];
    sink[blockIdx.x] = t;
  }
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src,
                                                   uint4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// The read pattern of the decode split kernel without its arithmetic: workgroup
// (b, h, s) of a [B, T, H, row] cache (row = 256 bytes per token and head, two
// buffers K and V) reads rows [s*chunk, min((s+1)*chunk, T)) of head h, the
// split index rotated by (b, h) as the decode kernel does; each wave takes
// 16-row tiles round-robin.  Per tile, lane (n = l%16, g = l/16) reads, like
// the matrix-core kernel: K 16 bytes of row n at byte 64c + 16g for c = 0..3
// (each instruction: 16 rows x 64 bytes, plain loads), V 16 bytes of row
// 4g + j at byte 16n for j = 0..3 (each instruction: 4 whole rows,
// non-temporal).  Like the kernel, a split of whole 64-row steps starts its
// sweep at step ((2b + s) mod 8) * (steps / 8) and wraps.  With `stamps`,
// thread 0 writes the workgroup's end time (s_memrealtime) and XCC_ID.
__global__ __launch_bounds__(256) void pattern_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                      int B, int T, int H, int S, int chunk,
                                                      uint32_t* __restrict__ sink, uint64_t* __restrict__ stamps) {
  const int wg = blockIdx.x;
  const int bh = wg / S;
  const int s = (wg - bh * S + bh) % S;
  const int h = bh % H, b = bh / H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int begin = min(s * chunk, T), end = min(begin + chunk, T);
  // 16-byte words: row (b, t, h) starts at ((b*T + t)*H + h)*16, 16 words per row
  const size_t base = ((size_t)b * T * H + h) * 16;
  const int ntiles = (end - begin + 15) / 16;
  const int r0 = (end - begin) % 64 == 0 ? 4 * (((2 * b + s) & 7) * (ntiles / 4 >> 3)) : 0;
  uint32_t acc = 0;
  for (int i = wave; i < ntiles; i += 4) {
    const int ti = i + r0 >= ntiles ? i + r0 - ntiles : i + r0;
    const int t = begin + 16 * ti;
    const size_t koff = base + (size_t)min(t + n, end - 1) * H * 16 + g;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 x = k[koff + 4 * c];
      const size_t voff = base + (size_t)min(t + 4 * g + c, end - 1) * H * 16 + n;
      const u32x4_t y = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(v + voff));
      acc ^= x.x ^ x.w ^ y.y ^ y.z;
    }
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int i = 0; i < 256; ++i) t ^= red[i];
    sink[wg] = t;
    if (stamps) {
      stamps[2 * (size_t)wg] = __builtin_amdgcn_s_memrealtime();
      stamps[2 * (size_t)wg + 1] = (uint32_t)__builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xfu;   // XCC_ID
    }
  }
}

// Contiguous streaming read of two buffers of n16 16-byte words each (the
// same K and V bytes as a decode call, in address order): the read ceiling
// of those bytes in one launch, whatever the access pattern.
__global__ __launch_bounds__(256) void read2_kernel(const uint4* __restrict__ a, const uint4* __restrict__ b,
                                                    size_t n16, uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a + i));
    const u32x4_t y = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(b + i));
    acc ^= x.x ^ x.w ^ y.y ^ y.z;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int i = 0; i < 256; ++i) t ^= red[i];
    sink[blockIdx.x] = t;
  }
}


// The int8 split kernel's code loads without its arithmetic: codes [B, T, H,
// 128] (128-byte rows), workgroup (b, h, s) reads rows [s*chunk, ..) of the
// window [T - W, T) (split index rotated by (b, h)); per 16-row tile, lane
// (n, g) reads K bytes [16g, 16g+16) and [64+16g, 64+16g+16) of row n
// (plain) and V bytes [8n, 8n+8) of rows 4g + j (non-temporal).  Like the
// kernel, the split's pairs of 64-row steps are visited from pair
// ((2b + s) mod 8) * (pairs / 8) on, wrapping.
__global__ __launch_bounds__(256) void i8_pattern_kernel(const int8_t* __restrict__ k, const int8_t* __restrict__ v,
                                                         int B, int T, int H, int S, int chunk, int W,
                                                         uint32_t* __restrict__ sink) {
  const int wg = blockIdx.x;
  const int bh = wg / S;
  const int s = (wg - bh * S + bh) % S;
  const int h = bh % H, b = bh / H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int w0 = T - W;
  const int begin = min(s * chunk, W), end = min(begin + chunk, W);
  const size_t base = ((size_t)b * T * H + h) * 128;
  const size_t rs = (size_t)H * 128;
  const int ntiles = (end - begin + 15) / 16;
  const int r0 = 8 * (((2 * b + s) & 7) * ((end - begin + 127) / 128 >> 3));   // in tiles, whole pairs
  uint32_t acc = 0;
  for (int i = wave; i < ntiles; i += 4) {
    const int ti = i + r0 >= ntiles ? i + r0 - ntiles : i + r0;
    const int t = begin + 16 * ti;
    const size_t kr = base + (size_t)(w0 + min(t + n, end - 1)) * rs;
    const uint4 x0 = *reinterpret_cast<const uint4*>(k + kr + 16 * g);
    const uint4 x1 = *reinterpret_cast<const uint4*>(k + kr + 64 + 16 * g);
    acc ^= x0.x ^ x1.w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const size_t vr = base + (size_t)(w0 + min(t + 4 * g + j, end - 1)) * rs + 8 * n;
      const u32x2_t y = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(v + vr));
      acc ^= y.x ^ y.y;
    }
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int i = 0; i < 256; ++i) t ^= red[i];
    sink[wg] = t;
  }
}

}  // namespace

// K and V [B, T, H, 128] bf16 (256-byte rows); grid B*H*S workgroups; sink
// holds one uint32 per workgroup; stamps (optional) two uint64 per workgroup.
extern "C" int hbm_probe_pattern(const void* k, const void* v, int B, int T, int H, int S, int chunk,
                                 uint32_t* sink, uint64_t* stamps, void* stream) {
  if (!k || !v || !sink || B <= 0 || T <= 0 || H <= 0 || S <= 0 || chunk <= 0) return -1;
  if ((reinterpret_cast<uintptr_t>(k) & 15u) || (reinterpret_cast<uintptr_t>(v) & 15u)) return -1;
  hipLaunchKernelGGL(pattern_kernel, dim3((unsigned)(B * H * S)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(k), static_cast<const uint4*>(v), B, T, H, S, chunk, sink, stamps);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// int8 codes K and V [B, T, H, 128]; grid B*H*S workgroups over the last W
// rows of each request; sink holds one uint32 per workgroup.
extern "C" int hbm_probe_i8_pattern(const void* k, const void* v, int B, int T, int H, int S, int chunk, int W,
                                    uint32_t* sink, void* stream) {
  if (!k || !v || !sink || B <= 0 || H <= 0 || S <= 0 || chunk <= 0 || W <= 0 || W > T) return -1;
  if ((reinterpret_cast<uintptr_t>(k) & 15u) || (reinterpret_cast<uintptr_t>(v) & 15u)) return -1;
  hipLaunchKernelGGL(i8_pattern_kernel, dim3((unsigned)(B * H * S)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const int8_t*>(k), static_cast<const int8_t*>(v), B, T, H, S, chunk, W, sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Two buffers of bytes_each (a multiple of 16) bytes; sink holds `grid` uint32 values.
extern "C" int hbm_probe_read2(const void* a, const void* b, uint64_t bytes_each, uint32_t* sink, int grid,
                               void* stream) {
  if (!a || !b || !sink || grid <= 0 || (bytes_each & 15u)) return -1;
  if ((reinterpret_cast<uintptr_t>(a) & 15u) || (reinterpret_cast<uintptr_t>(b) & 15u)) return -1;
  hipLaunchKernelGGL(read2_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(a), static_cast<const uint4*>(b), (size_t)(bytes_each / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// bytes must be a multiple of 16; sink holds `grid` uint32 values.
extern "C" int hbm_probe_read(const void* src, uint64_t bytes, uint32_t* sink, int grid,
                              void* stream) {
  if (!src || !sink || grid <= 0 || (bytes & 15u)) return -1;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), (size_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int hbm_probe_copy(const void* src, void* dst, uint64_t bytes, int grid, void* stream) {
  if (!src || !dst || grid <= 0 || (bytes & 15u)) return -1;
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), (size_t)(bytes / 16));
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
