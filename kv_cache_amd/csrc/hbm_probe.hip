// Measurement aid (not on the decode path): plain streaming kernels that give
// the box's practical HBM ceiling and a copy of known size against which the
// profiler's FETCH_SIZE / WRITE_SIZE counters are calibrated.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

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

}  // namespace

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
