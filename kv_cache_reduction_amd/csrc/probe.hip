// HBM probes (measurement only): a streaming read with 16-byte loads and a
// plain copy.  The read probe's rate is the practical ceiling for the K
// stream; the copy kernel has known traffic (bytes read + bytes written) and
// calibrates the FETCH_SIZE / WRITE_SIZE counters.
#include "common.hpp"
#include "internal.hpp"

namespace slim {

constexpr int kProbeBlocks = 2048;   // copy probe
constexpr int kReadBlocks = 256;     // read probe: one contiguous slab per workgroup
constexpr int kReadThreads = 512;

// Each workgroup streams one contiguous slab with non-temporal 16-byte
// loads, four in flight per thread (the fastest plain streaming read found
// on MI355X).
__global__ void __launch_bounds__(kReadThreads) probe_read_kernel(const u32x4* __restrict__ src, size_t n,
                                                                  float* __restrict__ sink) {
  const size_t per = (n + gridDim.x - 1) / gridDim.x;
  const size_t beg = (size_t)blockIdx.x * per, end = beg + per < n ? beg + per : n;
  const size_t T = blockDim.x;
  uint32_t x = 0;
  size_t i = beg + threadIdx.x;
  for (; i + 3 * T < end; i += 4 * T) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + T);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * T);
    const u32x4 e = __builtin_nontemporal_load(src + i + 3 * T);
    x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ e.x ^ e.y ^ e.z ^ e.w;
  }
  for (; i < end; i += T) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  __shared__ uint32_t red[kReadThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int k = 0; k < kReadThreads / 64; ++k) r ^= red[k];
    sink[blockIdx.x] = __uint_as_float(r);
  }
}

__global__ void __launch_bounds__(256) probe_copy_kernel(uint4* __restrict__ dst,
                                                         const uint4* __restrict__ src, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

int probe_sink_floats() { return kReadBlocks; }

hipError_t launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(kReadBlocks), dim3(kReadThreads), 0, s,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  hipLaunchKernelGGL(probe_copy_kernel, dim3(kProbeBlocks), dim3(256), 0, s, static_cast<uint4*>(dst),
                     static_cast<const uint4*>(src), bytes / 16);
  return hipGetLastError();
}

}  // namespace slim
