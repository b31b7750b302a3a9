// measure.hip -- a plain streaming read of device memory, the reference rate the decode kernels' HBM fractions are
// read against (the published 8 TB/s is a peak that no read stream reaches).  Not part of the layer.
#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;

// Grid-stride read of n16 16-byte chunks, four loads in flight per thread; the chunks are XOR-folded into *out so
// that no load is dead.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4_t* __restrict__ src, long long n16,
                                                                   uint32_t* out) {
  const long long stride = (long long)gridDim.x * kReadThreads;
  long long i = (long long)blockIdx.x * kReadThreads + threadIdx.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4_t v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = *(gbl_u32x4_t*)(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= *(gbl_u32x4_t*)(src + i);
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  if ((threadIdx.x & 63) == 0 && x) atomicXor(out, x);
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* out, int workgroups, hipStream_t st) {
  clear_stale_error();
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kReadThreads), 0, st, (const u32x4_t*)src,
                     (long long)(bytes / 16), out);
  return hipGetLastError();
}

}  // namespace lca
