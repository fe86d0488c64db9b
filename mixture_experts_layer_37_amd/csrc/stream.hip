// Read-bandwidth yardstick: one pass of 16-byte loads over a device buffer.
//
// Not part of the layer.  The HBM-bound workloads (small expert row blocks:
// every weight byte is read once per forward) are measured against what a
// plain read stream reaches on the same device, which this kernel gives:
// each thread keeps four 16-byte loads in flight over a grid-stride walk
// and folds the words into one XOR per workgroup, written to sink so the
// loads cannot be dropped.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* src, size_t n16,
                                                          uint32_t* sink) {
  __shared__ uint32_t red[4];
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= src[i];
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks,
                              hipStream_t s) {
  if (bytes < 16 || blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, s,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moe
