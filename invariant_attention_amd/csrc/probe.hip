// probe.hip -- a plain streaming read of a device buffer: the achievable-HBM
// reference beside which the decode kernel's KV-read rate is judged (the
// decode kernel streams pages from HBM and should approach what a kernel that
// does nothing but read reaches).  Not part of the attention path.
//
// Each thread reads 16-byte words in a grid-stride loop, kUnroll loads in
// flight, consecutive threads on consecutive words (a wave reads 1 KiB runs),
// and folds them with xor; each workgroup writes one word so that no load can
// be dropped.  The grid is a fixed number of workgroups per compute unit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace ia {

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;
constexpr int kReadBlocksPerCu = 8;
constexpr int kComputeUnitsProbe = 256;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* __restrict__ src, size_t words,
                                                                   uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  uint4 acc = make_uint4(0u, 0u, 0u, 0u);
  for (; i + (kReadUnroll - 1) * stride < words; i += kReadUnroll * stride) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      acc.x ^= v[u].x;
      acc.y ^= v[u].y;
      acc.z ^= v[u].z;
      acc.w ^= v[u].w;
    }
  }
  for (; i < words; i += stride) {
    const uint4 v = src[i];
    acc.x ^= v.x;
    acc.y ^= v.y;
    acc.z ^= v.z;
    acc.w ^= v.w;
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  // One word per workgroup (no atomics): a wave-level xor fold, then lane 0
  // of wave 0 stores its wave's fold.
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  if (threadIdx.x == 0) sink[blockIdx.x] = x;
}

}  // namespace

int stream_read_blocks() { return kComputeUnitsProbe * kReadBlocksPerCu; }

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st) {
  const size_t words = bytes / 16;
  if (words == 0) return hipSuccess;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)stream_read_blocks()), dim3(kReadThreads), 0, st,
                     static_cast<const uint4*>(src), words, sink);
  return hipGetLastError();
}

}  // namespace ia
