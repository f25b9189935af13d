// probe.hip -- a plain streaming read of a device buffer: the achievable-HBM
// reference beside which the decode kernel's KV-read rate is judged (the
// decode kernel streams pages from HBM and should approach what a kernel that
// does nothing but read reaches).  Not part of the attention path.
//
// Each workgroup reads one contiguous share of the buffer, 16-byte words with
// kReadUnroll nontemporal loads in flight per thread (consecutive threads on
// consecutive words, so a wave reads 1 KiB runs), and folds them with xor;
// each workgroup writes one word so that no load can be dropped.  The grid is
// a fixed number of workgroups per compute unit.  (Measured on MI355X over
// 4 GiB: nontemporal loads in contiguous shares reach ~7.0 TB/s; plain loads
// ~6.2-6.4 TB/s.)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"
#include "pages.hpp"

namespace ia {

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;
constexpr int kReadBlocksPerCu = 16;
constexpr int kComputeUnitsProbe = 256;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* __restrict__ src, size_t words,
                                                                   uint32_t* __restrict__ sink) {
  const size_t per = (words + gridDim.x - 1) / gridDim.x;
  const size_t w0 = (size_t)blockIdx.x * per;
  const size_t w1 = w0 + per < words ? w0 + per : words;
  uint32_t x = 0;
  size_t i = w0 + threadIdx.x;
  for (; i + (size_t)(kReadUnroll - 1) * kReadThreads < w1; i += (size_t)kReadUnroll * kReadThreads) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      load_stream(reinterpret_cast<const uint8_t*>(src + i + (size_t)u * kReadThreads), v[u]);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < w1; i += kReadThreads) {
    uint4 v;
    load_stream(reinterpret_cast<const uint8_t*>(src + i), v);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
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
