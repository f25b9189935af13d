// kv_append.hip -- writes new K/V rows into their page slots before the
// attention call that reads them (Defeating Nondeterminism in LLM Inference,
// summary page, Overview: the KV cache is updated before the attention
// kernel, which then reads every key through the cache).  bf16 rows are
// copied; for e4m3 pages each value is quantised with the static scale of its
// kv head (Detent, discussion of fp8 scales: batch-invariant fp8 needs static
// or per-token scales, never dynamic per-tensor ones).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "arith.hpp"
#include "launch.hpp"

namespace ia {

template <int D, bool FP8>
__device__ __forceinline__ uint8_t quant_e4m3(float x) {
  // x already divided by the scale.  Round to nearest even onto OCP e4m3,
  // saturating at +-448.  (Inputs are finite by contract.)
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (u >> 31) << 7;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return (uint8_t)(sign | 0x7E);  // |x| >= 448
  if (a < 0x3C800000u) {                                 // |x| < 2^-6: subnormal codes m * 2^-9
    const float f = __builtin_bit_cast(float, a) * 512.0f;  // exact
    const uint32_t m = (uint32_t)__builtin_rintf(f);      // ties to even; 8 = smallest normal
    return (uint8_t)(sign | m);
  }
  int e = (int)(a >> 23) - 127;
  uint32_t q = (a >> 20) & 7;
  const uint32_t rem = a & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (q & 1))) ++q;
  if (q == 8) {
    q = 0;
    ++e;
  }
  return (uint8_t)(sign | (uint32_t)((e + 7) << 3) | q);
}

template <int D, bool FP8>
__global__ __launch_bounds__(256) void kv_append_kernel(const __bf16* __restrict__ k_new,
                                                        const __bf16* __restrict__ v_new,
                                                        const int64_t* __restrict__ slots, int T, uint8_t* kc,
                                                        uint8_t* vc, int num_pages, int Hkv,
                                                        const float* __restrict__ k_scale,
                                                        const float* __restrict__ v_scale) {
  constexpr int kChunks = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)T * Hkv * kChunks;
  if (idx >= total) return;
  const int c = (int)(idx % kChunks);
  const int h = (int)((idx / kChunks) % Hkv);
  const int t = (int)(idx / kChunks / Hkv);
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= (int64_t)num_pages * 16) return;
  const int64_t pg = slot >> 4;
  const int tok = (int)(slot & 15);
  const size_t src = ((size_t)t * Hkv + h) * D + 8 * c;
  const uint4 kw = *reinterpret_cast<const uint4*>(k_new + src);
  const uint4 vw = *reinterpret_cast<const uint4*>(v_new + src);
  const bf16x8 kv8 = __builtin_bit_cast(bf16x8, kw);
  const bf16x8 vv8 = __builtin_bit_cast(bf16x8, vw);
  const size_t head = (size_t)pg * Hkv + h;
  const size_t ke = ((head * kChunks + c) * 16 + tok) * 8;
  const size_t ve = (head * D + 8 * c) * 16 + tok;
  if constexpr (FP8) {
    const float ks = k_scale[h], vs = v_scale[h];
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) lo |= (uint32_t)quant_e4m3<D, FP8>((float)kv8[j] / ks) << (8 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j) hi |= (uint32_t)quant_e4m3<D, FP8>((float)kv8[4 + j] / ks) << (8 * j);
    *reinterpret_cast<uint2*>(kc + ke) = make_uint2(lo, hi);
#pragma unroll
    for (int j = 0; j < 8; ++j) vc[ve + 16 * j] = quant_e4m3<D, FP8>((float)vv8[j] / vs);
  } else {
    *reinterpret_cast<uint4*>(kc + ke * 2) = kw;
    __bf16* vb = reinterpret_cast<__bf16*>(vc);
#pragma unroll
    for (int j = 0; j < 8; ++j) vb[ve + 16 * j] = vv8[j];
  }
}

template <int D, bool FP8>
static hipError_t launch_append_t(const AppendArgs& a, hipStream_t st) {
  const int64_t total = (int64_t)a.T * a.Hkv * (D / 8);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL((kv_append_kernel<D, FP8>), dim3((unsigned)blocks), dim3(256), 0, st, a.k_new, a.v_new,
                     a.slots, a.T, a.k_cache, a.v_cache, a.num_pages, a.Hkv, a.k_scale, a.v_scale);
  return hipGetLastError();
}

hipError_t launch_kv_append(int D, bool fp8, const AppendArgs& a, hipStream_t st) {
  if (D == 128 && fp8) return launch_append_t<128, true>(a, st);
  if (D == 128) return launch_append_t<128, false>(a, st);
  if (D == 64 && fp8) return launch_append_t<64, true>(a, st);
  if (D == 64) return launch_append_t<64, false>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace ia
