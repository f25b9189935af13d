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
#include "pages.hpp"

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

// One workgroup per (group of 16 consecutive input rows, kv head); thread
// (r, c) holds row r's 8-dim chunk c of K and of V.  When the group's 16
// slots are one whole page in order (slot[t0 + i] = 16 pg + i -- the usual
// case when a prompt's rows are appended), the group is transposed through
// LDS and written as whole runs: K as 16-byte units filling each chunk row
// (in K slot order), V as 8-token runs of each dim row.  Otherwise every row is
// written to its own slot.  Either way each stored value is the row's value
// (bf16) or its code (e4m3) at its slot.
template <int D, bool FP8>
__device__ __forceinline__ void store_k_unit(uint8_t* kc, size_t head, int c, int tok, uint4 w, float ks) {
  constexpr int kChunks = D / 8;
  const size_t ke = ((head * kChunks + c) * 16 + k_slot(tok)) * 8;  // element index
  if constexpr (FP8) {
    const bf16x8 x = __builtin_bit_cast(bf16x8, w);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) lo |= (uint32_t)quant_e4m3<D, FP8>((float)x[j] / ks) << (8 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j) hi |= (uint32_t)quant_e4m3<D, FP8>((float)x[4 + j] / ks) << (8 * j);
    *reinterpret_cast<uint2*>(kc + ke) = make_uint2(lo, hi);
  } else {
    *reinterpret_cast<uint4*>(kc + ke * 2) = w;
  }
}

template <int D, bool FP8>
__global__ __launch_bounds__(16 * (D / 8)) void kv_append_kernel(const __bf16* __restrict__ k_new,
                                                                 const __bf16* __restrict__ v_new,
                                                                 const int64_t* __restrict__ slots, int T,
                                                                 uint8_t* kc, uint8_t* vc, int num_pages, int Hkv,
                                                                 const float* __restrict__ k_scale,
                                                                 const float* __restrict__ v_scale) {
  constexpr int kChunks = D / 8;
  __shared__ uint4 kl[16 * kChunks];  // [row][chunk]
  __shared__ uint4 vl[16 * kChunks];
  const int tid = threadIdx.x;
  const int h = blockIdx.x % Hkv;
  const int t0 = (blockIdx.x / Hkv) * 16;
  const int r = tid / kChunks, c = tid % kChunks;
  const int t = t0 + r;
  const int64_t limit = (int64_t)num_pages * 16;
  int64_t slot = -1;
  uint4 kw = make_uint4(0u, 0u, 0u, 0u), vw = kw;
  if (t < T) {
    slot = slots[t];
    const size_t src = ((size_t)t * Hkv + h) * D + 8 * c;
    kw = *reinterpret_cast<const uint4*>(k_new + src);
    vw = *reinterpret_cast<const uint4*>(v_new + src);
  }
  const float ks = FP8 ? k_scale[h] : 1.f, vs = FP8 ? v_scale[h] : 1.f;
  const int64_t s0 = t0 < T ? slots[t0] : -1;
  const bool whole = t < T && s0 >= 0 && (s0 & 15) == 0 && s0 + 15 < limit && slot == s0 + r;
  if (__syncthreads_and(whole)) {
    kl[tid] = kw;
    vl[tid] = vw;
    __syncthreads();
    const size_t head = (size_t)(s0 >> 4) * Hkv + h;
    // K: thread (c', tok) = (tid / 16, tid % 16) writes unit [tok][c'].
    const int cw = tid >> 4, tok = tid & 15;
    store_k_unit<D, FP8>(kc, head, cw, tok, kl[tok * kChunks + cw], ks);
    // V: thread (dim, half) = (tid / 2, tid % 2) writes tokens 8 half .. + 7 of its dim row.
    const int dim = tid >> 1, half = tid & 1;
    const __bf16* vb = reinterpret_cast<const __bf16*>(vl);
    const size_t ve = (head * D + dim) * 16 + 8 * half;  // element index
    if constexpr (FP8) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) lo |= (uint32_t)quant_e4m3<D, FP8>((float)vb[(8 * half + j) * D + dim] / vs) << (8 * j);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        hi |= (uint32_t)quant_e4m3<D, FP8>((float)vb[(8 * half + 4 + j) * D + dim] / vs) << (8 * j);
      *reinterpret_cast<uint2*>(vc + ve) = make_uint2(lo, hi);
    } else {
      bf16x8 x;
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = vb[(8 * half + j) * D + dim];
      *reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(vc) + ve) = x;
    }
    return;
  }
  if (slot < 0 || slot >= limit) return;  // padding row, or no row
  const size_t head = (size_t)(slot >> 4) * Hkv + h;
  const int tok = (int)(slot & 15);
  store_k_unit<D, FP8>(kc, head, c, tok, kw, ks);
  const bf16x8 vv8 = __builtin_bit_cast(bf16x8, vw);
  const size_t ve = (head * D + 8 * c) * 16 + tok;
  if constexpr (FP8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) vc[ve + 16 * j] = quant_e4m3<D, FP8>((float)vv8[j] / vs);
  } else {
    __bf16* vb = reinterpret_cast<__bf16*>(vc);
#pragma unroll
    for (int j = 0; j < 8; ++j) vb[ve + 16 * j] = vv8[j];
  }
}

template <int D, bool FP8>
static hipError_t launch_append_t(const AppendArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const int64_t groups = ((int64_t)a.T + 15) / 16;
  hipLaunchKernelGGL((kv_append_kernel<D, FP8>), dim3((unsigned)(groups * a.Hkv)), dim3(16 * (D / 8)), 0, st,
                     a.k_new, a.v_new, a.slots, a.T, a.k_cache, a.v_cache, a.num_pages, a.Hkv, a.k_scale,
                     a.v_scale);
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
