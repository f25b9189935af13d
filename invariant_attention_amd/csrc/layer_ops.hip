// layer_ops.hip -- batch-invariant RMSNorm and fixed-tile bf16 GEMM, the
// other operators of a layer ("Deterministic inference: results independent
// of the batch", "Batch invariance: fixed splits": normalisation reduces each
// row in one block in a fixed order; matrix multiplication uses no split-K,
// so the accumulation order along K is independent of M.  Vosti, Figure 3:
// the matmul contract with fixed B_M x B_N tiles and the K loop in order).
//
// RMSNorm.  One workgroup per row.  Thread t sums the squares of its 8-element
// chunks t, t + 256, ... in order; a wave folds its 64 partial sums by a
// fixed xor butterfly and the 4 wave sums are added in wave order.  Then
// r = 1 / sqrt(mean + eps) and y = bf16((x * r) * w).  A row's operations
// depend on nothing but the row.
//
// GEMM.  C[M][N] = A[M][K] W[N][K]^T, bf16 in, fp32 accumulation, bf16 out.
// One tile shape for every call: 256 x 128 outputs per workgroup, 64-wide
// K steps, 4 waves of 128 x 64, v_mfma_f32_32x32x16_bf16.  Every output
// element is one MFMA accumulator chain over k = 0, 16, 32, ... in order, so
// its bits depend on its row of A and its row of W only -- not on M, on the
// row's place in a tile, or on the other rows.  K/W tiles go from memory
// straight into a 3-slot LDS ring (global_load_lds), two K steps ahead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace ia {

namespace {

typedef __bf16 lbf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float lf32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef __attribute__((address_space(3))) void lds_ptr_t;
typedef const __attribute__((address_space(1))) void gbl_ptr_t;

// ------------------------------------------------------------------ RMSNorm

constexpr int kNormThreads = 256;
constexpr int kNormMaxChunks = 8;  // 8-element chunks per thread: H <= 16384

__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const __bf16* __restrict__ x,
                                                               const __bf16* __restrict__ w,
                                                               __bf16* __restrict__ y, int H, float eps) {
  __shared__ float part[kNormThreads / 64];
  const int tid = threadIdx.x;
  const int nchunk = H / 8;
  const __bf16* xr = x + (size_t)blockIdx.x * H;
  __bf16* yr = y + (size_t)blockIdx.x * H;
  uint4 v[kNormMaxChunks];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i) {
    const int c = tid + kNormThreads * i;
    v[i] = c < nchunk ? *reinterpret_cast<const uint4*>(xr + 8 * c) : make_uint4(0u, 0u, 0u, 0u);
    const lbf16x8 b = __builtin_bit_cast(lbf16x8, v[i]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float f = (float)b[j];
      s = s + f * f;  // a zero chunk past the row adds +0, which changes nothing
    }
  }
  // Wave fold: after the step with offset o every lane holds the sum of its
  // 2o-lane group; a + b = b + a exactly, so all lanes agree.
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s = s + __shfl_xor(s, o);
  if ((tid & 63) == 0) part[tid >> 6] = s;
  __syncthreads();
  float total = part[0];
#pragma unroll
  for (int i = 1; i < kNormThreads / 64; ++i) total = total + part[i];
  const float ms = total / (float)H;
  const float r = 1.0f / __builtin_sqrtf(ms + eps);
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i) {
    const int c = tid + kNormThreads * i;
    if (c < nchunk) {
      const lbf16x8 b = __builtin_bit_cast(lbf16x8, v[i]);
      const lbf16x8 g = *reinterpret_cast<const lbf16x8*>(w + 8 * c);
      lbf16x8 o;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float t = (float)b[j] * r;
        o[j] = (__bf16)(t * (float)g[j]);
      }
      *reinterpret_cast<lbf16x8*>(yr + 8 * c) = o;
    }
  }
}

// --------------------------------------------------------------------- GEMM

constexpr int kBM = 256, kBN = 128, kBK = 64;
constexpr int kGemmWaves = 4;
constexpr int kStages = 3;
constexpr int kRowBytes = kBK * 2;                   // one tile row: 64 bf16 = 8 chunks of 16 B
constexpr int kATileBytes = kBM * kRowBytes;         // 32 KiB
constexpr int kBTileBytes = kBN * kRowBytes;         // 16 KiB
constexpr int kStageBytes = kATileBytes + kBTileBytes;
constexpr int kALoads = kBM / 8 / kGemmWaves;       // 1 KiB copies per wave per stage (8 rows each)
constexpr int kBLoads = kBN / 8 / kGemmWaves;
constexpr int kLoadsPerStage = kALoads + kBLoads;    // 12

// A tile row holds its 8 chunks (16 B = 8 k) at positions c ^ ((row >> 1) & 7),
// so the 16 rows a quarter-wave reads for one chunk fall on 16 distinct bank
// groups.
__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row >> 1) & 7); }

// Issues the copies of K step kt of A rows m0.. and W rows n0.. into a slot.
// Copy i of wave w fills tile rows 8 (i * 4 + w) .. +7; lane l writes row
// + l / 8, position l % 8, from chunk swz(row, l % 8) of that row.  Rows past
// M read row M - 1 (never stored).
__device__ __forceinline__ void gemm_issue(uint8_t* slot, const __bf16* a, const __bf16* wt, int M, int K, int m0,
                                           int n0, int kt, int w, int lane) {
  const int k0 = kt * kBK;
#pragma unroll
  for (int i = 0; i < kALoads; ++i) {
    const int r0 = (i * kGemmWaves + w) * 8;
    const int row = r0 + (lane >> 3);
    int m = m0 + row;
    m = m < M ? m : M - 1;
    const __bf16* src = a + (size_t)m * K + k0 + 8 * swz(row, lane & 7);
    __builtin_amdgcn_global_load_lds((gbl_ptr_t*)src, (lds_ptr_t*)(slot + r0 * kRowBytes), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < kBLoads; ++i) {
    const int r0 = (i * kGemmWaves + w) * 8;
    const int row = r0 + (lane >> 3);
    const __bf16* src = wt + (size_t)(n0 + row) * K + k0 + 8 * swz(row, lane & 7);
    __builtin_amdgcn_global_load_lds((gbl_ptr_t*)src, (lds_ptr_t*)(slot + kATileBytes + r0 * kRowBytes), 16, 0, 0);
  }
}

// Waits until this wave's copies of the step to be consumed have landed (N
// copies of later steps may stay in flight), then meets the other waves.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  static_assert(N == 0 || N == kLoadsPerStage, "wait counts");
  if constexpr (N == 0)
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__global__ __launch_bounds__(64 * kGemmWaves, 1) void gemm_kernel(const __bf16* __restrict__ a,
                                                                  const __bf16* __restrict__ wt,
                                                                  __bf16* __restrict__ c, int M, int N, int K) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;  // the wave's 128 x 64 block of the tile
  const int ntn = N / kBN;
  const int n0 = (blockIdx.x % ntn) * kBN;
  const int m0 = (blockIdx.x / ntn) * kBM;
  const int KT = K / kBK;
  auto slot = [&](int kt) { return lds + (kt % kStages) * kStageBytes; };

  lf32x16 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = lf32x16{};

  gemm_issue(slot(0), a, wt, M, K, m0, n0, 0, w, lane);
  if (KT > 1) gemm_issue(slot(1), a, wt, M, K, m0, n0, 1, w, lane);
  const int r32 = lane & 31, kh = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT)
      stage_barrier<kLoadsPerStage>();
    else
      stage_barrier<0>();
    if (kt + 2 < KT) gemm_issue(slot(kt + 2), a, wt, M, K, m0, n0, kt + 2, w, lane);
    const uint8_t* sa = slot(kt);
    const uint8_t* sb = sa + kATileBytes;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int ch = 2 * ks + kh;  // the lane's 8 k of this 16-k step
      lbf16x8 af[4], bf[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int row = wm * 128 + mi * 32 + r32;
        af[mi] = *reinterpret_cast<const lbf16x8*>(sa + row * kRowBytes + swz(row, ch) * 16);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int row = wn * 64 + ni * 32 + r32;
        bf[ni] = *reinterpret_cast<const lbf16x8*>(sb + row * kRowBytes + swz(row, ch) * 16);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
    }
  }
  // Output element (row, col) of a 32 x 32 accumulator sits in lane col +
  // 32 * ((row / 4) % 2), register 4 * (row / 8) + row % 4.
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + wm * 128 + mi * 32 + 8 * (i / 4) + 4 * kh + (i % 4);
        const int n = n0 + wn * 64 + ni * 32 + r32;
        if (m < M) c[(size_t)m * N + n] = (__bf16)acc[mi][ni][i];
      }
}

}  // namespace

int gemm_tile_m() { return kBM; }
int gemm_tile_n() { return kBN; }
int gemm_tile_k() { return kBK; }
int rmsnorm_max_h() { return kNormThreads * kNormMaxChunks * 8; }

hipError_t launch_rmsnorm(const __bf16* x, const __bf16* w, __bf16* y, int M, int H, float eps, hipStream_t st) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)M), dim3(kNormThreads), 0, st, x, w, y, H, eps);
  return hipGetLastError();
}

hipError_t launch_gemm(const __bf16* a, const __bf16* wt, __bf16* c, int M, int N, int K, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const int lds = kStages * kStageBytes;  // 144 KiB
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const int64_t tiles = (int64_t)(N / kBN) * ((M + kBM - 1) / kBM);
  hipLaunchKernelGGL(gemm_kernel, dim3((unsigned)tiles), dim3(64 * kGemmWaves), lds, st, a, wt, c, M, N, K);
  return hipGetLastError();
}

}  // namespace ia
