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
// GEMM.  C[M][N] = A[M][K] W[N][K]^T, bf16 in, fp32 accumulation, bf16 out,
// on v_mfma_f32_32x32x16_bf16.  Every output element is one MFMA accumulator
// chain over k = 0, 16, 32, ... in order, so its bits depend on its row of A
// and its row of W only -- not on M, on the tile that computes it, on the
// row's place in that tile, or on the other rows.  Two tiles, chosen from M,
// N and K only to fill the chip (the same bits either way):
//  - 256 x 256 outputs, 8 waves of 128 x 64 (two per SIMD), when it gives at
//    least one workgroup per compute unit; K steps of 64 when K % 64 == 0,
//    else 32;
//  - 64 x 64 outputs, 4 waves of 32 x 32, otherwise; K steps of 128 when
//    K % 128 == 0, else 32.
// A/W tiles go from memory straight into a two-slot LDS ring
// (global_load_lds), one K step ahead; each stage is waited for with
// vmcnt(0) before the barrier that publishes it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

constexpr int kComputeUnits = 256;              // MI355X
constexpr int kBK = 32;                          // K granularity of every tile (and the big tile's K step)

// A workgroup tile of BM x BN outputs over WM x WN waves, K steps of BK; each
// wave owns a (BM / WM) x (BN / WN) block as 32 x 32 MFMA tiles.  Every
// configuration computes each output with the same MFMA chain over k in
// ascending 16-wide steps, so neither the tile nor its K step changes a bit.
template <int BM_, int BN_, int WM_, int WN_, int BK_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_;
  static constexpr int kStages = 2;  // LDS ring slots
  static constexpr int kWaves = WM * WN;
  static constexpr int kMI = BM / WM / 32, kNI = BN / WN / 32;
  static constexpr int kChunks = BK / 8;                 // 16-byte chunks (8 k) per tile row
  static constexpr int kRowBytes = BK * 2;
  static constexpr int kRowsPerCopy = 1024 / kRowBytes;  // rows one 1 KiB copy fills
  static constexpr int kATileBytes = BM * kRowBytes;
  static constexpr int kStageBytes = (BM + BN) * kRowBytes;
  static constexpr int kALoads = BM / kRowsPerCopy / kWaves;  // 1 KiB copies per wave per stage
  static constexpr int kBLoads = BN / kRowsPerCopy / kWaves;
  static constexpr int kLoadsPerStage = kALoads + kBLoads;
  static_assert(BK % kBK == 0 && kChunks <= 16, "K step");
  static_assert(kMI >= 1 && kNI >= 1 && kALoads >= 1 && kBLoads >= 1, "tile must divide over the waves");
  static_assert(BM % (kRowsPerCopy * kWaves) == 0 && BN % (kRowsPerCopy * kWaves) == 0, "copies per wave");
  // A tile row holds its chunks at positions c ^ ((row / (16 / kChunks)) %
  // kChunks), so the 16 rows a quarter-wave reads for one chunk fall on 16
  // distinct 16-byte bank groups (256 bytes span the 64 banks).
  static __device__ __forceinline__ int swz(int row, int c) { return c ^ ((row / (16 / kChunks)) & (kChunks - 1)); }
};
using BigTile = Tile<256, 256, 2, 4, 32>;       // 8 waves of 128 x 64
using BigTileK64 = Tile<256, 256, 2, 4, 64>;    // the same, K steps of 64 (K % 64 == 0)
using SmallTile = Tile<64, 64, 2, 2, 32>;       // 4 waves of 32 x 32, for calls with few big tiles
using SmallTileK128 = Tile<64, 64, 2, 2, 128>;  // the same with 4x the work between barriers

// A wave-uniform pointer made opaque to the optimiser (an empty asm on its
// SGPR pair): a 32-bit lane offset added to it then stays a VGPR offset on a
// scalar base (the loads' saddr form), instead of a 64-bit per-lane address
// recomputed at every use.
__device__ __forceinline__ const uint8_t* uniform_base(const uint8_t* p) {
  uint64_t v = reinterpret_cast<uint64_t>(p);
  asm volatile("" : "+s"(v));
  return reinterpret_cast<const uint8_t*>(v);
}

// Waits until every copy this wave has issued has landed in LDS, then meets
// the other waves: after it, the slot about to be read is complete.  The wait
// is explicit (the copies write LDS behind the compiler's back) and counts
// down to zero: waiting for only the older copies would assume that the
// copies land in the order they were issued.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Every address the K loop needs is formed before it: each copy is a scalar
// base (the tile's first row at the K step) plus the lane's 32-bit offset, and
// each fragment read is a per-lane LDS address of (slot, 16-k step) plus an
// immediate for the 32-row block.  The loop itself then issues copies, LDS
// reads and MFMAs with no vector address arithmetic.  (A wave's VALU and MFMA
// instructions in this loop hardly overlap, so every VALU instruction adds to
// the step's time; forming the addresses in the loop measured ~5% slower.)
template <class T>
__global__ __launch_bounds__(64 * T::kWaves) void gemm_kernel(const __bf16* __restrict__ a,
                                                               const __bf16* __restrict__ wt,
                                                               __bf16* __restrict__ c, int M, int N, int K) {
  constexpr int MI = T::kMI, NI = T::kNI, KS = T::BK / 16;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / T::WN, wn = w % T::WN;  // the wave's block of the tile
  const int ntn = N / T::BN;
  const int n0 = (blockIdx.x % ntn) * T::BN;
  const int m0 = (blockIdx.x / ntn) * T::BM;
  const int KT = K / T::BK;

  // Copy i of wave w fills the kRowsPerCopy tile rows from r0 = kRowsPerCopy
  // (i * waves + w); lane l writes row r0 + l / kChunks, position l %
  // kChunks, from chunk swz(row, l % kChunks) of that row.  Rows past M read
  // row M - 1 (never stored).  Offsets are bytes from the tile's first row
  // at k = 0; row * K * 2 < 2^32 for every supported K.
  const int crow = lane / T::kChunks, cpos = lane % T::kChunks;
  uint32_t offa[T::kALoads], offb[T::kBLoads];
#pragma unroll
  for (int i = 0; i < T::kALoads; ++i) {
    const int row = (i * T::kWaves + w) * T::kRowsPerCopy + crow;
    const int m = m0 + row < M ? row : M - 1 - m0;
    offa[i] = ((uint32_t)m * (uint32_t)K + 8u * (uint32_t)T::swz(row, cpos)) * 2u;
  }
#pragma unroll
  for (int i = 0; i < T::kBLoads; ++i) {
    const int row = (i * T::kWaves + w) * T::kRowsPerCopy + crow;
    offb[i] = ((uint32_t)row * (uint32_t)K + 8u * (uint32_t)T::swz(row, cpos)) * 2u;
  }
  const uint8_t* ga = reinterpret_cast<const uint8_t*>(a + (size_t)m0 * K);
  const uint8_t* gb = reinterpret_cast<const uint8_t*>(wt + (size_t)n0 * K);
  // Issues the copies of K step kt into slot s.
  auto issue = [&](int s, int kt) {
    uint8_t* slot = lds + s * T::kStageBytes;
    const uint8_t* ba = uniform_base(ga + (size_t)kt * (T::BK * 2));
    const uint8_t* bb = uniform_base(gb + (size_t)kt * (T::BK * 2));
    // (The empty asm keeps each offset a 32-bit value at its use, so that the
    // load takes the scalar base + 32-bit offset form rather than a 64-bit
    // address formed in vector registers.)
#pragma unroll
    for (int i = 0; i < T::kALoads; ++i) asm volatile("" : "+v"(offa[i]));
#pragma unroll
    for (int i = 0; i < T::kBLoads; ++i) asm volatile("" : "+v"(offb[i]));
#pragma unroll
    for (int i = 0; i < T::kALoads; ++i)
      __builtin_amdgcn_global_load_lds((gbl_ptr_t*)(ba + offa[i]),
                                       (lds_ptr_t*)(slot + (i * T::kWaves + w) * T::kRowsPerCopy * T::kRowBytes), 16,
                                       0, 0);
#pragma unroll
    for (int i = 0; i < T::kBLoads; ++i)
      __builtin_amdgcn_global_load_lds(
          (gbl_ptr_t*)(bb + offb[i]),
          (lds_ptr_t*)(slot + T::kATileBytes + (i * T::kWaves + w) * T::kRowsPerCopy * T::kRowBytes), 16, 0, 0);
  };
  // Fragment reads: the lane's 8 k of 16-k step ks sit in chunk ch = 2 ks +
  // kh of its row, at position swz(row, ch) = ch ^ x: rows of the wave's
  // blocks differ from the lane's first row by multiples of 32, which leave x
  // unchanged.  The 32-row block index is an immediate offset.
  const int r32 = lane & 31, kh = lane >> 5;
  const int x = (r32 / (16 / T::kChunks)) & (T::kChunks - 1);
  uint32_t ra[2][KS], rb[2][KS];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t pos = (uint32_t)(((2 * ks + kh) ^ x) * 16);
      ra[s][ks] = (uint32_t)(s * T::kStageBytes + (wm * 32 * MI + r32) * T::kRowBytes) + pos;
      rb[s][ks] = (uint32_t)(s * T::kStageBytes + T::kATileBytes + (wn * 32 * NI + r32) * T::kRowBytes) + pos;
      // Opaque to the optimiser, so that the addresses stay in registers
      // instead of being formed again by adds inside the loop.
      asm volatile("" : "+v"(ra[s][ks]), "+v"(rb[s][ks]));
    }

  lf32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = lf32x16{};

  if (KT > 0) issue(0, 0);
  // One K step from slot S (a compile-time constant: the loop is unrolled by
  // the ring's two slots).
  auto step = [&](auto slot_c, int kt) {
    constexpr int S = decltype(slot_c)::value;
    // Step kt's copies have landed; those of step kt + 1 go to the other
    // slot, which every wave has finished reading.
    stage_barrier();
    if (kt + 1 < KT) issue(S ^ 1, kt + 1);
    auto frags = [&](int ks, lbf16x8 (&af)[MI], lbf16x8 (&bf)[NI]) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        af[mi] = *reinterpret_cast<const lbf16x8*>(lds + ra[S][ks] + mi * 32 * T::kRowBytes);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        bf[ni] = *reinterpret_cast<const lbf16x8*>(lds + rb[S][ks] + ni * 32 * T::kRowBytes);
    };
    lbf16x8 af[2][MI], bf[2][NI];
    frags(0, af[0], bf[0]);
    // The two waves of a SIMD meet at every stage barrier; a wave issuing its
    // MFMAs takes precedence over the other's fragment reads and copies.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) frags(ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][mi], bf[ks & 1][ni], acc[mi][ni], 0, 0, 0);
      if constexpr (MI * NI >= MI + NI) {
        if (ks + 1 < KS) {
          // One LDS read after each of the first MFMAs of this step.
#pragma unroll
          for (int i = 0; i < MI + NI; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, MI * NI - (MI + NI), 0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  for (int kt = 0; kt < KT; kt += 2) {
    step(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < KT) step(std::integral_constant<int, 1>{}, kt + 1);
  }
  // Output element (row, col) of a 32 x 32 accumulator sits in lane col +
  // 32 * ((row / 4) % 2), register 4 * (row / 8) + row % 4.  A wave whose
  // rows all exist stores without row checks.
  const int mw = m0 + wm * (32 * MI);
  auto store = [&](bool check) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = mw + mi * 32 + 8 * (i / 4) + 4 * kh + (i % 4);
          const int n = n0 + wn * (32 * NI) + ni * 32 + r32;
          if (!check || m < M) c[(size_t)m * N + n] = (__bf16)acc[mi][ni][i];
        }
  };
  if (mw + 32 * MI <= M)
    store(false);
  else
    store(true);
}

template <class T>
hipError_t launch_gemm_t(const __bf16* a, const __bf16* wt, __bf16* c, int M, int N, int K, hipStream_t st) {
  const int lds = T::kStages * T::kStageBytes;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<T>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const int64_t tiles = (int64_t)(N / T::BN) * ((M + T::BM - 1) / T::BM);
  hipLaunchKernelGGL(gemm_kernel<T>, dim3((unsigned)tiles), dim3(64 * T::kWaves), lds, st, a, wt, c, M, N, K);
  return hipGetLastError();
}

}  // namespace

int gemm_tile_m() { return BigTile::BM; }
int gemm_tile_n() { return BigTile::BN; }
int gemm_tile_k() { return kBK; }
int rmsnorm_max_h() { return kNormThreads * kNormMaxChunks * 8; }

hipError_t launch_rmsnorm(const __bf16* x, const __bf16* w, __bf16* y, int M, int H, float eps, hipStream_t st) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)M), dim3(kNormThreads), 0, st, x, w, y, H, eps);
  return hipGetLastError();
}

// The big tile when it gives at least one workgroup per compute unit (K steps
// of 64 when K allows: half the barriers of 32-wide steps), else the small one
// with K steps of 128 when K allows (else 32).  Same bits every way.
hipError_t launch_gemm(const __bf16* a, const __bf16* wt, __bf16* c, int M, int N, int K, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const int64_t big = (int64_t)(N / BigTile::BN) * ((M + BigTile::BM - 1) / BigTile::BM);
  if (big >= kComputeUnits) {
    if (K % BigTileK64::BK == 0) return launch_gemm_t<BigTileK64>(a, wt, c, M, N, K, st);
    return launch_gemm_t<BigTile>(a, wt, c, M, N, K, st);
  }
  if (K % SmallTileK128::BK == 0) return launch_gemm_t<SmallTileK128>(a, wt, c, M, N, K, st);
  return launch_gemm_t<SmallTile>(a, wt, c, M, N, K, st);
}

}  // namespace ia
