// prefill.hip -- chunked / whole prefill (causal, grouped-query) with K/V
// tiles staged in LDS and shared by the 8 waves of a workgroup.  All
// value-relevant arithmetic is in arith.hpp; each row runs exactly the
// decode row's operations at its position (Vosti §5.3, App. A.1-A.5).
//
// Rows.  A wave owns 16 rows = 16/g consecutive positions x the g query
// heads of one kv head; a workgroup of 8 waves owns 8 * 16/g consecutive
// positions of one sequence.  The workgroup walks 64-key tiles 0..T of the
// keys its last row can see; splits of S keys start a fresh state, and at a
// split's end every row that reaches into it folds the split's state into its
// running merge (ascending order, as in decode).  Tiles past all of a wave's
// positions are skipped, which is the identity on its rows' states.
//
// Staging.  While the waves compute tile t from LDS buffer t&1, the
// workgroup's global loads of tile t+1 are in flight; after the compute they
// are zero filled past the sequence end (and, for e4m3 pages, converted to
// bf16, exactly) and written to buffer (t+1)&1; one barrier per tile.
//   LDS K: [4 blocks][D/8 chunks][16 tokens] x 16 B   (the pages' own layout)
//   LDS V: [2 key halves][D dims][4 quads][2 blocks] x 8 B
// so every MFMA operand fragment is one conflict-free 16-byte LDS read.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "arith.hpp"
#include "launch.hpp"
#include "pages.hpp"

namespace ia {

constexpr int kPrefillWaves = 8;
constexpr int kPrefillThreads = 64 * kPrefillWaves;

// LDS bytes of one staged tile: K and V, 64 keys x D dims x 2 bytes each.
template <int D>
constexpr int tile_lds_bytes() {
  return 2 * kTileKeys * D * 2;
}

// Source 16-byte units of one tile, and their staging registers.
template <int D, bool FP8>
struct Stage {
  static constexpr int kUnits = 2 * kTileKeys * D * Raw<FP8>::kElemBytes / 16;
  static constexpr int kPerThread = kUnits / kPrefillThreads;
  static_assert(kUnits % kPrefillThreads == 0, "tile units must divide over the workgroup");
  uint4 w[kPerThread];
  int nv[kPerThread];  // keys among the unit's page block (tokens past it are zero filled)
};

// Whether unit i of thread tid is a V unit: units [0, kUnits/2) of a tile are
// K, the rest V (known at compile time per i when a half spans whole rounds of
// the workgroup, else uniform per wave).
template <int D, bool FP8>
__device__ __forceinline__ bool unit_is_v(int i, int tid) {
  constexpr int kHalf = Stage<D, FP8>::kUnits / 2;
  if constexpr (kHalf >= kPrefillThreads) return i >= kHalf / kPrefillThreads;
  else return tid >= kHalf;
}

// Issues the global loads of the tile at t0 for this thread's units.  Unit c
// of a tile: units [0, kUnits/2) are K, the rest V; each half is 4 page
// blocks of kUnits/8 units in the pages' own order (a page block of one kv
// head is D * 16 contiguous elements in both pools).  btv holds the tile's
// block-table entries in lanes 0..3.
template <int D, bool FP8>
__device__ __forceinline__ void stage_load(Stage<D, FP8>& st, const uint8_t* kc, const uint8_t* vc, int btv, int t0,
                                           int n, int num_pages, int kvh, int Hkv, int tid) {
  constexpr int kHalf = Stage<D, FP8>::kUnits / 2;
  constexpr int kBlk = kHalf / 4;
  constexpr size_t kHeadBytes = (size_t)D * 16 * Raw<FP8>::kElemBytes;
#pragma unroll
  for (int i = 0; i < Stage<D, FP8>::kPerThread; ++i) {
    const int c = tid + kPrefillThreads * i;
    const bool is_v = unit_is_v<D, FP8>(i, tid);
    const int cc = is_v ? c - kHalf : c;
    const int blk = cc / kBlk, u = cc % kBlk;
    int pg;
    block_page(__shfl(btv, blk), t0 + 16 * blk, n, num_pages, pg, st.nv[i]);
    const uint8_t* base = (is_v ? vc : kc) + ((size_t)pg * Hkv + kvh) * kHeadBytes;
    st.w[i] = *reinterpret_cast<const uint4*>(base + (uint32_t)u * 16);
  }
}

// Zero-fills tokens >= valid of 8 consecutive bf16 tokens starting at tok0.
__device__ __forceinline__ uint4 mask8_bf16(uint4 w, int nv) {
  // nv = valid tokens among the 8 (may be <= 0 or >= 8); 2 tokens per dword.
  w.x = nv >= 2 ? w.x : (nv == 1 ? (w.x & 0xFFFFu) : 0u);
  w.y = nv >= 4 ? w.y : (nv == 3 ? (w.y & 0xFFFFu) : 0u);
  w.z = nv >= 6 ? w.z : (nv == 5 ? (w.z & 0xFFFFu) : 0u);
  w.w = nv >= 8 ? w.w : (nv == 7 ? (w.w & 0xFFFFu) : 0u);
  return w;
}

__device__ __forceinline__ uint2 fp8x8_to_bf16(uint32_t lo, uint32_t hi, uint2* second) {
  const bf16x2 a = fp8x2_to_bf16(lo, false), b = fp8x2_to_bf16(lo, true);
  const bf16x2 c = fp8x2_to_bf16(hi, false), d = fp8x2_to_bf16(hi, true);
  bf16x4 x, y;
  x[0] = a[0]; x[1] = a[1]; x[2] = b[0]; x[3] = b[1];
  y[0] = c[0]; y[1] = c[1]; y[2] = d[0]; y[3] = d[1];
  *second = __builtin_bit_cast(uint2, y);
  return __builtin_bit_cast(uint2, x);
}

// Writes staged unit c (masked, as bf16) into the LDS tile; nv = keys in
// its page block.
template <int D, bool FP8>
__device__ __forceinline__ void stage_store_unit(uint8_t* lds, int c, bool is_v, uint4 w, int nv) {
  constexpr int kHalf = Stage<D, FP8>::kUnits / 2;
  constexpr int kBlk = kHalf / 4;
  constexpr int kKBytes = kTileKeys * D * 2;  // LDS K region
  const int cc = is_v ? c - kHalf : c;
  const int blk = cc / kBlk, u = cc % kBlk;
  if constexpr (!FP8) {
    if (!is_v) {
      // K unit u = chunk u / 16, token u % 16: 8 dims of one token.
      const bool keep = (u & 15) < nv;
      w.x = keep ? w.x : 0u;
      w.y = keep ? w.y : 0u;
      w.z = keep ? w.z : 0u;
      w.w = keep ? w.w : 0u;
      *reinterpret_cast<uint4*>(lds + ((size_t)blk * (D / 8) * 16 + u) * 16) = w;
    } else {
      // V unit u = dim u / 2, tokens 8 (u % 2) .. +7 (quads g = 2 (u % 2), +1).
      const int dim = u >> 1, half = u & 1;
      w = mask8_bf16(w, nv - 8 * half);
      const int ks2 = blk >> 1, hb = blk & 1;
      uint8_t* dst = lds + kKBytes + ((size_t)(ks2 * D + dim) * 4 + 2 * half) * 16 + hb * 8;
      *reinterpret_cast<uint2*>(dst) = make_uint2(w.x, w.y);
      *reinterpret_cast<uint2*>(dst + 16) = make_uint2(w.z, w.w);
    }
  } else {
    if (!is_v) {
      // K unit u = chunk u / 8, tokens 2 (u % 8), +1: 8 codes each.
      const int chunk = u >> 3, tok = 2 * (u & 7);
      const bool k0 = tok < nv, k1 = tok + 1 < nv;
      uint2 a1, b1;
      const uint2 a0 = fp8x8_to_bf16(k0 ? w.x : 0u, k0 ? w.y : 0u, &a1);
      const uint2 b0 = fp8x8_to_bf16(k1 ? w.z : 0u, k1 ? w.w : 0u, &b1);
      uint8_t* dst = lds + ((size_t)(blk * (D / 8) + chunk) * 16 + tok) * 16;
      *reinterpret_cast<uint4*>(dst) = make_uint4(a0.x, a0.y, a1.x, a1.y);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(b0.x, b0.y, b1.x, b1.y);
    } else {
      // V unit u = dim u: its 16 tokens.
      const int dim = u;
      const int ks2 = blk >> 1, hb = blk & 1;
      const uint32_t src[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int k = nv - 4 * qd;
        const uint32_t x = k >= 4 ? src[qd] : (k <= 0 ? 0u : (src[qd] & ((1u << (8 * k)) - 1u)));
        const bf16x2 a = fp8x2_to_bf16(x, false), b = fp8x2_to_bf16(x, true);
        bf16x4 y;
        y[0] = a[0]; y[1] = a[1]; y[2] = b[0]; y[3] = b[1];
        uint8_t* dst = lds + kKBytes + ((size_t)(ks2 * D + dim) * 4 + qd) * 16 + hb * 8;
        *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, y);
      }
    }
  }
}

template <int D, bool FP8>
__device__ __forceinline__ void stage_store(uint8_t* lds, const Stage<D, FP8>& st, int tid) {
#pragma unroll
  for (int i = 0; i < Stage<D, FP8>::kPerThread; ++i)
    stage_store_unit<D, FP8>(lds, tid + kPrefillThreads * i, unit_is_v<D, FP8>(i, tid), st.w[i], st.nv[i]);
}

// Operand fragments of one tile from LDS.
template <int D>
__device__ __forceinline__ void lds_k_block(const uint8_t* lds, int blk, int r, int g, bf16x8 (&kf)[D / 32]) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    kf[ks] = __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const uint4*>(lds + ((size_t)(blk * (D / 8) + 4 * ks + g) * 16 + r) * 16));
}
template <int D>
__device__ __forceinline__ void lds_v_block(const uint8_t* lds, int mb, int r, int g, bf16x8 (&vf)[2]) {
  constexpr int kKBytes = kTileKeys * D * 2;
#pragma unroll
  for (int ks2 = 0; ks2 < 2; ++ks2)
    vf[ks2] = __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const uint4*>(lds + kKBytes + ((size_t)(ks2 * D + 16 * mb + r) * 4 + g) * 16));
}

template <int D, bool FP8>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
  constexpr int kTileBytes = tile_lds_bytes<D>();
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  // Heaviest row blocks first: block index -> (row block from the end, b, kvh).
  const int unit = blockIdx.x;
  const int kvh = unit % a.Hkv;
  const int b = (unit / a.Hkv) % a.B;
  const int rb = a.max_row_blocks - 1 - unit / a.Hkv / a.B;
  const int q0 = a.cu_q_lens[b];
  const int n = clamp_len(a.seq_lens[b], a.max_seq_len);
  int ql = a.cu_q_lens[b + 1] - q0;
  ql = ql < 0 ? 0 : (ql > a.max_q_len ? a.max_q_len : ql);
  if (q0 < 0 || q0 > a.total_q - ql) return;  // inconsistent cu_q_lens: stay in bounds
  const int ppw = kRows / a.group;         // positions per wave
  const int ppg = ppw * kPrefillWaves;     // positions per workgroup
  const int i0 = rb * ppg;
  if (i0 >= ql || n - ql + i0 < 0) return;  // uniform over the workgroup
  const int pmax_wg = n - ql + min(i0 + ppg, ql) - 1;

  // This wave's rows.
  const int iw = i0 + w * ppw;             // first position of the wave
  const int i = iw + r / a.group;
  const bool row_ok = r < ppw * a.group && i < ql;
  const int p = n - ql + i;
  const int limit = row_ok ? p : -1;
  const int hq = kvh * a.group + r % a.group;
  const QFrag<D> q = load_q<D>(a.q + ((size_t)(q0 + (row_ok ? i : i0)) * a.Hq + hq) * D, row_ok, g);
  const int pmax_w = iw < ql ? n - ql + min(iw + ppw, ql) - 1 : -1;  // last position of the wave
  float c = a.c;
  if constexpr (FP8) c = c * a.k_scale[kvh];
  const int S = a.split_tokens;

  const int32_t* bt_row = a.block_table + (size_t)b * a.bt_stride;
  const int nblk = (n + 15) >> 4;
  const int T = pmax_wg / kTileKeys;  // last tile
  // Block-table entries run one tile ahead of the staging loads, which run one
  // tile ahead of the compute.
  auto bt_of = [&](int t) { return load_tile_bt(bt_row, kTileKeys * (t < T ? t : T), nblk, lane); };
  int bt_next = bt_of(1);
  Stage<D, FP8> stg;
  stage_load<D, FP8>(stg, a.k_cache, a.v_cache, bt_of(0), 0, n, a.num_pages, kvh, a.Hkv, tid);
  stage_store<D, FP8>(lds_raw, stg, tid);
  __syncthreads();

  RowState<D> st;
  st.init();
  float M = 0.f, Z = 0.f;
  f32x4 U[D / 16];
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) U[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t = 0; t <= T; ++t) {
    const int t0 = t * kTileKeys;
    if (t < T) stage_load<D, FP8>(stg, a.k_cache, a.v_cache, bt_next, t0 + kTileKeys, n, a.num_pages, kvh, a.Hkv, tid);
    const int bt_after = bt_of(t + 2);
    if (t0 <= pmax_w) {
      const uint8_t* tile = lds_raw + (t & 1) * kTileBytes;
      f32x4 sc[4];
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        bf16x8 kf[D / 32];
        lds_k_block<D>(tile, blk, r, g, kf);
        sc[blk] = block_scores<D>(kf, q);
      }
      // The tile is whole for the wave when its last key is visible to the
      // wave's first position (and so to every stored row of the wave).
      const TileStep ts = t0 + kTileKeys - 1 <= n - ql + iw ? tile_softmax<false>(st.m, st.z, sc, c, t0, limit, g)
                                                           : tile_softmax<true>(st.m, st.z, sc, c, t0, limit, g);
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb) {
        bf16x8 vf[2];
        lds_v_block<D>(tile, mb, r, g, vf);
        st.u[mb] = pv_block(st.u[mb], vf, ts);
      }
      commit_scalars(st.m, st.z, ts);
    }
    // Split end: fold this split's state into the rows that reach into it.
    const int s = t0 / S;
    if (t == T || (t0 + kTileKeys) % S == 0) {
      if (limit >= s * S) {
        if (s == 0) {
          M = st.m;
          Z = st.z;
#pragma unroll
          for (int mb = 0; mb < D / 16; ++mb) U[mb] = st.u[mb];
        } else {
          float wa, wb;
          merge_scalars(M, Z, st.m, st.z, wa, wb);
#pragma unroll
          for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) U[mb][j] = merge_value(U[mb][j], st.u[mb][j], wa, wb);
        }
      }
      st.init();
    }
    if (t < T) {
      stage_store<D, FP8>(lds_raw + ((t + 1) & 1) * kTileBytes, stg, tid);
      __syncthreads();
    }
    bt_next = bt_after;
  }
  if (!row_ok) return;
  const float rz = final_rz(Z);
  const float vs = FP8 ? a.v_scale[kvh] : 1.0f;
  __bf16* out = a.out + ((size_t)(q0 + i) * a.Hq + hq) * D;
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) {
    bf16x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = finalize(U[mb][j], vs, rz);
    *reinterpret_cast<bf16x4*>(out + 16 * mb + 4 * g) = o;
  }
}

template <int D, bool FP8>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  if (a.B == 0 || a.max_q_len == 0) return hipSuccess;
  const int64_t units = (int64_t)a.B * a.max_row_blocks * a.Hkv;
  const size_t lds = 2 * (size_t)tile_lds_bytes<D>();
  hipLaunchKernelGGL((prefill_kernel<D, FP8>), dim3((unsigned)units), dim3(kPrefillThreads), lds, st, a);
  return hipGetLastError();
}

int prefill_positions_per_block(int group) { return (kRows / group) * kPrefillWaves; }

hipError_t launch_prefill(int D, bool fp8, const PrefillArgs& a, hipStream_t st) {
  if (D == 128 && fp8) return launch_prefill_t<128, true>(a, st);
  if (D == 128) return launch_prefill_t<128, false>(a, st);
  if (D == 64 && fp8) return launch_prefill_t<64, true>(a, st);
  if (D == 64) return launch_prefill_t<64, false>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace ia
