// attention.hip -- kv_append, decode (split + merge) and prefill kernels for
// gfx950, and their launchers.  All value-relevant arithmetic is in arith.hpp.
//
// Page layout (page size 16):
//   K: [num_pages][Hkv][D/8][16][8]   a 16-byte chunk = 8 dims of one token
//   V: [num_pages][Hkv][D][16]        the 16 tokens of one dim are contiguous
// With this layout every fragment load is a contiguous run: a K fragment load
// (one 16-byte chunk per lane, 4 chunks x 16 tokens per instruction) reads
// 1 KiB in one piece; a V^T fragment load (4 tokens per lane) reads 16 dims x
// 32 bytes = 512 bytes of one page in one piece.  One key block of 16 keys is
// exactly one page, so a block needs one block-table entry.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "arith.hpp"
#include "launch.hpp"

namespace ia {

// ------------------------------------------------------------------ loads

template <bool FP8>
struct Elem;
template <>
struct Elem<false> {
  static constexpr int kBytes = 2;
};
template <>
struct Elem<true> {
  static constexpr int kBytes = 1;
};

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = (__bf16)0.f;
  return z;
}

// 8 consecutive K elements (one chunk of one token) as bf16.
template <bool FP8>
__device__ __forceinline__ bf16x8 load_k8(const uint8_t* base, size_t elem) {
  if constexpr (FP8) {
    const uint2 w = *reinterpret_cast<const uint2*>(base + elem);
    bf16x8 r;
    const bf16x2 a = fp8x2_to_bf16(w.x, false), b = fp8x2_to_bf16(w.x, true);
    const bf16x2 c = fp8x2_to_bf16(w.y, false), d = fp8x2_to_bf16(w.y, true);
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(base + elem * 2);
    return __builtin_bit_cast(bf16x8, w);
  }
}

// 4 consecutive V elements (4 tokens of one dim) as bf16.
template <bool FP8>
__device__ __forceinline__ bf16x4 load_v4(const uint8_t* base, size_t elem) {
  if constexpr (FP8) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(base + elem);
    const bf16x2 a = fp8x2_to_bf16(w, false), b = fp8x2_to_bf16(w, true);
    bf16x4 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    return r;
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(base + elem * 2);
    return __builtin_bit_cast(bf16x4, w);
  }
}

// Tile geometry for one (sequence, kv head): the physical page of each of the
// 4 key blocks and how many of its 16 tokens are keys (< n).  Blocks without
// valid keys, or with an out-of-range page id, load as zeros.
struct TilePages {
  int page[4];
  int valid[4];
};

__device__ __forceinline__ TilePages tile_pages(const int32_t* bt_row, int tile_key0, int n, int num_pages) {
  TilePages tp;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    const int k0 = tile_key0 + 16 * blk;
    int v = n - k0;
    v = v < 0 ? 0 : (v > 16 ? 16 : v);
    int pg = v > 0 ? bt_row[k0 >> 4] : -1;
    if (pg < 0 || pg >= num_pages) {
      pg = 0;
      v = 0;
    }
    tp.page[blk] = pg;
    tp.valid[blk] = v;
  }
  return tp;
}

// Loads the K and V^T fragments of one tile.  Keys >= n (and keys of invalid
// pages) read as zeros, so stale or unwritten slots never reach the products.
template <int D, bool FP8>
__device__ __forceinline__ void load_tile(KTile<D>& kt, VTile<D>& vt, const uint8_t* kc, const uint8_t* vc,
                                          const TilePages& tp, int kvh, int Hkv, int lane) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    const size_t head = (size_t)tp.page[blk] * Hkv + kvh;
    const bool ok = r < tp.valid[blk];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const size_t e = ((head * (D / 8) + (4 * ks + g)) * 16 + r) * 8;
      kt.f[blk][ks] = ok ? load_k8<FP8>(kc, e) : zero8();
    }
  }
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) {
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      bf16x8 f;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int blk = 2 * ks2 + hb;
        const size_t head = (size_t)tp.page[blk] * Hkv + kvh;
        const int nv = tp.valid[blk] - 4 * g;  // valid tokens among this lane's 4
        bf16x4 v4;
        if (nv >= 4) {
          v4 = load_v4<FP8>(vc, (head * D + 16 * mb + r) * 16 + 4 * g);
        } else if (nv <= 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) v4[j] = (__bf16)0.f;
        } else {
          v4 = load_v4<FP8>(vc, (head * D + 16 * mb + r) * 16 + 4 * g);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (j >= nv) v4[j] = (__bf16)0.f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) f[4 * hb + j] = v4[j];
      }
      vt.f[mb][ks2] = f;
    }
  }
}

template <int D>
__device__ __forceinline__ QFrag<D> load_q(const __bf16* qrow, bool ok, int g) {
  QFrag<D> q;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    q.f[ks] = ok ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g)) : zero8();
  return q;
}

// Split length for sequence b: the fixed deployment constant, or (comparison
// variant only) the load-based length roundup(ceil(n / k), 64) with
// k = max(1, min(64, 256 / B)).
__device__ __forceinline__ int split_len(int policy, int S, int n, int B) {
  if (policy == 0) return S;
  int k = 256 / (B > 0 ? B : 1);
  k = k < 1 ? 1 : (k > 64 ? 64 : k);
  int len = (n + k - 1) / k;
  len = (len + 63) & ~63;
  return len < 64 ? 64 : len;
}

__device__ __forceinline__ int clamp_len(int n, int max_len) { return n < 0 ? 0 : (n > max_len ? max_len : n); }

// ------------------------------------------------------------ kv_append

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

// -------------------------------------------------------------- decode

// One wave per (sequence b, kv head, split s): the g query heads of the group
// are the rows; rows >= g are idle.  Writes the split's partial state.
template <int D, bool FP8>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int unit = blockIdx.x;
  const int s = unit % a.max_splits;
  const int kvh = (unit / a.max_splits) % a.Hkv;
  const int b = unit / a.max_splits / a.Hkv;
  const int n = clamp_len(a.seq_lens[b], a.max_seq_len);
  const int S = split_len(a.policy, a.split_tokens, n, a.B);
  const int nsplit = (n + S - 1) / S;
  if (s >= nsplit) return;
  const int p = n - 1;
  const bool row_ok = r < a.group;
  const int limit = row_ok ? p : -1;
  const int hq = kvh * a.group + (row_ok ? r : 0);
  const QFrag<D> q = load_q<D>(a.q + ((size_t)b * a.Hq + hq) * D, row_ok, g);
  float c = a.c;
  if constexpr (FP8) c = c * a.k_scale[kvh];
  RowState<D> st;
  st.init();
  const int32_t* bt_row = a.block_table + (size_t)b * a.bt_stride;
  const int key_hi = min((s + 1) * S, n);
  for (int t0 = s * S; t0 < key_hi; t0 += kTileKeys) {
    const TilePages tp = tile_pages(bt_row, t0, n, a.num_pages);
    KTile<D> kt;
    VTile<D> vt;
    load_tile<D, FP8>(kt, vt, a.k_cache, a.v_cache, tp, kvh, a.Hkv, lane);
    f32x4 sc[4];
    tile_scores<D>(kt, q, sc);
    tile_update<D>(st, sc, vt, c, t0, limit, g);
  }
  if (row_ok) {
    const size_t row = ((size_t)b * a.max_splits + s) * a.Hq + hq;
    float* u = a.ws_u + row * D;
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) *reinterpret_cast<f32x4*>(u + 16 * mb + 4 * g) = st.u[mb];
    if (g == 0) *reinterpret_cast<f32x2*>(a.ws_ml + row * 2) = f32x2{st.m, st.z};
  }
}

// One wave per (sequence, query head): folds the split partials in ascending
// split order and writes the bf16 output row.
template <int D, bool FP8>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  constexpr int kPer = D / 64;
  const int lane = threadIdx.x;
  const int hq = blockIdx.x % a.Hq;
  const int b = blockIdx.x / a.Hq;
  const int n = clamp_len(a.seq_lens[b], a.max_seq_len);
  const int S = split_len(a.policy, a.split_tokens, n, a.B);
  const int nsplit = n > 0 ? (n + S - 1) / S : 0;
  __bf16* out = a.out + ((size_t)b * a.Hq + hq) * D + kPer * lane;
  if (nsplit == 0) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) out[k] = (__bf16)0.f;
    return;
  }
  const size_t row0 = (size_t)b * a.max_splits * a.Hq + hq;
  const f32x2 ml0 = *reinterpret_cast<const f32x2*>(a.ws_ml + row0 * 2);
  float M = ml0[0], Z = ml0[1];
  float U[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) U[k] = a.ws_u[row0 * D + kPer * lane + k];
  for (int s = 1; s < nsplit; ++s) {
    const size_t row = row0 + (size_t)s * a.Hq;
    const f32x2 ml = *reinterpret_cast<const f32x2*>(a.ws_ml + row * 2);
    float wa, wb;
    merge_scalars(M, Z, ml[0], ml[1], wa, wb);
#pragma unroll
    for (int k = 0; k < kPer; ++k) U[k] = merge_value(U[k], a.ws_u[row * D + kPer * lane + k], wa, wb);
  }
  const float rz = final_rz(Z);
  const float vs = FP8 ? a.v_scale[hq / a.group] : 1.0f;
#pragma unroll
  for (int k = 0; k < kPer; ++k) out[k] = finalize(U[k], vs, rz);
}

// ------------------------------------------------------------- prefill

// One wave per (sequence b, block of 16/g consecutive query positions, kv
// head): row r holds position offset r / g and head r % g of the group.  The
// wave walks splits 0..floor(pmax/S) and, in each, the split's tiles in
// ascending order with the decode arithmetic; tiles and splits past a row's
// position leave its state untouched.  Each row folds the states of its own
// splits 0..floor(p/S) in ascending order and is finalised.
template <int D, bool FP8>
__global__ __launch_bounds__(64) void prefill_kernel(PrefillArgs a) {
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int unit = blockIdx.x;
  const int kvh = unit % a.Hkv;
  const int rb = (unit / a.Hkv) % a.max_row_blocks;
  const int b = unit / a.Hkv / a.max_row_blocks;
  const int q0 = a.cu_q_lens[b];
  const int n = clamp_len(a.seq_lens[b], a.max_seq_len);
  int ql = a.cu_q_lens[b + 1] - q0;
  ql = ql < 0 ? 0 : (ql > a.max_q_len ? a.max_q_len : ql);
  if (q0 < 0 || q0 > a.total_q - ql) return;  // inconsistent cu_q_lens: stay in bounds
  const int ppb = kRows / a.group;  // positions per wave
  const int i0 = rb * ppb;
  if (i0 >= ql) return;
  const int i = i0 + r / a.group;
  const bool row_ok = r < ppb * a.group && i < ql && n - ql + i >= 0;
  const int p = n - ql + i;
  const int limit = row_ok ? p : -1;
  const int hq = kvh * a.group + r % a.group;
  const QFrag<D> q = load_q<D>(a.q + ((size_t)(q0 + (row_ok ? i : 0)) * a.Hq + hq) * D, row_ok, g);
  const int pmax = n - ql + min(i0 + ppb, ql) - 1;
  if (pmax < 0) return;
  float c = a.c;
  if constexpr (FP8) c = c * a.k_scale[kvh];
  const int S = a.split_tokens;
  const int32_t* bt_row = a.block_table + (size_t)b * a.bt_stride;
  RowState<D> st;
  float M = 0.f, Z = 0.f;
  f32x4 U[D / 16];
  for (int s = 0; s * S <= pmax; ++s) {
    st.init();
    const int key_hi = min((s + 1) * S, pmax + 1);
    for (int t0 = s * S; t0 < key_hi; t0 += kTileKeys) {
      const TilePages tp = tile_pages(bt_row, t0, n, a.num_pages);
      KTile<D> kt;
      VTile<D> vt;
      load_tile<D, FP8>(kt, vt, a.k_cache, a.v_cache, tp, kvh, a.Hkv, lane);
      f32x4 sc[4];
      tile_scores<D>(kt, q, sc);
      tile_update<D>(st, sc, vt, c, t0, limit, g);
    }
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

// ------------------------------------------------------------ launchers

template <int D, bool FP8>
static hipError_t launch_append_t(const AppendArgs& a, hipStream_t st) {
  const int64_t total = (int64_t)a.T * a.Hkv * (D / 8);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL((kv_append_kernel<D, FP8>), dim3((unsigned)blocks), dim3(256), 0, st, a.k_new, a.v_new,
                     a.slots, a.T, a.k_cache, a.v_cache, a.num_pages, a.Hkv, a.k_scale, a.v_scale);
  return hipGetLastError();
}

template <int D, bool FP8>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const int64_t units = (int64_t)a.B * a.Hkv * a.max_splits;
  hipLaunchKernelGGL((decode_split_kernel<D, FP8>), dim3((unsigned)units), dim3(64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D, FP8>), dim3((unsigned)((int64_t)a.B * a.Hq)), dim3(64), 0, st, a);
  return hipGetLastError();
}

template <int D, bool FP8>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  if (a.B == 0 || a.max_q_len == 0) return hipSuccess;
  const int64_t units = (int64_t)a.B * a.max_row_blocks * a.Hkv;
  hipLaunchKernelGGL((prefill_kernel<D, FP8>), dim3((unsigned)units), dim3(64), 0, st, a);
  return hipGetLastError();
}

#define IA_DISPATCH(fn, D, FP8, ...)                     \
  do {                                                   \
    if (D == 128 && FP8) return fn<128, true>(__VA_ARGS__);   \
    if (D == 128) return fn<128, false>(__VA_ARGS__);         \
    if (D == 64 && FP8) return fn<64, true>(__VA_ARGS__);     \
    if (D == 64) return fn<64, false>(__VA_ARGS__);           \
    return hipErrorInvalidValue;                         \
  } while (0)

hipError_t launch_kv_append(int D, bool fp8, const AppendArgs& a, hipStream_t st) {
  IA_DISPATCH(launch_append_t, D, fp8, a, st);
}
hipError_t launch_decode(int D, bool fp8, const DecodeArgs& a, hipStream_t st) {
  IA_DISPATCH(launch_decode_t, D, fp8, a, st);
}
hipError_t launch_prefill(int D, bool fp8, const PrefillArgs& a, hipStream_t st) {
  IA_DISPATCH(launch_prefill_t, D, fp8, a, st);
}

}  // namespace ia
