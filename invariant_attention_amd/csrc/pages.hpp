// pages.hpp -- paged K/V addressing and loads shared by the attention kernels.
// Data movement only: nothing here changes a value except the zero fill of
// keys that do not exist (Vosti App. A.2: out-of-range loads are
// zero-padded).
//
// Page layout (page size 16, one page = one 16-key MFMA block):
//   K: [num_pages][Hkv][D/8][16 slots][8]  a 16-byte chunk = 8 dims of one
//      token; token t in slot k_slot(t) (bits 2 and 3 of t exchanged)
//   V: [num_pages][Hkv][D][16]             the 16 tokens of one dim are
//      contiguous, in token order
// Key j of a sequence lives in page block_table[j / 16], token j % 16 (Vosti
// App. A.1: K_X[j] = K_phys[pi(floor(j / P)), j mod P]).  The K slot order
// puts the 8 tokens of one page that a score block takes (tokens 0-3 and
// 8-11, or 4-7 and 12-15) in 8 consecutive slots: one 128-byte run per chunk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "arith.hpp"

namespace ia {

// Address-space pointer types of the direct global -> LDS copy builtin.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

// ---------------------------------------------------------------- raw types

// Raw page words of one K chunk (8 dims of one token), of one V quad (4
// tokens of one dim) and of one V run (8 tokens of one dim: a lane's V^T
// operand of the value product): bf16 bits, or e4m3 codes.
template <bool FP8>
struct Raw;
template <>
struct Raw<false> {
  using K = uint4;
  using V = uint2;
  using V8 = uint4;
  static constexpr int kElemBytes = 2;
};
template <>
struct Raw<true> {
  using K = uint2;
  using V = uint32_t;
  using V8 = uint2;
  static constexpr int kElemBytes = 1;
};

// Loads of page data that a kernel reads exactly once (the decode kernels
// stream each split's K and V): nontemporal, so the caches treat them as
// streaming data.  The hint changes where the bytes are cached, never their
// values.
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int nt_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void load_stream(const uint8_t* p, uint4& out) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  out = make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void load_stream(const uint8_t* p, uint2& out) {
  const nt_u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x2*>(p));
  out = make_uint2(v.x, v.y);
}

// A page load: nontemporal when NT, else an ordinary (cached) load.
template <bool NT, class T>
__device__ __forceinline__ void load_page(const uint8_t* p, T& out) {
  if constexpr (NT)
    load_stream(p, out);
  else
    out = *reinterpret_cast<const T*>(p);
}

// K chunk -> bf16x8; `keep` false gives +0 (a token that is not a key).
__device__ __forceinline__ bf16x8 k_to_bf16(uint4 w, bool keep) {
  w.x = keep ? w.x : 0u;
  w.y = keep ? w.y : 0u;
  w.z = keep ? w.z : 0u;
  w.w = keep ? w.w : 0u;
  return __builtin_bit_cast(bf16x8, w);
}
__device__ __forceinline__ bf16x8 k_to_bf16(uint2 w, bool keep) {
  w.x = keep ? w.x : 0u;
  w.y = keep ? w.y : 0u;
  const bf16x2 a = fp8x2_to_bf16(w.x, false), b = fp8x2_to_bf16(w.x, true);
  const bf16x2 c = fp8x2_to_bf16(w.y, false), d = fp8x2_to_bf16(w.y, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// V quad with only the first nv of its 4 tokens kept (nv may be <= 0 or
// >= 4); the others become zero bits.
__device__ __forceinline__ uint2 v_keep(uint2 w, int nv) {
  w.x = nv >= 2 ? w.x : (nv == 1 ? (w.x & 0xFFFFu) : 0u);
  w.y = nv >= 4 ? w.y : (nv == 3 ? (w.y & 0xFFFFu) : 0u);
  return w;
}
__device__ __forceinline__ uint32_t v_keep(uint32_t w, int nv) {
  return nv >= 4 ? w : (nv <= 0 ? 0u : (w & ((1u << (8 * nv)) - 1u)));
}

// V quad -> bf16x4; only the first nv of the 4 tokens are keys (nv may be
// <= 0 or >= 4), the rest become +0.
__device__ __forceinline__ bf16x4 v_to_bf16(uint2 w, int nv) { return __builtin_bit_cast(bf16x4, v_keep(w, nv)); }
__device__ __forceinline__ bf16x4 v_to_bf16(uint32_t w, int nv) {
  w = v_keep(w, nv);
  const bf16x2 a = fp8x2_to_bf16(w, false), b = fp8x2_to_bf16(w, true);
  bf16x4 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  return r;
}

// V run with only the first nv of its 8 tokens kept (nv may be <= 0 or
// >= 8); the others become zero bits.
__device__ __forceinline__ uint4 v8_keep(uint4 w, int nv) {
  const uint2 lo = v_keep(make_uint2(w.x, w.y), nv), hi = v_keep(make_uint2(w.z, w.w), nv - 4);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}
__device__ __forceinline__ uint2 v8_keep(uint2 w, int nv) {
  return make_uint2(v_keep((uint32_t)w.x, nv), v_keep((uint32_t)w.y, nv - 4));
}

// V run -> bf16x8 (a V^T operand); only the first nv of the 8 tokens are
// keys, the rest become +0.
__device__ __forceinline__ bf16x8 v8_to_bf16(uint4 w, int nv) { return __builtin_bit_cast(bf16x8, v8_keep(w, nv)); }
__device__ __forceinline__ bf16x8 v8_to_bf16(uint2 w, int nv) {
  w = v8_keep(w, nv);
  const bf16x2 a = fp8x2_to_bf16(w.x, false), b = fp8x2_to_bf16(w.x, true);
  const bf16x2 c = fp8x2_to_bf16(w.y, false), d = fp8x2_to_bf16(w.y, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Operand addressing in the page layout for the key-to-slot mapping of
// arith.hpp.  K operand of score block sb, k-step ks, lane (r, g): page block
// 2*(sb/2) + r/8 of the tile, token k_token(sb, r) (in K slot
// 8*(sb%2) + r%8), chunk 4*ks + g.  V^T
// operand of dim block mb, k-step ks2, lane (r, g): page block 2*ks2 + g/2,
// dim 16*mb + r, tokens 8*(g%2) .. 8*(g%2) + 7.
__device__ __forceinline__ int k_block(int sb, int r) { return 2 * (sb >> 1) + (r >> 3); }
__device__ __forceinline__ int k_token(int sb, int r) { return 8 * ((r >> 2) & 1) + 4 * (sb & 1) + (r & 3); }
// K slot of token t of a page (and, the map being its own inverse, token of
// slot t): bits 2 and 3 exchanged.  Score block sb's tokens of a page fill
// slots 8 (sb % 2) .. 8 (sb % 2) + 7.
__device__ __forceinline__ int k_slot(int t) { return (t & ~12) | ((t >> 1) & 4) | ((t << 1) & 8); }
__device__ __forceinline__ int v_block(int ks2, int g) { return 2 * ks2 + (g >> 1); }
// Byte offset, inside one (page, kv head) block, of a lane's K chunk and of
// its V run.
template <int D, bool FP8>
__device__ __forceinline__ uint32_t k_frag_off(int sb, int ks, int r, int g) {
  return (uint32_t)((((4 * ks + g) * 16 + k_slot(k_token(sb, r))) * 8) * Raw<FP8>::kElemBytes);
}
template <int D, bool FP8>
__device__ __forceinline__ uint32_t v_frag_off(int mb, int r, int g) {
  return (uint32_t)((((16 * mb + r) * 16) + 8 * (g & 1)) * Raw<FP8>::kElemBytes);
}

// ------------------------------------------------------------ block table

struct TilePages {
  int page[4];
  int valid[4];
};

// Page and key count of the 16-key block starting at key k0 whose
// block-table entry is e.  A block without keys, or whose page id is out of
// range, is marked empty (valid = 0) and addressed at page 0, so every load
// stays in bounds.
__device__ __forceinline__ void block_page(int e, int k0, int n, int num_pages, int& pg, int& v) {
  v = n - k0;
  v = v < 0 ? 0 : (v > 16 ? 16 : v);
  pg = e;
  if (v == 0 || pg < 0 || pg >= num_pages) {
    pg = 0;
    v = 0;
  }
}

// The 4 blocks of the tile starting at key t0, from their entries.
__device__ __forceinline__ TilePages tile_pages_of(const int4& e, int t0, int n, int num_pages) {
  TilePages tp;
  block_page(e.x, t0, n, num_pages, tp.page[0], tp.valid[0]);
  block_page(e.y, t0 + 16, n, num_pages, tp.page[1], tp.valid[1]);
  block_page(e.z, t0 + 32, n, num_pages, tp.page[2], tp.valid[2]);
  block_page(e.w, t0 + 48, n, num_pages, tp.page[3], tp.valid[3]);
  return tp;
}

// Block-table entry of block (lane & 3) of the tile starting at key t0, for
// one lane; the index is clamped to the sequence's last block so the load is
// in bounds and unconditional (blocks past the last one hold no keys and
// never use their entry).
__device__ __forceinline__ int load_tile_bt(const int32_t* bt_row, int t0, int nblk, int lane) {
  int e = (t0 >> 4) + (lane & 3);
  e = e < nblk ? e : nblk - 1;
  return bt_row[e];
}

__device__ __forceinline__ int clamp_len(int n, int max_len) { return n < 0 ? 0 : (n > max_len ? max_len : n); }

template <int D>
__device__ __forceinline__ QFrag<D> load_q(const __bf16* qrow, bool ok, int g) {
  QFrag<D> q;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    uint4 w = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g);
    q.f[ks] = k_to_bf16(w, ok);
  }
  return q;
}

}  // namespace ia
