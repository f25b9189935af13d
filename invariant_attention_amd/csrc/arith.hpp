// arith.hpp -- the one arithmetic core shared by every attention kernel.
//
// Every value-relevant operation of a query row lives here, so decode, prefill
// and the split merge apply the same operations in the same order (Vosti:
// Specifying, Implementing, and Verifying Deterministic LLM Inference, App. A.2:
// each operation keeps its floating-point type, its operands and its place in
// the order of evaluation).  The library is compiled with -ffp-contract=off: no
// product is fused into an add unless written as such here.
//
// Wave geometry (gfx950, wave64).  A wave owns one block of 16 query rows and
// walks 64-key tiles.  Both contractions run on v_mfma_f32_16x16x32_bf16 with
// the query rows as the N (column) index, so a row's arithmetic never depends
// on its column slot or on the other rows:
//   scores   D[key][row] = sum_d K[key][d] * Q[row][d]     A = K tile, B = Q^T
//   values   D[dim][row] = sum_key V^T[dim][key] * P^T[key][row]
//                                                          A = V^T,    B = P^T
// Keys.  A 64-key tile is four 16-key pages; keys 32*h .. 32*h + 31 (pages
// 2h and 2h + 1) form the pair h.  The value product takes the pair h as its
// k-step ks2 = h, and MFMA k-slot j (0..7) of lane group g is key
// 32*h + 8*g + j there: 8 consecutive tokens of one page (page 2h + g/2,
// tokens 8*(g%2) .. 8*(g%2) + 7), so a lane's V^T operand is one 16-byte
// run of the page layout.  The score product computes the same pair as two
// score blocks sb = 2h (half 0) and 2h + 1 (half 1): MFMA row m of score block
// sb is key 32*h + 8*(m/4) + 4*(sb%2) + m%4 (score_row_key), so the block's
// output leaves in lane group g the keys 32*h + 8*g + 4*(sb%2) + j, j = 0..3
// (tile_key) -- exactly the k-slots 4*(sb%2) + j of the value product.  The
// weights a lane produces are thus the B operand it feeds into the value
// product, with no cross-lane shuffle.
// Lane l (group g = l / 16) holds, for its row l % 16:
//   scores of keys tile_key(sb, g, j)          (sb = 0..3, j = 0..3)
//   accumulators of dims 16*mb + 4*g + j       (mb = 0..d/16-1, j = 0..3)
// MFMA k-slot j of lane group g in k-step ks of the score product is dim
// 32*ks + 8*g + j.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ia {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x2 __attribute__((__vector_size__(2 * sizeof(float))));

constexpr int kTileKeys = 64;   // B_N: keys per tile (4 pages of 16)
constexpr int kBlockKeys = 16;  // keys per MFMA block (one page)
constexpr int kRows = 16;       // query rows per wave

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Key (offset in its tile) of element j (0..3) that lane group g holds in
// score block sb, and key of MFMA row m of score block sb (the K operand row).
__device__ __forceinline__ int tile_key(int sb, int g, int j) { return 32 * (sb >> 1) + 8 * g + 4 * (sb & 1) + j; }
__device__ __forceinline__ int score_row_key(int sb, int m) {
  return 32 * (sb >> 1) + 8 * (m >> 2) + 4 * (sb & 1) + (m & 3);
}

// The single exp2 of the library (v_exp_f32).  exp2(0) = 1 and
// exp2(-inf) = 0 exactly.
__device__ __forceinline__ float ia_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Row reductions over the 4 lanes that share a row (lanes l, l^16, l^32,
// l^48), as two swap steps on the VALU (gfx950 v_permlane16_swap /
// v_permlane32_swap).  Swapping a register with itself hands each lane the
// pair (x[lo], x[hi]) of its butterfly partners in the same order in both
// lanes, so all four lanes end with the same bits.
__device__ __forceinline__ void swap16(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ float row_max(float v) {
  float a, b;
  swap16(v, a, b);
  v = fmaxf(a, b);
  swap32(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float row_sum(float v) {
  float a, b;
  swap16(v, a, b);
  v = a + b;
  swap32(v, a, b);
  return a + b;
}

// Online-softmax state of one row (replicated in its 4 lanes) plus the lane's
// D/4 accumulators.
template <int D>
struct RowState {
  float m;              // running max of scaled scores (base-2 units)
  float z;              // running sum of weights
  f32x4 u[D / 16];      // weighted values, dims 16*mb + 4*g + j
  __device__ __forceinline__ void init() {
    m = neg_inf();
    z = 0.f;
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) u[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// Q^T fragments of the wave's rows: qf[ks] = B operand of k-step ks.
template <int D>
struct QFrag {
  bf16x8 f[D / 32];
};

// Scores of one score block (16 keys) for the wave's rows: s[j] = <q_row,
// k_{tile_key(sb, g, j)}> as one MFMA chain over the D/32 k-steps of the head
// dim, in ascending order.  Which wave computes a block does not change its
// bits: a column of the product depends only on its own operands.
template <int D>
__device__ __forceinline__ f32x4 block_scores(const bf16x8 (&kf)[D / 32], const QFrag<D>& q) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) acc = mfma(kf[ks], q.f[ks], acc);
  return acc;
}

// The softmax half of one tile's update for one row (Vosti App. A.2, with
// the lazy reference of raise_max):
//   s  = dot(Q, K^T),  masked lanes -> -inf
//   m^ = raise_max(m, max_b(s) * c),  alpha = exp2(m - m^)
//   A  = select(mask, exp2(fma(s, c, -m^)), 0)
//   z^ = z * alpha + sum_b A
// c > 0, so max_b(s) * c is the maximum of the rounded scaled scores s * c
// (rounding is monotone) and one multiply per row serves the maximum.  The
// exponent's argument s * c - m^ is one fused multiply-add (one rounding,
// where App. A.2's G = s * c then G - m^ rounds twice).
// The row sees keys lo..limit: limit is its position p (keys beyond it, and
// every key of a row that does not exist, limit < 0, are masked) and lo is 0,
// or p - w + 1 under a sliding window of w keys (Vosti App. A.5: the mask
// adds j > p - w).  tile_key0 is the absolute index of the tile's first key.
// A tile with no visible key keeps the state bit for bit.  z sums the fp32
// weights.  The
// weights leave as the B operands of the value product: each fp32 weight is
// the unevaluated sum of two bf16 numbers, A_hi = bf16(A) and
// A_lo = bf16(A - A_hi) (A - A_hi is exact).  Vosti casts the weights once to
// the cache type; with a single bf16 cast a row over a few keys whose values
// cancel misses the 2e-3 + 1e-2 |ref| oracle tolerance (the weight carries
// only 8 significant bits), while the hi/lo pair carries ~16.
struct TileStep {
  float m_new, z_new, alpha;
  bool any_visible;   // the tile holds a key <= limit; otherwise the state is kept bit for bit
  bf16x8 phi[2], plo[2];
};

// Splits weights w0, w1 into bf16 hi parts and bf16 lo parts, both rounded
// to nearest even.  The residual w - hi is exact in fp32; it is formed by
// v_dot2_f32_bf16 as hi . (-1, -0) + w0 and hi . (-0, -1) + w1, whose products
// and sums are exact here, so no unpacking of hi to fp32 is needed.  (The
// zero halves are -0 so that neither constant is an inline constant: for
// packed bf16 operands the compiler's reading of the inline constant -1.0
// differs from the hardware's.)
__device__ __forceinline__ void split_hi_lo(float w0, float w1, bf16x2& hi, bf16x2& lo) {
  hi = __builtin_convertvector((f32x2{w0, w1}), bf16x2);
  const bf16x2 neg0 = {(__bf16)-1.0f, (__bf16)-0.0f};
  const bf16x2 neg1 = {(__bf16)-0.0f, (__bf16)-1.0f};
  const float r0 = __builtin_amdgcn_fdot2_f32_bf16(hi, neg0, w0, false);
  const float r1 = __builtin_amdgcn_fdot2_f32_bf16(hi, neg1, w1, false);
  lo = __builtin_convertvector((f32x2{r0, r1}), bf16x2);
}

// The row maximum half of a tile step: s = masked scores (unscaled), mx =
// the maximum of the scaled scores over the row's 64 keys (lane values first,
// then the butterfly, then the scale).
struct TileMax {
  float s[4][4];
  float mx;
  bool any_visible;  // the tile holds a key the row sees
};

__device__ __forceinline__ bool key_visible(int key, int lo, int limit) { return key <= limit && key >= lo; }

// MASK = false is the same computation for a tile whose keys are all visible
// to every row that will be stored (the selects below are then identities);
// rows that are never stored may compute anything there.
template <bool MASK>
__device__ __forceinline__ TileMax tile_max(const f32x4 (&s)[4], float c, int tile_key0, int lo, int limit,
                                            int lane_group) {
  TileMax tm;
  float mx = neg_inf();
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = tile_key0 + tile_key(blk, lane_group, j);
      tm.s[blk][j] = (!MASK || key_visible(key, lo, limit)) ? s[blk][j] : neg_inf();
      mx = fmaxf(mx, tm.s[blk][j]);
    }
  }
  tm.mx = row_max(mx) * c;
  tm.any_visible = !MASK || (tile_key0 <= limit && tile_key0 + kTileKeys - 1 >= lo);
  return tm;
}

// The running reference m after a tile whose maximum scaled score is mx.
// Vosti App. A.2 takes m^ = max(m, mx) at every tile; here m is raised only
// when mx exceeds it by more than kMaxSlack (base-2 units), to mx.  The
// result is the same softmax in exact arithmetic (every weight and sum is
// relative to m); the weights are bounded by 2^kMaxSlack instead of 1, and a
// tile that does not raise m has alpha = exp2(0) = 1, so a kernel can skip
// rescaling U (U * 1 = U exactly).  The first visible tile always sets m
// (m = -inf before it).  A tile the row does not see leaves m unchanged
// (mx = -inf, or any_visible = false).
constexpr float kMaxSlack = 8.0f;
__device__ __forceinline__ float raise_max(float m, float mx) { return mx > m + kMaxSlack ? mx : m; }
__device__ __forceinline__ float max_update(float m, float mx, bool any_visible) {
  return any_visible ? raise_max(m, mx) : m;
}

// The running sum after a tile: z^ = z * alpha + sum_b A (two roundings).
__device__ __forceinline__ float z_update(float z, float alpha, float sum) {
  const float t = z * alpha;
  return t + sum;
}

// The weight half of a tile step, given the running maximum m before the
// tile: m^, alpha, the weights (as hi/lo bf16 B operands) and their row sum.
// z_new is left to the caller (z_update), so a kernel that has m before each
// tile but not yet z can form the weights of many tiles at once.
template <bool MASK>
__device__ __forceinline__ TileStep tile_weights(float m, const TileMax& tm, float c, int tile_key0, int lo,
                                                 int limit, int lane_group, float& row_sum_out) {
  TileStep ts;
  ts.any_visible = tm.any_visible;
  ts.m_new = raise_max(m, tm.mx);
  ts.alpha = ia_exp2(m - ts.m_new);
  const float neg_m = -ts.m_new;
  float a[4][4];
  float sum = 0.f;
  // A masked key's score is -inf: when the tile has a key the row sees, m^
  // is finite and its weight exp2(-inf) = 0 exactly.  When it has none, the
  // step is discarded (any_visible), whatever the weights are.
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[blk][j] = ia_exp2(__builtin_fmaf(tm.s[blk][j], c, neg_m));
      sum = sum + a[blk][j];
    }
  }
  row_sum_out = row_sum(sum);
#pragma unroll
  for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        bf16x2 hi, lo2;
        split_hi_lo(a[2 * ks2 + hb][j], a[2 * ks2 + hb][j + 1], hi, lo2);
        ts.phi[ks2][4 * hb + j] = hi[0];
        ts.phi[ks2][4 * hb + j + 1] = hi[1];
        ts.plo[ks2][4 * hb + j] = lo2[0];
        ts.plo[ks2][4 * hb + j + 1] = lo2[1];
      }
    }
  }
  return ts;
}

// The whole softmax half of a tile step for one row (the two halves above).
template <bool MASK>
__device__ __forceinline__ TileStep tile_softmax(float m, float z, const f32x4 (&s)[4], float c, int tile_key0,
                                                 int lo, int limit, int lane_group) {
  const TileMax tm = tile_max<MASK>(s, c, tile_key0, lo, limit, lane_group);
  float sum;
  TileStep ts = tile_weights<MASK>(m, tm, c, tile_key0, lo, limit, lane_group, sum);
  ts.z_new = z_update(z, ts.alpha, sum);
  return ts;
}

// The value half of the update for one dim block mb of a row:
//   U^ = U * alpha, then per key k-step ks2 (ascending) U^ += V^T A_hi, U^ += V^T A_lo
// (one MFMA each, hi first); the block keeps U when the tile is fully masked.
// MASK = false: a tile every stored row sees, so the update always applies.
// pv_rescale and pv_accumulate are its two halves, for a kernel that skips
// the rescale of a wave whose rows all have alpha = 1 (U * 1 = U exactly).
template <bool MASK = true>
__device__ __forceinline__ f32x4 pv_rescale(const f32x4& u, const TileStep& ts) {
  f32x4 un;
#pragma unroll
  for (int j = 0; j < 4; ++j) un[j] = u[j] * ts.alpha;
  if constexpr (MASK) return ts.any_visible ? un : u;
  return un;
}
template <bool MASK = true>
__device__ __forceinline__ f32x4 pv_accumulate(const f32x4& u, const bf16x8 (&vf)[2], const TileStep& ts) {
  f32x4 un = u;
#pragma unroll
  for (int ks2 = 0; ks2 < 2; ++ks2) {
    un = mfma(vf[ks2], ts.phi[ks2], un);
    un = mfma(vf[ks2], ts.plo[ks2], un);
  }
  if constexpr (MASK) return ts.any_visible ? un : u;
  return un;
}
template <bool MASK = true>
__device__ __forceinline__ f32x4 pv_block(const f32x4& u, const bf16x8 (&vf)[2], const TileStep& ts) {
  return pv_accumulate<MASK>(pv_rescale<MASK>(u, ts), vf, ts);
}
// Whether this lane's row needs pv_rescale for this tile: a visible tile
// whose alpha is not 1.  A kernel skips the rescale only when no lane of the
// wave needs it (a wave-uniform branch).
template <bool MASK = true>
__device__ __forceinline__ bool rescale_lane(const TileStep& ts) {
  return (!MASK || ts.any_visible) && ts.alpha != 1.0f;
}

// Commits the scalar half of a tile step.
template <bool MASK = true>
__device__ __forceinline__ void commit_scalars(float& m, float& z, const TileStep& ts) {
  if (!MASK || ts.any_visible) {
    m = ts.m_new;
    z = ts.z_new;
  }
}

// Folds split partial (m_s, z_s, U_s) into the running merged state (M, Z, U);
// splits are folded in ascending order, the first one seeding the state
// (fixed-size split-KV with the LSE merge of "Deterministic inference: results
// independent of the batch", split-KV decode example).
__device__ __forceinline__ void merge_scalars(float& M, float& Z, float m_s, float z_s, float& a, float& b) {
  const float M_new = fmaxf(M, m_s);
  a = ia_exp2(M - M_new);
  b = ia_exp2(m_s - M_new);
  const float t1 = Z * a;
  const float t2 = z_s * b;
  Z = t1 + t2;
  M = M_new;
}
__device__ __forceinline__ float merge_value(float U, float U_s, float a, float b) {
  const float t1 = U * a;
  const float t2 = U_s * b;
  return t1 + t2;
}

// Reciprocal of the final sum: select(z > 0, 1/z, 0) (Vosti App. A.2), with
// IEEE division.
__device__ __forceinline__ float final_rz(float Z) { return Z > 0.f ? 1.0f / Z : 0.f; }

// O = bf16((U * v_scale) * rz); v_scale is 1 for bf16 pages and the static
// per-head scale for fp8 pages (scaling by 2^k commutes with rounding).
__device__ __forceinline__ __bf16 finalize(float U, float v_scale, float rz) {
  const float t = U * v_scale;
  return to_bf16(t * rz);
}

// e4m3 (OCP) -> bf16, exact: 2 codes per instruction.
__device__ __forceinline__ bf16x2 fp8x2_to_bf16(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
            : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
}

}  // namespace ia
