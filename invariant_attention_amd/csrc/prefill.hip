// prefill.hip -- chunked / whole prefill (causal, grouped-query) with K/V
// tiles staged in LDS and shared by the 4 waves of a workgroup.  All
// value-relevant arithmetic is in arith.hpp; each row runs exactly the
// decode row's operations at its position (Vosti §5.3, App. A.1-A.5).
//
// Rows.  A row block is 16 rows = 16/g consecutive positions x the g query
// heads of one kv head.  A wave owns two consecutive row blocks (bf16 pages;
// one for e4m3 pages), and every K and V fragment it reads from LDS feeds the
// MFMAs of both, which halves the LDS reads per flop; a workgroup of 4 waves
// owns 4 x 2 x 16/g consecutive positions of one sequence, so each staged
// tile serves 128 rows.  Two workgroups share a compute unit (2 x 64 KiB of
// LDS, 2 waves per SIMD, <= 256 VGPRs each) and run out of step with each
// other, so one's value products overlap the other's softmax.  The workgroup
// walks 64-key tiles 0..T of the keys its last row can see; splits of S keys
// start a fresh state, and at a split's end every row that reaches into it
// folds the split's state into its merge (ascending order, as in decode).
// The merge so far of a row that sees several splits waits in the workspace
// between its splits (holding it in registers would not fit two row blocks
// in 256 VGPRs); the fold of a row's last split writes the row.  Tiles past
// all of a wave's positions are skipped, which is the identity on its rows'
// states.
//
// Small launches.  A launch of fewer row-block workgroups than compute units
// takes one row block per wave (twice the workgroups).  A sequence of few
// row blocks whose keys reach a second split (decode rows co-batched with
// prompts, short chunks of long prompts) can run split grid: one workgroup
// per (row block, kv head, split) walks only that split's tiles and stores
// its rows' split states, and prefill_merge_kernel folds them in ascending
// order.  A row's operations and their order are the same in every case.
//
// Staging.  Tiles pass through two LDS slots: while the waves compute tile t,
// the workgroup's loads of tile t+1 are in flight into the other slot; one
// barrier per tile.  bf16 pages go from memory straight into LDS
// (global_load_lds, 1 KiB runs of K and V), with a zero fill of the keys past
// the sequence end only in a tile that has them; e4m3 pages go through
// registers, where they are zero filled and converted to bf16 (exactly).
// K and V keep the pages' own order, in 1 KiB runs of one page block each:
//   LDS K: [4 blocks][D/8 chunks][16 positions] x 16 B, K slot s of a page
//          at position s (even page blocks) or s ^ 8 (odd ones)
//   LDS V: [4 blocks][D/32 runs][2 dim halves][2 token halves][16 dims]
//          x 16 B: run j holds dims 32 j .. 32 j + 31 of the block, unit
//          32 (dl / 16) + 16 h + dl % 16 tokens 8 h .. 8 h + 7 of dim 32 j + dl
// so every copy reads one page block (a scalar page base and a fixed lane
// offset), and every operand fragment is one 16-byte LDS read per lane.  A K
// read takes 8 consecutive slots of each of two page blocks (arith.hpp's
// key-to-slot mapping); the swap of 128-byte halves in odd page blocks puts
// them on disjoint banks.  A V read (lane 16 g + r: dim 16 mb + r, tokens
// 8 (g % 2) .. of page block 2 ks2 + g / 2, its V^T operand of the value
// product) takes 512 contiguous bytes of one run in each half-wave, which
// the LDS serves as fast as a read in lane order (measured on MI355X: a
// 32-byte lane stride inside the run halves the rate).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "arith.hpp"
#include "launch.hpp"
#include "pages.hpp"

namespace ia {

constexpr int kPrefillWaves = 4;       // per workgroup; two workgroups per compute unit
constexpr int kPrefillThreads = 64 * kPrefillWaves;
// 16-row blocks per wave, sharing every K/V fragment read: two for bf16
// pages; one for e4m3 pages, whose staging registers leave no room for a
// second block within the 256 VGPRs of two waves per SIMD.  bf16 launches
// of fewer row-block workgroups than compute units take one block per wave
// instead, which doubles their workgroups (a row's operations do not depend
// on the other rows of its wave, so the bits are the same).
template <bool FP8>
constexpr int row_blocks_per_wave() {
  return FP8 ? 1 : 2;
}
constexpr int kSmallLaunchUnits = 256;
constexpr int kStageTiles = 1;         // tiles per LDS slot (two slots)
constexpr int kXcds = 8;  // accelerator complex dies of an MI355X, each with its own L2

// First key position p sees: 0, or p - w + 1 under a sliding window of w keys
// (Vosti App. A.5).
__device__ __forceinline__ int first_key(int p, int window) {
  if (window <= 0) return 0;
  return p - window + 1 > 0 ? p - window + 1 : 0;
}

// LDS bytes of one staged tile: K and V, 64 keys x D dims x 2 bytes each.
template <int D>
constexpr int tile_lds_bytes() {
  return 2 * kTileKeys * D * 2;
}

// LDS position of K slot s in a page block's chunk row: halves swap in odd
// blocks (the map is its own inverse).
__device__ __forceinline__ int k_pos(int blk, int s) { return s ^ ((blk & 1) << 3); }

// Dim (within its 32-dim run) and token half held by unit l of an LDS V run.
__device__ __forceinline__ int v_run_dim(int l) { return 16 * (l >> 5) + (l & 15); }
__device__ __forceinline__ int v_run_half(int l) { return (l >> 4) & 1; }

// The page block, and the byte offset inside its (page, kv head) block, of
// the 8 tokens held by 16-byte unit c of a tile's LDS V (run c / 64 = block
// p, dims 32 j..; unit c % 64 of the run).
template <int D, bool FP8>
__device__ __forceinline__ void v_unit(int c, int& blk, uint32_t& off, int& first_tok) {
  const int run = c >> 6, l = c & 63;
  blk = run / (D / 32);
  const int dim = 32 * (run % (D / 32)) + v_run_dim(l);
  first_tok = 8 * v_run_half(l);
  off = (uint32_t)((dim * 16 + first_tok) * Raw<FP8>::kElemBytes);
}

// Staging registers of one thread for one tile (e4m3 pages).
//  K: the tile's K is 4 page blocks of D * 16 elements in the pages' own
//     order; 16-byte units of it are copied as they are (kKUnits units).
//  V: LDS unit c of the V region (16 bytes of bf16 = 8 tokens of one dim)
//     comes from the 8 codes of the same tokens in the page.
template <int D, bool FP8>
struct Stage {
  static constexpr int kKUnits = kTileKeys * D * Raw<FP8>::kElemBytes / 16;
  static constexpr int kKPer = (kKUnits + kPrefillThreads - 1) / kPrefillThreads;
  static constexpr int kVUnits = 4 * D * 2;
  static constexpr int kVPer = kVUnits / kPrefillThreads;
  static_assert(kKUnits % 64 == 0 && kVUnits % kPrefillThreads == 0, "tile must divide over the waves");
  uint4 k[kKPer];
  int knv[kKPer];                  // keys in the unit's page block
  typename Raw<FP8>::V8 v[kVPer];
  int vnv[kVPer];                  // keys among the unit's 8 tokens
};

// x[blk] for a lane-varying blk in 0..3, as two levels of selects on its bits
// (no branches).
__device__ __forceinline__ int select4(int blk, const int (&x)[4]) {
  const int lo = (blk & 1) ? x[1] : x[0];
  const int hi = (blk & 1) ? x[3] : x[2];
  return (blk & 2) ? hi : lo;
}

// Issues the global loads of the tile at t0 for this thread's share, given
// the tile's 4 block-table entries e.
template <int D, bool FP8>
__device__ __forceinline__ void stage_load(Stage<D, FP8>& st, const uint8_t* kc, const uint8_t* vc, const int4& e, int t0,
                                           int n, int num_pages, int kvh, int Hkv, int tid) {
  using S = Stage<D, FP8>;
  constexpr int EB = Raw<FP8>::kElemBytes;
  constexpr size_t kHeadBytes = (size_t)D * 16 * EB;
  const TilePages tp = tile_pages_of(e, t0, n, num_pages);
#pragma unroll
  for (int i = 0; i < S::kKPer; ++i) {
    const int c = tid + kPrefillThreads * i;
    const int cc = c < S::kKUnits ? c : S::kKUnits - 1;
    const int blk = cc / (S::kKUnits / 4), u = cc % (S::kKUnits / 4);
    st.knv[i] = select4(blk, tp.valid);
    const uint8_t* base = kc + ((size_t)select4(blk, tp.page) * Hkv + kvh) * kHeadBytes;
    st.k[i] = *reinterpret_cast<const uint4*>(base + (uint32_t)u * 16);
  }
#pragma unroll
  for (int i = 0; i < S::kVPer; ++i) {
    const int c = tid + kPrefillThreads * i;
    int blk, first;
    uint32_t off;
    v_unit<D, FP8>(c, blk, off, first);
    st.vnv[i] = select4(blk, tp.valid) - first;
    const uint8_t* base = vc + ((size_t)select4(blk, tp.page) * Hkv + kvh) * kHeadBytes;
    st.v[i] = *reinterpret_cast<const typename Raw<FP8>::V8*>(base + off);
  }
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

// Writes the staged share (keys past the sequence end zero filled, e4m3
// converted to bf16 exactly) into the LDS tile.
template <int D, bool FP8>
__device__ __forceinline__ void stage_store(uint8_t* lds, const Stage<D, FP8>& st, int tid) {
  using S = Stage<D, FP8>;
  constexpr int kKBytes = kTileKeys * D * 2;  // LDS K region
#pragma unroll
  for (int i = 0; i < S::kKPer; ++i) {
    const int c = tid + kPrefillThreads * i;
    if (S::kKUnits % kPrefillThreads != 0 && c >= S::kKUnits) continue;  // uniform per wave
    const int blk = c / (S::kKUnits / 4), u = c % (S::kKUnits / 4);
    uint4 w = st.k[i];
    if constexpr (!FP8) {
      // unit u = chunk u / 16, slot u % 16: 8 dims of one token
      const int slot = u & 15;
      const bool keep = k_slot(slot) < st.knv[i];
      w.x = keep ? w.x : 0u;
      w.y = keep ? w.y : 0u;
      w.z = keep ? w.z : 0u;
      w.w = keep ? w.w : 0u;
      *reinterpret_cast<uint4*>(lds + ((size_t)(blk * (D / 8) + (u >> 4)) * 16 + k_pos(blk, slot)) * 16) = w;
    } else {
      // unit u = chunk u / 8, slots 2 (u % 8) and +1: 8 codes each (tokens
      // k_slot(slot) and + 1; the positions stay adjacent under k_pos)
      const int chunk = u >> 3, slot = 2 * (u & 7), tok = k_slot(slot);
      const bool k0 = tok < st.knv[i], k1 = tok + 1 < st.knv[i];
      uint2 a1, b1;
      const uint2 a0 = fp8x8_to_bf16(k0 ? w.x : 0u, k0 ? w.y : 0u, &a1);
      const uint2 b0 = fp8x8_to_bf16(k1 ? w.z : 0u, k1 ? w.w : 0u, &b1);
      uint8_t* dst = lds + ((size_t)(blk * (D / 8) + chunk) * 16 + k_pos(blk, slot)) * 16;
      *reinterpret_cast<uint4*>(dst) = make_uint4(a0.x, a0.y, a1.x, a1.y);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(b0.x, b0.y, b1.x, b1.y);
    }
  }
#pragma unroll
  for (int i = 0; i < S::kVPer; ++i) {
    const int c = tid + kPrefillThreads * i;
    *reinterpret_cast<bf16x8*>(lds + kKBytes + (size_t)c * 16) = v8_to_bf16(st.v[i], st.vnv[i]);
  }
}

// A wave-uniform pointer made opaque to the optimiser (an empty asm on its
// SGPR pair), so that a lane offset added to it is not folded into a 64-bit
// per-lane address hoisted out of the tile loop: such hoisted addresses cost
// two VGPRs each for the whole loop.
__device__ __forceinline__ const uint8_t* sgpr_base(const uint8_t* p) {
  uint64_t v = reinterpret_cast<uint64_t>(p);
  asm volatile("" : "+s"(v));
  return reinterpret_cast<const uint8_t*>(v);
}

// ---- bf16 tiles: direct global -> LDS loads (global_load_lds) --------------
// The data moves from the pages to LDS without passing through registers.
// Each instruction of a wave fills a contiguous 1 KiB LDS run, 16 bytes per
// lane in lane order, each lane from an address of its own.  A page block's
// K (D x 16 values) is contiguous in its page, so a tile's K is 4 blocks x
// D/32 copies of 4 chunk rows (the lanes of an odd block fetch their row's
// tokens in k_pos order); a V copy fills one 32-dim run of one page block,
// each lane fetching the 16 bytes v_unit assigns it.
template <int D>
__device__ __forceinline__ void direct_issue(uint8_t* slot, const uint8_t* kc, const uint8_t* vc, const TilePages& tp,
                                             int kvh, int Hkv, int w, int lane) {
  constexpr size_t kHeadBytes = (size_t)D * 16 * 2;          // one (page, kv head) block
  constexpr int kChunks = kTileKeys * D * 2 / 1024;           // 1 KiB copies per tile and tensor
  constexpr int kKBytes = kTileKeys * D * 2;
  static_assert(kChunks % kPrefillWaves == 0, "chunks must divide over waves");
  auto head = [&](const uint8_t* pool, int pg) { return pool + ((size_t)pg * Hkv + kvh) * kHeadBytes; };
  // Each address is a wave-uniform base plus a 32-bit lane offset.  The lane
  // offset of a K copy: the lane's 16 bytes of the 1 KiB run, in k_pos order
  // for an odd page block.  A V copy's lane offset: the dim and token half
  // its LDS unit holds (v_run_dim, v_run_half), the same in every run.
  __builtin_assume(w >= 0 && w < kPrefillWaves);  // so that the chunk -> page block map folds
  uint32_t k_even = (uint32_t)lane * 16;
  uint32_t k_odd = (uint32_t)((lane & ~15) | k_pos(1, lane & 15)) * 16;
  uint32_t v_lane = (uint32_t)((v_run_dim(lane) * 16 + 8 * v_run_half(lane)) * 2);
  // Opaque 32-bit offsets: each copy then takes the scalar base + 32-bit
  // offset form, instead of a 64-bit address formed in vector registers.
  asm volatile("" : "+v"(k_even), "+v"(k_odd), "+v"(v_lane));
#pragma unroll
  for (int i = 0; i < kChunks / kPrefillWaves; ++i) {
    const int ch = i * kPrefillWaves + w;  // wave-uniform
    const int blk = ch / (kChunks / 4), part = ch % (kChunks / 4);
    const int pg = blk == 0 ? tp.page[0] : (blk == 1 ? tp.page[1] : (blk == 2 ? tp.page[2] : tp.page[3]));
    const uint8_t* kb = sgpr_base(head(kc, pg) + part * 1024);
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(kb + ((blk & 1) ? k_odd : k_even)), (lds_void_t*)(slot + ch * 1024),
                                     16, 0, 0);
    // V run ch: dims 32 j .. of page block p, 1 KiB of one page.
    const int p = ch / (D / 32), j = ch % (D / 32);
    const int vpg = p == 0 ? tp.page[0] : (p == 1 ? tp.page[1] : (p == 2 ? tp.page[2] : tp.page[3]));
    const uint8_t* vb = sgpr_base(head(vc, vpg) + j * 1024);
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(vb + v_lane), (lds_void_t*)(slot + kKBytes + ch * 1024), 16, 0, 0);
  }
}

// Zero fills the V of tokens past each block's key count in a landed tile
// (only tiles that reach past the sequence end, or hold an invalid page).
// Their K needs no fill: a key's score column depends only on its own K row,
// and a masked score is replaced by the mask, never used.
template <int D>
__device__ __forceinline__ void direct_fixup(uint8_t* slot, const TilePages& tp, int tid) {
  constexpr int kKBytes = kTileKeys * D * 2;
  constexpr int kVUnits = 4 * D * 2;
  static_assert(kVUnits % kPrefillThreads == 0, "V units must divide over the threads");
#pragma unroll
  for (int i = 0; i < kVUnits / kPrefillThreads; ++i) {
    const int c = tid + kPrefillThreads * i;
    int blk, first;
    uint32_t off;
    v_unit<D, false>(c, blk, off, first);
    uint4* p = reinterpret_cast<uint4*>(slot + kKBytes + (size_t)c * 16);
    *p = v8_keep(*p, select4(blk, tp.valid) - first);
  }
}

// Operand fragments of one tile from LDS: the K of k-step ks of score block
// sb (the key of MFMA row r lies in page block k_block(sb, r)), and the V^T
// run of k-step ks2 of dim block mb.
template <int D>
__device__ __forceinline__ bf16x8 lds_k_frag(const uint8_t* lds, int sb, int ks, int r, int g) {
  const int blk = k_block(sb, r);
  const int pos = k_pos(blk, k_slot(k_token(sb, r)));
  return __builtin_bit_cast(
      bf16x8, *reinterpret_cast<const uint4*>(lds + ((size_t)(blk * (D / 8) + 4 * ks + g) * 16 + pos) * 16));
}
template <int D>
__device__ __forceinline__ bf16x8 lds_v_frag(const uint8_t* lds, int mb, int ks2, int r, int g) {
  constexpr int kKBytes = kTileKeys * D * 2;
  const int run = v_block(ks2, g) * (D / 32) + (mb >> 1);
  const int unit = 32 * (mb & 1) + 16 * (g & 1) + r;
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(lds + kKBytes + run * 1024 + unit * 16));
}

// Folds the state of one split into the merge of the lane's row (row index
// ridx = query row * Hq + query head): the first split seeds the merge
// (M, Z, U) = (m, z, u); a later one merges into the merge so far, which
// waits in the workspace between splits (Vosti App. A.3: the split states
// are folded in ascending order).  After the row's last split the merge is
// finalised into the output row; otherwise it goes (back) to the workspace.
// Only rows that see more than one split touch the workspace.
template <int D>
__device__ __forceinline__ void fold_split(const PrefillArgs& a, RowState<D>& st, size_t ridx, bool first, bool last,
                                           float vs, int g) {
  // The merge is formed in place in st (which the caller then resets).  (The
  // empty asm keeps the row's addresses from being computed ahead of the tile
  // loop and held through it.)
  asm volatile("" : "+v"(ridx));
  float M = st.m, Z = st.z, wa = 0.f, wb = 0.f;
  float* wu = a.ws_u + ridx * D + 4 * g;
  if (!first) {
    // All of the row's stored merge is loaded before any of it is used or
    // overwritten: one wait for the loads, not one per dim block.
    f32x4 prev[D / 16];
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) prev[mb] = *reinterpret_cast<const f32x4*>(wu + 16 * mb);
    const f32x2 mz = *reinterpret_cast<const f32x2*>(a.ws_mz + 2 * ridx);
    M = mz[0];
    Z = mz[1];
    merge_scalars(M, Z, st.m, st.z, wa, wb);
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) st.u[mb][j] = merge_value(prev[mb][j], st.u[mb][j], wa, wb);
  }
  if (last) {
    const float rz = final_rz(Z);
    __bf16* out = a.out + ridx * D + 4 * g;
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      bf16x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = finalize(st.u[mb][j], vs, rz);
      *reinterpret_cast<bf16x4*>(out + 16 * mb) = o;
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) *reinterpret_cast<f32x4*>(wu + 16 * mb) = st.u[mb];
  }
  if (!last && g == 0) *reinterpret_cast<f32x2*>(a.ws_mz + 2 * ridx) = f32x2{M, Z};
}

// Split grid: the state of one split for the lane's row, to entry `e` of
// the state arrays (u, mz): the layout fold_split uses for a row's merge.
template <int D>
__device__ __forceinline__ void store_split(float* u, float* mz, const RowState<D>& st, size_t e, int g) {
  asm volatile("" : "+v"(e));  // (as in fold_split: keep the address out of the tile loop)
  float* wu = u + e * D + 4 * g;
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) *reinterpret_cast<f32x4*>(wu + 16 * mb) = st.u[mb];
  if (g == 0) *reinterpret_cast<f32x2*>(mz + 2 * e) = f32x2{st.m, st.z};
}

// Positions one prefill workgroup of the launch covers.
__device__ __forceinline__ int positions_per_workgroup(const PrefillArgs& a) {
  return (kRows / a.group) * a.rb * kPrefillWaves;
}

// Whether a sequence runs split grid: the launch splits sequences of at most
// split_rbs row blocks, and its keys reach a second split.
__device__ __forceinline__ bool split_sequence(const PrefillArgs& a, int n, int ql, int ppg) {
  return a.split_rbs > 0 && n > a.split_tokens && ql <= a.split_rbs * ppg;
}

// Entry of split s >= 1 of row i of sequence b (split grid).
__device__ __forceinline__ size_t split_entry(const PrefillArgs& a, int b, int i, int s, int hq, int ppg) {
  return (((size_t)b * (a.split_rbs * ppg) + i) * (a.max_splits - 1) + (s - 1)) * a.Hq + hq;
}

// Split grid: one wave per (sequence, row, query head) of the split
// sequences folds the row's split states in ascending split order -- the
// first seeds the merge, each later one is merged into it (merge_scalars /
// merge_value), as fold_split does inside a workgroup -- and writes the
// finalised bf16 row.  Waves of other sequences and rows return at once.
constexpr int kMergeWaves = 4;

template <int D, bool FP8>
__global__ __launch_bounds__(64 * kMergeWaves) void prefill_merge_kernel(PrefillArgs a) {
  constexpr int kPer = D / 64;
  const int lane = threadIdx.x & 63;
  const int ppg = positions_per_workgroup(a);
  const int rows = a.split_rbs * ppg;
  const int64_t item = (int64_t)blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  const int hq = (int)(item % a.Hq);
  const int i = (int)((item / a.Hq) % rows);
  const int b = (int)(item / a.Hq / rows);
  if (b >= a.B) return;
  const int q0 = a.cu_q_lens[b];
  const int n = clamp_len(a.seq_lens[b], a.max_seq_len);
  int ql = a.cu_q_lens[b + 1] - q0;
  ql = ql < 0 ? 0 : (ql > a.max_q_len ? a.max_q_len : ql);
  if (q0 < 0 || q0 > a.total_q - ql || i >= ql || !split_sequence(a, n, ql, ppg)) return;
  // Rows of a row-block workgroup whose first position is negative
  // (inconsistent lengths) are not computed, as in prefill_kernel.
  if (n - ql + (i - i % ppg) < 0) return;
  const int p = n - ql + i;
  const int S = a.split_tokens;
  const int s0 = first_key(p, a.window) / S, s1 = p / S;
  const size_t e0 = (size_t)(q0 + i) * a.Hq + hq;
  auto u_of = [&](int s) { return s == 0 ? a.ws_u + e0 * D : a.sg_u + split_entry(a, b, i, s, hq, ppg) * D; };
  auto mz_of = [&](int s) { return s == 0 ? a.ws_mz + 2 * e0 : a.sg_mz + 2 * split_entry(a, b, i, s, hq, ppg); };
  const f32x2 mz0 = *reinterpret_cast<const f32x2*>(mz_of(s0));
  float M = mz0[0], Z = mz0[1];
  float U[kPer];
  const float* u0 = u_of(s0);
#pragma unroll
  for (int k = 0; k < kPer; ++k) U[k] = u0[kPer * lane + k];
  for (int s = s0 + 1; s <= s1; ++s) {
    const f32x2 mz = *reinterpret_cast<const f32x2*>(mz_of(s));
    const float* us = u_of(s);
    float wa, wb;
    merge_scalars(M, Z, mz[0], mz[1], wa, wb);
#pragma unroll
    for (int k = 0; k < kPer; ++k) U[k] = merge_value(U[k], us[kPer * lane + k], wa, wb);
  }
  const float rz = final_rz(Z);
  const float vs = FP8 ? a.v_scale[hq / a.group] : 1.0f;
  __bf16* out = a.out + e0 * D + kPer * lane;
#pragma unroll
  for (int k = 0; k < kPer; ++k) out[k] = finalize(U[k], vs, rz);
}

template <int D, bool FP8, int kRB>
__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_kernel(PrefillArgs a) {
  static_assert(kRB >= 1 && kRB <= row_blocks_per_wave<FP8>(), "row blocks per wave");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
  constexpr int kTileBytes = tile_lds_bytes<D>();
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  // Block index -> (sequence b, kv head, workgroup row block).  Workgroups go
  // to the 8 XCDs round robin (block i to XCD i mod 8), each XCD with its own
  // L2.  The (b, kvh) pairs are dealt to the XCDs, and each XCD runs its pairs
  // one after another, every pair's row blocks heaviest (last) first: the
  // workgroups resident on an XCD at a time are mostly row blocks of one pair
  // and walk the same K/V tiles, which its L2 then serves.  When the pair
  // count is not a multiple of 8 the order is simply row block (from the
  // end), b, kvh.
  // Split grid: past the row-block grid come the workgroups of splits 1,
  // 2, ... of the first split_rbs row blocks of every (sequence, kv head);
  // those of sequences that are not split return at once.  In a split
  // sequence each workgroup walks only the tiles of its split (split 0: the
  // row-block grid's workgroup).
  const int pairs = a.B * a.Hkv;
  const int units = pairs * a.max_row_blocks;
  int pair, wrb, sp_grid = 0;
  if ((int)blockIdx.x < units) {
    const int bid = blockIdx.x;
    int rbi;
    if (pairs % kXcds == 0) {
      const int xcd = bid % kXcds, k = bid / kXcds;
      pair = xcd + kXcds * (k / a.max_row_blocks);
      rbi = k % a.max_row_blocks;
    } else {
      pair = bid % pairs;
      rbi = bid / pairs;
    }
    wrb = a.max_row_blocks - 1 - rbi;
  } else {
    const int e = blockIdx.x - units, per = pairs * a.split_rbs;
    sp_grid = 1 + e / per;
    pair = (e % per) % pairs;
    wrb = (e % per) / pairs;
  }
  const int kvh = pair % a.Hkv;
  const int b = pair / a.Hkv;
  const int q0 = a.cu_q_lens[b];
  const int n = clamp_len(a.seq_lens[b], a.max_seq_len);
  int ql = a.cu_q_lens[b + 1] - q0;
  ql = ql < 0 ? 0 : (ql > a.max_q_len ? a.max_q_len : ql);
  if (q0 < 0 || q0 > a.total_q - ql) return;  // inconsistent cu_q_lens: stay in bounds
  const int ppr = kRows / a.group;                 // positions per row block
  const int ppw = ppr * kRB;         // positions per wave
  const int ppg = ppw * kPrefillWaves;             // positions per workgroup
  const int i0 = wrb * ppg;
  if (i0 >= ql || n - ql + i0 < 0) return;  // uniform over the workgroup
  const int pmax_wg = n - ql + min(i0 + ppg, ql) - 1;

  // This wave's rows: row block k holds positions iw + k ppr .. + ppr - 1.
  const int iw = i0 + w * ppw;  // first position of the wave
  const int hq = kvh * a.group + r % a.group;
  int limit[kRB], lo[kRB], ii[kRB];
  bool row_ok[kRB];
  QFrag<D> q[kRB];
#pragma unroll
  for (int k = 0; k < kRB; ++k) {
    ii[k] = iw + k * ppr + r / a.group;
    row_ok[k] = r < ppr * a.group && ii[k] < ql;
    const int p = n - ql + ii[k];
    limit[k] = row_ok[k] ? p : -1;
    // Visible keys: lo..p per row, lo = 0 or p - w + 1 under a sliding
    // window of w keys (Vosti App. A.5).
    lo[k] = first_key(p, a.window);
    q[k] = load_q<D>(a.q + ((size_t)(q0 + (row_ok[k] ? ii[k] : i0)) * a.Hq + hq) * D, row_ok[k], g);
  }
  const int pmax_w = iw < ql ? n - ql + min(iw + ppw, ql) - 1 : -1;  // last position of the wave
  const int p_first = n - ql + iw;                                     // first position of the wave
  const int lo_first = first_key(p_first, a.window);
  const int lo_last = first_key(pmax_w, a.window);
  // Whether the wave has a row that sees some key of tile t.
  auto needs = [&](int t) { return t * kTileKeys <= pmax_w && t * kTileKeys + kTileKeys - 1 >= lo_first; };
  float c = a.c;
  if constexpr (FP8) c = c * a.k_scale[kvh];
  const int S = a.split_tokens;
  const bool split_grid = split_sequence(a, n, ql, ppg);
  if (sp_grid > 0 && !split_grid) return;  // uniform over the workgroup

  const int32_t* bt_row = a.block_table + (size_t)b * a.bt_stride;
  const int nblk = (n + 15) >> 4;
  int T = pmax_wg / kTileKeys;                            // last tile
  int T0 = first_key(n - ql + i0, a.window) / kTileKeys;  // first tile
  if (split_grid) {
    T0 = max(T0, sp_grid * (S / kTileKeys));
    T = min(T, (sp_grid + 1) * (S / kTileKeys) - 1);
    if (T0 > T) return;  // uniform over the workgroup
  }
  // Pipeline.  Tiles go in stages of kStageTiles (stage s = tiles 2s, 2s + 1)
  // through two LDS slots: while the waves compute stage s from one slot,
  // stage s + 1 loads into the other -- bf16 pages straight from memory into
  // LDS, e4m3 pages through registers (converted to bf16 after the compute).
  // One barrier per stage publishes the next stage; a tile reaching past the
  // sequence end gets its V zero filled between two barriers.  Tiles outside
  // T0..T are never loaded nor computed.  Block-table entries run one stage
  // ahead of the loads.
  auto buf = [&](int t) {
    return lds_raw + ((t / kStageTiles) & 1) * (kStageTiles * kTileBytes) + (t % kStageTiles) * kTileBytes;
  };
  auto in_range = [&](int t) { return t >= T0 && t <= T; };
  // A tile's 4 block-table entries, by scalar loads (wave-uniform indices,
  // clamped to the sequence's last block: blocks past it hold no keys).  The
  // table is read through the constant address space, which is what lets the
  // loads be scalar: nothing writes it during the call.
  const __attribute__((address_space(4))) int32_t* bt_const =
      (const __attribute__((address_space(4))) int32_t*)bt_row;
  auto bt_of = [&](int t) {
    const int e0 = (t < T ? t : T) * (kTileKeys / 16);
    auto ent = [&](int j) { return bt_const[e0 + j < nblk ? e0 + j : nblk - 1]; };
    return make_int4(ent(0), ent(1), ent(2), ent(3));
  };
  auto pages_of = [&](const int4& e, int t) { return tile_pages_of(e, t * kTileKeys, n, a.num_pages); };
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int S0 = T0 / kStageTiles, S1 = T / kStageTiles;
  Stage<D, FP8> stg[kStageTiles];
  // Issues the loads of stage s (its tiles in T0..T); e4m3 pages land in stg.
  auto issue = [&](int s, const int4 (&btv)[kStageTiles]) {
#pragma unroll
    for (int k = 0; k < kStageTiles; ++k) {
      const int t = s * kStageTiles + k;
      if (!in_range(t)) continue;  // uniform
      if constexpr (FP8)
        stage_load<D, FP8>(stg[k], a.k_cache, a.v_cache, btv[k], t * kTileKeys, n, a.num_pages, kvh, a.Hkv, tid);
      else
        direct_issue<D>(buf(t), a.k_cache, a.v_cache, pages_of(btv[k], t), kvh, a.Hkv, wu, lane);
    }
  };
  // After the stage's loads have landed and a barrier: e4m3 tiles are stored
  // (FP8), bf16 tiles reaching past the sequence end are zero filled.
  // Whether tile t needs a V zero fill: some block of it holds fewer than 16
  // keys, i.e. the tile reaches past the sequence end or one of its entries
  // is out of range (such a block reads page 0 and holds no keys).  Scalar
  // compares on the entries.
  auto tile_short = [&](const int4& e, int t) {
    const int np = a.num_pages;
    return (t + 1) * kTileKeys > n || e.x < 0 || e.x >= np || e.y < 0 || e.y >= np || e.z < 0 || e.z >= np ||
           e.w < 0 || e.w >= np;
  };
  auto land = [&](int s, const int4 (&btv)[kStageTiles]) {
    if constexpr (FP8) {
#pragma unroll
      for (int k = 0; k < kStageTiles; ++k)
        if (in_range(s * kStageTiles + k)) stage_store<D, FP8>(buf(s * kStageTiles + k), stg[k], tid);
    } else {
      bool partial = false;
#pragma unroll
      for (int k = 0; k < kStageTiles; ++k) {
        const int t = s * kStageTiles + k;
        if (in_range(t) && tile_short(btv[k], t)) {
          direct_fixup<D>(buf(t), pages_of(btv[k], t), tid);
          partial = true;
        }
      }
      if (partial) __syncthreads();
    }
  };
  int4 btn[kStageTiles];
  {
    int4 bt0[kStageTiles];
#pragma unroll
    for (int k = 0; k < kStageTiles; ++k) bt0[k] = bt_of(S0 * kStageTiles + k);
    issue(S0, bt0);
    __syncthreads();
    if constexpr (FP8) {
      land(S0, bt0);
      __syncthreads();
    } else {
      land(S0, bt0);
    }
#pragma unroll
    for (int k = 0; k < kStageTiles; ++k) btn[k] = bt_of((S0 + 1) * kStageTiles + k);
  }

  RowState<D> st[kRB];
#pragma unroll
  for (int k = 0; k < kRB; ++k) st[k].init();
  const float vs = FP8 ? a.v_scale[kvh] : 1.0f;

  for (int s = S0; s <= S1; ++s) {
    const bool more = s < S1;
    int4 bta[kStageTiles];
#pragma unroll
    for (int k = 0; k < kStageTiles; ++k) bta[k] = bt_of((s + 2) * kStageTiles + k);
    if (more) issue(s + 1, btn);
#pragma unroll 1
    for (int kt = 0; kt < kStageTiles; ++kt) {
      const int t = s * kStageTiles + kt;
      if (!in_range(t)) continue;  // uniform
      const int t0 = t * kTileKeys;
      const uint8_t* tile = buf(t);
      // The tile is whole for the wave when all its keys are visible to every
      // stored row: its last key to the first position, its first key to the
      // last position's window.
      const bool whole = t0 + kTileKeys - 1 <= p_first && t0 >= lo_last;
      // One tile step of the wave's row blocks; MASK = false for a whole tile.
      // Each K and V fragment read from LDS feeds the MFMAs of both row
      // blocks; LDS reads run one block ahead of the MFMAs that use them.
      auto step = [&](auto mask) {
        constexpr bool MASK = decltype(mask)::value;
        // Scores: each row block's chain over the head dim in ascending k-steps
        // (block_scores' order), one K fragment feeding both chains.
        f32x4 sc[kRB][4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
          for (int k = 0; k < kRB; ++k) sc[k][blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) {
            const bf16x8 kf = lds_k_frag<D>(tile, blk, ks, r, g);
#pragma unroll
            for (int k = 0; k < kRB; ++k) sc[k][blk] = mfma(kf, q[k].f[ks], sc[k][blk]);
          }
        }
        TileStep ts[kRB];
        bool need = false;
#pragma unroll
        for (int k = 0; k < kRB; ++k) {
          ts[k] = tile_softmax<MASK>(st[k].m, st[k].z, sc[k], c, t0, lo[k], limit[k], g);
          need = need || rescale_lane<MASK>(ts[k]);
        }
        // Once a row's maximum settles its alpha is 1 and the rescale is the
        // identity; a wave whose rows all have alpha = 1 skips it.
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
          for (int k = 0; k < kRB; ++k)
#pragma unroll
            for (int mb = 0; mb < D / 16; ++mb) st[k].u[mb] = pv_rescale<MASK>(st[k].u[mb], ts[k]);
        }
#pragma unroll
        for (int mb = 0; mb < D / 16; ++mb) {
          bf16x8 vf[2];
#pragma unroll
          for (int ks2 = 0; ks2 < 2; ++ks2) vf[ks2] = lds_v_frag<D>(tile, mb, ks2, r, g);
#pragma unroll
          for (int k = 0; k < kRB; ++k) st[k].u[mb] = pv_accumulate<MASK>(st[k].u[mb], vf, ts[k]);
        }
#pragma unroll
        for (int k = 0; k < kRB; ++k) commit_scalars<MASK>(st[k].m, st[k].z, ts[k]);
      };
      if (needs(t)) {
        if (whole)
          step(std::false_type{});
        else
          step(std::true_type{});
      }
      // Split end: fold this split's state into the rows that see a key of
      // it.  A row's first such split seeds its merge; a row that sees a
      // later split finds the merge so far in the workspace.  The fold of a
      // row's last split finalises the row.
      const int sp = t0 / S;
      if (t == T || (t0 + kTileKeys) % S == 0) {
#pragma unroll
        for (int k = 0; k < kRB; ++k) {
          if (limit[k] >= sp * S && lo[k] < sp * S + S) {
            const size_t ridx = (size_t)(q0 + ii[k]) * a.Hq + hq;
            if (split_grid && sp == 0)
              store_split<D>(a.ws_u, a.ws_mz, st[k], ridx, g);
            else if (split_grid)
              store_split<D>(a.sg_u, a.sg_mz, st[k], split_entry(a, b, ii[k], sp, hq, ppg), g);
            else
              fold_split<D>(a, st[k], ridx, sp == lo[k] / S, sp == limit[k] / S, vs, g);
          }
          st[k].init();
        }
      }
    }
    if (more) {
      __syncthreads();
      land(s + 1, btn);
      if constexpr (FP8) __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < kStageTiles; ++k) btn[k] = bta[k];
  }
}

template <int D, bool FP8, int RB>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  if (a.B == 0 || a.max_q_len == 0) return hipSuccess;
  const int64_t pairs = (int64_t)a.B * a.Hkv;
  const int64_t units = pairs * a.max_row_blocks + (a.split_rbs ? pairs * a.split_rbs * (a.max_splits - 1) : 0);
  const int lds = 2 * kStageTiles * tile_lds_bytes<D>();  // two slots of a stage (64 KiB at head_dim 128)
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<D, FP8, RB>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((prefill_kernel<D, FP8, RB>), dim3((unsigned)units), dim3(kPrefillThreads), lds, st, a);
  if (!a.split_rbs) return hipGetLastError();
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t items = (int64_t)a.B * a.split_rbs * prefill_positions_per_block(a.group, RB) * a.Hq;
  hipLaunchKernelGGL((prefill_merge_kernel<D, FP8>), dim3((unsigned)((items + kMergeWaves - 1) / kMergeWaves)),
                     dim3(64 * kMergeWaves), 0, st, a);
  return hipGetLastError();
}

int prefill_rows_per_wave(bool fp8, int64_t units_two_blocks) {
  return fp8 || units_two_blocks < kSmallLaunchUnits ? 1 : row_blocks_per_wave<false>();
}

int prefill_positions_per_block(int group, int rb) { return (kRows / group) * rb * kPrefillWaves; }

hipError_t launch_prefill(int D, bool fp8, const PrefillArgs& a, hipStream_t st) {
  if (a.rb != 1 && (fp8 || a.rb != row_blocks_per_wave<false>())) return hipErrorInvalidValue;
  if (D == 128 && fp8) return launch_prefill_t<128, true, 1>(a, st);
  if (D == 128 && a.rb == 1) return launch_prefill_t<128, false, 1>(a, st);
  if (D == 128) return launch_prefill_t<128, false, 2>(a, st);
  if (D == 64 && fp8) return launch_prefill_t<64, true, 1>(a, st);
  if (D == 64 && a.rb == 1) return launch_prefill_t<64, false, 1>(a, st);
  if (D == 64) return launch_prefill_t<64, false, 2>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace ia
