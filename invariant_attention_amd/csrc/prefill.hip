// prefill.hip -- chunked / whole prefill (causal, grouped-query) with K/V
// tiles staged in LDS and shared by the 4 waves of a workgroup.  All
// value-relevant arithmetic is in arith.hpp; each row runs exactly the
// decode row's operations at its position (Vosti §5.3, App. A.1-A.5).
//
// Rows.  A wave owns 16 rows = 16/g consecutive positions x the g query
// heads of one kv head; a workgroup of 4 waves owns 4 * 16/g consecutive
// positions of one sequence.  Two workgroups share a compute unit (2 x 64 KiB
// of LDS, 2 waves per SIMD) and run out of step with each other, so one's
// value products overlap the other's softmax; one workgroup of 8 waves per
// compute unit, whose waves meet at every tile's barrier, measured ~3% slower.  The workgroup walks 64-key tiles 0..T of the
// keys its last row can see; splits of S keys start a fresh state, and at a
// split's end every row that reaches into it folds the split's state into its
// running merge (ascending order, as in decode).  Tiles past all of a wave's
// positions are skipped, which is the identity on its rows' states.
//
// Staging.  Tiles pass through two LDS slots: while the waves compute tile t,
// the workgroup's loads of tile t+1 are in flight into the other slot; one
// barrier per tile.  bf16 pages go from memory straight into LDS
// (global_load_lds, 1 KiB runs of K and V), with a zero fill of the keys past
// the sequence end only in a tile that has them; e4m3 pages go through
// registers, where they are zero filled and converted to bf16 (exactly).
// K keeps the pages' own layout; V is staged in operand order:
//   LDS K: [4 blocks][D/8 chunks][16 positions] x 16 B, K slot s of a page
//          at position s (even page blocks) or s ^ 8 (odd ones)
//   LDS V: [2 k-steps][D/16 dim blocks][64 lanes] x 16 B, lane 16 g + r
//          holding dim 16 mb + r, tokens 8 (g % 2) .. + 7 of page block
//          2 ks2 + g / 2 (its V^T operand of the value product)
// Every operand fragment is one 16-byte LDS read per lane.  A K read takes 8
// consecutive slots of each of two page blocks (arith.hpp's key-to-slot
// mapping); the swap of 128-byte halves in odd page blocks puts them on
// disjoint banks.  A V read is 1 KiB in lane order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "arith.hpp"
#include "launch.hpp"
#include "pages.hpp"

namespace ia {

constexpr int kPrefillWaves = 4;  // per workgroup; 2 workgroups per compute unit
constexpr int kPrefillThreads = 64 * kPrefillWaves;
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

// The page block, and the byte offset of the V run inside its (page, kv head)
// block, held by 16-byte unit c of a tile's LDS V (unit c = run c / 64 =
// (ks2, mb), lane c % 64 of that run's operand).
template <int D, bool FP8>
__device__ __forceinline__ void v_unit(int c, int& blk, uint32_t& off, int& first_tok) {
  const int run = c >> 6, l = c & 63;
  const int ks2 = run / (D / 16), mb = run % (D / 16);
  const int r = l & 15, g = l >> 4;
  blk = v_block(ks2, g);
  off = v_frag_off<D, FP8>(mb, r, g);
  first_tok = 8 * (g & 1);
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

// Issues the global loads of the tile at t0 for this thread's share.  btv
// holds the tile's block-table entries in lanes 0..3.
template <int D, bool FP8>
__device__ __forceinline__ void stage_load(Stage<D, FP8>& st, const uint8_t* kc, const uint8_t* vc, int btv, int t0,
                                           int n, int num_pages, int kvh, int Hkv, int tid) {
  using S = Stage<D, FP8>;
  constexpr int EB = Raw<FP8>::kElemBytes;
  constexpr size_t kHeadBytes = (size_t)D * 16 * EB;
  const int4 e = make_int4(__builtin_amdgcn_readlane(btv, 0), __builtin_amdgcn_readlane(btv, 1),
                           __builtin_amdgcn_readlane(btv, 2), __builtin_amdgcn_readlane(btv, 3));
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

// ---- bf16 tiles: direct global -> LDS loads (global_load_lds) --------------
// The data moves from the pages to LDS without passing through registers.
// Each instruction of a wave fills a contiguous 1 KiB LDS run, 16 bytes per
// lane in lane order, each lane from an address of its own.  A page block's
// K (D x 16 values) is contiguous in its page, so a tile's K is 4 blocks x
// D/32 copies of 4 chunk rows (the lanes of an odd block fetch their row's
// tokens in k_pos order); a V copy fills one operand run of the V region,
// each lane fetching the 16 bytes v_unit assigns it.
template <int D>
__device__ __forceinline__ void direct_issue(uint8_t* slot, const uint8_t* kc, const uint8_t* vc, const TilePages& tp,
                                             int kvh, int Hkv, int w, int lane) {
  constexpr size_t kHeadBytes = (size_t)D * 16 * 2;          // one (page, kv head) block
  constexpr int kChunks = kTileKeys * D * 2 / 1024;           // 1 KiB copies per tile and tensor
  constexpr int kKBytes = kTileKeys * D * 2;
  static_assert(kChunks % kPrefillWaves == 0, "chunks must divide over waves");
  auto head = [&](const uint8_t* pool, int pg) { return pool + ((size_t)pg * Hkv + kvh) * kHeadBytes; };
  const int kl = (lane & ~15) | k_pos(1, lane & 15);  // the source position of an odd block's lane
#pragma unroll
  for (int i = 0; i < kChunks / kPrefillWaves; ++i) {
    const int ch = i * kPrefillWaves + w;  // wave-uniform
    const int blk = ch / (kChunks / 4), part = ch % (kChunks / 4);
    const int pg = blk == 0 ? tp.page[0] : (blk == 1 ? tp.page[1] : (blk == 2 ? tp.page[2] : tp.page[3]));
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(head(kc, pg) + part * 1024 + ((blk & 1) ? kl : lane) * 16),
                                     (lds_void_t*)(slot + ch * 1024), 16, 0, 0);
    // V: run ch; the lane's run lies in page block 2 ks2 + (lane / 32).
    int vb, first;
    uint32_t off;
    v_unit<D, false>(ch * 64 + lane, vb, off, first);
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(head(vc, select4(vb, tp.page)) + off),
                                     (lds_void_t*)(slot + kKBytes + ch * 1024), 16, 0, 0);
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

__device__ __forceinline__ bool tile_partial(const TilePages& tp) {
  return (tp.valid[0] & tp.valid[1] & tp.valid[2] & tp.valid[3]) != 16;
}

// Operand fragments of one tile from LDS: the K of score block sb (the key
// of MFMA row r lies in page block k_block(sb, r)), and the V^T runs of dim
// block mb (lane order).
template <int D>
__device__ __forceinline__ void lds_k_block(const uint8_t* lds, int sb, int r, int g, bf16x8 (&kf)[D / 32]) {
  const int blk = k_block(sb, r);
  const int pos = k_pos(blk, k_slot(k_token(sb, r)));
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    kf[ks] = __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const uint4*>(lds + ((size_t)(blk * (D / 8) + 4 * ks + g) * 16 + pos) * 16));
}
template <int D>
__device__ __forceinline__ void lds_v_block(const uint8_t* lds, int mb, int r, int g, bf16x8 (&vf)[2]) {
  constexpr int kKBytes = kTileKeys * D * 2;
#pragma unroll
  for (int ks2 = 0; ks2 < 2; ++ks2)
    vf[ks2] = __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const uint4*>(lds + kKBytes + (ks2 * (D / 16) + mb) * 1024 + (16 * g + r) * 16));
}

// Scores of one tile for the wave's rows, from the LDS copy of its K.
template <int D>
__device__ __forceinline__ void lds_tile_scores(const uint8_t* tile, const QFrag<D>& q, int r, int g,
                                                f32x4 (&sc)[4]) {
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    bf16x8 kf[D / 32];
    lds_k_block<D>(tile, blk, r, g, kf);
    sc[blk] = block_scores<D>(kf, q);
  }
}

template <int D, bool FP8>
__global__ __launch_bounds__(kPrefillThreads, 8 / kPrefillWaves) void prefill_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
  constexpr int kTileBytes = tile_lds_bytes<D>();
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  // Block index -> (sequence b, kv head, row block).  Workgroups go to the 8
  // XCDs round robin (block i to XCD i mod 8), each XCD with its own L2.  The
  // (b, kvh) pairs are dealt to the XCDs, and each XCD runs its pairs one
  // after another, every pair's row blocks heaviest (last) first: the
  // workgroups resident on an XCD at a time are mostly row blocks of one pair
  // and walk the same K/V tiles, which its L2 then serves.  When the pair count
  // is not a multiple of 8 the order is simply row block (from the end), b, kvh.
  const int pairs = a.B * a.Hkv;
  int pair, rbi;
  if (pairs % kXcds == 0) {
    const int xcd = blockIdx.x % kXcds, k = blockIdx.x / kXcds;
    pair = xcd + kXcds * (k / a.max_row_blocks);
    rbi = k % a.max_row_blocks;
  } else {
    pair = blockIdx.x % pairs;
    rbi = blockIdx.x / pairs;
  }
  const int kvh = pair % a.Hkv;
  const int b = pair / a.Hkv;
  const int rb = a.max_row_blocks - 1 - rbi;
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
  const int p_first = n - ql + iw;                                     // first position of the wave
  // Visible keys: lo..p per row, lo = 0 or p - w + 1 under a sliding window
  // of w keys (Vosti App. A.5).  lo_first / lo_last bound the wave's rows.
  const int lo = first_key(p, a.window);
  const int lo_first = first_key(p_first, a.window);
  const int lo_last = first_key(pmax_w, a.window);
  // Whether the wave has a row that sees some key of tile t.
  auto needs = [&](int t) { return t * kTileKeys <= pmax_w && t * kTileKeys + kTileKeys - 1 >= lo_first; };
  float c = a.c;
  if constexpr (FP8) c = c * a.k_scale[kvh];
  const int S = a.split_tokens;

  const int32_t* bt_row = a.block_table + (size_t)b * a.bt_stride;
  const int nblk = (n + 15) >> 4;
  const int T = pmax_wg / kTileKeys;                                   // last tile
  const int T0 = first_key(n - ql + i0, a.window) / kTileKeys;         // first tile
  // Pipeline.  LDS holds two tiles.  While the waves compute tile t from one
  // slot, tile t+1 loads into the other: bf16 pages straight from memory into
  // LDS, e4m3 pages through registers (converted to bf16 after the compute).
  // One barrier per tile publishes the next tile; a tile reaching past the
  // sequence end gets its K and V zero filled between two barriers.
  // Block-table entries run one tile ahead of the loads.
  auto buf = [&](int t) { return lds_raw + (t & 1) * kTileBytes; };
  auto bt_of = [&](int t) { return load_tile_bt(bt_row, kTileKeys * (t < T ? t : T), nblk, lane); };
  auto pages_of = [&](int btv, int t) {
    const int4 e = make_int4(__builtin_amdgcn_readlane(btv, 0), __builtin_amdgcn_readlane(btv, 1),
                             __builtin_amdgcn_readlane(btv, 2), __builtin_amdgcn_readlane(btv, 3));
    return tile_pages_of(e, t * kTileKeys, n, a.num_pages);
  };
  const int wu = __builtin_amdgcn_readfirstlane(w);
  Stage<D, FP8> stg;
  {
    const int bt0 = bt_of(T0);
    const TilePages tp0 = pages_of(bt0, T0);
    if constexpr (FP8) {
      stage_load<D, FP8>(stg, a.k_cache, a.v_cache, bt0, T0 * kTileKeys, n, a.num_pages, kvh, a.Hkv, tid);
      stage_store<D, FP8>(buf(T0), stg, tid);
      __syncthreads();
    } else {
      direct_issue<D>(buf(T0), a.k_cache, a.v_cache, tp0, kvh, a.Hkv, wu, lane);
      __syncthreads();
      if (tile_partial(tp0)) {
        direct_fixup<D>(buf(T0), tp0, tid);
        __syncthreads();
      }
    }
  }
  int bt_next = bt_of(T0 + 1);

  RowState<D> st;
  st.init();
  float M = 0.f, Z = 0.f;
  f32x4 U[D / 16];
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) U[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t = T0; t <= T; ++t) {
    const int t0 = t * kTileKeys;
    const bool more = t < T;
    const int bt_after = bt_of(t + 2);
    const TilePages tpn = pages_of(bt_next, t + 1);
    const uint8_t* tile = buf(t);
    if (more) {
      if constexpr (FP8)
        stage_load<D, FP8>(stg, a.k_cache, a.v_cache, bt_next, t0 + kTileKeys, n, a.num_pages, kvh, a.Hkv, tid);
      else
        direct_issue<D>(buf(t + 1), a.k_cache, a.v_cache, tpn, kvh, a.Hkv, wu, lane);
    }
    // The tile is whole for the wave when all its keys are visible to every
    // stored row: its last key to the first position, its first key to the
    // last position's window.
    const bool whole = t0 + kTileKeys - 1 <= p_first && t0 >= lo_last;
    // One tile step of the wave's rows; MASK = false for a whole tile.  LDS
    // reads run one block ahead of the MFMAs that use them; the first V block
    // is read before the softmax.
    auto step = [&](auto mask) {
      constexpr bool MASK = decltype(mask)::value;
      f32x4 sc[4];
      bf16x8 kf[2][D / 32];
      lds_k_block<D>(tile, 0, r, g, kf[0]);
      // A wave issuing its score or value MFMAs takes precedence over the
      // other wave of its SIMD (another workgroup's), whose softmax then
      // fills the issue slots between the MFMAs.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        if (blk < 3) lds_k_block<D>(tile, blk + 1, r, g, kf[(blk + 1) & 1]);
        sc[blk] = block_scores<D>(kf[blk & 1], q);
      }
      __builtin_amdgcn_s_setprio(0);
      bf16x8 vf[2][2];
      lds_v_block<D>(tile, 0, r, g, vf[0]);
      const TileStep ts = tile_softmax<MASK>(st.m, st.z, sc, c, t0, lo, limit, g);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb) {
        if (mb + 1 < D / 16) lds_v_block<D>(tile, mb + 1, r, g, vf[(mb + 1) & 1]);
        st.u[mb] = pv_block<MASK>(st.u[mb], vf[mb & 1], ts);
      }
      __builtin_amdgcn_s_setprio(0);
      commit_scalars<MASK>(st.m, st.z, ts);
    };
    if (needs(t)) {
      if (whole)
        step(std::false_type{});
      else
        step(std::true_type{});
    }
    if constexpr (FP8) {
      if (more) stage_store<D, FP8>(buf(t + 1), stg, tid);
    }
    // Split end: fold this split's state into the rows that see a key of it;
    // a row's first such split seeds its merge.
    const int s = t0 / S;
    if (t == T || (t0 + kTileKeys) % S == 0) {
      if (limit >= s * S && lo < s * S + S) {
        if (s == lo / S) {
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
    if (more) {
      __syncthreads();
      if constexpr (!FP8) {
        if (tile_partial(tpn)) {
          direct_fixup<D>(buf(t + 1), tpn, tid);
          __syncthreads();
        }
      }
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
  const int lds = 2 * tile_lds_bytes<D>();  // two tile slots (64 KiB at head_dim 128)
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<D, FP8>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
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
