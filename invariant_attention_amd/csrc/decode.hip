// decode.hip -- decode attention: the fixed-split kernel and the ascending
// split merge.  All value-relevant arithmetic is in arith.hpp.
//
// One workgroup of 4 waves per (sequence b, kv head, split s).  The g query
// heads of the group are the rows (padded to 16).  Per 64-key tile, wave w
// computes the scores of score block w (its own 16 keys, all head dims),
// the 4 waves exchange scores through LDS, every wave runs the same softmax
// step on the whole tile, and wave w applies it to dim blocks
// [w * D/64, (w + 1) * D/64) of the value accumulators.  A row's operations
// and their order are those of a single wave's tile step, so the bits equal
// prefill's at the same position; splitting the blocks over waves only
// changes where each operation runs.  Each wave loads exactly the operand
// fragments it consumes, straight from the pages into registers, one tile
// ahead of the compute; nontemporal loads when the host asks for them (each
// byte is read once per call; see ia_config.kv_cache_hint).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "arith.hpp"
#include "launch.hpp"
#include "pages.hpp"

namespace ia {

constexpr int kDecodeWaves = 4;
constexpr int kBtWindowTiles = 256;  // block-table entries staged per LDS refill: 4 per tile
constexpr int kOrderBuckets = 64;  // last-split lengths, in tiles; longer ones share bucket 0
// Launches of at most kSelfOrderMaxB sequences, more than kSelfOrderMinUnits
// units and fewer than take the dispatch-order list have each workgroup find
// its own unit in that order (measured on the Llama-3-8B shape, contexts
// U[512, 8192]: +2.5% at batch 16, +2.8% at batch 48, the same at 32 and 64;
// at batch 8, one round of units, 1.5% slower, hence the lower bound).
constexpr int kSelfOrderMaxB = 64;
constexpr int64_t kSelfOrderMinUnits = 256;

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

// Raw fragments one wave needs for one tile: score block w's K (all k-steps)
// and the V^T runs of its D/64 dim blocks (one per k-step), plus the key
// count of every page block for the zero fill of V.
template <int D, bool FP8>
struct DecodeFrags {
  static constexpr int MB = D / 64;
  typename Raw<FP8>::K k[D / 32];
  typename Raw<FP8>::V8 v[MB][2];
  int valid[4];
};

// Loads the fragments of the tile at t0 given its 4 block-table entries
// (nontemporal loads when NT).  Addresses are a page base chosen per lane
// among two pages plus a 32-bit per-lane offset that is the same for every
// tile.
template <int D, bool FP8, bool NT>
__device__ __forceinline__ void load_decode_frags(DecodeFrags<D, FP8>& f, const uint8_t* kc, const uint8_t* vc,
                                                  const int4& e, int t0, int n, int num_pages, int kvh, int Hkv,
                                                  int w, int r, int g) {
  constexpr int MB = D / 64;
  constexpr int EB = Raw<FP8>::kElemBytes;
  constexpr size_t kHeadBytes = (size_t)D * 16 * EB;  // one (page, kv head) block
  const TilePages tp = tile_pages_of(e, t0, n, num_pages);
  // Score block w: the lane's key lies in page block 2 (w / 2) + r / 8.
  const int kpa = (w >> 1) == 0 ? tp.page[0] : tp.page[2];
  const int kpb = (w >> 1) == 0 ? tp.page[1] : tp.page[3];
  const uint8_t* kp = kc + ((size_t)((r >> 3) ? kpb : kpa) * Hkv + kvh) * kHeadBytes;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) load_page<NT>(kp + k_frag_off<D, FP8>(w, ks, r, g), f.k[ks]);
#pragma unroll
  for (int ks2 = 0; ks2 < 2; ++ks2) {
    // The lane's V run lies in page block 2 ks2 + g / 2.
    const int pg = (g >> 1) ? tp.page[2 * ks2 + 1] : tp.page[2 * ks2];
    const uint8_t* vp = vc + ((size_t)pg * Hkv + kvh) * kHeadBytes;
#pragma unroll
    for (int mbi = 0; mbi < MB; ++mbi) load_page<NT>(vp + v_frag_off<D, FP8>(w * MB + mbi, r, g), f.v[mbi][ks2]);
  }
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) f.valid[blk] = tp.valid[blk];
}

// One tile of a decode unit: wave w's scores of key block w go through LDS
// buffer `xb` to all 4 waves; each wave runs the softmax step of the whole
// tile and the value step of its own dim blocks.  FULL: every key of the tile
// exists (t0 + 64 <= n), so no key is masked and nothing needs zero filling;
// otherwise keys >= n get -inf scores and zero values.  (Their K needs no
// fill: a key's score column depends only on its own K row, and a masked
// score is replaced, never used.)
template <int D, bool FP8, bool FULL>
__device__ __forceinline__ void decode_tile(const DecodeFrags<D, FP8>& f, const QFrag<D>& q, f32x4 (*xb)[64],
                                            float& m, float& z, f32x4 (&u)[D / 64], float c, int t0, int lo,
                                            int limit, int w, int lane, int r, int g) {
  constexpr int MB = D / 64;
  bf16x8 kf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) kf[ks] = k_to_bf16(f.k[ks], true);
  xb[w][lane] = block_scores<D>(kf, q);
  __syncthreads();
  f32x4 sc[4];
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) sc[blk] = xb[blk][lane];
  const TileStep ts = tile_softmax<!FULL>(m, z, sc, c, t0, lo, limit, g);
#pragma unroll
  for (int mbi = 0; mbi < MB; ++mbi) {
    bf16x8 vf[2];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
      vf[ks2] = v8_to_bf16(f.v[mbi][ks2], FULL ? 8 : ((g >> 1) ? f.valid[2 * ks2 + 1] : f.valid[2 * ks2]) - 8 * (g & 1));
    u[mbi] = pv_block(u[mbi], vf, ts);
  }
  commit_scalars(m, z, ts);
}

template <int D, bool FP8>
__device__ __forceinline__ void decode_tile_any(const DecodeFrags<D, FP8>& f, const QFrag<D>& q, f32x4 (*xb)[64],
                                                float& m, float& z, f32x4 (&u)[D / 64], float c, int t0, int n,
                                                int lo, int limit, int w, int lane, int r, int g) {
  if (t0 >= lo && t0 + kTileKeys <= n)
    decode_tile<D, FP8, true>(f, q, xb, m, z, u, c, t0, lo, limit, w, lane, r, g);
  else
    decode_tile<D, FP8, false>(f, q, xb, m, z, u, c, t0, lo, limit, w, lane, r, g);
}

// First key a decode row at position p sees: 0, or p - w + 1 under a sliding
// window of w keys (Vosti App. A.5).
__device__ __forceinline__ int first_key(int p, int window) {
  if (window <= 0) return 0;
  return p - window + 1 > 0 ? p - window + 1 : 0;
}

template <int D, bool FP8, bool NT>
__global__ __launch_bounds__(256, 3) void decode_split_kernel(DecodeArgs a) {
  constexpr int MB = D / 64;
  __shared__ f32x4 xs[2][4][64];  // score exchange, double buffered by tile parity
  __shared__ __attribute__((aligned(16))) int bt_lds[4 * kBtWindowTiles];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  // Which (sequence, split) the workgroup runs: the order list of
  // decode_order_kernel when the launch has one (longest units first), else
  // split-major (every sequence's first split before any second split, and
  // so on).  The choice moves work between workgroups, never changes it.
  const int unit = blockIdx.x;
  const int kvh = unit % a.Hkv;
  int b, s;
  if (a.order) {
    const int e = a.order[unit / a.Hkv];
    if (e < 0) return;  // past the listed units; uniform over the workgroup
    b = e / a.max_splits;
    s = e % a.max_splits;
  } else if (a.self_order) {
    // The same order for a launch of few sequences, found by every
    // workgroup itself instead of by decode_order_kernel: whole splits first
    // (by sequence), then the last splits by decreasing length in tiles (by
    // sequence among equal lengths).  Thread t takes sequence t.
    __shared__ int nf_s[kSelfOrderMaxB], q_s[kSelfOrderMaxB], pick[2];
    const int t = threadIdx.x;
    if (t == 0) pick[0] = -1;
    if (t < a.B) {
      const int nt = clamp_len(a.seq_lens[t], a.max_seq_len);
      const int St = split_len(a.policy, a.split_tokens, nt, a.B);
      const int nf = nt / St;
      const int tiles = (nt - nf * St + kTileKeys - 1) / kTileKeys;
      nf_s[t] = nf;
      q_s[t] = tiles > 0 ? kOrderBuckets - (tiles < kOrderBuckets ? tiles : kOrderBuckets) : -1;
    }
    __syncthreads();
    const int e = unit / a.Hkv;
    if (t < a.B) {
      int f0 = 0, whole = 0, rank = 0;
      const int qt = q_s[t];
      for (int i = 0; i < a.B; ++i) {
        const int nfi = nf_s[i], qi = q_s[i];
        whole += nfi;
        f0 += i < t ? nfi : 0;
        rank += (qi >= 0 && (qi < qt || (qi == qt && i < t))) ? 1 : 0;
      }
      if (e >= f0 && e < f0 + nf_s[t]) {
        pick[0] = t;
        pick[1] = e - f0;
      }
      if (qt >= 0 && e == whole + rank) {
        pick[0] = t;
        pick[1] = nf_s[t];
      }
    }
    __syncthreads();
    b = pick[0];
    s = pick[1];
    if (b < 0) return;  // past the listed units; uniform over the workgroup
  } else {
    b = (unit / a.Hkv) % a.B;
    s = unit / a.Hkv / a.B;
  }
  const int n = clamp_len(a.seq_lens[b], a.max_seq_len);
  const int S = split_len(a.policy, a.split_tokens, n, a.B);
  const int nsplit = (n + S - 1) / S;
  const int p = n - 1;
  const int lo = first_key(p, a.window);
  // Splits past the sequence, and (sliding window) splits before the window,
  // hold no visible key: no unit runs for them and the merge skips them.
  if (s >= nsplit || (s + 1) * S <= lo) return;  // uniform over the workgroup
  const bool row_ok = r < a.group;
  const int limit = row_ok ? p : -1;
  const int hq = kvh * a.group + (row_ok ? r : 0);
  const QFrag<D> q = load_q<D>(a.q + ((size_t)b * a.Hq + hq) * D, row_ok, g);
  float c = a.c;
  if constexpr (FP8) c = c * a.k_scale[kvh];

  const int k_begin = max(s * S, lo & ~(kTileKeys - 1));  // the window's first tile, if later
  const int k_end = min(s * S + S, n);
  const int ntiles = (k_end - k_begin + kTileKeys - 1) / kTileKeys;
  const int32_t* bt_row = a.block_table + (size_t)b * a.bt_stride;
  const int nblk = (n + 15) >> 4;

  float m = neg_inf(), z = 0.f;
  f32x4 u[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) u[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The split's block-table entries are staged in LDS, kBtWindowTiles tiles
  // at a time, so page lookups never wait on the memory loads in flight.
  const int tid = threadIdx.x;
  const uint8_t* kc = a.k_cache;
  const uint8_t* vc = a.v_cache;
  const int np = a.num_pages;
  DecodeFrags<D, FP8> fa, fb;
  for (int w0 = 0; w0 < ntiles; w0 += kBtWindowTiles) {
    const int wn = min(ntiles - w0, kBtWindowTiles);
    __syncthreads();
    const int e0 = (k_begin >> 4) + 4 * w0;
    for (int i = tid; i < 4 * wn; i += 64 * kDecodeWaves) {
      const int e = e0 + i < nblk ? e0 + i : nblk - 1;
      bt_lds[i] = bt_row[e];
    }
    __syncthreads();

    // Software pipeline over the window's tiles, unrolled by two so no
    // register set is ever copied: while tile lt computes from one fragment
    // set, tile lt+1 loads into the other.  A tile index past the window
    // clamps to its last tile (a re-read that hits the cache), so every load
    // is unconditional and a wait for one tile's operands never drains the
    // next tile's loads.
    const int last = wn - 1;
    auto load = [&](DecodeFrags<D, FP8>& f, int lt) {
      lt = lt < last ? lt : last;
      const int4 e = *reinterpret_cast<const int4*>(&bt_lds[4 * lt]);
      const int4 eu = make_int4(__builtin_amdgcn_readfirstlane(e.x), __builtin_amdgcn_readfirstlane(e.y),
                                __builtin_amdgcn_readfirstlane(e.z), __builtin_amdgcn_readfirstlane(e.w));
      load_decode_frags<D, FP8, NT>(f, kc, vc, eu, k_begin + kTileKeys * (w0 + lt), n, np, kvh, a.Hkv, w, r, g);
    };
    load(fa, 0);
    for (int lt = 0; lt < wn; lt += 2) {
      load(fb, lt + 1);
      __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before waiting on this tile
      decode_tile_any<D, FP8>(fa, q, xs[0], m, z, u, c, k_begin + kTileKeys * (w0 + lt), n, lo, limit, w, lane, r,
                            g);
      if (lt + 1 >= wn) break;
      load(fa, lt + 2);
      __builtin_amdgcn_sched_barrier(0);
      decode_tile_any<D, FP8>(fb, q, xs[1], m, z, u, c, k_begin + kTileKeys * (w0 + lt + 1), n, lo, limit, w, lane,
                            r, g);
    }
  }

  if (row_ok) {
    const size_t row = ((size_t)b * a.max_splits + s) * a.Hq + hq;
    float* uo = a.ws_u + row * D;
#pragma unroll
    for (int mbi = 0; mbi < MB; ++mbi) *reinterpret_cast<f32x4*>(uo + 16 * (w * MB + mbi) + 4 * g) = u[mbi];
    if (w == 0 && g == 0) *reinterpret_cast<f32x2*>(a.ws_ml + row * 2) = f32x2{m, z};
  }
}

// ---------------------------------------------------------------------------
// The wide decode kernel: bitwise equal to decode_split_kernel, for launches
// with few units.
//
// Within a split the split kernel is one chain of tile steps, and with few
// units the machine waits on that chain.  Most of a step does not need the
// chain's state: the scores of a tile, its row maximum, and -- given the
// running maximum before the tile -- its weights and their row sum.  The
// running maximum before tile t is a fold of fmaxf over the earlier tiles'
// row maxima, which every wave can form exactly in the same order.  So here
// the 8 waves of a unit take a chunk of 8 tiles at a time:
//   A. wave i scores tile i of the chunk and forms its row maxima;
//   B. after a barrier, wave i folds the running maximum up to its tile and
//      forms the tile's weights (hi/lo B operands) and row sum, into LDS;
//   C. after a barrier, wave w runs the value chain of dim block w over the
//      chunk's tiles (U * alpha, then the four MFMAs of pv_block) and every
//      wave folds z = z * alpha + sum.
// Every operation on a row's values is the split kernel's, with the same
// operands in the same order (tile_max, max_update, tile_weights, z_update
// and pv_block are the functions tile_softmax and the split kernel use), so
// the partial (m, z, U) of each split and hence the output bits are the same;
// only the schedule differs.  The partials go to the same workspace and the
// same merge kernel folds them.
constexpr int kWideWaves = 8;
constexpr int kWideChunk = kWideWaves;  // tiles per chunk: one per wave in A and B
constexpr int kWideMaxTiles = 256;      // longest split the wide kernel takes: 16384 keys

template <int D, bool FP8>
struct WideK {  // K of one tile: 4 score blocks x D/32 k-steps
  typename Raw<FP8>::K k[4][D / 32];
};
template <int D, bool FP8>
struct WideV {  // V^T of one dim block of one tile: one run per k-step
  typename Raw<FP8>::V8 v[2];
};

template <int D, bool FP8>
__global__ __launch_bounds__(64 * kWideWaves) void decode_wide_kernel(DecodeArgs a) {
  constexpr int EB = Raw<FP8>::kElemBytes;
  constexpr size_t kHeadBytes = (size_t)D * 16 * EB;
  constexpr int kDimBlocks = D / 16;
  __shared__ __attribute__((aligned(16))) uint4 pw[kWideChunk][4][64];  // weights of each tile, per lane
  __shared__ float mxs[kWideChunk][16];                                   // row maxima
  __shared__ __attribute__((aligned(16))) float als[16][kWideChunk];     // alpha per row and tile
  __shared__ __attribute__((aligned(16))) float sms[16][kWideChunk];     // row sums per row and tile
  __shared__ __attribute__((aligned(16))) int bts[4 * kWideMaxTiles];    // the split's block-table entries
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  // The dim block whose V the wave loads: its own (waves past the last dim
  // block at head_dim 64 load a copy they never use, so that every wave
  // issues the same loads and each wait covers exactly the loads it needs).
  const int wd = w % kDimBlocks;
  const int unit = blockIdx.x;  // split-major, as the split kernel without an order list
  const int kvh = unit % a.Hkv;
  const int b = (unit / a.Hkv) % a.B;
  const int s = unit / a.Hkv / a.B;
  const int n = clamp_len(a.seq_lens[b], a.max_seq_len);
  const int S = split_len(a.policy, a.split_tokens, n, a.B);
  const int nsplit = (n + S - 1) / S;
  const int p = n - 1;
  const int lo = first_key(p, a.window);
  if (s >= nsplit || (s + 1) * S <= lo) return;  // uniform over the workgroup
  const bool row_ok = r < a.group;
  const int limit = row_ok ? p : -1;
  const int hq = kvh * a.group + (row_ok ? r : 0);
  const QFrag<D> q = load_q<D>(a.q + ((size_t)b * a.Hq + hq) * D, row_ok, g);
  float c = a.c;
  if constexpr (FP8) c = c * a.k_scale[kvh];
  const int k_begin = max(s * S, lo & ~(kTileKeys - 1));
  const int k_end = min(s * S + S, n);
  const int ntiles = (k_end - k_begin + kTileKeys - 1) / kTileKeys;
  const int32_t* bt_row = a.block_table + (size_t)b * a.bt_stride;
  const int nblk = (n + 15) >> 4;
  const uint8_t* kc = a.k_cache;
  const uint8_t* vc = a.v_cache;
  // A tile takes the masked step unless all its keys exist and lie in the
  // window (the split kernel's rule), and a masked tile with no visible key
  // leaves the row's state as it is.
  auto full = [&](int t0) { return t0 >= lo && t0 + kTileKeys <= n; };
  auto visible = [&](int t0) { return full(t0) || (t0 <= limit && t0 + kTileKeys - 1 >= lo); };
  // The split's block-table entries, staged in LDS once (clamped to the
  // sequence's last block); a tile index past the split reads the last tile's.
  {
    const int e0 = k_begin >> 4;
    // (The host launches this kernel only for splits of at most
    // kWideMaxTiles tiles; the bound keeps LDS in range regardless.)
    for (int i = threadIdx.x; i < 4 * min(ntiles, kWideMaxTiles); i += 64 * kWideWaves) {
      const int e = e0 + i < nblk ? e0 + i : nblk - 1;
      bts[i] = bt_row[e];
    }
  }
  __syncthreads();
  auto pages = [&](int t) {
    t = t < ntiles ? t : ntiles - 1;
    t = t < kWideMaxTiles ? t : kWideMaxTiles - 1;
    const int4 e = *reinterpret_cast<const int4*>(&bts[4 * t]);
    const int4 eu = make_int4(__builtin_amdgcn_readfirstlane(e.x), __builtin_amdgcn_readfirstlane(e.y),
                              __builtin_amdgcn_readfirstlane(e.z), __builtin_amdgcn_readfirstlane(e.w));
    return tile_pages_of(eu, k_begin + kTileKeys * t, n, a.num_pages);
  };

  // Loads run one chunk ahead: the K of a wave's tile in the next chunk is
  // issued once this chunk's scores are formed, the V of its dim block once
  // this chunk's value chain is done.  A tile past the split re-reads the
  // split's last tile, which stays in bounds and is never used.
  // vv[i] packs the key counts of tile i's 4 page blocks, 5 bits each.
  auto load_v = [&](WideV<D, FP8> (&vr)[kWideChunk], int (&vv)[kWideChunk], int c0) {
#pragma unroll
    for (int i = 0; i < kWideChunk; ++i) {
      const TilePages tp = pages(c0 + i);
      vv[i] = tp.valid[0] | (tp.valid[1] << 5) | (tp.valid[2] << 10) | (tp.valid[3] << 15);
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const int pg = (g >> 1) ? tp.page[2 * ks2 + 1] : tp.page[2 * ks2];
        const uint8_t* base = vc + ((size_t)pg * a.Hkv + kvh) * kHeadBytes;
        load_page<false>(base + v_frag_off<D, FP8>(wd, r, g), vr[i].v[ks2]);
      }
    }
  };
  auto load_k = [&](WideK<D, FP8>& kr, int c0) {
    const TilePages kp = pages(c0 + w);
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const int pg = (r >> 3) ? kp.page[2 * (sb >> 1) + 1] : kp.page[2 * (sb >> 1)];
      const uint8_t* base = kc + ((size_t)pg * a.Hkv + kvh) * kHeadBytes;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) load_page<false>(base + k_frag_off<D, FP8>(sb, ks, r, g), kr.k[sb][ks]);
    }
  };

  float m = neg_inf(), z = 0.f;  // the running state after the chunks so far
  f32x4 u = {0.f, 0.f, 0.f, 0.f};  // dim block w (waves w < D/16)
  WideV<D, FP8> vr[kWideChunk];
  int vvalid[kWideChunk];
  WideK<D, FP8> kr;
  // (K before V, the order of the loop's own prefetches, so the wait for a
  // chunk's K never has to drain its V.)
  load_k(kr, 0);
  __builtin_amdgcn_sched_barrier(0);
  load_v(vr, vvalid, 0);
  __builtin_amdgcn_sched_barrier(0);
  for (int c0 = 0; c0 < ntiles; c0 += kWideChunk) {
    const int nt = min(kWideChunk, ntiles - c0);
    // A: scores and row maxima of tile w of the chunk.
    const bool mine = w < nt;
    const int tw0 = k_begin + kTileKeys * (c0 + (mine ? w : 0));
    TileMax tm = {};
    if (mine) {
      f32x4 sc[4];
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        bf16x8 kf[D / 32];
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) kf[ks] = k_to_bf16(kr.k[blk][ks], true);
        sc[blk] = block_scores<D>(kf, q);
      }
      tm = full(tw0) ? tile_max<false>(sc, c, tw0, lo, limit, g) : tile_max<true>(sc, c, tw0, lo, limit, g);
      if (g == 0) mxs[w][r] = tm.mx;
    }
    __builtin_amdgcn_sched_barrier(0);
    load_k(kr, c0 + kWideChunk);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    // B: the running maximum before tile w, then its weights and row sum.
    if (mine) {
      float mp = m;
      for (int i = 0; i < w; ++i) mp = max_update(mp, mxs[i][r], visible(k_begin + kTileKeys * (c0 + i)));
      float sum;
      const TileStep ts = full(tw0) ? tile_weights<false>(mp, tm, c, tw0, lo, limit, g, sum)
                                    : tile_weights<true>(mp, tm, c, tw0, lo, limit, g, sum);
      pw[w][0][lane] = __builtin_bit_cast(uint4, ts.phi[0]);
      pw[w][1][lane] = __builtin_bit_cast(uint4, ts.plo[0]);
      pw[w][2][lane] = __builtin_bit_cast(uint4, ts.phi[1]);
      pw[w][3][lane] = __builtin_bit_cast(uint4, ts.plo[1]);
      if (g == 0) {
        als[r][w] = ts.alpha;
        sms[r][w] = sum;
      }
    }
    for (int i = 0; i < nt; ++i) m = max_update(m, mxs[i][r], visible(k_begin + kTileKeys * (c0 + i)));
    // Zero fill of the chunk's V past the sequence end, in place (only a tile
    // that is not full has such keys: a uniform branch).
#pragma unroll
    for (int i = 0; i < kWideChunk; ++i) {
      if (!full(k_begin + kTileKeys * (c0 + i))) {
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2)
          vr[i].v[ks2] = v8_keep(vr[i].v[ks2], ((vvalid[i] >> (5 * v_block(ks2, g))) & 31) - 8 * (g & 1));
      }
    }
    __syncthreads();
    // C: the z chain and the value chain of dim block w, tile by tile, with
    // no branch: a slot past the chunk (i >= nt) is a step with no visible
    // key, which pv_block and the z update turn into the identity.
    float alv[kWideChunk], smv[kWideChunk];
#pragma unroll
    for (int i = 0; i < kWideChunk; i += 4) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(&als[r][i]);
      const f32x4 s4 = *reinterpret_cast<const f32x4*>(&sms[r][i]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        alv[i + j] = a4[j];
        smv[i + j] = s4[j];
      }
    }
    bool vis[kWideChunk];
#pragma unroll
    for (int i = 0; i < kWideChunk; ++i) {
      const int t0 = k_begin + kTileKeys * (c0 + i);
      vis[i] = (i < nt) & (full(t0) | ((t0 <= limit) & (t0 + kTileKeys - 1 >= lo)));
      z = vis[i] ? z_update(z, alv[i], smv[i]) : z;
    }
    if (w < kDimBlocks) {
#pragma unroll
      for (int i = 0; i < kWideChunk; ++i) {
        TileStep ts;
        ts.alpha = alv[i];
        ts.any_visible = vis[i];
        ts.phi[0] = __builtin_bit_cast(bf16x8, pw[i][0][lane]);
        ts.plo[0] = __builtin_bit_cast(bf16x8, pw[i][1][lane]);
        ts.phi[1] = __builtin_bit_cast(bf16x8, pw[i][2][lane]);
        ts.plo[1] = __builtin_bit_cast(bf16x8, pw[i][3][lane]);
        bf16x8 vf[2];
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) vf[ks2] = v8_to_bf16(vr[i].v[ks2], 8);  // already zero filled
        // The masked form's final select is the identity where every key is
        // visible, so one form serves full and masked tiles.
        u = pv_block<true>(u, vf, ts);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_v(vr, vvalid, c0 + kWideChunk);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // the next chunk rewrites the LDS tables
  }

  if (row_ok) {
    const size_t row = ((size_t)b * a.max_splits + s) * a.Hq + hq;
    if (w < kDimBlocks) *reinterpret_cast<f32x4*>(a.ws_u + row * D + 16 * w + 4 * g) = u;
    if (w == 0 && g == 0) *reinterpret_cast<f32x2*>(a.ws_ml + row * 2) = f32x2{m, z};
  }
}

// ---------------------------------------------------------------------------
// The spread decode kernels: bitwise equal to decode_split_kernel, for
// launches with few split units.
//
// A split unit of the split kernel is one chain of tile steps on one compute
// unit, and a compute unit streams only a few tens of GB/s, so a launch of a
// few dozen units (one sequence, or a handful) leaves most of the chip idle
// and most of HBM unused.  Here a split's work is spread over many compute
// units in three launches (Vosti, Discussion: a decode kernel that gives one
// sequence several compute units for partially filled waves, with the same
// accumulation order as the kernel for full waves):
//   decode_score_kernel, one wave per (unit, tile): loads the tile's K and
//     forms its scores (block_scores) and tile_max (masked scaled scores and
//     their row maximum) for the stored rows;
//   decode_weight_kernel, one wave per (unit, tile): folds the running
//     maximum before its tile from the earlier tiles' row maxima (an exact
//     fmaxf fold in tile order, the split kernel's max updates), then runs
//     tile_weights: alpha, the weights as hi/lo bf16 B operands, and their
//     row sum;
//   decode_value_kernel, one wave per (unit, 16-dim block): walks the split's
//     tiles in order running the only true chain, the z update and pv_block
//     on its own dims' V.
// Every value is formed by the functions the split kernel's tile step uses,
// from the same operands, in the same order, and an fp32 or bf16 value
// stored and read back keeps its bits; so each split partial, and the merged
// output, is the split kernel's.  Slots are indexed
// ((b * max_splits + s) * Hkv + kvh) * tps + tile, tps being the longest
// split of the launch in tiles; a slot past its split's tiles is never
// written or read.  A slot holds, per stored row, 64 fp32 scores, which the
// weight kernel then overwrites with the row's hi/lo weights (the same 256
// bytes); plus the row maximum, and alpha with the row sum.

// (b, s, kvh) of a unit in the spread kernels' order.
struct SpreadUnit {
  int b, s, kvh;
};
__device__ __forceinline__ SpreadUnit spread_unit(const DecodeArgs& a, int us) {
  SpreadUnit u;
  u.kvh = us % a.Hkv;
  const int bs = us / a.Hkv;
  u.s = bs % a.max_splits;
  u.b = bs / a.max_splits;
  return u;
}

// Offset (in floats) of lane (r, g)'s 16 bytes of part `part` (a key block's
// four scores, later one of the four weight operands) in a slot:
// [4 parts][4 lane groups][group rows][16 bytes].
__device__ __forceinline__ size_t spread_x_off(size_t slot, int group, int part, int g, int r) {
  return ((slot * 16 + (size_t)(4 * part + g)) * group + r) * 4;
}

// The split geometry of one unit, as every decode kernel computes it.
struct SpreadSplit {
  int n, p, lo, k_begin, ntiles;
  bool live;  // the split holds a key the row sees
};
__device__ __forceinline__ SpreadSplit spread_split(const DecodeArgs& a, const SpreadUnit& un) {
  SpreadSplit sp;
  sp.n = clamp_len(a.seq_lens[un.b], a.max_seq_len);
  const int S = split_len(a.policy, a.split_tokens, sp.n, a.B);
  const int nsplit = (sp.n + S - 1) / S;
  sp.p = sp.n - 1;
  sp.lo = first_key(sp.p, a.window);
  sp.live = !(un.s >= nsplit || (un.s + 1) * S <= sp.lo);
  sp.k_begin = max(un.s * S, sp.lo & ~(kTileKeys - 1));
  const int k_end = min(un.s * S + S, sp.n);
  sp.ntiles = sp.live ? (k_end - sp.k_begin + kTileKeys - 1) / kTileKeys : 0;
  return sp;
}

// The split kernel's rules for a tile at t0: unmasked step when all its keys
// exist and lie in the window; a tile holds a key the row sees.
__device__ __forceinline__ bool tile_full(int t0, int lo, int n) { return t0 >= lo && t0 + kTileKeys <= n; }
__device__ __forceinline__ bool tile_visible(int t0, int lo, int n, int limit) {
  return tile_full(t0, lo, n) || (t0 <= limit && t0 + kTileKeys - 1 >= lo);
}

template <int D, bool FP8>
__global__ __launch_bounds__(64) void decode_score_kernel(DecodeArgs a) {
  constexpr int EB = Raw<FP8>::kElemBytes;
  constexpr size_t kHeadBytes = (size_t)D * 16 * EB;
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const size_t slot = blockIdx.x;
  const int lt = (int)(slot % a.tps);
  const SpreadUnit un = spread_unit(a, (int)(slot / a.tps));
  const SpreadSplit sp = spread_split(a, un);
  if (lt >= sp.ntiles) return;  // uniform over the wave (no tile, or no live split)
  const bool row_ok = r < a.group;
  const int limit = row_ok ? sp.p : -1;
  const int hq = un.kvh * a.group + (row_ok ? r : 0);
  const QFrag<D> q = load_q<D>(a.q + ((size_t)un.b * a.Hq + hq) * D, row_ok, g);
  float c = a.c;
  if constexpr (FP8) c = c * a.k_scale[un.kvh];
  const int t0 = sp.k_begin + kTileKeys * lt;
  const int32_t* bt_row = a.block_table + (size_t)un.b * a.bt_stride;
  const int btv = load_tile_bt(bt_row, t0, (sp.n + 15) >> 4, lane);
  const int4 e = make_int4(__builtin_amdgcn_readlane(btv, 0), __builtin_amdgcn_readlane(btv, 1),
                           __builtin_amdgcn_readlane(btv, 2), __builtin_amdgcn_readlane(btv, 3));
  const TilePages tp = tile_pages_of(e, t0, sp.n, a.num_pages);
  // The K of all 4 score blocks, then their scores (the split kernel's
  // key-to-slot mapping: lane (r, g) holds chunk 4 ks + g of the key of MFMA
  // row r).
  typename Raw<FP8>::K kr[4][D / 32];
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    const int pg = (r >> 3) ? tp.page[2 * (sb >> 1) + 1] : tp.page[2 * (sb >> 1)];
    const uint8_t* base = a.k_cache + ((size_t)pg * a.Hkv + un.kvh) * kHeadBytes;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) load_page<false>(base + k_frag_off<D, FP8>(sb, ks, r, g), kr[sb][ks]);
  }
  f32x4 sc[4];
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    bf16x8 kf[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) kf[ks] = k_to_bf16(kr[blk][ks], true);
    sc[blk] = block_scores<D>(kf, q);
  }
  const bool full = tile_full(t0, sp.lo, sp.n);
  TileMax tm;
  if (full)
    tm = tile_max<false>(sc, c, t0, sp.lo, limit, g);
  else
    tm = tile_max<true>(sc, c, t0, sp.lo, limit, g);
  if (row_ok) {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
      *reinterpret_cast<f32x4*>(a.ws_x + spread_x_off(slot, a.group, blk, g, r)) =
          f32x4{tm.s[blk][0], tm.s[blk][1], tm.s[blk][2], tm.s[blk][3]};
    if (g == 0) a.ws_mx[slot * 16 + r] = tm.mx;
  }
}

// The weights of one tile from its stored scores and the running maximum m
// before it; MASK as in the split kernel's step.
template <bool MASK>
__device__ __forceinline__ void spread_weights(const DecodeArgs& a, size_t slot, float m, float c, int t0, int lo,
                                               int limit, int rr, bool row_ok, int g, int r) {
  TileMax tm;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(a.ws_x + spread_x_off(slot, a.group, blk, g, rr));
#pragma unroll
    for (int j = 0; j < 4; ++j) tm.s[blk][j] = x[j];
  }
  tm.mx = a.ws_mx[slot * 16 + rr];
  tm.any_visible = !MASK || (t0 <= limit && t0 + kTileKeys - 1 >= lo);
  float sum;
  const TileStep ts = tile_weights<MASK>(m, tm, c, t0, lo, limit, g, sum);
  if (row_ok) {
    // The scores were read above into registers the weights depend on; the
    // slot's 256 bytes per row now take the four weight operands.
    *reinterpret_cast<uint4*>(a.ws_x + spread_x_off(slot, a.group, 0, g, r)) = __builtin_bit_cast(uint4, ts.phi[0]);
    *reinterpret_cast<uint4*>(a.ws_x + spread_x_off(slot, a.group, 1, g, r)) = __builtin_bit_cast(uint4, ts.plo[0]);
    *reinterpret_cast<uint4*>(a.ws_x + spread_x_off(slot, a.group, 2, g, r)) = __builtin_bit_cast(uint4, ts.phi[1]);
    *reinterpret_cast<uint4*>(a.ws_x + spread_x_off(slot, a.group, 3, g, r)) = __builtin_bit_cast(uint4, ts.plo[1]);
    if (g == 0) *reinterpret_cast<f32x4*>(a.ws_as + (slot * 16 + r) * 4) = f32x4{ts.alpha, sum, tm.mx, 0.f};
  }
}

template <int D, bool FP8>
__global__ __launch_bounds__(64) void decode_weight_kernel(DecodeArgs a) {
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const size_t slot = blockIdx.x;
  const int lt = (int)(slot % a.tps);
  const SpreadUnit un = spread_unit(a, (int)(slot / a.tps));
  const SpreadSplit sp = spread_split(a, un);
  if (lt >= sp.ntiles) return;  // uniform over the wave
  const bool row_ok = r < a.group;
  const int rr = row_ok ? r : 0;  // padding lanes read row 0's slots (never stored)
  const int limit = row_ok ? sp.p : -1;
  float c = a.c;
  if constexpr (FP8) c = c * a.k_scale[un.kvh];
  // The running maximum before this tile: the split kernel's max updates
  // over the split's earlier tiles, in order.
  const size_t slot0 = slot - lt;
  constexpr int kMaxChunk = 32;  // earlier tiles' maxima loaded at once
  float mx[kMaxChunk];
  float m = neg_inf();
  for (int i0 = 0; i0 < lt; i0 += kMaxChunk) {
#pragma unroll
    for (int i = 0; i < kMaxChunk; ++i) mx[i] = a.ws_mx[(slot0 + min(i0 + i, lt - 1)) * 16 + rr];
#pragma unroll
    for (int i = 0; i < kMaxChunk; ++i) {
      const int t0 = sp.k_begin + kTileKeys * (i0 + i);
      m = (i0 + i < lt) ? max_update(m, mx[i], tile_visible(t0, sp.lo, sp.n, limit)) : m;
    }
  }
  const int t0 = sp.k_begin + kTileKeys * lt;
  if (tile_full(t0, sp.lo, sp.n))
    spread_weights<false>(a, slot, m, c, t0, sp.lo, limit, rr, row_ok, g, r);
  else
    spread_weights<true>(a, slot, m, c, t0, sp.lo, limit, rr, row_ok, g, r);
}

template <bool FP8>
struct SpreadFrag {  // one tile's operands for one wave of decode_value_kernel
  uint4 w[4];                    // phi[0], plo[0], phi[1], plo[1]
  f32x4 asm4;                    // alpha, row sum, row maximum, 0
  typename Raw<FP8>::V8 v[2];    // V^T runs of the wave's dim block
};

// The chain half of the split kernel's tile step, for one dim block: the z
// and running-maximum commits, and pv_block.  FULL: the unmasked step (every
// key of the tile exists); otherwise the V of keys past n is zero filled.
template <bool FULL, bool FP8>
__device__ __forceinline__ void spread_chain(const SpreadFrag<FP8>& f, int valid, bool vis, float& m, float& z,
                                             f32x4& u, int g) {
  TileStep ts;
  ts.alpha = f.asm4[0];
  ts.any_visible = vis;
  ts.phi[0] = __builtin_bit_cast(bf16x8, f.w[0]);
  ts.plo[0] = __builtin_bit_cast(bf16x8, f.w[1]);
  ts.phi[1] = __builtin_bit_cast(bf16x8, f.w[2]);
  ts.plo[1] = __builtin_bit_cast(bf16x8, f.w[3]);
  ts.m_new = raise_max(m, f.asm4[2]);
  ts.z_new = z_update(z, f.asm4[0], f.asm4[1]);
  bf16x8 vf[2];
#pragma unroll
  for (int ks2 = 0; ks2 < 2; ++ks2) {
    const int nv = FULL ? 8 : ((valid >> (5 * v_block(ks2, g))) & 31) - 8 * (g & 1);
    vf[ks2] = v8_to_bf16(f.v[ks2], nv);
  }
  u = pv_block(u, vf, ts);
  commit_scalars(m, z, ts);
}

// The value kernel is a workgroup of 4 waves per (unit, 16-dim block).  It
// stages a group of up to GT tiles' operands in LDS with direct global -> LDS
// copies (global_load_lds), each wave copying a quarter of the tiles (a wave
// keeps at most 63 memory instructions in flight), waits for all of them, then
// wave 0 runs the chain over the group from LDS.  GT covers a whole
// 2048-key split at up to 4 query heads per kv head.  Copies per tile: the
// V^T of the dim block from its 4 pages (4 x 512 B bf16 in two copies,
// 4 x 256 B e4m3 in one), the slot's weights (group x 256 B in WC copies of
// 1 KiB), and the rows' (alpha, sum, max) (16 x 16 B in one copy of 4 B per
// lane).
template <int WC>
struct SpreadRing {
  static constexpr int GT = WC == 1 ? 32 : 16;  // tiles per group
  static constexpr int kWaves = 4;
  static constexpr int TPW = GT / kWaves;       // tiles each wave copies
};

template <int D, bool FP8, int WC>
__global__ __launch_bounds__(256) void decode_value_kernel(DecodeArgs a) {
  constexpr int EB = Raw<FP8>::kElemBytes;
  constexpr size_t kHeadBytes = (size_t)D * 16 * EB;
  constexpr int kDimBlocks = D / 16;
  constexpr int GT = SpreadRing<WC>::GT;
  constexpr int TPW = SpreadRing<WC>::TPW;
  constexpr int kVBytes = 4 * 16 * 16 * EB;         // V of one dim block of one tile
  constexpr int kWBytes = WC * 1024;
  constexpr int kSlotBytes = kVBytes + kWBytes + 256;
  static_assert(4 * TPW <= 64, "a wave's block-table entries fit its lanes");
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];  // GT slots, then GT x 4 block-table entries
  int* bt_lds = reinterpret_cast<int*>(ring + GT * kSlotBytes);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int mb = blockIdx.x % kDimBlocks;
  const int us = blockIdx.x / kDimBlocks;
  const SpreadUnit un = spread_unit(a, us);
  const SpreadSplit sp = spread_split(a, un);
  if (!sp.live) return;  // uniform over the workgroup
  const int n = sp.n, lo = sp.lo, k_begin = sp.k_begin, ntiles = sp.ntiles;
  const bool row_ok = r < a.group;
  const int rr = row_ok ? r : 0;  // padding lanes read row 0's values (never stored)
  const int limit = row_ok ? sp.p : -1;
  const int hq = un.kvh * a.group + rr;
  const size_t slot0 = (size_t)us * a.tps;
  const int32_t* bt_row = a.block_table + (size_t)un.b * a.bt_stride;
  const int nblk = (n + 15) >> 4;
  const int np = a.num_pages;
  const int wbytes = a.group * 256;  // one slot's weights
  // This lane's source byte within a slot's weights for copy i (lanes past
  // the slot's rows re-read its last 16 bytes: in bounds, never used).
  auto w_src = [&](int i) { return min(i * 1024 + lane * 16, wbytes - 16); };
  auto pages = [&](int j) {  // group tile j's entries, staged in LDS
    const int4 e = *reinterpret_cast<const int4*>(&bt_lds[4 * j]);
    return make_int4(__builtin_amdgcn_readfirstlane(e.x), __builtin_amdgcn_readfirstlane(e.y),
                     __builtin_amdgcn_readfirstlane(e.z), __builtin_amdgcn_readfirstlane(e.w));
  };

  float m = neg_inf(), z = 0.f;
  f32x4 u = {0.f, 0.f, 0.f, 0.f};  // dims 16 mb + 4 g + j of the row (wave 0)
  for (int g0 = 0; g0 < ntiles; g0 += GT) {
    const int cnt = min(GT, ntiles - g0);
    const int j0 = w * TPW;                       // this wave's first tile of the group
    const int jn = min(TPW, cnt - j0);            // and how many (may be <= 0)
    __syncthreads();                              // the previous group's chain is done with LDS
    // Weights and (alpha, sum, max): they need no page.
    for (int jj = 0; jj < jn; ++jj) {
      const int j = j0 + jj;
      uint8_t* dst = ring + j * kSlotBytes;
      const size_t slot = slot0 + g0 + j;
      const uint8_t* wsrc = reinterpret_cast<const uint8_t*>(a.ws_x + spread_x_off(slot, a.group, 0, 0, 0));
#pragma unroll
      for (int i = 0; i < WC; ++i)
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(wsrc + w_src(i)), (lds_void_t*)(dst + kVBytes + i * 1024),
                                         16, 0, 0);
      const uint8_t* asrc = reinterpret_cast<const uint8_t*>(a.ws_as + slot * 16 * 4);
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(asrc + lane * 4), (lds_void_t*)(dst + kVBytes + kWBytes), 4, 0,
                                       0);
    }
    // The wave's block-table entries (clamped to the sequence's last block),
    // one per lane, then the V copies of its tiles.
    int btv = 0;
    if (jn > 0) {
      const int e = (k_begin >> 4) + 4 * (g0 + j0) + (lane < 4 * jn ? lane : 4 * jn - 1);
      btv = bt_row[e < nblk ? e : nblk - 1];
    }
    for (int jj = 0; jj < jn; ++jj) {
      const int j = j0 + jj;
      const int4 ent = make_int4(__builtin_amdgcn_readlane(btv, 4 * jj), __builtin_amdgcn_readlane(btv, 4 * jj + 1),
                                 __builtin_amdgcn_readlane(btv, 4 * jj + 2), __builtin_amdgcn_readlane(btv, 4 * jj + 3));
      const TilePages tp = tile_pages_of(ent, k_begin + kTileKeys * (g0 + j), n, np);
      uint8_t* dst = ring + j * kSlotBytes;
      const size_t vdim = (size_t)16 * mb * 16 * EB;  // the dim block's bytes inside a page block
      if constexpr (FP8) {
        // 4 page blocks x 256 B: lanes 16 q .. 16 q + 15 copy block q.
        const int q = lane >> 4;
        const int pg = q == 0 ? tp.page[0] : (q == 1 ? tp.page[1] : (q == 2 ? tp.page[2] : tp.page[3]));
        const uint8_t* src = a.v_cache + ((size_t)pg * a.Hkv + un.kvh) * kHeadBytes + vdim + (lane & 15) * 16;
        __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)dst, 16, 0, 0);
      } else {
        // 4 page blocks x 512 B: copy h takes blocks 2 h (lanes 0..31) and 2 h + 1.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int pg = (lane < 32) ? (h == 0 ? tp.page[0] : tp.page[2]) : (h == 0 ? tp.page[1] : tp.page[3]);
          const uint8_t* src = a.v_cache + ((size_t)pg * a.Hkv + un.kvh) * kHeadBytes + vdim + (lane & 31) * 16;
          __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)(dst + h * 1024), 16, 0, 0);
        }
      }
    }
    if (jn > 0 && lane < 4 * jn) bt_lds[4 * j0 + lane] = btv;  // for the chain's key counts
    __syncthreads();  // (waits for every copy of this wave first) the group has landed
    if (w != 0) continue;
    // Wave 0: the chain over the group, operands read from LDS (no copy is
    // in flight now, so these are ordinary LDS reads), four tiles' reads at a
    // time ahead of their value products.
    auto read = [&](int j, SpreadFrag<FP8>& f) {
      const uint8_t* src = ring + j * kSlotBytes;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
        f.v[ks2] = *reinterpret_cast<const typename Raw<FP8>::V8*>(src + v_block(ks2, g) * (kVBytes / 4) +
                                                                    (r * 16 + 8 * (g & 1)) * EB);
#pragma unroll
      for (int part = 0; part < 4; ++part)
        f.w[part] = *reinterpret_cast<const uint4*>(src + kVBytes + ((4 * part + g) * a.group + rr) * 16);
      f.asm4 = *reinterpret_cast<const f32x4*>(src + kVBytes + kWBytes + rr * 16);
    };
    auto chain = [&](int j, const SpreadFrag<FP8>& f) {
      const int t0 = k_begin + kTileKeys * (g0 + j);
      const bool vis = tile_visible(t0, lo, n, limit);
      if (tile_full(t0, lo, n)) {
        spread_chain<true, FP8>(f, 0, vis, m, z, u, g);
      } else {
        const TilePages tp = tile_pages_of(pages(j), t0, n, np);
        const int valid = tp.valid[0] | (tp.valid[1] << 5) | (tp.valid[2] << 10) | (tp.valid[3] << 15);
        spread_chain<false, FP8>(f, valid, vis, m, z, u, g);
      }
    };
    for (int j = 0; j < cnt; j += 4) {
      SpreadFrag<FP8> f[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j + i < cnt) read(j + i, f[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j + i < cnt) chain(j + i, f[i]);
    }
  }

  if (w == 0 && row_ok) {
    const size_t row = ((size_t)un.b * a.max_splits + un.s) * a.Hq + hq;
    *reinterpret_cast<f32x4*>(a.ws_u + row * D + 16 * mb + 4 * g) = u;
    if (mb == 0 && g == 0) *reinterpret_cast<f32x2*>(a.ws_ml + row * 2) = f32x2{m, z};
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
  const int s0 = first_key(n - 1, a.window) / S;  // first split with a visible key
  const size_t row0 = ((size_t)b * a.max_splits + s0) * a.Hq + hq;
  const f32x2 ml0 = *reinterpret_cast<const f32x2*>(a.ws_ml + row0 * 2);
  float M = ml0[0], Z = ml0[1];
  float U[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) U[k] = a.ws_u[row0 * D + kPer * lane + k];
  for (int s = s0 + 1; s < nsplit; ++s) {
    const size_t row = row0 + (size_t)(s - s0) * a.Hq;
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

// ---------------------------------------------------------------------------
// Longest-first dispatch of the split units.
//
// A launch's units are whole splits (S keys) except each sequence's last
// split, which holds the remaining n mod S keys.  Workgroups start in grid
// order as compute units free up, so a long unit that starts late sets the
// end of the launch.  This one-workgroup kernel writes the list the split
// kernel takes its units from: every whole split first, then the last splits
// by decreasing length in 64-key tiles, then -1 for the unused grid entries.
// Entry = b * max_splits + s.  Places inside the list are claimed with LDS
// atomics, so the order among sequences may differ between calls; it decides
// only which workgroup runs a unit, never what the unit computes.  Batches
// above kOrderMaxB, and launches with fewer than kOrderMinUnits units (where
// most units start at once), keep the split-major grid order.
constexpr int kOrderThreads = 1024;
constexpr int kOrderMaxB = kOrderThreads;
constexpr int kOrderMinUnits = 2048;

__global__ __launch_bounds__(kOrderThreads) void decode_order_kernel(DecodeArgs a) {
  __shared__ int full_next;             // next free place in the whole-split part
  __shared__ int next[kOrderBuckets];   // last splits per bucket, then each bucket's next place
  __shared__ int listed;
  const int tid = threadIdx.x;
  if (tid == 0) full_next = 0;
  if (tid < kOrderBuckets) next[tid] = 0;
  __syncthreads();
  int nf = 0, q = -1;  // q: bucket of the last split (0 = longest), -1 = none
  if (tid < a.B) {
    const int n = clamp_len(a.seq_lens[tid], a.max_seq_len);
    const int S = split_len(a.policy, a.split_tokens, n, a.B);
    nf = n / S;
    const int tiles = (n - nf * S + kTileKeys - 1) / kTileKeys;
    if (tiles > 0) q = kOrderBuckets - (tiles < kOrderBuckets ? tiles : kOrderBuckets);
  }
  const int f0 = nf > 0 ? atomicAdd(&full_next, nf) : 0;
  if (q >= 0) atomicAdd(&next[q], 1);
  __syncthreads();
  if (tid == 0) {
    int run = full_next;
    for (int i = 0; i < kOrderBuckets; ++i) {
      const int c = next[i];
      next[i] = run;
      run += c;
    }
    listed = run;
  }
  __syncthreads();
  for (int s = 0; s < nf; ++s) a.order[f0 + s] = tid * a.max_splits + s;
  if (q >= 0) a.order[atomicAdd(&next[q], 1)] = tid * a.max_splits + nf;
  for (int i = listed + tid; i < a.B * a.max_splits; i += kOrderThreads) a.order[i] = -1;
}

// Whether every split of the launch is at most kWideMaxTiles tiles long (the
// split kernel, with the same bits, runs the others).
static bool wide_fits(const DecodeArgs& a) {
  int64_t len = a.split_tokens;
  if (a.policy != 0) {
    int k = 256 / (a.B > 0 ? a.B : 1);
    k = k < 1 ? 1 : (k > 64 ? 64 : k);
    len = ((a.max_seq_len + k - 1) / k + 63) / 64 * 64;
  }
  return len <= (int64_t)kWideMaxTiles * kTileKeys;
}

template <int D, bool FP8, int WC>
static hipError_t launch_value(const DecodeArgs& a, int64_t units, hipStream_t st) {
  constexpr int kSlotBytes = 4 * 16 * 16 * (FP8 ? 1 : 2) + WC * 1024 + 256;
  const int lds = SpreadRing<WC>::GT * (kSlotBytes + 16);  // slots, then 4 block-table entries per tile
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&decode_value_kernel<D, FP8, WC>), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((decode_value_kernel<D, FP8, WC>), dim3((unsigned)(units * (D / 16))),
                     dim3(64 * SpreadRing<WC>::kWaves), lds, st, a);
  return hipGetLastError();
}

template <int D, bool FP8>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const int64_t units = (int64_t)a.B * a.Hkv * a.max_splits;
  if (a.kernel == 2) {
    hipLaunchKernelGGL((decode_score_kernel<D, FP8>), dim3((unsigned)(units * a.tps)), dim3(64), 0, st, a);
    hipError_t se = hipGetLastError();
    if (se != hipSuccess) return se;
    hipLaunchKernelGGL((decode_weight_kernel<D, FP8>), dim3((unsigned)(units * a.tps)), dim3(64), 0, st, a);
    se = hipGetLastError();
    if (se != hipSuccess) return se;
    if (a.group <= 4)
      se = launch_value<D, FP8, 1>(a, units, st);
    else if (a.group <= 8)
      se = launch_value<D, FP8, 2>(a, units, st);
    else
      se = launch_value<D, FP8, 4>(a, units, st);
    if (se != hipSuccess) return se;
  } else if (a.kernel == 1 && wide_fits(a)) {
    hipLaunchKernelGGL((decode_wide_kernel<D, FP8>), dim3((unsigned)units), dim3(64 * kWideWaves), 0, st, a);
  } else {
    DecodeArgs sa = a;
    sa.self_order = 0;
    if (a.order && a.B <= kOrderMaxB && units >= kOrderMinUnits) {
      hipLaunchKernelGGL(decode_order_kernel, dim3(1), dim3(kOrderThreads), 0, st, a);
      const hipError_t oe = hipGetLastError();
      if (oe != hipSuccess) return oe;
    } else {
      sa.order = nullptr;
      sa.self_order = a.B <= kSelfOrderMaxB && units > kSelfOrderMinUnits;
    }
    if (a.nt)
      hipLaunchKernelGGL((decode_split_kernel<D, FP8, true>), dim3((unsigned)units), dim3(64 * kDecodeWaves), 0, st, sa);
    else
      hipLaunchKernelGGL((decode_split_kernel<D, FP8, false>), dim3((unsigned)units), dim3(64 * kDecodeWaves), 0, st,
                         sa);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D, FP8>), dim3((unsigned)((int64_t)a.B * a.Hq)), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode(int D, bool fp8, const DecodeArgs& a, hipStream_t st) {
  if (D == 128 && fp8) return launch_decode_t<128, true>(a, st);
  if (D == 128) return launch_decode_t<128, false>(a, st);
  if (D == 64 && fp8) return launch_decode_t<64, true>(a, st);
  if (D == 64) return launch_decode_t<64, false>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace ia
