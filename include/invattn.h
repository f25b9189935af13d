/*
 * invattn.h -- C ABI of libinvattn.so, a batch-invariant paged-attention
 * library for AMD Instinct MI355X (gfx950).
 *
 * Every (sequence, head, query position) is reduced in one fixed order that
 * depends only on that row's logical inputs, so output bits do not depend on
 * batch composition, query length, chunk split points, prefix reuse or
 * physical page placement.  Sources for the contracts:
 *
 *  - Vosti: Specifying, Implementing, and Verifying Deterministic LLM
 *    Inference (arXiv:2609.38981): §5.3 and App. A.1 (the causal contract:
 *    query row i of an invocation with query length s and key length n sits
 *    at position p = n - s + i; equal queries and equal logical K/V through p
 *    give bitwise-equal output rows), App. A.2 (the tile arithmetic), §4.1-4.3
 *    and Figure 2 (prefix sharing, write isolation, leaf-only eviction), §4.1
 *    "Fixed kernel choices" (an immutable configuration, no autotuning, a
 *    missing configuration is rejected).
 *  - Deterministic inference: results independent of the batch (AI infra
 *    handbook), "Batch invariance: fixed splits that don't change with load":
 *    attention splits its KV by a fixed length, never into a fixed number of
 *    pieces.
 *  - Defeating Nondeterminism in LLM Inference (summary), Overview: fixed-size
 *    split-KV plus a KV cache updated before the attention kernel.
 *
 * Conventions
 *  - All tensors are row-major.  "dev" pointers are device memory on the
 *    current HIP device; "host" pointers are host memory.  The caller owns
 *    every buffer.  The library never allocates or frees device memory, never
 *    synchronises, and enqueues work only on the `stream` argument (a
 *    hipStream_t; NULL is the default stream).  Device buffers must stay alive
 *    until that work completes.
 *  - Status codes are returned; no C++ exception crosses the ABI.  Every
 *    host-checkable argument is validated before anything is launched; on
 *    error nothing is launched and ia_last_error() (thread-local) describes
 *    why.  There is no fallback path.
 *  - Device-resident preconditions are not checked on the hot path (they
 *    would need a synchronisation): 1 <= q_len <= seq_len <= max_seq_len,
 *    block-table entries of positions < seq_len in [0, num_pages), write slots
 *    in range and pairwise disjoint, finite K/V/Q.  The kernels stay memory
 *    safe when they are violated (out-of-range page ids and lengths are
 *    clamped or read as zeros) but the results are then unspecified.
 *
 * Page layout (per KV pool; element = bf16, or one e4m3 byte for fp8):
 *    K: [num_pages][num_kv_heads][head_dim/8][16 slots][8]
 *    V: [num_pages][num_kv_heads][head_dim][16 tokens]
 *  Token t of physical page pg holds logical position j with
 *  block_table[b][j / page_size] = pg and t = j % page_size; slot = pg *
 *  page_size + t.  V keeps the tokens of a dim row in order; K stores token
 *  t in slot t with bits 2 and 3 exchanged (tokens 0-3, 8-11, 4-7, 12-15 in
 *  slots 0..15), so that the 8 tokens of a page that one MFMA score block
 *  takes are one contiguous 128-byte run of each chunk row.
 */
#ifndef INVATTN_H_
#define INVATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IA_OK = 0,
  IA_ERR_INVALID_ARG = 1,
  IA_ERR_UNSUPPORTED_CONFIG = 2,
  IA_ERR_WORKSPACE_TOO_SMALL = 3,
  IA_ERR_OUT_OF_PAGES = 4,
  IA_ERR_PAGE_REFERENCED = 5,
  IA_ERR_HIP = 6,
  IA_ERR_INTERNAL = 7
} ia_status;

typedef enum { IA_KV_BF16 = 0, IA_KV_FP8_E4M3 = 1 } ia_kv_dtype;

/* IA_SPLIT_FIXED: decode splits each sequence's keys at absolute multiples of
 * split_tokens (batch invariant).  IA_SPLIT_BY_COUNT: decode cuts sequence b
 * into k = max(1, min(64, 256 / B)) pieces, each roundup(ceil(n_b / k), 64)
 * tokens long -- the load-based heuristic of the handbook's split-KV example
 * with 256 compute units in place of 132 SMs.  It is NOT batch invariant and
 * exists only to measure what invariance costs.  Prefill always uses the
 * fixed split. */
typedef enum { IA_SPLIT_FIXED = 0, IA_SPLIT_BY_COUNT = 1 } ia_split_policy;

/* Which decode kernel runs the splits.  All produce bit-identical partial
 * states and outputs (the same operations on the same operands in the same
 * order) and differ only in schedule.  This is the pages' open item of
 * dispatch among bitwise-equivalent kernels (Vosti, Discussion,
 * "Cross-kernel relational verification": one decode kernel for full waves,
 * one that gives a sequence several compute units for partially filled
 * waves, with the same accumulation order).
 *   IA_DECODE_SPLIT walks each split's tiles as one chain of steps on one
 *     compute unit (4 waves per split).
 *   IA_DECODE_WIDE lets 8 waves of one compute unit score and weight 8 tiles
 *     of a split at once (the running maximum before a tile is an exact fmaxf
 *     fold of the earlier tiles' maxima) and keeps only the z and value
 *     updates as a chain.  It takes splits of at most 16384 keys; longer ones
 *     run on SPLIT.  Selectable only: it is not faster than SPLIT.
 *   IA_DECODE_SPREAD spreads a split over many compute units in three
 *     launches: one wave per (split, tile) forms the tile's scores and row
 *     maxima; one wave per (split, tile) folds the running maximum before its
 *     tile from the earlier tiles' maxima and forms the tile's weights, alpha
 *     and row sum; one wave per (split, 16-dim block) runs the chain of z and
 *     value updates for its dims.  The intermediate values live in the
 *     workspace.  Launches whose buffer would exceed 32768 (split, tile)
 *     slots run on SPLIT.
 *   IA_DECODE_AUTO runs SPREAD for launches of at most 32 split units
 *     (batch x kv heads x splits of max_seq_len) whose splits are at most 32
 *     tiles (2048 keys) with at most 4 query heads per kv head, and SPLIT
 *     otherwise (measured: outside that range SPLIT is faster). */
typedef enum { IA_DECODE_AUTO = 0, IA_DECODE_SPLIT = 1, IA_DECODE_WIDE = 2, IA_DECODE_SPREAD = 3 } ia_decode_kernel;

/* Cache policy of the decode split kernel's K/V page loads.  It changes only
 * where bytes are cached, never a value or an order, so it is free to differ
 * between calls.
 *   IA_KV_HINT_STREAM loads every page nontemporally: each byte of a call is
 *     read once, and streaming loads keep the caches from holding it (a plain
 *     streaming read of HBM reaches ~7.0 TB/s this way against ~6.3 TB/s).
 *   IA_KV_HINT_CACHED uses ordinary loads: for batches whose sequences share
 *     pages (a common prefix), where the cached copy of a shared page serves
 *     every sequence that reads it (measured: 128 sequences on a 16384-token
 *     prefix decode at 12.1 TB/s of logical KV bytes cached, 6.8 streamed).
 *   IA_KV_HINT_AUTO streams launches of at least 512 split units (measured
 *     faster there on private pages) and caches smaller ones, whose working
 *     set the caches can hold across calls. */
typedef enum { IA_KV_HINT_AUTO = 0, IA_KV_HINT_STREAM = 1, IA_KV_HINT_CACHED = 2 } ia_kv_cache_hint;

/* How a prefill launch whose rows can see two splits spreads its work.  Every
 * choice folds a row's split states in ascending split order with the same
 * operations, so all give the same bits.
 *   IA_PREFILL_FOLD: one workgroup per (sequence, row block, kv head) walks
 *     its rows' whole range of keys and folds each split into the rows'
 *     merge at the split's end.
 *   IA_PREFILL_AUTO: as FOLD, except that a sequence of at most 4 row blocks
 *     whose keys reach a second split runs one workgroup per (row block, kv
 *     head, split), each walking that split's keys and storing its rows'
 *     split states, and a merge kernel then folds every row's states.  That
 *     serves few rows over long keys (decode rows co-batched with prompts,
 *     short chunks of long prompts), which FOLD leaves on a few workgroups.
 *     A row block holds floor(16 / (Hq / Hkv)) x 8 positions for bf16
 *     pages, half as many for e4m3 ones.
 *   IA_PREFILL_SPLIT: as AUTO for sequences of any number of row blocks.
 * AUTO and SPLIT apply to launches of fewer than 8192 (sequence, row block,
 * kv head) workgroups whose workspace holds the split states (within 128 MiB;
 * the bound halves the row blocks split per sequence until they fit); other
 * launches run FOLD, and so do launches whose total_q leaves no room for a
 * sequence short enough to split (total_q > (B - 1) * max_q_len + the
 * positions of the row blocks split). */
typedef enum { IA_PREFILL_AUTO = 0, IA_PREFILL_FOLD = 1, IA_PREFILL_SPLIT = 2 } ia_prefill_grid;

typedef struct {
  int32_t num_q_heads;   /* Hq; a multiple of num_kv_heads, Hq / Hkv <= 16 */
  int32_t num_kv_heads;  /* Hkv */
  int32_t head_dim;      /* d: 64 or 128 */
  int32_t page_size;     /* P: 16 */
  int32_t split_tokens;  /* S: a positive multiple of 64 (the key tile) */
  int32_t kv_dtype;      /* ia_kv_dtype */
  int32_t split_policy;  /* ia_split_policy */
  float sm_scale;        /* softmax scale, e.g. 1/sqrt(d); scores use
                            c = fp32(sm_scale * log2(e)) and exp2 (Vosti App. A.2,
                            "shared base-two scale c") */
  int32_t sliding_window; /* 0: full causal attention.  w > 0: position p sees
                             keys p - w < j <= p (Vosti App. A.5, sliding-window
                             attention).  Splits and tiles with no visible key
                             are skipped, which is the identity on a row's state,
                             so decode = prefill and batch invariance hold as for
                             full attention. */
  int32_t decode_kernel;  /* ia_decode_kernel (0 = AUTO) */
  int32_t kv_cache_hint;  /* ia_kv_cache_hint (0 = AUTO): how the decode split
                             kernel's page loads use the caches; never a value */
  int32_t prefill_grid;   /* ia_prefill_grid (0 = AUTO); never a value */
} ia_config;

typedef struct ia_ctx ia_ctx;
typedef struct ia_pool ia_pool;
typedef struct ia_seq ia_seq;

/* Validates and freezes a configuration (Vosti §4.1: fixed kernel choices,
 * no runtime autotuning; an unsupported configuration is rejected with
 * IA_ERR_UNSUPPORTED_CONFIG rather than served by another kernel).  The
 * context is immutable and may be used from several threads at once. */
ia_status ia_create(const ia_config* cfg, ia_ctx** out);
void ia_destroy(ia_ctx* ctx);

/* Thread-local description of the last error of this thread ("" if none). */
const char* ia_last_error(void);

/* Library version string. */
const char* ia_version(void);

/* Device workspace (bytes) that ia_paged_attn_decode needs for `batch`
 * sequences of at most max_seq_len keys: one fp32 partial state
 * (max, sum, head_dim accumulators) per (sequence, split, query head), one
 * int32 per (sequence, split) for the order in which the split units are
 * dispatched (longest first; the order never changes a result bit), and,
 * when the launch runs the spread kernels, one slot per (sequence, split,
 * kv head, tile): group x 64 fp32 scores (later the weights), 16 row
 * maxima, and 16 rows of (alpha, row sum, row maximum, 0).  Under
 * IA_DECODE_AUTO a workspace large enough for the split kernel but not for
 * the score slots runs the split kernel (the same bits). */
size_t ia_decode_workspace_bytes(const ia_ctx* ctx, int32_t batch, int32_t max_seq_len);

/* Device workspace for ia_paged_attn_prefill: 0 when max_seq_len <=
 * split_tokens (no row can see keys of two splits; NULL / 0 is then fine).
 * Otherwise one fp32 row state of d + 2 floats per (query row, query head):
 * total_q * Hq * d floats of U, then total_q * Hq * 2 floats of (M, Z), each
 * array rounded up to 256 bytes (the merge of the row's splits so far, or
 * its split-0 state under the split grid); the launch refuses less.  When
 * the launch can run the split grid (ia_prefill_grid) the size also holds,
 * in two more arrays laid out the same way, B * r * (positions per row block)
 * * (ceil(max_seq_len / split_tokens) - 1) * Hq states for the splits past
 * the first, r = the row blocks it splits per sequence; a workspace without
 * them runs in-workgroup folds (the same bits).  A workspace serves one call
 * at a time. */
size_t ia_prefill_workspace_bytes(const ia_ctx* ctx, int32_t B, int32_t total_q, int32_t max_q_len,
                                  int32_t max_seq_len);

/*
 * kv_append: writes T new K/V rows into their page slots.  Enqueue it on the
 * same stream before the attention call that reads them (Defeating
 * Nondeterminism, Overview: the cache is updated before the attention kernel,
 * which then reads every key through the cache).
 *   k_new, v_new   dev [T][Hkv][d] bf16
 *   slot_mapping   dev [T] int64, slot = page * P + offset; a negative slot
 *                  skips the row (padding)
 *   k_cache,v_cache dev page pools (layout above) of num_pages pages
 *   k_scale,v_scale dev [Hkv] fp32 static per-KV-head scales for
 *                  IA_KV_FP8_E4M3 (stored code = e4m3_rne(clamp(x / s, +-448)),
 *                  value = code * s); must be NULL for IA_KV_BF16.
 * Slots must be pairwise disjoint and must not belong to pages another
 * sequence reads (shared pages are immutable, Vosti §4.3).
 */
ia_status ia_kv_append(const ia_ctx* ctx, const void* k_new, const void* v_new, const int64_t* slot_mapping,
                       int32_t T, void* k_cache, void* v_cache, int32_t num_pages, const float* k_scale,
                       const float* v_scale, void* stream);

/*
 * Decode attention: one query row per sequence, at position p = seq_len - 1
 * (its own K/V already appended).  Keys are cut into splits at absolute
 * multiples of split_tokens; each split is walked in 64-key tiles in
 * ascending order with the online-softmax update of Vosti App. A.2 (fp32
 * state m, z, U; z sums the fp32 weights).  Departures from App. A.2, each
 * taken by every kernel alike (so invariance is unaffected):
 *  - it casts the weights once to the cache type before the PV product;
 *    here each fp32 weight w enters the PV product as two bf16 numbers,
 *    hi = bf16(w) and lo = bf16(w - hi), in two MFMAs (hi first), so a
 *    weight carries about 16 significant bits instead of 8 (a single cast
 *    misses the 2e-3 + 1e-2 |ref| tolerance on rows over a few keys whose
 *    values cancel);
 *  - the running reference m is raised only when a tile's maximum scaled
 *    score exceeds it by more than 8 (base-2 units), so weights are at most
 *    2^8 and most tiles have alpha = 1 (the same softmax in exact
 *    arithmetic);
 *  - a weight's exponent is one fused multiply-add, exp2(fma(s, c, -m)), of
 *    the raw score s (one rounding where scaling then subtracting rounds
 *    twice).  The split states
 * are then folded in ascending split order and the row is finalised as
 * O = bf16(U * select(z > 0, 1/z, 0)).
 *   q            dev [B][Hq][d] bf16
 *   block_table  dev [B][bt_stride] int32
 *   seq_lens     dev [B] int32, n_b >= 1 keys including the current token
 *   max_seq_len  host upper bound of seq_lens; sizes the grid only and never
 *                changes a row's arithmetic; bt_stride * P >= max_seq_len
 *   out          dev [B][Hq][d] bf16
 *   workspace    dev, >= ia_decode_workspace_bytes(ctx, B, max_seq_len)
 * Bitwise equal to ia_paged_attn_prefill's row at the same position.
 */
ia_status ia_paged_attn_decode(const ia_ctx* ctx, const void* q, const void* k_cache, const void* v_cache,
                               int32_t num_pages, const float* k_scale, const float* v_scale,
                               const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                               int32_t B, int32_t max_seq_len, void* out, void* workspace, size_t ws_bytes,
                               void* stream);

/*
 * Decode attention that allocates nothing, for callers that cannot allocate
 * device memory or be handed a workspace: code under HIP graph capture,
 * serving loops and harnesses that forbid hipMalloc.  Same arguments (minus
 * the workspace), same kernels and the same output bits as
 * ia_paged_attn_decode; the workspace is a fixed device array inside the
 * library, one per GPU, of ia_decode_noalloc_scratch_bytes() bytes (32 MiB:
 * enough for 256 sequences of up to 8192 keys at 32 query heads and head_dim
 * 128), held from the library's load until the process ends.  A launch whose
 * workspace would exceed it is rejected with IA_ERR_WORKSPACE_TOO_SMALL
 * before anything is enqueued (under IA_DECODE_AUTO a launch that fits only
 * without the spread kernels' slots runs the split kernel, the same bits).
 * Nothing in the array needs to start at zero: every call writes what it
 * later reads.  Calls on one GPU share its array, so calls that may overlap
 * on one GPU (other streams, other threads) race and must be serialised by
 * the caller.
 */
ia_status ia_paged_attn_decode_noalloc(const ia_ctx* ctx, const void* q, const void* k_cache, const void* v_cache,
                                       int32_t num_pages, const float* k_scale, const float* v_scale,
                                       const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                                       int32_t B, int32_t max_seq_len, void* out, void* stream);

/* Bytes of the fixed workspace ia_paged_attn_decode_noalloc uses. */
size_t ia_decode_noalloc_scratch_bytes(void);

/*
 * Chunked / whole prefill (and mixed batches): packed ragged query rows,
 * causal, grouped-query.  Sequence b owns rows cu_q_lens[b] ..
 * cu_q_lens[b+1]-1; row i of it is position p = seq_lens[b] - q_len_b + i and
 * attends keys 0..p, all read from the pages (append the chunk's own K/V
 * first).  Each row visits the same splits and tiles, in the same order and
 * with the same arithmetic, as a decode row at that position; tiles past a
 * row's position leave its state bit-identical (Vosti App. A.3-A.5).
 *   q            dev [total_q][Hq][d] bf16
 *   cu_q_lens    dev [B+1] int32 (cu_q_lens[0] = 0, total_q = cu_q_lens[B])
 *   seq_lens     dev [B] int32, seq_len_b >= q_len_b
 *   max_q_len    host upper bound of q lengths (grid only)
 *   max_seq_len  host upper bound of seq_lens (grid only)
 *   out          dev [total_q][Hq][d] bf16
 *   workspace    dev, ia_prefill_workspace_bytes(ctx, B, total_q, max_q_len,
 *                max_seq_len) bytes, 16-byte aligned (NULL when that is 0);
 *                one without the split states runs in-workgroup folds, one
 *                smaller than the row states is refused with
 *                IA_ERR_WORKSPACE_TOO_SMALL
 */
ia_status ia_paged_attn_prefill(const ia_ctx* ctx, const void* q, const int32_t* cu_q_lens,
                                const int32_t* seq_lens, const void* k_cache, const void* v_cache,
                                int32_t num_pages, const float* k_scale, const float* v_scale,
                                const int32_t* block_table, int32_t bt_stride, int32_t B, int32_t total_q,
                                int32_t max_q_len, int32_t max_seq_len, void* out, void* workspace,
                                size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Batch-invariant layer operators: the other reductions of a layer, each
 * computing an output row from its own input row in one fixed order, so a
 * row's bits do not depend on how many rows share the call ("Deterministic
 * inference: results independent of the batch", "Batch invariance: fixed
 * splits": normalisation reduced by one block per row in a fixed order, and
 * matrix multiplication without split-K; Vosti, Figure 3, the matmul
 * contract).  Neither needs a context.  On error nothing is launched.
 */

/*
 * RMSNorm: y[m][i] = bf16((x[m][i] * r_m) * w[i]), r_m = 1 / sqrt(mean_i
 * x[m][i]^2 + eps), fp32 arithmetic; the sum of squares of a row runs in one
 * workgroup in a fixed order.
 *   x       dev [M][H] bf16, 16-byte aligned
 *   weight  dev [H] bf16
 *   out     dev [M][H] bf16 (may not alias x)
 *   H       a multiple of 8, 8 <= H <= 16384; eps finite, >= 0
 */
ia_status ia_rmsnorm(const void* x, const void* weight, int32_t M, int32_t H, float eps, void* out, void* stream);

/*
 * C = A W^T: c[m][n] = bf16(sum_k a[m][k] w[n][k]), fp32 accumulation, no
 * split-K.  Every output is one MFMA accumulator chain over k in ascending
 * 16-wide steps (v_mfma_f32_32x32x16_bf16), whatever tile computes it, so a
 * row of C depends on its row of A and on W only, never on M.  Two tiles
 * (chosen from M, N and K only to fill the chip; the same bits either way):
 *  - 256 x 256 outputs, 8 waves, when it gives at least one workgroup per
 *    compute unit: K steps of 64 when K % 64 == 0, else 32;
 *  - 64 x 64 outputs, 4 waves, otherwise: K steps of 128 when K % 128 == 0,
 *    else 32.
 * Both go through a two-slot LDS ring, one K step ahead.
 *   a  dev [M][K] bf16 (row-major activations, one row per token)
 *   w  dev [N][K] bf16 (a linear layer's weight, one row per output feature)
 *   c  dev [M][N] bf16
 *   N  a positive multiple of 256; K a positive multiple of 32; M >= 0
 */
ia_status ia_gemm_bf16(const void* a, const void* w, int32_t M, int32_t N, int32_t K, void* c, void* stream);

/* ------------------------------------------------------------------------
 * Host page table with prefix sharing (host memory only; one pool is not
 * thread safe).  Vosti §4.1-4.3, Figure 2:
 *  - a cached page is reused only for the token prefix that produced it: a
 *    rolling hash finds candidates, then exact tokens, depth and physical
 *    parent page are checked, so a hash collision never justifies reuse;
 *  - hits are resolved when a sequence begins, before it registers the pages
 *    it will produce; new K/V go to private pages; a page is published for
 *    reuse after it is full and its K/V are computed (ia_seq_commit);
 *  - published pages are immutable and refcounted; when the last reference
 *    ends they are retained; only unreferenced leaves of the parent chain are
 *    evicted (least recently released first, ties by page id), so a parent is
 *    never recycled while a retained child refers to it.
 * Free pages are handed out lowest id first.  A prompt always keeps at least
 * one token to compute.  A full page identical to a published one, or whose
 * parent is not published, stays private.
 * ------------------------------------------------------------------------ */

/* flags: 0, or IA_POOL_CONSTANT_HASH (every page hashes alike -- a test hook
 * that forces collisions; reuse must still be exact). */
#define IA_POOL_CONSTANT_HASH 1
ia_status ia_pool_create(int32_t num_pages, int32_t page_size, int32_t flags, ia_pool** out);
void ia_pool_destroy(ia_pool* pool);

/* Starts a sequence with prompt tokens[0..n) (host) and attaches its longest
 * exactly-matching published prefix; *cached_len = tokens already in cache
 * (a multiple of page_size, < n). */
ia_status ia_seq_begin(ia_pool* pool, const int32_t* tokens, int32_t n, ia_seq** out, int32_t* cached_len);

/* Appends generated tokens (host) to the sequence's history. */
ia_status ia_seq_append_tokens(ia_pool* pool, ia_seq* seq, const int32_t* tokens, int32_t n);

/* Reserves private write slots for the next n_new history positions and
 * writes them to slot_mapping_out (host [n_new] int64).  Allocates pages,
 * evicting unreferenced leaves if the free list runs short;
 * IA_ERR_OUT_OF_PAGES (nothing allocated) if that is not enough. */
ia_status ia_seq_reserve(ia_pool* pool, ia_seq* seq, int32_t n_new, int64_t* slot_mapping_out);

/* Marks n_done reserved positions as computed and publishes pages that became
 * full. */
ia_status ia_seq_commit(ia_pool* pool, ia_seq* seq, int32_t n_done);

/* Copies the sequence's page ids in logical order to out (host, capacity cap);
 * *n_pages = their number (IA_ERR_INVALID_ARG if cap is too small). */
ia_status ia_seq_block_table(const ia_seq* seq, int32_t* out, int32_t cap, int32_t* n_pages);

/* Positions computed so far. */
int32_t ia_seq_len(const ia_seq* seq);

/* Ends the sequence: drops its references (published pages are retained,
 * private pages freed) and frees the handle. */
ia_status ia_seq_end(ia_pool* pool, ia_seq* seq);

/* Evicts up to `want` unreferenced leaf pages; *evicted = how many. */
ia_status ia_pool_evict(ia_pool* pool, int32_t want, int32_t* evicted);

/* Introspection: refcount of a page (-1 if out of range), whether it is
 * published, number of free pages. */
int32_t ia_pool_page_refs(const ia_pool* pool, int32_t page);
int32_t ia_pool_page_published(const ia_pool* pool, int32_t page);
int32_t ia_pool_num_free(const ia_pool* pool);

/* ------------------------------------------------------------------------
 * Opt-in host validators of the device-resident preconditions that the
 * launches leave unchecked (Vosti §4.3 "Sharing and write isolation": new
 * K/V go only to private, pairwise disjoint slots and shared pages are never
 * written; App. A.1: every key of a row is read through its block-table
 * entry).  The caller copies the arrays to host memory first; nothing here
 * touches the GPU, so a deployment runs them when it wants the guarantee,
 * off the hot path.  The first violation found is reported through
 * ia_last_error().
 * ------------------------------------------------------------------------ */

/* kv_append slots (host [T] int64; negative entries are padding and skipped).
 * Taken in slot order, the first slot at or past num_pages * page_size gives
 * IA_ERR_INVALID_ARG, and, with a pool (may be NULL), the first slot on a
 * published page gives IA_ERR_PAGE_REFERENCED (published pages are shared
 * and immutable); failing both, a slot listed twice gives IA_ERR_INVALID_ARG.
 * The pool must have num_pages pages of page_size tokens. */
ia_status ia_validate_slots(const ia_pool* pool, const int64_t* slot_mapping, int32_t T, int32_t num_pages,
                            int32_t page_size);

/* Attention launch arguments (all host arrays): cu_q_lens [B+1] with
 * cu_q_lens[0] = 0 and cu_q_lens[B] = total_q (NULL for decode, where each
 * q_len is 1); for every sequence 1 <= q_len <= seq_lens[b] <= max_seq_len,
 * its ceil(seq_len / page_size) pages fit a block-table row of bt_stride
 * entries, and each of those entries names a page in [0, num_pages).
 * IA_OK, or IA_ERR_INVALID_ARG with the first violation. */
ia_status ia_validate_attention_args(const int32_t* cu_q_lens, const int32_t* seq_lens, int32_t B, int32_t total_q,
                                     const int32_t* block_table, int32_t bt_stride, int32_t num_pages,
                                     int32_t page_size, int32_t max_seq_len);

/* ------------------------------------------------------------------------
 * Measurement reference (not part of the attention path): a kernel that does
 * nothing but stream `bytes` of device memory from buf (16-byte nontemporal
 * loads, 8 in flight per thread, one contiguous share per workgroup, 16
 * workgroups of 256 threads per compute unit) and xor
 * them into one word per workgroup in sink, so that the decode kernel's
 * KV-read rate can be set beside what a plain read reaches on the same GPU.
 *   buf   dev, 16-byte aligned, bytes a multiple of 16
 *   sink  dev, >= ia_stream_read_sink_bytes() bytes (its contents are
 *         meaningless)
 */
size_t ia_stream_read_sink_bytes(void);
ia_status ia_stream_read(const void* buf, size_t bytes, void* sink, size_t sink_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* INVATTN_H_ */
