// capi.hip -- the C ABI of libinvattn.so: configuration, argument validation
// and launches.  Every host-checkable argument is checked before anything is
// enqueued; on error nothing is launched (Detent, §5 "Legal values": a failed
// precondition stops with an error and runs no kernel; Vosti §4.1: a missing
// configuration is rejected, never autotuned or replaced).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/invattn.h"
#include "errors.hpp"
#include "launch.hpp"

struct ia_ctx {
  ia_config cfg;
  float c;  // fp32(sm_scale * log2 e), rounded once from double
  int group;
};

namespace {
thread_local char g_err[512] = "";
}  // namespace

ia_status ia::fail(ia_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

ia_status ia::ok() {
  g_err[0] = '\0';
  return IA_OK;
}

namespace {
using ia::fail;
using ia::ok;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kTileKeys = 64;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t decode_max_splits(const ia_ctx* ctx, int64_t batch, int64_t max_seq_len) {
  if (ctx->cfg.split_policy == IA_SPLIT_FIXED) return ceil_div(max_seq_len, ctx->cfg.split_tokens);
  int64_t k = 256 / (batch > 0 ? batch : 1);
  k = k < 1 ? 1 : (k > 64 ? 64 : k);
  const int64_t by_tile = ceil_div(max_seq_len, kTileKeys);
  return k < by_tile ? k : by_tile;
}

// The spread decode pair (decode_score_kernel + decode_value_kernel) serves
// launches with few split units, where one compute unit per split leaves the
// chip idle; it gives the split kernel's bits, so the choice below decides
// speed only.  Its score buffer holds one slot per (unit, tile).
constexpr int64_t kSpreadMaxUnits = 32;        // IA_DECODE_AUTO: at most this many split units
constexpr int64_t kSpreadMaxSlots = 1 << 15;   // slots: <= 128 MiB of scores at 16 rows
// IA_KV_HINT_AUTO: nontemporal page loads for launches of at least this many
// split units (measured faster from about 700 units up on private pages, and
// slower at 340 and below).
constexpr int64_t kStreamMinUnits = 512;

// Tiles of the longest split a launch can have: the fixed split, or the
// split-by-count length for the longest sequence.
int64_t decode_split_tiles(const ia_ctx* ctx, int64_t batch, int64_t max_seq_len) {
  if (ctx->cfg.split_policy == IA_SPLIT_FIXED) return ctx->cfg.split_tokens / kTileKeys;
  int64_t k = 256 / (batch > 0 ? batch : 1);
  k = k < 1 ? 1 : (k > 64 ? 64 : k);
  const int64_t len = ceil_div(ceil_div(max_seq_len, k), kTileKeys);
  return len < 1 ? 1 : len;
}

// Which decode kernel a launch of this size runs: 0 split, 1 wide, 2 spread.
int decode_kernel_for(const ia_ctx* ctx, int64_t B, int64_t max_seq_len) {
  const int64_t units = B * ctx->cfg.num_kv_heads * decode_max_splits(ctx, B, max_seq_len);
  const bool spread_fits = units * decode_split_tiles(ctx, B, max_seq_len) <= kSpreadMaxSlots;
  switch (ctx->cfg.decode_kernel) {
    case IA_DECODE_WIDE: return 1;
    case IA_DECODE_SPLIT: return 0;
    case IA_DECODE_SPREAD: return spread_fits ? 2 : 0;
    default: {
      // Measured: the spread kernels win for a few dozen units when a split's
      // tiles fit one staging group of the value kernel (at most 32 tiles, up
      // to 4 query heads per kv head); otherwise the split kernel is faster.
      const bool one_group = ctx->group <= 4 && decode_split_tiles(ctx, B, max_seq_len) <= 32;
      return spread_fits && one_group && units <= kSpreadMaxUnits ? 2 : 0;
    }
  }
}

// Bytes of the workspace arrays: U accumulators, (m, z) pairs, the dispatch
// order of the split units, and (spread kernels only) the score / weight
// slots, their row maxima, and their alphas and row sums.
void decode_ws_parts(const ia_ctx* ctx, int64_t B, int64_t max_seq_len, size_t* u_bytes, size_t* ml_bytes,
                     size_t* order_bytes, size_t* x_bytes, size_t* mx_bytes) {
  const int64_t ms = decode_max_splits(ctx, B, max_seq_len);
  const int64_t rows = B * ms * ctx->cfg.num_q_heads;
  *u_bytes = align_up((size_t)rows * ctx->cfg.head_dim * sizeof(float));
  *ml_bytes = align_up((size_t)rows * 2 * sizeof(float));
  *order_bytes = align_up((size_t)(B * ms) * sizeof(int32_t));
  *x_bytes = *mx_bytes = 0;
  if (decode_kernel_for(ctx, B, max_seq_len) == 2) {
    const int64_t slots = B * ms * ctx->cfg.num_kv_heads * decode_split_tiles(ctx, B, max_seq_len);
    *x_bytes = align_up((size_t)slots * 16 * ctx->group * 4 * sizeof(float));
    // row maxima [slot][16], then (alpha, row sum, row maximum, 0) [slot][16][4]
    *mx_bytes = align_up((size_t)slots * 16 * sizeof(float)) + align_up((size_t)slots * 16 * 4 * sizeof(float));
  }
}

ia_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(IA_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

ia_status check_scales(const ia_ctx* ctx, const float* k_scale, const float* v_scale) {
  if (ctx->cfg.kv_dtype == IA_KV_FP8_E4M3) {
    if (!k_scale || !v_scale) return fail(IA_ERR_INVALID_ARG, "fp8 pages need k_scale and v_scale");
  } else if (k_scale || v_scale) {
    return fail(IA_ERR_INVALID_ARG, "k_scale/v_scale must be NULL for bf16 pages");
  }
  return IA_OK;
}

ia_status check_pages(const void* k_cache, const void* v_cache, int32_t num_pages) {
  if (!k_cache || !v_cache) return fail(IA_ERR_INVALID_ARG, "k_cache/v_cache is NULL");
  if (num_pages <= 0) return fail(IA_ERR_INVALID_ARG, "num_pages must be positive (got %d)", num_pages);
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(IA_ERR_INVALID_ARG, "page pools must be 16-byte aligned");
  return IA_OK;
}

// Workspace of ia_paged_attn_decode_noalloc: one fixed array per GPU, held
// from the library's load until the process ends.  Host code never uses the
// array's name as an address (on the host it only names the symbol); each
// device's own address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that address reaches kernels.
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// The current device's address of `scratch` (looked up on its first use).
ia_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(IA_ERR_HIP, "hipGetDevice: HIP error %d (%s)", (int)e, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(IA_ERR_INTERNAL, "device %d is past the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(IA_ERR_HIP, "hipGetSymbolAddress(scratch): HIP error %d (%s)", (int)e, hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return IA_OK;
}

}  // namespace

extern "C" {

const char* ia_last_error(void) { return g_err; }

const char* ia_version(void) { return "invattn 0.1 gfx950"; }

ia_status ia_create(const ia_config* cfg, ia_ctx** out) {
  if (!cfg || !out) return fail(IA_ERR_INVALID_ARG, "cfg and out must be non-NULL");
  *out = nullptr;
  const ia_config& c = *cfg;
  if (c.num_kv_heads <= 0 || c.num_q_heads <= 0 || c.num_q_heads % c.num_kv_heads != 0)
    return fail(IA_ERR_UNSUPPORTED_CONFIG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                c.num_q_heads, c.num_kv_heads);
  const int group = c.num_q_heads / c.num_kv_heads;
  if (group > 16) return fail(IA_ERR_UNSUPPORTED_CONFIG, "query heads per kv head must be <= 16 (got %d)", group);
  if (c.head_dim != 64 && c.head_dim != 128)
    return fail(IA_ERR_UNSUPPORTED_CONFIG, "head_dim must be 64 or 128 (got %d)", c.head_dim);
  if (c.page_size != 16) return fail(IA_ERR_UNSUPPORTED_CONFIG, "page_size must be 16 (got %d)", c.page_size);
  if (c.split_tokens <= 0 || c.split_tokens % kTileKeys != 0)
    return fail(IA_ERR_UNSUPPORTED_CONFIG, "split_tokens must be a positive multiple of %d (got %d)", kTileKeys,
                c.split_tokens);
  if (c.kv_dtype != IA_KV_BF16 && c.kv_dtype != IA_KV_FP8_E4M3)
    return fail(IA_ERR_UNSUPPORTED_CONFIG, "unknown kv_dtype %d", c.kv_dtype);
  if (c.split_policy != IA_SPLIT_FIXED && c.split_policy != IA_SPLIT_BY_COUNT)
    return fail(IA_ERR_UNSUPPORTED_CONFIG, "unknown split_policy %d", c.split_policy);
  if (!(c.sm_scale > 0.f) || !std::isfinite(c.sm_scale))
    return fail(IA_ERR_UNSUPPORTED_CONFIG, "sm_scale must be finite and positive");
  if (c.sliding_window < 0)
    return fail(IA_ERR_UNSUPPORTED_CONFIG, "sliding_window must be >= 0 (got %d)", c.sliding_window);
  if (c.decode_kernel != IA_DECODE_AUTO && c.decode_kernel != IA_DECODE_SPLIT && c.decode_kernel != IA_DECODE_WIDE &&
      c.decode_kernel != IA_DECODE_SPREAD)
    return fail(IA_ERR_UNSUPPORTED_CONFIG, "unknown decode_kernel %d", c.decode_kernel);
  if (c.kv_cache_hint != IA_KV_HINT_AUTO && c.kv_cache_hint != IA_KV_HINT_STREAM &&
      c.kv_cache_hint != IA_KV_HINT_CACHED)
    return fail(IA_ERR_UNSUPPORTED_CONFIG, "unknown kv_cache_hint %d", c.kv_cache_hint);
  if (c.prefill_grid != IA_PREFILL_AUTO && c.prefill_grid != IA_PREFILL_FOLD && c.prefill_grid != IA_PREFILL_SPLIT)
    return fail(IA_ERR_UNSUPPORTED_CONFIG, "unknown prefill_grid %d", c.prefill_grid);
  ia_ctx* ctx = new (std::nothrow) ia_ctx;
  if (!ctx) return fail(IA_ERR_INTERNAL, "out of host memory");
  ctx->cfg = c;
  ctx->group = group;
  ctx->c = (float)((double)c.sm_scale * 1.4426950408889634073599246810018921);  // log2(e)
  *out = ctx;
  return ok();
}

void ia_destroy(ia_ctx* ctx) { delete ctx; }

size_t ia_decode_workspace_bytes(const ia_ctx* ctx, int32_t batch, int32_t max_seq_len) {
  if (!ctx || batch <= 0 || max_seq_len <= 0) return 0;
  size_t u, ml, ord, x, mx;
  decode_ws_parts(ctx, batch, max_seq_len, &u, &ml, &ord, &x, &mx);
  return u + ml + ord + x + mx;
}

// Prefill workspace, when some row can see keys of two splits (max_seq_len >
// split_tokens).  First one fp32 row state of d + 2 floats per (query row,
// query head): U of every entry, then (M, Z) of every entry -- the merge of
// the row's splits so far under in-workgroup folds, the state of split 0
// under the split grid.  Then, for the split grid, the states of splits 1 ..
// of the first split_rbs row blocks of every sequence.  The split grid is
// offered to launches of fewer than kSplitMaxUnits row-block workgroups, for
// sequences of at most kSplitMaxRowBlocks row blocks (few rows over long
// keys: decode rows co-batched with prompts, short chunks of long prompts),
// with its states in at most kSplitMaxBytes.
constexpr size_t kSplitMaxBytes = (size_t)128 << 20;
constexpr int64_t kSplitMaxUnits = 8192;
constexpr int kSplitMaxRowBlocks = 4;

static size_t prefill_state_bytes(const ia_ctx* ctx, int64_t entries) {
  return align_up((size_t)entries * ctx->cfg.head_dim * sizeof(float)) + align_up((size_t)entries * 2 * sizeof(float));
}

static int prefill_max_splits(const ia_ctx* ctx, int32_t max_seq_len) {
  return (int)ceil_div(max_seq_len, ctx->cfg.split_tokens);
}

// Row blocks per wave (2 for bf16 pages, 1 for launches that would leave
// compute units idle with 2, and for e4m3 pages), and positions per
// workgroup.
static int prefill_rb(const ia_ctx* ctx, int32_t B, int32_t max_q_len) {
  const int64_t units2 = (int64_t)B * ceil_div(max_q_len, ia::prefill_positions_per_block(ctx->group, 2)) *
                         ctx->cfg.num_kv_heads;
  return ia::prefill_rows_per_wave(ctx->cfg.kv_dtype == IA_KV_FP8_E4M3, units2);
}

static int64_t prefill_ppg(const ia_ctx* ctx, int32_t B, int32_t max_q_len) {
  return ia::prefill_positions_per_block(ctx->group, prefill_rb(ctx, B, max_q_len));
}

static int64_t prefill_row_blocks(const ia_ctx* ctx, int32_t B, int32_t max_q_len) {
  return ceil_div(max_q_len, prefill_ppg(ctx, B, max_q_len));
}

// Entries of the split states of splits 1 .. for split_rbs row blocks.
static int64_t prefill_split_entries(const ia_ctx* ctx, int32_t B, int32_t max_q_len, int32_t max_seq_len, int rbs) {
  return (int64_t)B * rbs * prefill_ppg(ctx, B, max_q_len) * (prefill_max_splits(ctx, max_seq_len) - 1) *
         ctx->cfg.num_q_heads;
}

// Row blocks per sequence that a launch splits (0: none), before the
// workspace is checked.  When max_q_len exceeds them, a sequence that fits
// leaves rows of the bound unused: total_q rows with none unused mean no
// sequence fits, and nothing is split.
static int prefill_split_rbs(const ia_ctx* ctx, int32_t B, int32_t total_q, int32_t max_q_len, int32_t max_seq_len) {
  if (ctx->cfg.prefill_grid == IA_PREFILL_FOLD || max_seq_len <= ctx->cfg.split_tokens || B <= 0 || max_q_len <= 0)
    return 0;
  const int64_t rb = prefill_row_blocks(ctx, B, max_q_len);
  if ((int64_t)B * rb * ctx->cfg.num_kv_heads >= kSplitMaxUnits) return 0;
  int64_t rbs = ctx->cfg.prefill_grid == IA_PREFILL_SPLIT ? rb : (rb < kSplitMaxRowBlocks ? rb : kSplitMaxRowBlocks);
  const int64_t ppg = prefill_ppg(ctx, B, max_q_len);
  if (rbs < rb && (int64_t)total_q > (int64_t)(B - 1) * max_q_len + rbs * ppg) return 0;
  while (rbs > 0 &&
         prefill_state_bytes(ctx, prefill_split_entries(ctx, B, max_q_len, max_seq_len, (int)rbs)) > kSplitMaxBytes)
    rbs /= 2;
  return (int)rbs;
}

size_t ia_prefill_workspace_bytes(const ia_ctx* ctx, int32_t B, int32_t total_q, int32_t max_q_len,
                                  int32_t max_seq_len) {
  if (!ctx || B <= 0 || total_q <= 0 || max_q_len <= 0 || max_seq_len <= ctx->cfg.split_tokens) return 0;
  const int rbs = prefill_split_rbs(ctx, B, total_q, max_q_len, max_seq_len);
  return prefill_state_bytes(ctx, (int64_t)total_q * ctx->cfg.num_q_heads) +
         (rbs ? prefill_state_bytes(ctx, prefill_split_entries(ctx, B, max_q_len, max_seq_len, rbs)) : 0);
}

ia_status ia_kv_append(const ia_ctx* ctx, const void* k_new, const void* v_new, const int64_t* slot_mapping,
                       int32_t T, void* k_cache, void* v_cache, int32_t num_pages, const float* k_scale,
                       const float* v_scale, void* stream) {
  if (!ctx) return fail(IA_ERR_INVALID_ARG, "ctx is NULL");
  if (T < 0) return fail(IA_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
  ia_status st = check_scales(ctx, k_scale, v_scale);
  if (st != IA_OK) return st;
  if ((st = check_pages(k_cache, v_cache, num_pages)) != IA_OK) return st;
  if (T == 0) return ok();
  if (!k_new || !v_new || !slot_mapping) return fail(IA_ERR_INVALID_ARG, "k_new/v_new/slot_mapping is NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return fail(IA_ERR_INVALID_ARG, "k_new/v_new must be 16-byte aligned");
  if ((int64_t)T * ctx->cfg.num_kv_heads * (ctx->cfg.head_dim / 8) / 256 >= (int64_t)1 << 31)
    return fail(IA_ERR_INVALID_ARG, "T too large for one launch");
  ia::AppendArgs a;
  a.k_new = static_cast<const __bf16*>(k_new);
  a.v_new = static_cast<const __bf16*>(v_new);
  a.slots = slot_mapping;
  a.T = T;
  a.k_cache = static_cast<uint8_t*>(k_cache);
  a.v_cache = static_cast<uint8_t*>(v_cache);
  a.num_pages = num_pages;
  a.Hkv = ctx->cfg.num_kv_heads;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  return hip_status(ia::launch_kv_append(ctx->cfg.head_dim, ctx->cfg.kv_dtype == IA_KV_FP8_E4M3, a,
                                         static_cast<hipStream_t>(stream)),
                    "kv_append launch");
}

ia_status ia_paged_attn_decode(const ia_ctx* ctx, const void* q, const void* k_cache, const void* v_cache,
                               int32_t num_pages, const float* k_scale, const float* v_scale,
                               const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                               int32_t B, int32_t max_seq_len, void* out, void* workspace, size_t ws_bytes,
                               void* stream) {
  if (!ctx) return fail(IA_ERR_INVALID_ARG, "ctx is NULL");
  if (B < 0) return fail(IA_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
  ia_status st = check_scales(ctx, k_scale, v_scale);
  if (st != IA_OK) return st;
  if (B == 0) return ok();
  if ((st = check_pages(k_cache, v_cache, num_pages)) != IA_OK) return st;
  if (!q || !block_table || !seq_lens || !out) return fail(IA_ERR_INVALID_ARG, "q/block_table/seq_lens/out is NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(IA_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  if (max_seq_len <= 0) return fail(IA_ERR_INVALID_ARG, "max_seq_len must be positive (got %d)", max_seq_len);
  if ((int64_t)bt_stride * ctx->cfg.page_size < max_seq_len)
    return fail(IA_ERR_INVALID_ARG, "bt_stride (%d) pages cannot hold max_seq_len (%d) keys", bt_stride, max_seq_len);
  size_t u_bytes, ml_bytes, order_bytes, x_bytes, mx_bytes;
  decode_ws_parts(ctx, B, max_seq_len, &u_bytes, &ml_bytes, &order_bytes, &x_bytes, &mx_bytes);
  int kernel = decode_kernel_for(ctx, B, max_seq_len);
  const size_t need_split = u_bytes + ml_bytes + order_bytes;
  // Under IA_DECODE_AUTO a workspace too small for the spread kernels' score
  // slots runs the split kernel instead (the same bits).
  if (kernel == 2 && ctx->cfg.decode_kernel == IA_DECODE_AUTO && workspace && ws_bytes >= need_split &&
      ws_bytes < need_split + x_bytes + mx_bytes)
    kernel = 0;
  const size_t need = need_split + (kernel == 2 ? x_bytes + mx_bytes : 0);
  if (!workspace || ws_bytes < need)
    return fail(IA_ERR_WORKSPACE_TOO_SMALL, "decode workspace needs %zu bytes (got %zu)", need, ws_bytes);
  if (!aligned(workspace, 16)) return fail(IA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const int64_t ms = decode_max_splits(ctx, B, max_seq_len);
  if ((int64_t)B * ctx->cfg.num_kv_heads * ms >= ((int64_t)1 << 31))
    return fail(IA_ERR_INVALID_ARG, "grid too large");
  ia::DecodeArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = static_cast<__bf16*>(out);
  a.ws_u = static_cast<float*>(workspace);
  a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + u_bytes);
  a.order = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + u_bytes + ml_bytes);
  a.ws_x = reinterpret_cast<float*>(static_cast<char*>(workspace) + u_bytes + ml_bytes + order_bytes);
  a.ws_mx = reinterpret_cast<float*>(static_cast<char*>(workspace) + u_bytes + ml_bytes + order_bytes + x_bytes);
  {
    const int64_t slots = (int64_t)B * ctx->cfg.num_kv_heads * decode_max_splits(ctx, B, max_seq_len) *
                          decode_split_tiles(ctx, B, max_seq_len);
    a.ws_as = a.ws_mx + align_up((size_t)slots * 16 * sizeof(float)) / sizeof(float);
  }
  a.c = ctx->c;
  a.B = B;
  a.Hq = ctx->cfg.num_q_heads;
  a.Hkv = ctx->cfg.num_kv_heads;
  a.group = ctx->group;
  a.bt_stride = bt_stride;
  a.num_pages = num_pages;
  a.max_seq_len = max_seq_len;
  a.max_splits = (int)ms;
  a.split_tokens = ctx->cfg.split_tokens;
  a.policy = ctx->cfg.split_policy;
  a.window = ctx->cfg.sliding_window;
  a.kernel = kernel;
  a.tps = (int)decode_split_tiles(ctx, B, max_seq_len);
  {
    const int64_t units = (int64_t)B * ctx->cfg.num_kv_heads * ms;
    const int hint = ctx->cfg.kv_cache_hint;
    a.nt = hint == IA_KV_HINT_STREAM || (hint == IA_KV_HINT_AUTO && units >= kStreamMinUnits);
  }
  return hip_status(ia::launch_decode(ctx->cfg.head_dim, ctx->cfg.kv_dtype == IA_KV_FP8_E4M3, a,
                                      static_cast<hipStream_t>(stream)),
                    "decode launch");
}

ia_status ia_paged_attn_decode_noalloc(const ia_ctx* ctx, const void* q, const void* k_cache, const void* v_cache,
                                       int32_t num_pages, const float* k_scale, const float* v_scale,
                                       const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                                       int32_t B, int32_t max_seq_len, void* out, void* stream) {
  if (!ctx) return fail(IA_ERR_INVALID_ARG, "ctx is NULL");
  void* ws = nullptr;
  ia_status st = scratch_address(&ws);
  if (st != IA_OK) return st;
  st = ia_paged_attn_decode(ctx, q, k_cache, v_cache, num_pages, k_scale, v_scale, block_table, bt_stride, seq_lens,
                            B, max_seq_len, out, ws, kScratchBytes, stream);
  if (st == IA_ERR_WORKSPACE_TOO_SMALL)
    return fail(IA_ERR_WORKSPACE_TOO_SMALL,
                "ia_paged_attn_decode_noalloc: batch %d at max_seq_len %d needs %zu bytes of workspace, more than "
                "the library's %zu-byte scratch; use ia_paged_attn_decode with a caller workspace",
                B, max_seq_len, ia_decode_workspace_bytes(ctx, B, max_seq_len), kScratchBytes);
  return st;
}

size_t ia_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

size_t ia_stream_read_sink_bytes(void) { return (size_t)ia::stream_read_blocks() * sizeof(uint32_t); }

ia_status ia_stream_read(const void* buf, size_t bytes, void* sink, size_t sink_bytes, void* stream) {
  if (bytes == 0) return ok();
  if (!buf || !sink) return fail(IA_ERR_INVALID_ARG, "buf/sink is NULL");
  if (!aligned(buf, 16) || bytes % 16 != 0) return fail(IA_ERR_INVALID_ARG, "buf and bytes must be 16-byte aligned");
  if (sink_bytes < ia_stream_read_sink_bytes())
    return fail(IA_ERR_WORKSPACE_TOO_SMALL, "sink needs %zu bytes (got %zu)", ia_stream_read_sink_bytes(), sink_bytes);
  return hip_status(ia::launch_stream_read(buf, bytes, static_cast<uint32_t*>(sink), static_cast<hipStream_t>(stream)),
                    "stream read launch");
}

ia_status ia_paged_attn_prefill(const ia_ctx* ctx, const void* q, const int32_t* cu_q_lens,
                                const int32_t* seq_lens, const void* k_cache, const void* v_cache,
                                int32_t num_pages, const float* k_scale, const float* v_scale,
                                const int32_t* block_table, int32_t bt_stride, int32_t B, int32_t total_q,
                                int32_t max_q_len, int32_t max_seq_len, void* out, void* workspace,
                                size_t ws_bytes, void* stream) {
  if (!ctx) return fail(IA_ERR_INVALID_ARG, "ctx is NULL");
  if (B < 0 || total_q < 0 || max_q_len < 0)
    return fail(IA_ERR_INVALID_ARG, "B, total_q and max_q_len must be >= 0");
  ia_status st = check_scales(ctx, k_scale, v_scale);
  if (st != IA_OK) return st;
  if (B == 0 || total_q == 0) return ok();
  if ((st = check_pages(k_cache, v_cache, num_pages)) != IA_OK) return st;
  if (!q || !cu_q_lens || !seq_lens || !block_table || !out)
    return fail(IA_ERR_INVALID_ARG, "q/cu_q_lens/seq_lens/block_table/out is NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(IA_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  if (max_q_len <= 0 || max_seq_len <= 0)
    return fail(IA_ERR_INVALID_ARG, "max_q_len and max_seq_len must be positive when total_q > 0");
  if ((int64_t)bt_stride * ctx->cfg.page_size < max_seq_len)
    return fail(IA_ERR_INVALID_ARG, "bt_stride (%d) pages cannot hold max_seq_len (%d) keys", bt_stride, max_seq_len);
  const int64_t row_blocks = prefill_row_blocks(ctx, B, max_q_len);
  if ((int64_t)B * row_blocks * ctx->cfg.num_kv_heads >= ((int64_t)1 << 31))
    return fail(IA_ERR_INVALID_ARG, "grid too large");
  if ((int64_t)total_q * ctx->cfg.num_q_heads >= ((int64_t)1 << 31))
    return fail(IA_ERR_INVALID_ARG, "total_q x num_q_heads must be below 2^31");
  const bool multi_split = max_seq_len > ctx->cfg.split_tokens;
  const size_t fold_bytes = multi_split ? prefill_state_bytes(ctx, (int64_t)total_q * ctx->cfg.num_q_heads) : 0;
  if (multi_split) {
    if (!workspace || ws_bytes < fold_bytes)
      return fail(IA_ERR_WORKSPACE_TOO_SMALL, "prefill workspace needs %zu bytes (got %zu)", fold_bytes, ws_bytes);
    if (!aligned(workspace, 16)) return fail(IA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  ia::PrefillArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.cu_q_lens = cu_q_lens;
  a.seq_lens = seq_lens;
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.out = static_cast<__bf16*>(out);
  a.max_splits = prefill_max_splits(ctx, max_seq_len);
  a.rb = prefill_rb(ctx, B, max_q_len);
  a.ws_u = a.ws_mz = a.sg_u = a.sg_mz = nullptr;
  a.split_rbs = 0;
  if (multi_split) {
    const size_t rows = (size_t)total_q * ctx->cfg.num_q_heads;
    char* base = static_cast<char*>(workspace);
    a.ws_u = reinterpret_cast<float*>(base);
    a.ws_mz = reinterpret_cast<float*>(base + align_up(rows * ctx->cfg.head_dim * sizeof(float)));
    // The split grid, when the workspace also holds its states (a workspace
    // of the size ia_prefill_workspace_bytes reports does).
    const int rbs = prefill_split_rbs(ctx, B, total_q, max_q_len, max_seq_len);
    if (rbs > 0) {
      const int64_t entries = prefill_split_entries(ctx, B, max_q_len, max_seq_len, rbs);
      const int64_t grid = (int64_t)B * ctx->cfg.num_kv_heads * (row_blocks + (int64_t)rbs * (a.max_splits - 1));
      if (ws_bytes >= fold_bytes + prefill_state_bytes(ctx, entries) && grid < ((int64_t)1 << 31)) {
        a.split_rbs = rbs;
        a.sg_u = reinterpret_cast<float*>(base + fold_bytes);
        a.sg_mz = reinterpret_cast<float*>(base + fold_bytes + align_up((size_t)entries * ctx->cfg.head_dim * sizeof(float)));
      }
    }
  }
  a.c = ctx->c;
  a.B = B;
  a.Hq = ctx->cfg.num_q_heads;
  a.Hkv = ctx->cfg.num_kv_heads;
  a.group = ctx->group;
  a.bt_stride = bt_stride;
  a.num_pages = num_pages;
  a.max_q_len = max_q_len;
  a.max_seq_len = max_seq_len;
  a.max_row_blocks = (int)row_blocks;
  a.split_tokens = ctx->cfg.split_tokens;
  a.total_q = total_q;
  a.window = ctx->cfg.sliding_window;
  return hip_status(ia::launch_prefill(ctx->cfg.head_dim, ctx->cfg.kv_dtype == IA_KV_FP8_E4M3, a,
                                       static_cast<hipStream_t>(stream)),
                    "prefill launch");
}

ia_status ia_rmsnorm(const void* x, const void* weight, int32_t M, int32_t H, float eps, void* out, void* stream) {
  if (M < 0) return fail(IA_ERR_INVALID_ARG, "M must be >= 0 (got %d)", M);
  if (H < 8 || H % 8 != 0 || H > ia::rmsnorm_max_h())
    return fail(IA_ERR_INVALID_ARG, "H must be a multiple of 8 in [8, %d] (got %d)", ia::rmsnorm_max_h(), H);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(IA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (M == 0) return ok();
  if (!x || !weight || !out) return fail(IA_ERR_INVALID_ARG, "x/weight/out is NULL");
  if (!aligned(x, 16) || !aligned(weight, 16) || !aligned(out, 16))
    return fail(IA_ERR_INVALID_ARG, "x, weight and out must be 16-byte aligned");
  return hip_status(ia::launch_rmsnorm(static_cast<const __bf16*>(x), static_cast<const __bf16*>(weight),
                                       static_cast<__bf16*>(out), M, H, eps, static_cast<hipStream_t>(stream)),
                    "rmsnorm launch");
}

ia_status ia_gemm_bf16(const void* a, const void* w, int32_t M, int32_t N, int32_t K, void* c, void* stream) {
  if (M < 0) return fail(IA_ERR_INVALID_ARG, "M must be >= 0 (got %d)", M);
  if (N <= 0 || N % ia::gemm_tile_n() != 0)
    return fail(IA_ERR_INVALID_ARG, "N must be a positive multiple of %d (got %d)", ia::gemm_tile_n(), N);
  if (K <= 0 || K % ia::gemm_tile_k() != 0)
    return fail(IA_ERR_INVALID_ARG, "K must be a positive multiple of %d (got %d)", ia::gemm_tile_k(), K);
  if (M == 0) return ok();
  if (!a || !w || !c) return fail(IA_ERR_INVALID_ARG, "a/w/c is NULL");
  if (!aligned(a, 16) || !aligned(w, 16) || !aligned(c, 16))
    return fail(IA_ERR_INVALID_ARG, "a, w and c must be 16-byte aligned");
  if ((int64_t)(N / ia::gemm_tile_n()) * ceil_div(M, ia::gemm_tile_m()) >= ((int64_t)1 << 31))
    return fail(IA_ERR_INVALID_ARG, "grid too large");
  return hip_status(ia::launch_gemm(static_cast<const __bf16*>(a), static_cast<const __bf16*>(w),
                                    static_cast<__bf16*>(c), M, N, K, static_cast<hipStream_t>(stream)),
                    "gemm launch");
}

}  // extern "C"
