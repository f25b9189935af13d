// launch.hpp -- kernel argument blocks and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ia {

struct AppendArgs {
  const __bf16* k_new;
  const __bf16* v_new;
  const int64_t* slots;
  int T;
  uint8_t* k_cache;
  uint8_t* v_cache;
  int num_pages;
  int Hkv;
  const float* k_scale;
  const float* v_scale;
};

struct DecodeArgs {
  const __bf16* q;            // [B][Hq][D]
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;  // [B][bt_stride]
  const int32_t* seq_lens;     // [B]
  __bf16* out;                 // [B][Hq][D]
  float* ws_u;                 // [B][max_splits][Hq][D]
  float* ws_ml;                // [B][max_splits][Hq][2]
  int32_t* order;              // [B * max_splits] dispatch order of the split units (workspace)
  float* ws_x;                 // spread: per slot [4 parts][4 lane groups][group][16 B]: scores, then weights
  float* ws_mx;                // spread: row maxima, [slot][16]
  float* ws_as;                // spread: (alpha, row sum, row maximum, 0), [slot][16][4]
  float c;                     // fp32(sm_scale * log2 e)
  int B, Hq, Hkv, group;
  int bt_stride, num_pages;
  int max_seq_len, max_splits;
  int split_tokens, policy;
  int window;                  // 0: full causal attention; w > 0: keys p - w < j <= p
  int kernel;                  // 0: decode_split_kernel, 1: decode_wide_kernel, 2: the spread kernels
                               // (score, weight, value); all give the same bits
  int tps;                     // spread: tile slots per split (the longest split of the launch, in tiles)
  int nt;                      // split kernel: nontemporal page loads (caching only, never values)
  int self_order;              // split kernel without an order list: each workgroup finds its unit
                               // in the list's order (B <= kSelfOrderMaxB)
};

struct PrefillArgs {
  const __bf16* q;            // [total_q][Hq][D]
  const int32_t* cu_q_lens;   // [B+1]
  const int32_t* seq_lens;    // [B]
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  __bf16* out;
  // Row states, entry (row, query head) of [total_q][Hq]: D fp32 of U (ws_u)
  // and (M, Z) (ws_mz).  In-workgroup folds: the merge of the row's splits so
  // far.  Split grid: the row's state at the end of split 0.
  float* ws_u;
  float* ws_mz;
  // Split grid: the states of splits 1 .. max_splits - 1 of the rows of split
  // sequences, entry ((b * split_rows + i) * (max_splits - 1) + s - 1) * Hq +
  // head, split_rows = split_rbs x positions per row block.
  float* sg_u;
  float* sg_mz;
  int split_rbs;              // sequences of at most this many row blocks whose keys reach a
                              // second split run one workgroup per split (0: none)
  int max_splits;             // ceil(max_seq_len / split_tokens)
  int rb;                     // 16-row blocks per wave (prefill_rows_per_wave)
  float c;
  int B, Hq, Hkv, group;
  int bt_stride, num_pages;
  int max_q_len, max_seq_len, max_row_blocks;
  int split_tokens;
  int total_q;
  int window;                 // 0: full causal attention; w > 0: keys p - w < j <= p
};

hipError_t launch_kv_append(int D, bool fp8, const AppendArgs& a, hipStream_t st);
hipError_t launch_decode(int D, bool fp8, const DecodeArgs& a, hipStream_t st);
hipError_t launch_prefill(int D, bool fp8, const PrefillArgs& a, hipStream_t st);
// Row blocks per wave of a prefill launch: fp8 pages 1; bf16 pages 2, or 1
// when the launch would have fewer than 256 workgroups with 2 (units_two_blocks:
// its (sequence, row block, kv head) count with 2).
int prefill_rows_per_wave(bool fp8, int64_t units_two_blocks);
// Query positions one prefill workgroup covers at rb row blocks per wave (its
// grid has ceil(max_q_len / this) row blocks per (sequence, kv head)).
int prefill_positions_per_block(int group, int rb);

// Layer operators (layer_ops.hip).
hipError_t launch_rmsnorm(const __bf16* x, const __bf16* w, __bf16* y, int M, int H, float eps, hipStream_t st);
hipError_t launch_gemm(const __bf16* a, const __bf16* wt, __bf16* c, int M, int N, int K, hipStream_t st);
// Measurement reference (probe.hip): a plain streaming read of `bytes`.
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st);
int stream_read_blocks();
int gemm_tile_m();
int gemm_tile_n();
int gemm_tile_k();
int rmsnorm_max_h();

}  // namespace ia
