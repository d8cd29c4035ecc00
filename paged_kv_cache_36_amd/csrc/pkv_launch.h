// Internal interface between the C-ABI host layer (pkv_api.cpp) and the HIP
// kernels (pkv_kernels.hip). Not installed; not part of the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

// pkv_decode and its workspace size (shared with the allocation-free entry
// point, which passes its static scratch array as the workspace).
size_t decode_workspace(const pkv_decode_params* params);
pkv_status decode_call(const pkv_decode_params* params, const void* q, const void* key_cache,
                       const void* value_cache, const int32_t* block_table,
                       const int32_t* seq_lens, void* out, float* out_f32, void* workspace,
                       size_t workspace_bytes, void* stream);

constexpr int kHeadSize = 256;   // D
constexpr int kGroup = 6;        // query heads per KV head
constexpr int kWaveTokens = 16;  // tokens one wave handles per step (MFMA rows)
constexpr int kWaves = 4;        // waves per split workgroup
constexpr int kTileTokens = kWaveTokens * kWaves;  // 64 tokens per workgroup step
constexpr int kMaxBalancedSeqs = 4096;             // sequences the balanced split handles
// The dispatcher deals workgroups to the 8 XCDs round robin (workgroup b to
// XCD b % 8), and on MI355X the balanced split's workgroups on odd XCDs
// stream 5-8 % more slowly than those on even ones (every box measured). Its
// odd workgroups therefore get a share 1/kOddShareDiv smaller and even ones a
// share 1/kOddShareDiv larger. (The fixed-partition grid, which the
// dispatcher refills as slots free up, measured faster without such a skew.)
constexpr int kOddShareDiv = 24;
constexpr int kMaxOrderedSeqs = 1024;              // sequences the ordered fixed split handles

// Everything a split/combine/debug launch needs, already validated.
struct LaunchArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* block_table;
  const int32_t* seq_lens;
  uint16_t* out;        // bf16 [S, Hq, D] or null
  float* out_f32;       // fp32 [S, Hq, D] or null
  float* o_part;        // fp32 [S, Hq, n_parts, D] (fixed P) or [slots, 6, D] (balanced)
  float* lse_part;      // fp32 [S, Hq, n_parts] (fixed P) or [slots, 6] (balanced)
  int32_t* prefix;      // balanced: [S + 1] tile prefix sums (x Hkv), written by the split
  int64_t k_page_stride;
  int64_t v_page_stride;
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t max_blocks;
  int32_t partition_tokens;
  int32_t n_parts;
  int32_t max_seq_len;
  int32_t balanced_grid;  // balanced split: workgroups G (0 = fixed partitions)
  int32_t resident_wgs;   // fixed split: workgroups resident at once (2 per CU); the
                          // ones dispatched before the last round store nontemporally
  float scale_log2;     // scale * log2(e)
  // debug walks only
  int64_t* dbg_offsets;   // resolve: int64 [S, max_seq_len]
  uint16_t* dbg_dense;    // gather: bf16 [S, max_seq_len, Hkv, D]
  int32_t dbg_kv_head;    // resolve: the KV head recorded
  int32_t dbg_which;      // gather: 0 = the K loader, 1 = the V loader
};

// How a decode call splits its work: the balanced share or fixed partitions,
// whether a segment may refetch its page list, and whether K is loaded as
// whole rows and staged through LDS (else straight into the MFMA operand).
struct SplitChoice {
  bool balanced;
  bool refetch;
  bool k_rows;
  bool ordered;   // fixed partitions in the ordered dispatch order
};

// split kernel: per (sequence, KV head, partition). direct=true writes the
// final bf16 (and optional fp32) output, valid only when n_parts == 1.
hipError_t launch_split(const LaunchArgs& a, bool direct, const SplitChoice& c,
                        hipStream_t stream);
// balanced split: G = a.balanced_grid workgroups share the tiles evenly.
hipError_t launch_balanced_split(const LaunchArgs& a, bool refetch, bool k_rows,
                                 hipStream_t stream);
// combine: per_run (balanced only) merges each (sequence, KV head) run's six
// query heads in one wave; otherwise one wave per (sequence, head, quarter)
hipError_t launch_combine(const LaunchArgs& a, bool balanced, bool per_run, hipStream_t stream);
bool partition_needs_refetch(int32_t partition_tokens, int32_t block_size);
// The split `c` walks its segments and records what decode reads: row
// offsets (a.dbg_offsets, a.dbg_kv_head) or rows through decode's loaders
// (a.dbg_dense, a.dbg_which).
hipError_t launch_debug_resolve(const LaunchArgs& a, const SplitChoice& c, hipStream_t stream);
hipError_t launch_debug_gather(const LaunchArgs& a, const SplitChoice& c, hipStream_t stream);
// KV append: one wave per new token, rows moved as 16-byte chunks.
struct AppendArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int64_t* slots;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int64_t k_new_stride, v_new_stride;   // elements
  int64_t k_page_stride, v_page_stride; // elements
  int64_t num_slots;                    // num_pages * block_size
  int32_t num_tokens;
  int32_t block_size;
  int32_t row_chunks;                   // Hkv * D / 8
};
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
// Tail-Q prefill of one sequence: num_q new tokens at positions seq_len - num_q ..
struct PrefillArgs {
  const uint16_t* q;            // [num_q, Hq, D]
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* block_table;   // [max_blocks] of this sequence
  uint16_t* out;                // bf16 [num_q, Hq, D] or null
  float* out_f32;               // fp32 [num_q, Hq, D] or null
  int64_t k_page_stride;
  int64_t v_page_stride;
  int32_t num_q;
  int32_t seq_len;
  int32_t num_kv_heads;
  int32_t block_size;
  float scale_log2;             // scale * log2(e)
  // key splits: 1 writes out / out_f32 directly; more write per-split partials
  // (o_part fp32 [key_splits, num_q, Hq, D], lse_part fp32 [key_splits, num_q,
  // Hq] in log2 units) that a second kernel merges into out / out_f32; the
  // short_blocks lowest query blocks use only key_splits - 1 of them
  int32_t key_splits;
  int32_t short_blocks;         // the lowest query blocks that take key_splits - 1 splits
  float* o_part;
  float* lse_part;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// Paged window compression: per-dimension softmax over each boundary token's
// window of state rows [values(D) | scores(D)], fp32, D = kCompressDim.
constexpr int kCompressDim = 512;
constexpr int kCompressMaxBlocks = 64;   // logical blocks one window part may touch
constexpr int kCompressMaxSplits = 64;   // window parts per output the combine merges
struct CompressArgs {
  const float* state;             // paged state cache
  const int32_t* token_to_req;    // [num_tokens]
  const int64_t* positions;       // [num_tokens]
  const int64_t* boundaries;      // [num_outputs] token indices
  const int32_t* block_table;     // [num_reqs, max_blocks]
  float* out;                     // [num_outputs, D]
  float* o_part;                  // [num_outputs, num_splits, D] (num_splits > 1)
  float* lse_part;                // same shape, log2 units
  int64_t block_stride;           // elements between state blocks
  int64_t row_stride;             // elements between rows of a block
  int32_t num_outputs;
  int32_t num_tokens;
  int32_t num_reqs;
  int32_t max_blocks;
  int32_t block_size;
  int32_t compress_ratio;
  int32_t num_splits;             // window parts per output
  int32_t part_rows;              // ceil(compress_ratio / num_splits)
  int32_t combine_lanes;          // lanes per (output, 4 dims) in the combine: 1, 2, 4 or 8
};
// split kernel, then (num_splits > 1) the combine kernel
hipError_t launch_compress(const CompressArgs& a, hipStream_t stream);
// The compression finalizer: RMSNorm, NOPE INT8 + scale bytes, GPT-J RoPE in
// bf16, written into 64-slot KV pages of 64 * (576 + 8) bytes.
constexpr int kKvBlockSize = 64;
constexpr int kKvTokenStride = 576;
constexpr int kKvScaleDim = 8;
struct FinalizeArgs {
  const float* compressed;        // [num_outputs, 512]
  const int64_t* positions;       // [num_tokens]
  const int64_t* boundaries;      // [num_outputs]
  const float* weight;            // [512]
  const float* cos_sin;           // [cos_sin_rows, 64]: cos 0..31, sin 32..63
  const int64_t* slots;           // [num_tokens]
  uint8_t* kv;                    // [num_kv_pages, kv_page_stride bytes]
  int64_t num_kv_pages;
  int64_t kv_page_stride;
  int32_t num_outputs;
  int32_t num_tokens;
  int32_t compress_ratio;
  int32_t cos_sin_rows;
  float eps;
};
hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t stream);
// pkv_compress_pack: the compression with the finalizer fused into its last
// kernel (the split kernel with one part per window, else the combine);
// f.compressed is unused and a.out may be null.
hipError_t launch_compress_pack(const CompressArgs& a, const FinalizeArgs& f, hipStream_t stream);
int32_t probe_sink_floats();
hipError_t launch_probe_read(const void* buf, size_t bytes, float* sink, hipStream_t stream);
hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

}  // namespace pkv
