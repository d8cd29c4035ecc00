// C-ABI host layer: argument validation and launch (the decode plan is in pkv_plan.cpp).
// Declarations and the contract of every entry point are in include/pkv.h.

#include "pkv.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "pkv_launch.h"
#include "pkv_plan.h"

namespace {

using pkv::base_args;
using pkv::check_params;
using pkv::kWorkspaceAlign;
using pkv::make_decode_plan;
using pkv::make_fixed_plan;
using pkv::Plan;
using pkv::split_choice;
using pkv::split_workgroups;

bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("PKV_LOG");
    return e != nullptr && e[0] != '\0' && e[0] != '0';
  }();
  return on;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }


void log_plan(const char* what, const pkv_decode_params* p, const Plan& pl) {
  if (!log_enabled()) return;
  std::fprintf(stderr,
               "[pkv] %s: S=%d Hq=%d Hkv=%d D=%d block_size=%d (64-token groups %d, tail %d) "
               "max_seq_len=%d %s P=%d partitions=%d split_wg=%lld refetch=%d k_rows=%d "
               "ordered=%d combine=%s workspace=%zu\n",
               what, p->num_seqs, p->num_q_heads, p->num_kv_heads, p->head_size, p->block_size,
               p->block_size / 64, p->block_size % 64, p->max_seq_len,
               pl.balanced ? "balanced" : "fixed", pl.P, pl.n_parts,
               static_cast<long long>(split_workgroups(p, pl)), pl.refetch ? 1 : 0,
               pl.k_rows ? 1 : 0, pl.ordered ? 1 : 0,
               (pl.balanced || pl.n_parts > 1) ? "yes" : "no", pl.workspace);
}

pkv_status check_inputs(const void* q, const void* k, const void* v, const int32_t* bt,
                        const int32_t* sl) {
  if (!q || !k || !v || !bt || !sl) return PKV_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(bt, 4) || !aligned(sl, 4))
    return PKV_ERR_NULL;
  return PKV_OK;
}

pkv_status hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

pkv_status check_workspace(const Plan& pl, const void* workspace, size_t workspace_bytes) {
  if (pl.workspace > 0 &&
      (workspace == nullptr || workspace_bytes < pl.workspace || !aligned(workspace, kWorkspaceAlign)))
    return PKV_ERR_WORKSPACE;
  return PKV_OK;
}

// Partials (and, for the balanced split, tile prefix sums) inside the workspace.
void carve_workspace(const Plan& pl, void* workspace, pkv::LaunchArgs& a) {
  char* ws = static_cast<char*>(workspace);
  a.o_part = reinterpret_cast<float*>(ws);
  a.lse_part = reinterpret_cast<float*>(ws + pl.o_part_bytes);
  if (pl.balanced) a.prefix = reinterpret_cast<int32_t*>(ws + pl.o_part_bytes + pl.lse_bytes);
}

}  // namespace

namespace {

// Prefill key splits: queries per workgroup of the prefill kernel, the most
// splits a call may ask for, and the CU count the automatic choice fills.
constexpr int64_t kPrefillQueries = 128;
constexpr int32_t kPrefillMaxSplits = 64;
// the CUs the automatic split count fills: pkv::plan_cus()

// Host checks shared by the prefill entry points.
pkv_status check_prefill_params(const pkv_prefill_params* p) {
  if (p->head_size != pkv::kHeadSize || p->num_kv_heads <= 0 ||
      p->num_q_heads != pkv::kGroup * p->num_kv_heads)
    return PKV_ERR_UNSUPPORTED;
  if (p->block_size <= 0) return PKV_ERR_BLOCK_SIZE;
  if (p->num_q_tokens < 1 || p->seq_len < p->num_q_tokens || p->max_blocks <= 0 ||
      static_cast<int64_t>(p->seq_len) > static_cast<int64_t>(p->max_blocks) * p->block_size ||
      !std::isfinite(p->scale))
    return PKV_ERR_SHAPE;
  const int64_t row = static_cast<int64_t>(p->num_kv_heads) * p->head_size;
  if (p->k_page_stride < p->block_size * row || p->v_page_stride < p->block_size * row ||
      p->k_page_stride % 8 != 0 || p->v_page_stride % 8 != 0)
    return PKV_ERR_STRIDE;
  if (p->key_splits < 0 || p->key_splits > kPrefillMaxSplits) return PKV_ERR_PARTITION;
  return PKV_OK;
}

// Key splits of a checked call: the caller's, else one while the launch
// already has two workgroups per CU, else the smallest count giving three
// (at most 16) that keeps 16 tiles in every split of the shortest block.
// Measured on MI355X (Q = 1500, L = 20000, 288 workgroups unsplit): 1 / 2 /
// 3 / 4 / 8 splits ran 1020 / 846 / 809 / 815 / 880 us; every split adds
// partials and per-workgroup start-up, so a few rounds of workgroups are enough.
int32_t prefill_key_splits(const pkv_prefill_params* p) {
  if (p->key_splits > 0) return p->key_splits;
  const int64_t nqb = (p->num_q_tokens + kPrefillQueries - 1) / kPrefillQueries;
  const int64_t wgs = nqb * p->num_q_heads;
  const int64_t cus = pkv::plan_cus();
  if (wgs >= 2 * cus) return 1;
  // keys of the shortest query block (block 0): up to its last query's position
  const int64_t kend0 = static_cast<int64_t>(p->seq_len) - p->num_q_tokens +
                        std::min<int64_t>(kPrefillQueries, p->num_q_tokens);
  const int64_t tiles0 = (kend0 + 63) / 64;
  int32_t k = 1;
  while (k < 16 && wgs * k < 3 * cus && tiles0 / (k + 1) >= 16) ++k;
  return k;
}

// Query blocks that take one key split fewer than the others: with an
// automatic count S >= 2, the fewest of the shortest (lowest) blocks that
// make the workgroup count Hq (nqb S - n) a whole number of rounds over the
// CUs, if some n < nqb does; 0 otherwise, and when the caller fixed the count.
// The last round then runs full instead of part empty (Q = 1500, L = 20000:
// 864 workgroups for 256 CUs with 3 splits everywhere; 768 with 2 splits for
// the 4 shortest of the 12 blocks).
int32_t prefill_short_blocks(const pkv_prefill_params* p, int32_t splits) {
  if (p->key_splits > 0 || splits < 2) return 0;
  const int64_t nqb = (p->num_q_tokens + kPrefillQueries - 1) / kPrefillQueries;
  const int64_t cus = pkv::plan_cus();
  for (int64_t n = 0; n < nqb; ++n)
    if ((static_cast<int64_t>(p->num_q_heads) * (nqb * splits - n)) % cus == 0)
      return static_cast<int32_t>(n);
  return 0;
}

size_t prefill_workspace(const pkv_prefill_params* p, int32_t splits) {
  if (splits <= 1) return 0;
  return static_cast<size_t>(splits) * p->num_q_tokens * p->num_q_heads *
         (pkv::kHeadSize + 1) * sizeof(float);
}

}  // namespace

namespace pkv {

size_t decode_workspace(const pkv_decode_params* params) {
  if (check_params(params) != PKV_OK) return 0;
  return make_decode_plan(params).workspace;
}

pkv_status decode_call(const pkv_decode_params* params, const void* q, const void* key_cache,
                       const void* value_cache, const int32_t* block_table,
                       const int32_t* seq_lens, void* out, float* out_f32, void* workspace,
                       size_t workspace_bytes, void* stream) {
  pkv_status st = check_params(params);
  if (st != PKV_OK) return st;
  if (params->num_seqs == 0) return PKV_OK;
  st = check_inputs(q, key_cache, value_cache, block_table, seq_lens);
  if (st != PKV_OK) return st;
  if (!out || !aligned(out, 16) || (out_f32 != nullptr && !aligned(out_f32, 16)))
    return PKV_ERR_NULL;
  const Plan pl = make_decode_plan(params);
  st = check_workspace(pl, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  log_plan("decode", params, pl);

  pkv::LaunchArgs a = base_args(params, pl);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(key_cache);
  a.v = static_cast<const uint16_t*>(value_cache);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = static_cast<uint16_t*>(out);
  a.out_f32 = out_f32;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!pl.balanced && pl.n_parts == 1)
    return hip_status(pkv::launch_split(a, /*direct=*/true, split_choice(pl), s));
  carve_workspace(pl, workspace, a);
  st = pl.balanced ? hip_status(pkv::launch_balanced_split(a, pl.refetch, pl.k_rows, s))
                   : hip_status(pkv::launch_split(a, /*direct=*/false, split_choice(pl), s));
  if (st != PKV_OK) return st;
  return hip_status(pkv::launch_combine(a, pl.balanced, pl.combine_per_run, s));
}

}  // namespace pkv

extern "C" {

const char* pkv_version(void) { return "pkv 0.2.0 (gfx950)"; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "null or misaligned pointer";
    case PKV_ERR_SHAPE: return "inconsistent shape";
    case PKV_ERR_BLOCK_SIZE: return "block_size must be positive (a multiple of 16 for decode)";
    case PKV_ERR_PARTITION:
      return "partition_tokens must be 0 or a multiple of 64 (prefill: key_splits 0..64)";
    case PKV_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case PKV_ERR_UNSUPPORTED: return "unsupported head geometry (need head_size 256, 6 query heads per KV head)";
    case PKV_ERR_HIP: return "HIP launch or runtime error";
    case PKV_ERR_STRIDE: return "page stride smaller than a page or not a multiple of 8";
    case PKV_ERR_SCRATCH:
      return "workspace needed exceeds the static scratch array of pkv_decode_noalloc (32 MiB)";
    default: return "unknown status";
  }
}

pkv_status pkv_plan(const pkv_decode_params* params, pkv_plan_info* info) {
  pkv_status st = check_params(params);
  if (st != PKV_OK) return st;
  if (info == nullptr) return PKV_ERR_NULL;
  const Plan fx = make_fixed_plan(params);
  const Plan dec = make_decode_plan(params);
  info->partition_tokens = fx.P;
  info->num_partitions = fx.n_parts;
  info->split_workgroups = static_cast<int32_t>(split_workgroups(params, dec));
  info->combine_workgroups =
      (dec.balanced && dec.combine_per_run) ? params->num_seqs * params->num_kv_heads
      : (dec.balanced || dec.n_parts > 1)   ? params->num_seqs * params->num_q_heads * 4
                                            : 0;
  info->balanced = dec.balanced ? 1 : 0;
  info->full_groups_per_page = params->block_size / 64;
  info->tail_tokens_per_page = params->block_size % 64;
  info->workspace_bytes = static_cast<int64_t>(dec.workspace);
  info->k_rows = dec.k_rows ? 1 : 0;
  info->ordered = (!dec.balanced && dec.ordered) ? 1 : 0;
  return PKV_OK;
}

size_t pkv_decode_workspace_bytes(const pkv_decode_params* params) {
  return pkv::decode_workspace(params);
}

pkv_status pkv_decode(const pkv_decode_params* params, const void* q, const void* key_cache,
                      const void* value_cache, const int32_t* block_table,
                      const int32_t* seq_lens, void* out, float* out_f32, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return pkv::decode_call(params, q, key_cache, value_cache, block_table, seq_lens, out, out_f32,
                          workspace, workspace_bytes, stream);
}

pkv_status pkv_split_balanced(const pkv_decode_params* params, const void* q,
                              const void* key_cache, const void* value_cache,
                              const int32_t* block_table, const int32_t* seq_lens,
                              void* workspace, size_t workspace_bytes, void* stream) {
  pkv_status st = check_params(params);
  if (st != PKV_OK) return st;
  const Plan pl = make_decode_plan(params);
  if (!pl.balanced) return params->num_seqs == 0 ? PKV_OK : PKV_ERR_UNSUPPORTED;
  st = check_inputs(q, key_cache, value_cache, block_table, seq_lens);
  if (st != PKV_OK) return st;
  st = check_workspace(pl, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  log_plan("split_balanced", params, pl);
  pkv::LaunchArgs a = base_args(params, pl);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(key_cache);
  a.v = static_cast<const uint16_t*>(value_cache);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  carve_workspace(pl, workspace, a);
  return hip_status(
      pkv::launch_balanced_split(a, pl.refetch, pl.k_rows, static_cast<hipStream_t>(stream)));
}

pkv_status pkv_combine_balanced(const pkv_decode_params* params, const int32_t* seq_lens,
                                const void* workspace, size_t workspace_bytes, void* out,
                                float* out_f32, void* stream) {
  pkv_status st = check_params(params);
  if (st != PKV_OK) return st;
  const Plan pl = make_decode_plan(params);
  if (!pl.balanced) return params->num_seqs == 0 ? PKV_OK : PKV_ERR_UNSUPPORTED;
  if (!seq_lens || !aligned(seq_lens, 4) || (out != nullptr && !aligned(out, 16)) ||
      (out_f32 != nullptr && !aligned(out_f32, 16)))
    return PKV_ERR_NULL;
  st = check_workspace(pl, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  pkv::LaunchArgs a = base_args(params, pl);
  a.seq_lens = seq_lens;
  a.out = static_cast<uint16_t*>(out);
  a.out_f32 = out_f32;
  carve_workspace(pl, const_cast<void*>(workspace), a);
  return hip_status(pkv::launch_combine(a, /*balanced=*/true, pl.combine_per_run,
                                               static_cast<hipStream_t>(stream)));
}

pkv_status pkv_decode_partials(const pkv_decode_params* params, const void* q,
                               const void* key_cache, const void* value_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               float* o_partial, float* lse_partial, float* out_f32, void* out,
                               void* stream) {
  pkv_status st = check_params(params);
  if (st != PKV_OK) return st;
  if (params->num_seqs == 0) return PKV_OK;
  st = check_inputs(q, key_cache, value_cache, block_table, seq_lens);
  if (st != PKV_OK) return st;
  if (!o_partial || !lse_partial || !out_f32 || !aligned(o_partial, 16) || !aligned(out_f32, 16) ||
      (out != nullptr && !aligned(out, 16)))
    return PKV_ERR_NULL;
  const Plan pl = make_fixed_plan(params);
  log_plan("decode_partials", params, pl);
  pkv::LaunchArgs a = base_args(params, pl);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(key_cache);
  a.v = static_cast<const uint16_t*>(value_cache);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.o_part = o_partial;
  a.lse_part = lse_partial;
  a.out = static_cast<uint16_t*>(out);
  a.out_f32 = out_f32;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(pkv::launch_split(a, /*direct=*/false, split_choice(pl), s));
  if (st != PKV_OK) return st;
  return hip_status(pkv::launch_combine(a, /*balanced=*/false, /*per_run=*/false, s));
}

pkv_status pkv_split(const pkv_decode_params* params, const void* q, const void* key_cache,
                     const void* value_cache, const int32_t* block_table,
                     const int32_t* seq_lens, float* o_partial, float* lse_partial,
                     void* stream) {
  pkv_status st = check_params(params);
  if (st != PKV_OK) return st;
  if (params->num_seqs == 0) return PKV_OK;
  st = check_inputs(q, key_cache, value_cache, block_table, seq_lens);
  if (st != PKV_OK) return st;
  if (!o_partial || !lse_partial || !aligned(o_partial, 16) || !aligned(lse_partial, 4))
    return PKV_ERR_NULL;
  const Plan pl = make_fixed_plan(params);
  log_plan("split", params, pl);
  pkv::LaunchArgs a = base_args(params, pl);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(key_cache);
  a.v = static_cast<const uint16_t*>(value_cache);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.o_part = o_partial;
  a.lse_part = lse_partial;
  return hip_status(
      pkv::launch_split(a, /*direct=*/false, split_choice(pl), static_cast<hipStream_t>(stream)));
}

pkv_status pkv_combine(const pkv_decode_params* params, const float* o_partial,
                       const float* lse_partial, const int32_t* seq_lens, void* out,
                       float* out_f32, void* stream) {
  pkv_status st = check_params(params);
  if (st != PKV_OK) return st;
  if (params->num_seqs == 0) return PKV_OK;
  if (!o_partial || !lse_partial || !seq_lens || !aligned(o_partial, 16) ||
      (out != nullptr && !aligned(out, 16)) || (out_f32 != nullptr && !aligned(out_f32, 16)))
    return PKV_ERR_NULL;
  const Plan pl = make_fixed_plan(params);
  pkv::LaunchArgs a = base_args(params, pl);
  a.seq_lens = seq_lens;
  a.o_part = const_cast<float*>(o_partial);
  a.lse_part = const_cast<float*>(lse_partial);
  a.out = static_cast<uint16_t*>(out);
  a.out_f32 = out_f32;
  return hip_status(pkv::launch_combine(a, /*balanced=*/false, /*per_run=*/false,
                                               static_cast<hipStream_t>(stream)));
}

pkv_status pkv_debug_resolve(const pkv_decode_params* params, int32_t kv_head,
                             const int32_t* block_table, const int32_t* seq_lens,
                             int64_t* row_offsets, void* stream) {
  pkv_status st = check_params(params);
  if (st != PKV_OK) return st;
  if (kv_head < 0 || kv_head >= params->num_kv_heads) return PKV_ERR_SHAPE;
  if (params->num_seqs == 0) return PKV_OK;
  if (!block_table || !seq_lens || !row_offsets || !aligned(row_offsets, 8)) return PKV_ERR_NULL;
  const Plan pl = make_decode_plan(params);
  pkv::LaunchArgs a = base_args(params, pl);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.dbg_offsets = row_offsets;
  a.dbg_kv_head = kv_head;
  return hip_status(
      pkv::launch_debug_resolve(a, split_choice(pl), static_cast<hipStream_t>(stream)));
}

pkv_status pkv_debug_gather(const pkv_decode_params* params, int32_t which, const void* cache,
                            const int32_t* block_table, const int32_t* seq_lens, void* dense,
                            void* stream) {
  pkv_status st = check_params(params);
  if (st != PKV_OK) return st;
  if (which != 0 && which != 1) return PKV_ERR_SHAPE;
  if (params->num_seqs == 0) return PKV_OK;
  if (!cache || !block_table || !seq_lens || !dense || !aligned(cache, 16) || !aligned(dense, 16))
    return PKV_ERR_NULL;
  const Plan pl = make_decode_plan(params);
  pkv::LaunchArgs a = base_args(params, pl);
  a.k = static_cast<const uint16_t*>(cache);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.dbg_dense = static_cast<uint16_t*>(dense);
  a.dbg_which = which;
  return hip_status(
      pkv::launch_debug_gather(a, split_choice(pl), static_cast<hipStream_t>(stream)));
}

int32_t pkv_probe_sink_floats(void) { return pkv::probe_sink_floats(); }

pkv_status pkv_probe_read(const void* buf, size_t bytes, float* sink, void* stream) {
  if (!buf || !sink || !aligned(buf, 16) || bytes % 16 != 0) return PKV_ERR_NULL;
  return hip_status(pkv::launch_probe_read(buf, bytes, sink, static_cast<hipStream_t>(stream)));
}

pkv_status pkv_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src || !aligned(dst, 16) || !aligned(src, 16) || bytes % 16 != 0)
    return PKV_ERR_NULL;
  return hip_status(pkv::launch_probe_copy(dst, src, bytes, static_cast<hipStream_t>(stream)));
}

pkv_status pkv_append(const pkv_append_params* p, const void* k_new, const void* v_new,
                      const int64_t* slot_mapping, void* key_cache, void* value_cache,
                      void* stream) {
  if (!p) return PKV_ERR_NULL;
  if (p->num_tokens < 0 || p->num_kv_heads <= 0 || p->head_size <= 0 || p->num_pages < 0)
    return PKV_ERR_SHAPE;
  if (p->block_size <= 0) return PKV_ERR_BLOCK_SIZE;
  const int64_t row_elems = static_cast<int64_t>(p->num_kv_heads) * p->head_size;
  if (row_elems % 8 != 0 || row_elems > (int64_t{1} << 20)) return PKV_ERR_UNSUPPORTED;
  if (p->k_page_stride < p->block_size * row_elems || p->v_page_stride < p->block_size * row_elems ||
      p->k_page_stride % 8 != 0 || p->v_page_stride % 8 != 0 || p->k_new_stride < row_elems ||
      p->v_new_stride < row_elems || p->k_new_stride % 8 != 0 || p->v_new_stride % 8 != 0)
    return PKV_ERR_STRIDE;
  if (p->num_pages > (int64_t{1} << 62) / p->block_size) return PKV_ERR_SHAPE;
  if (p->num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !key_cache || !value_cache || !aligned(k_new, 16) ||
      !aligned(v_new, 16) || !aligned(slot_mapping, 8) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16))
    return PKV_ERR_NULL;
  pkv::AppendArgs a;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.slots = slot_mapping;
  a.k_cache = static_cast<uint16_t*>(key_cache);
  a.v_cache = static_cast<uint16_t*>(value_cache);
  a.k_new_stride = p->k_new_stride;
  a.v_new_stride = p->v_new_stride;
  a.k_page_stride = p->k_page_stride;
  a.v_page_stride = p->v_page_stride;
  a.num_slots = p->num_pages * p->block_size;
  a.num_tokens = p->num_tokens;
  a.block_size = p->block_size;
  a.row_chunks = static_cast<int32_t>(row_elems / 8);
  return hip_status(pkv::launch_append(a, static_cast<hipStream_t>(stream)));
}

int32_t pkv_prefill_key_splits(const pkv_prefill_params* p) {
  if (!p) return PKV_ERR_NULL;
  const pkv_status st = check_prefill_params(p);
  if (st != PKV_OK) return st;
  return prefill_key_splits(p);
}

int32_t pkv_prefill_short_blocks(const pkv_prefill_params* p) {
  if (!p) return PKV_ERR_NULL;
  const pkv_status st = check_prefill_params(p);
  if (st != PKV_OK) return st;
  return prefill_short_blocks(p, prefill_key_splits(p));
}

size_t pkv_prefill_workspace_bytes(const pkv_prefill_params* p) {
  if (!p || check_prefill_params(p) != PKV_OK) return 0;
  return prefill_workspace(p, prefill_key_splits(p));
}

pkv_status pkv_prefill(const pkv_prefill_params* p, const void* q, const void* key_cache,
                       const void* value_cache, const int32_t* block_table, void* out,
                       float* out_f32, void* workspace, size_t workspace_bytes, void* stream) {
  if (!p) return PKV_ERR_NULL;
  const pkv_status st = check_prefill_params(p);
  if (st != PKV_OK) return st;
  if (!q || !key_cache || !value_cache || !block_table || (!out && !out_f32) || !aligned(q, 16) ||
      !aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(block_table, 4) ||
      (out && !aligned(out, 16)) || (out_f32 && !aligned(out_f32, 16)))
    return PKV_ERR_NULL;
  const int32_t splits = prefill_key_splits(p);
  const size_t need = prefill_workspace(p, splits);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
    return PKV_ERR_WORKSPACE;
  pkv::PrefillArgs a;
  a.key_splits = splits;
  a.short_blocks = prefill_short_blocks(p, splits);
  a.o_part = need > 0 ? static_cast<float*>(workspace) : nullptr;
  a.lse_part = need > 0 ? static_cast<float*>(workspace) +
                              static_cast<int64_t>(splits) * p->num_q_tokens * p->num_q_heads *
                                  pkv::kHeadSize
                        : nullptr;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(key_cache);
  a.v = static_cast<const uint16_t*>(value_cache);
  a.block_table = block_table;
  a.out = static_cast<uint16_t*>(out);
  a.out_f32 = out_f32;
  a.k_page_stride = p->k_page_stride;
  a.v_page_stride = p->v_page_stride;
  a.num_q = p->num_q_tokens;
  a.seq_len = p->seq_len;
  a.num_kv_heads = p->num_kv_heads;
  a.block_size = p->block_size;
  a.scale_log2 = static_cast<float>(static_cast<double>(p->scale) * 1.4426950408889634);
  return hip_status(pkv::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Window parts per output: the caller's S, else the smallest power of two that
// gives at least one workgroup per CU (pkv::plan_cus(), 256 on MI355X) while
// parts keep 16 rows or more.
// Measured on MI355X over the 12 shapes (1/4/8 requests, C = 128/256/512):
// more parts than that only add partials and the combine launch (4 x 32768
// tokens, C = 128: 1 / 2 / 4 parts ran 24.6 / 29.2 / 32.2 us), and a target of
// 1024 workgroups was up to 24 % slower on every shape it split. Every part
// must touch at most kCompressMaxBlocks logical blocks (its ids sit one per
// lane), and an output has at most kCompressMaxSplits parts (the combine's
// lanes). Returns a negative status for invalid params.

int32_t compress_splits(const pkv_compress_params* p) {
  if (!p) return PKV_ERR_NULL;
  if (p->head_dim != pkv::kCompressDim) return PKV_ERR_UNSUPPORTED;
  if (p->block_size <= 0) return PKV_ERR_BLOCK_SIZE;
  if (p->num_outputs < 0 || p->num_tokens < 0 || p->num_reqs < 0 || p->max_blocks < 0 ||
      p->compress_ratio < 1 || (p->num_outputs > 0 && (p->num_tokens < 1 || p->num_reqs < 1 ||
                                                        p->max_blocks < 1)) ||
      static_cast<int64_t>(p->max_blocks) * p->block_size > INT32_MAX)
    return PKV_ERR_SHAPE;
  if (p->row_stride < 2 * p->head_dim || p->row_stride % 4 != 0 ||
      p->block_stride < p->block_size * p->row_stride || p->block_stride % 4 != 0)
    return PKV_ERR_STRIDE;
  const int64_t c = p->compress_ratio;
  auto blocks_touched = [&](int64_t s) {
    const int64_t rows = (c + s - 1) / s;
    return (rows - 1 + p->block_size - 1) / p->block_size + 1;
  };
  int64_t s = p->num_splits;
  if (s < 0 || s > c || s > pkv::kCompressMaxSplits) return PKV_ERR_PARTITION;
  if (s > 0) {
    if (blocks_touched(s) > pkv::kCompressMaxBlocks) return PKV_ERR_PARTITION;
  } else {
    s = 1;
    while (blocks_touched(s) > pkv::kCompressMaxBlocks) s *= 2;
    const int64_t target = pkv::plan_cus();
    while (static_cast<int64_t>(p->num_outputs) * s < target &&
           (c + 2 * s - 1) / (2 * s) >= 16)
      s *= 2;
    if (s > c) s = c;
    if (s > pkv::kCompressMaxSplits) return PKV_ERR_UNSUPPORTED;
  }
  if (static_cast<int64_t>(p->num_outputs) * s > INT32_MAX) return PKV_ERR_SHAPE;
  return static_cast<int32_t>(s);
}

// Launch arguments of a checked compression call with s parts; the workspace
// (need bytes, s > 1) holds the parts' outputs, then their log2-sum-exps.
pkv::CompressArgs compress_args(const pkv_compress_params* p, int32_t s, const float* state_cache,
                                const int32_t* token_to_req, const int64_t* positions,
                                const int64_t* boundary_token_indices, const int32_t* block_table,
                                float* compressed, void* workspace, size_t need) {
  pkv::CompressArgs a;
  a.state = state_cache;
  a.token_to_req = token_to_req;
  a.positions = positions;
  a.boundaries = boundary_token_indices;
  a.block_table = block_table;
  a.out = compressed;
  a.o_part = need > 0 ? static_cast<float*>(workspace) : nullptr;
  a.lse_part = need > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + need / 2)
                        : nullptr;
  a.block_stride = p->block_stride;
  a.row_stride = p->row_stride;
  a.num_outputs = p->num_outputs;
  a.num_tokens = p->num_tokens;
  a.num_reqs = p->num_reqs;
  a.max_blocks = p->max_blocks;
  a.block_size = p->block_size;
  a.compress_ratio = p->compress_ratio;
  a.num_splits = s;
  a.part_rows = (p->compress_ratio + s - 1) / s;
  a.combine_lanes = 1;
  while (a.combine_lanes * 8 < s) a.combine_lanes *= 2;
  return a;
}

pkv_status check_finalize_params(const pkv_finalize_params* p) {
  if (p->num_outputs < 0 || p->num_tokens < 0 || p->compress_ratio < 1 || p->cos_sin_rows < 0 ||
      p->num_kv_pages < 0 || (p->num_outputs > 0 && p->num_tokens < 1) ||
      !std::isfinite(p->rms_norm_eps) || p->rms_norm_eps < 0.f ||
      p->num_kv_pages > INT64_MAX / (pkv::kKvBlockSize * 2))
    return PKV_ERR_SHAPE;
  if (p->kv_page_stride < pkv::kKvBlockSize * (pkv::kKvTokenStride + pkv::kKvScaleDim) ||
      p->kv_page_stride % 16 != 0)
    return PKV_ERR_STRIDE;
  return PKV_OK;
}

bool finalize_pointers_ok(const int64_t* positions, const int64_t* boundary_token_indices,
                          const float* rms_norm_weight, const float* cos_sin_cache,
                          const int64_t* kv_slot_mapping, const void* kv_cache) {
  return positions && boundary_token_indices && rms_norm_weight && cos_sin_cache &&
         kv_slot_mapping && kv_cache && aligned(rms_norm_weight, 16) &&
         aligned(cos_sin_cache, 16) && aligned(kv_cache, 16) && aligned(positions, 8) &&
         aligned(boundary_token_indices, 8) && aligned(kv_slot_mapping, 8);
}

// Finalizer arguments of a checked call (`compressed` left null: the caller
// sets it, or the fused path hands the values over inside its last kernel).
pkv::FinalizeArgs finalize_args(const pkv_finalize_params* p, const int64_t* positions,
                                const int64_t* boundary_token_indices, const float* rms_norm_weight,
                                const float* cos_sin_cache, const int64_t* kv_slot_mapping,
                                void* kv_cache) {
  pkv::FinalizeArgs a;
  a.compressed = nullptr;
  a.positions = positions;
  a.boundaries = boundary_token_indices;
  a.weight = rms_norm_weight;
  a.cos_sin = cos_sin_cache;
  a.slots = kv_slot_mapping;
  a.kv = static_cast<uint8_t*>(kv_cache);
  a.num_kv_pages = p->num_kv_pages;
  a.kv_page_stride = p->kv_page_stride;
  a.num_outputs = p->num_outputs;
  a.num_tokens = p->num_tokens;
  a.compress_ratio = p->compress_ratio;
  a.cos_sin_rows = p->cos_sin_rows;
  a.eps = p->rms_norm_eps;
  return a;
}

}  // namespace

extern "C" {

int32_t pkv_compress_splits(const pkv_compress_params* params) { return compress_splits(params); }

size_t pkv_compress_workspace_bytes(const pkv_compress_params* params) {
  const int32_t s = compress_splits(params);
  if (s <= 1) return 0;
  const size_t part = static_cast<size_t>(params->num_outputs) * s * pkv::kCompressDim * 4;
  return 2 * ((part + 255) / 256 * 256);
}

pkv_status pkv_compress(const pkv_compress_params* p, const float* state_cache,
                        const int32_t* token_to_req, const int64_t* positions,
                        const int64_t* boundary_token_indices, const int32_t* block_table,
                        float* compressed, void* workspace, size_t workspace_bytes,
                        void* stream) {
  const int32_t s = compress_splits(p);
  if (s < 0) return static_cast<pkv_status>(s);
  if (p->num_outputs == 0) return PKV_OK;
  if (!state_cache || !token_to_req || !positions || !boundary_token_indices || !block_table ||
      !compressed || !aligned(state_cache, 16) || !aligned(compressed, 16) ||
      !aligned(token_to_req, 4) || !aligned(positions, 8) || !aligned(boundary_token_indices, 8) ||
      !aligned(block_table, 4))
    return PKV_ERR_NULL;
  const size_t need = pkv_compress_workspace_bytes(p);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return PKV_ERR_WORKSPACE;
  const pkv::CompressArgs a = compress_args(p, s, state_cache, token_to_req, positions,
                                            boundary_token_indices, block_table, compressed,
                                            workspace, need);
  return hip_status(pkv::launch_compress(a, static_cast<hipStream_t>(stream)));
}

pkv_status pkv_compress_finalize(const pkv_finalize_params* p, const float* compressed,
                                 const int64_t* positions, const int64_t* boundary_token_indices,
                                 const float* rms_norm_weight, const float* cos_sin_cache,
                                 const int64_t* kv_slot_mapping, void* kv_cache, void* stream) {
  if (!p) return PKV_ERR_NULL;
  const pkv_status st = check_finalize_params(p);
  if (st != PKV_OK || p->num_outputs == 0) return st;
  if (!compressed || !aligned(compressed, 16) ||
      !finalize_pointers_ok(positions, boundary_token_indices, rms_norm_weight, cos_sin_cache,
                            kv_slot_mapping, kv_cache))
    return PKV_ERR_NULL;
  pkv::FinalizeArgs a = finalize_args(p, positions, boundary_token_indices, rms_norm_weight,
                                      cos_sin_cache, kv_slot_mapping, kv_cache);
  a.compressed = compressed;
  return hip_status(pkv::launch_finalize(a, static_cast<hipStream_t>(stream)));
}

pkv_status pkv_compress_pack(const pkv_compress_params* p, const pkv_finalize_params* fp,
                             const float* state_cache, const int32_t* token_to_req,
                             const int64_t* positions, const int64_t* boundary_token_indices,
                             const int32_t* block_table, const float* rms_norm_weight,
                             const float* cos_sin_cache, const int64_t* kv_slot_mapping,
                             void* kv_cache, float* compressed, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!p || !fp) return PKV_ERR_NULL;
  const int32_t s = compress_splits(p);
  if (s < 0) return static_cast<pkv_status>(s);
  const pkv_status st = check_finalize_params(fp);
  if (st != PKV_OK) return st;
  // both halves describe the same outputs, tokens and window length
  if (fp->num_outputs != p->num_outputs || fp->num_tokens != p->num_tokens ||
      fp->compress_ratio != p->compress_ratio)
    return PKV_ERR_SHAPE;
  if (p->num_outputs == 0) return PKV_OK;
  if (!state_cache || !token_to_req || !block_table || !aligned(state_cache, 16) ||
      !aligned(token_to_req, 4) || !aligned(block_table, 4) ||
      (compressed && !aligned(compressed, 16)) ||
      !finalize_pointers_ok(positions, boundary_token_indices, rms_norm_weight, cos_sin_cache,
                            kv_slot_mapping, kv_cache))
    return PKV_ERR_NULL;
  const size_t need = pkv_compress_workspace_bytes(p);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return PKV_ERR_WORKSPACE;
  const pkv::CompressArgs a = compress_args(p, s, state_cache, token_to_req, positions,
                                            boundary_token_indices, block_table, compressed,
                                            workspace, need);
  const pkv::FinalizeArgs f = finalize_args(fp, positions, boundary_token_indices,
                                            rms_norm_weight, cos_sin_cache, kv_slot_mapping,
                                            kv_cache);
  return hip_status(pkv::launch_compress_pack(a, f, static_cast<hipStream_t>(stream)));
}

int32_t pkv_page_tokens(int64_t state_page_bytes, int64_t attn_bytes_per_token,
                        int32_t alignment_tokens) {
  if (state_page_bytes <= 0 || attn_bytes_per_token <= 0 || alignment_tokens <= 0) return -1;
  if (attn_bytes_per_token > INT64_MAX / alignment_tokens) return -1;
  const int64_t unit = attn_bytes_per_token * alignment_tokens;
  const int64_t units = state_page_bytes / unit + (state_page_bytes % unit != 0 ? 1 : 0);
  if (units > INT32_MAX / alignment_tokens) return -1;
  return static_cast<int32_t>(units * alignment_tokens);
}

}  // extern "C"
