// The decode plan: validation of the geometry, the split (balanced share or
// fixed partitions, and their partition size), and the kernel variants each
// split launches (page-list refetch, K load layout, dispatch order). Host
// only; the launches live in pkv_api.cpp.

#include "pkv_plan.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstring>
#include <mutex>

namespace pkv {
namespace {

// Automatic partition size: about one (sequence, partition, KV head)
// workgroup per CU (plan_cus()) for the longest sequence in every batch slot,
// between 64 and 1024 tokens. Measured on MI355X: fewer, longer partitions
// cost less in per-workgroup start-up and in partials, as long as every CU
// gets work.
constexpr int32_t kAutoMinPartition = 64;
constexpr int32_t kAutoMaxPartition = 1024;
// (sequence, KV head) runs from which the balanced combine takes one wave per run
constexpr int64_t kCombinePerRunMin = 256;

// K load layout. Whole rows (full 128-byte lines, staged through LDS for the
// MFMA operand) stream faster than the operand layout's half-line reads, at
// the cost of one more LDS round trip per block; a batch has enough blocks in
// flight to hide it, a single sequence's short decode does not.
bool k_rows_for(const pkv_decode_params* p) { return p->num_seqs > 1; }

}  // namespace

int64_t plan_cus() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int64_t cus[kMaxDevices] = {};
  static bool no_device = false;
  std::lock_guard<std::mutex> lock(mu);
  if (no_device) return kDefaultCUs;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    no_device = true;
    return kDefaultCUs;
  }
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = static_cast<int>(kDefaultCUs);
    cus[dev] = n;
  }
  return cus[dev];
}

pkv_status check_params(const pkv_decode_params* p) {
  if (p == nullptr) return PKV_ERR_NULL;
  if (p->num_seqs < 0 || p->num_kv_heads < 1 || p->num_q_heads < 1 || p->max_seq_len < 0 ||
      p->max_blocks_per_seq < 1)
    return PKV_ERR_SHAPE;
  if (p->head_size != kHeadSize) return PKV_ERR_UNSUPPORTED;
  if (p->num_q_heads != p->num_kv_heads * kGroup) return PKV_ERR_UNSUPPORTED;
  if (p->num_kv_heads > 64) return PKV_ERR_SHAPE;
  if (p->block_size < 16 || p->block_size % 16 != 0) return PKV_ERR_BLOCK_SIZE;
  if (static_cast<int64_t>(p->max_seq_len) >
      static_cast<int64_t>(p->max_blocks_per_seq) * p->block_size)
    return PKV_ERR_SHAPE;
  const int64_t page_elems = static_cast<int64_t>(p->block_size) * p->num_kv_heads * p->head_size;
  if (p->k_page_stride < page_elems || p->v_page_stride < page_elems || p->k_page_stride % 8 != 0 ||
      p->v_page_stride % 8 != 0)
    return PKV_ERR_STRIDE;
  if (p->partition_tokens < 0 || p->partition_tokens % 64 != 0) return PKV_ERR_PARTITION;
  if (!std::isfinite(p->scale)) return PKV_ERR_SHAPE;
  return PKV_OK;
}

// Fixed partitions (pkv_split, pkv_decode_partials, and pkv_decode with an
// explicit partition size).
Plan make_fixed_plan(const pkv_decode_params* p) {
  Plan pl;
  int32_t P = p->partition_tokens;
  if (P == 0) {
    // Enough (sequence, KV head, partition) workgroups to give every CU a few,
    // counting the longest sequence for every slot of the batch.
    const int64_t token_heads =
        static_cast<int64_t>(p->num_seqs) * p->num_kv_heads * static_cast<int64_t>(p->max_seq_len);
    const int64_t target = plan_cus();
    int64_t want = (token_heads + target - 1) / target;
    want = (want + 63) / 64 * 64;
    if (want < kAutoMinPartition) want = kAutoMinPartition;
    if (want > kAutoMaxPartition) want = kAutoMaxPartition;
    P = static_cast<int32_t>(want);
  }
  pl.P = P;
  pl.n_parts = p->max_seq_len > 0 ? (p->max_seq_len + P - 1) / P : 1;
  pl.refetch = partition_needs_refetch(P, p->block_size);
  pl.k_rows = k_rows_for(p);
  // Several sequences of several partitions each: the dispatch order of
  // ordered_coord (full partitions first, the shorter last ones at the end,
  // no empty workgroups among the live ones). It needs the lengths before
  // the first loads, which one sequence's short decode cannot afford.
  pl.ordered = p->num_seqs > 1 && p->num_seqs <= kMaxOrderedSeqs && pl.n_parts > 1;
  if (pl.n_parts > 1) {
    const size_t rows = static_cast<size_t>(p->num_seqs) * p->num_q_heads * pl.n_parts;
    pl.o_part_bytes = round_up(rows * kHeadSize * sizeof(float), kWorkspaceAlign);
    pl.lse_bytes = round_up(rows * sizeof(float), kWorkspaceAlign);
    pl.workspace = pl.o_part_bytes + pl.lse_bytes;
  }
  return pl;
}

// The plan pkv_decode runs: the balanced split when the partition size is
// left to the library and the batch has several sequences (within the
// balanced kernel's limits); fixed partitions otherwise. One sequence is
// split evenly by fixed partitions already, and they start one memory round
// trip sooner (no prefix sums over the lengths before the page list).
Plan make_decode_plan(const pkv_decode_params* p) {
  const int64_t tiles_per_seq = (static_cast<int64_t>(p->max_seq_len) + kTileTokens - 1) /
                                kTileTokens;
  const int64_t t_max = static_cast<int64_t>(p->num_seqs) * p->num_kv_heads * tiles_per_seq;
  if (p->partition_tokens != 0 || p->num_seqs == 1 || p->num_seqs > kMaxBalancedSeqs ||
      t_max < 1 ||
      t_max > (int64_t{1} << 30))
    return make_fixed_plan(p);
  Plan pl;
  pl.balanced = true;
  // One workgroup per CU: each already keeps all of its first two blocks per
  // wave in flight, and a second workgroup per CU measured slower at every
  // batch size tried (more partials, no more bandwidth).
  int64_t g = plan_cus();
  if (g > t_max) g = t_max;
  pl.grid = static_cast<int32_t>(g);
  // longest run of one (sequence, KV head) a workgroup can get
  const int64_t seg_tokens = std::min<int64_t>(
      p->max_seq_len, ((t_max + g - 1) / g + 1) * kTileTokens);
  pl.refetch = partition_needs_refetch(static_cast<int32_t>((seg_tokens + 63) / 64 * 64),
                                            p->block_size);
  pl.k_rows = k_rows_for(p);
  // Many (sequence, KV head) runs: each has one or two partials, and one
  // combine wave per run (its 6 heads) starts a fraction of the waves of one
  // per (sequence, head, quarter). Few runs keep the finer combine, whose
  // waves then have more partials each to load in parallel.
  pl.combine_per_run = static_cast<int64_t>(p->num_seqs) * p->num_kv_heads >= kCombinePerRunMin;
  const size_t slots = static_cast<size_t>(g) + static_cast<size_t>(p->num_seqs) * p->num_kv_heads;
  pl.o_part_bytes = round_up(slots * kGroup * kHeadSize * sizeof(float), kWorkspaceAlign);
  pl.lse_bytes = round_up(slots * kGroup * sizeof(float), kWorkspaceAlign);
  pl.workspace = pl.o_part_bytes + pl.lse_bytes +
                 round_up((static_cast<size_t>(p->num_seqs) + 1) * sizeof(int32_t), kWorkspaceAlign);
  return pl;
}

LaunchArgs base_args(const pkv_decode_params* p, const Plan& pl) {
  LaunchArgs a;
  std::memset(&a, 0, sizeof(a));
  a.k_page_stride = p->k_page_stride;
  a.v_page_stride = p->v_page_stride;
  a.num_seqs = p->num_seqs;
  a.num_kv_heads = p->num_kv_heads;
  a.block_size = p->block_size;
  a.max_blocks = p->max_blocks_per_seq;
  a.partition_tokens = pl.P;
  a.n_parts = pl.n_parts;
  a.max_seq_len = p->max_seq_len;
  a.balanced_grid = pl.balanced ? pl.grid : 0;
  a.resident_wgs = static_cast<int32_t>(2 * plan_cus());
  a.scale_log2 = static_cast<float>(static_cast<double>(p->scale) * 1.4426950408889634);
  return a;
}

int64_t split_workgroups(const pkv_decode_params* p, const Plan& pl) {
  if (pl.balanced) return pl.grid;
  return static_cast<int64_t>(p->num_seqs) * p->num_kv_heads * pl.n_parts;
}

SplitChoice split_choice(const Plan& pl) {
  SplitChoice c;
  c.balanced = pl.balanced;
  c.refetch = pl.refetch;
  c.k_rows = pl.k_rows;
  c.ordered = pl.ordered;
  return c;
}

}  // namespace pkv
