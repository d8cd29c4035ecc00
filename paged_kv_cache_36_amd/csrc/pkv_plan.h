// Internal interface of the decode plan (pkv_plan.cpp): how a decode call
// splits its work and which kernel variants it launches. Not installed; not
// part of the C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pkv.h"
#include "pkv_launch.h"

namespace pkv {

// Compute units the plans fill: the current device's count, read once per
// device; 256 (every gfx950 part: MI350X and MI355X) when no device can be
// queried, as in host-only planning on a machine without a GPU.
constexpr int64_t kDefaultCUs = 256;
int64_t plan_cus();
constexpr size_t kWorkspaceAlign = 256;

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Plan {
  bool balanced = false;
  int32_t P = 0;            // fixed partitions: tokens per partition
  int32_t n_parts = 0;      // fixed partitions: ceil(max_seq_len / P)
  int32_t grid = 0;         // balanced: workgroups G
  bool refetch = false;     // a segment may span more than the walker's 64 page ids
  bool k_rows = false;      // K loaded as whole rows and staged through LDS
  bool ordered = false;     // fixed partitions taken full ones first, tails last
  bool combine_per_run = false;   // balanced: one combine wave per (sequence, KV head)
  size_t o_part_bytes = 0;
  size_t lse_bytes = 0;
  size_t workspace = 0;
};

// Geometry checks that need no pointers.
pkv_status check_params(const pkv_decode_params* p);
// Fixed partitions (pkv_split, pkv_decode_partials, and pkv_decode with an
// explicit partition size).
Plan make_fixed_plan(const pkv_decode_params* p);
// The plan pkv_decode runs (balanced or fixed).
Plan make_decode_plan(const pkv_decode_params* p);
LaunchArgs base_args(const pkv_decode_params* p, const Plan& pl);
SplitChoice split_choice(const Plan& pl);
int64_t split_workgroups(const pkv_decode_params* p, const Plan& pl);

}  // namespace pkv
