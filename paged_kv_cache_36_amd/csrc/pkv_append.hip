// HIP kernels for the KV append over a paged cache, gfx950: each new token's
// K and V rows are written into the cache row its slot names (page = slot /
// B, offset = slot % B), the slot-to-page arithmetic of "From Attention to KV
// Cache Compression: Notes from a KernelGen Optimization" ("Gather and
// Scatter", "How One Output Is Produced") on the page layout of "海光 DCU 上的
// 长上下文 Attention：从 page784 到 page832 的 KV Cache 对齐与访存优化" (§4).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

// ---------------------------------------------------------------------------
// KV append: token b's K and V rows go to the cache row of slot slots[b]
// (page = slot / B, offset = slot % B). One wave per token; a lane moves
// 16-byte chunks, all of a token's loads issued before its stores. Padding
// (negative) and out-of-cache slots write nothing.
// ---------------------------------------------------------------------------
constexpr int kAppendThreads = 256;
constexpr int kAppendTokensPerBlock = kAppendThreads / 64;
constexpr int32_t kAppendPairChunks = 128;    // 16-byte chunks of a 4 x 256 bf16 row
constexpr int32_t kAppendPairTokens = 2048;   // from this many tokens, two per wave

__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  const int lane = lane_id();
  const int64_t b = static_cast<int64_t>(blockIdx.x) * kAppendTokensPerBlock + wave_id();
  if (b >= a.num_tokens) return;
  const int64_t slot = a.slots[b];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t page = slot / a.block_size;
  const int64_t offset = slot - page * a.block_size;
  const int64_t row_elems = static_cast<int64_t>(a.row_chunks) * 8;
  const u32x4* ks = reinterpret_cast<const u32x4*>(a.k_new + b * a.k_new_stride);
  const u32x4* vs = reinterpret_cast<const u32x4*>(a.v_new + b * a.v_new_stride);
  u32x4* kd = reinterpret_cast<u32x4*>(a.k_cache + page * a.k_page_stride + offset * row_elems);
  u32x4* vd = reinterpret_cast<u32x4*>(a.v_cache + page * a.v_page_stride + offset * row_elems);
  // rows of up to 4 KiB in one pass (2 chunks per lane each for K and V);
  // every byte is read once and written once, so both stream (nontemporal)
  int c = lane;
  for (; c + 64 < a.row_chunks; c += 128) {
    const u32x4 k0 = __builtin_nontemporal_load(ks + c), k1 = __builtin_nontemporal_load(ks + c + 64);
    const u32x4 v0 = __builtin_nontemporal_load(vs + c), v1 = __builtin_nontemporal_load(vs + c + 64);
    __builtin_nontemporal_store(k0, kd + c);
    __builtin_nontemporal_store(k1, kd + c + 64);
    __builtin_nontemporal_store(v0, vd + c);
    __builtin_nontemporal_store(v1, vd + c + 64);
  }
  if (c < a.row_chunks) {
    const u32x4 k0 = __builtin_nontemporal_load(ks + c), v0 = __builtin_nontemporal_load(vs + c);
    __builtin_nontemporal_store(k0, kd + c);
    __builtin_nontemporal_store(v0, vd + c);
  }
}

// Rows of exactly 128 chunks (4 KV heads x 256 dims) for long appends: a wave
// moves tokens 2 b and 2 b + 1 and issues all 8 of its loads before the
// stores, which keeps twice the bytes in flight per wave.
__global__ __launch_bounds__(kAppendThreads) void append_pairs_kernel(AppendArgs a) {
  const int lane = lane_id();
  const int64_t b0 = (static_cast<int64_t>(blockIdx.x) * kAppendTokensPerBlock + wave_id()) * 2;
  if (b0 >= a.num_tokens) return;
  const int64_t row_elems = kAppendPairChunks * 8;
  u32x4 kv[2][4];
  u32x4* dk[2];
  u32x4* dv[2];
  bool go[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t b = b0 + j;
    const int64_t slot = b < a.num_tokens ? a.slots[b] : -1;
    go[j] = slot >= 0 && slot < a.num_slots;
    const int64_t page = go[j] ? slot / a.block_size : 0;
    const int64_t offset = go[j] ? slot - page * a.block_size : 0;
    // a token that stores nothing re-reads the first token's row (the loads
    // then wait for the slots: measured faster than issuing them at once)
    const int64_t src = go[j] ? b : b0;
    const u32x4* ks = reinterpret_cast<const u32x4*>(a.k_new + src * a.k_new_stride);
    const u32x4* vs = reinterpret_cast<const u32x4*>(a.v_new + src * a.v_new_stride);
    dk[j] = reinterpret_cast<u32x4*>(a.k_cache + page * a.k_page_stride + offset * row_elems);
    dv[j] = reinterpret_cast<u32x4*>(a.v_cache + page * a.v_page_stride + offset * row_elems);
    kv[j][0] = __builtin_nontemporal_load(ks + lane);
    kv[j][1] = __builtin_nontemporal_load(ks + lane + 64);
    kv[j][2] = __builtin_nontemporal_load(vs + lane);
    kv[j][3] = __builtin_nontemporal_load(vs + lane + 64);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (!go[j]) continue;
    __builtin_nontemporal_store(kv[j][0], dk[j] + lane);
    __builtin_nontemporal_store(kv[j][1], dk[j] + lane + 64);
    __builtin_nontemporal_store(kv[j][2], dv[j] + lane);
    __builtin_nontemporal_store(kv[j][3], dv[j] + lane + 64);
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  if (a.num_tokens <= 0) return hipSuccess;
  if (a.row_chunks == kAppendPairChunks && a.num_tokens >= kAppendPairTokens) {
    const int64_t per_block = 2 * kAppendTokensPerBlock;
    const int64_t blocks = (static_cast<int64_t>(a.num_tokens) + per_block - 1) / per_block;
    hipLaunchKernelGGL(append_pairs_kernel, dim3(static_cast<uint32_t>(blocks)),
                       dim3(kAppendThreads), 0, stream, a);
    return hipGetLastError();
  }
  const int64_t blocks = (static_cast<int64_t>(a.num_tokens) + kAppendTokensPerBlock - 1) /
                         kAppendTokensPerBlock;
  hipLaunchKernelGGL(append_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kAppendThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace pkv
