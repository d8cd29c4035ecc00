// The parts of the tail-Q prefill (gfx950) around its inner loop: the grid's
// mapping of workgroups to (query head, query block, key split) and its size,
// the direct-to-LDS load, and the constants of the 64-key tiles the kernel
// streams through LDS in a blocked, swizzled layout.
//
// A workgroup serves one query head and a block of 128 queries; a tile is 64
// consecutive keys of one KV head (32 KiB of K and 32 KiB of V), stored as
// 1 KiB blocks of 8 rows x 8 pieces of 16 bytes so that every direct load
// reads whole 128-byte lines of a row ("海光 DCU 上的长上下文 Attention：从
// page784 到 page832 的 KV Cache 对齐与访存优化", §6 for the tail-Q shape).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"

namespace pkv {
namespace {

constexpr int kPfQueries = 128;                 // queries per workgroup
constexpr int kPfWaveKeys = 32;                 // keys per wave and tile (one key half)
constexpr int kPfKeys = 2 * kPfWaveKeys;        // keys per tile
constexpr int kXcds = 8;                        // XCDs workgroups are dealt to, round robin
constexpr int kBlockBytes = 1024;               // 8 rows x 8 pieces of 16 bytes
constexpr int kTileBytes = kPfKeys * kHeadSize * 2;   // 32 KiB of K (or of V)

// The running max is only moved when a tile's max exceeds it by more than
// this (log2 units): the weights exp2(x - m) then stay below 2^8, which bf16
// holds with the same relative rounding as any weight and fp32 sums cannot
// overflow, while the accumulator rescale becomes rare.
constexpr float kRescaleLog2 = 8.f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// One direct-to-LDS load (64 lanes x 16 bytes into 1 KiB of LDS at lds_dst).
// Written as asm so the compiler does not order later LDS reads behind it:
// the kernel waits for these loads itself (vmcnt(0) before each
// barrier), and they only ever fill a stage no wave is reading.
// M0 (the LDS base of the load) is declared clobbered; clang warns that M0
// is reserved, and no other code of the kernel uses it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, const void* lds_dst) {
  const uint32_t dst = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)lds_dst)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(dst)
               : "m0");
}
#pragma clang diagnostic pop

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Key splits of query block qb: one fewer for the short_blocks shortest
// (lowest) blocks.
__device__ __forceinline__ int splits_of(int qb, int nsplit, int short_blocks) {
  return qb < short_blocks ? nsplit - 1 : nsplit;
}

// (query head, query block, key split) of workgroup b and the block's split
// count; false for grid padding. XCD x serves KV head x % hkv, so one L2 sees
// every request for that head's tiles. The largest shares go out first, the
// splits of one block together.
__device__ __forceinline__ bool block_of(int b, int hkv, int nqb, int nsplit, int short_blocks,
                                         int& h, int& qb, int& split, int& ns) {
  const int per_kv = kGroup * (nqb * nsplit - short_blocks);
  int j;
  if (kXcds % hkv == 0) {
    const int x = b % kXcds;
    j = (b / kXcds) * (kXcds / hkv) + x / hkv;
    if (j >= per_kv) return false;
    h = (x % hkv) * kGroup + j % kGroup;
  } else {
    const int hq = hkv * kGroup;
    h = b % hq;
    j = (b / hq) * kGroup;
  }
  const int t = j / kGroup;
  // the short blocks' nsplit - 1 splits go first (each a larger share of its
  // block than a longer block's split), then the longer blocks' nsplit splits,
  // each group longest block first
  const int short_items = short_blocks * (nsplit - 1);
  if (t < short_items) {
    qb = short_blocks - 1 - t / (nsplit - 1);
    split = t % (nsplit - 1);
    ns = nsplit - 1;
  } else {
    const int u = t - short_items;
    qb = nqb - 1 - u / nsplit;
    split = u % nsplit;
    ns = nsplit;
  }
  return true;
}

// Grid size of a prefill launch: every XCD gets the same number of slots when
// the KV heads divide the XCDs (slots past a head's list exit at once).
inline int64_t prefill_grid(int num_q, int num_kv_heads, int key_splits, int short_blocks) {
  const int64_t nqb = (num_q + kPfQueries - 1) / kPfQueries;
  const int64_t per_kv = kGroup * (nqb * key_splits - short_blocks);
  int64_t blocks = static_cast<int64_t>(num_kv_heads) * per_kv;
  if (kXcds % num_kv_heads == 0) {
    const int64_t per_xcd = (per_kv + kXcds / num_kv_heads - 1) / (kXcds / num_kv_heads);
    blocks = per_xcd * kXcds;
  }
  return blocks;
}

}  // namespace
}  // namespace pkv
