// HIP kernel for tail-Q chunked prefill over a paged KV cache, gfx950.
//
// The q new tokens of one sequence are its last q cached tokens: query i sits
// at position L - q + i and attends keys 0 .. L - q + i (causal), for 24 query
// heads over 4 KV heads of size 256, bf16 in and out ("海光 DCU 上的长上下文
// Attention：从 page784 到 page832 的 KV Cache 对齐与访存优化", §6; the formula:
// "From Attention to KV Cache Compression: Notes from a KernelGen
// Optimization", "Starting from Attention"; the online max / denominator /
// numerator update: same page, "Online Softmax: Streaming Away the Window").
//
// Work split. One workgroup (4 waves) per (query head, block of 128 queries);
// the blocks with the longest causal ranges are launched first. Wave w owns
// 32 queries, the 32 columns of its MFMA tiles. Per tile of 32 keys (small
// enough that the whole working set, accumulator included, stays in VGPRs):
//  - the workgroup stages the K and V rows of the tile in LDS (rows looked up
//    through the block table one by one, so any page size works); the next
//    tile's rows are loaded into registers while the current one is used,
//  - S^T (32 keys x 32 queries) = K Q^T by 16 v_mfma_f32_32x32x16_bf16, K (A
//    operand) and the wave's Q^T fragments (B operand) read from LDS, where
//    the block's queries are staged once; lane l then holds query l % 32 and
//    16 of the tile's keys,
//  - online softmax in log2 units per query (one lane pair), the causal mask
//    only on tiles that reach past the block's first query,
//  - O^T (256 dims x 32 queries) += V^T P^T by 16 MFMAs: p is rounded to bf16
//    straight from the S^T registers (the B operand needs exactly the keys the
//    lane holds, in the order k = keys 4h..4h+3, 8+4h..8+4h+3 of each 16-key
//    chunk, h = l / 32), and V^T comes from LDS through the transposing read
//    in that same key order.
// The accumulator belongs to the lane's query, so the rescale is per lane.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kPfThreads = 256;                 // 4 waves
constexpr int kPfCols = 32;                     // queries per wave
constexpr int kPfQueries = 4 * kPfCols;         // queries per workgroup
constexpr int kPfKeys = 32;                     // keys per tile (one MFMA block)
// LDS row strides (elements). K: 528 bytes, so the 16 rows one A-operand
// read touches per 16 lanes start 4 banks apart. V: 576 bytes, so the 4 rows x
// 2 dim groups of a transposing read cover distinct banks.
constexpr int kPfKStride = kHeadSize + 8;
constexpr int kPfVStride = kHeadSize + 32;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct PrefillLds {
  uint16_t q[kPfQueries * kPfKStride];   // the block's queries (same padded rows as K)
  uint16_t k[kPfKeys * kPfKStride];
  uint16_t v[kPfKeys * kPfVStride];
};

// The running max is only moved when a tile's max exceeds it by more than
// this (log2 units): the weights exp2(x - m) then stay below 2^8, which bf16
// holds with the same relative rounding as any weight and fp32 sums cannot
// overflow, while the accumulator rescale becomes rare.
constexpr float kRescaleLog2 = 8.f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__global__ __launch_bounds__(kPfThreads, 1) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) PrefillLds lds;
  const int hq = a.num_kv_heads * kGroup;
  const int nqb = (a.num_q + kPfQueries - 1) / kPfQueries;
  const int h = blockIdx.x % hq;
  const int qb = nqb - 1 - static_cast<int>(blockIdx.x / hq);   // longest ranges first
  const int g = h / kGroup;
  const int lane = lane_id();
  const int w = wave_id();
  const int col = lane & 31;
  const int half = lane >> 5;
  const int q0 = qb * kPfQueries;
  const int qi = q0 + kPfCols * w + col;              // this lane's query
  const bool q_valid = qi < a.num_q;
  const int first_pos = a.seq_len - a.num_q;          // position of query 0
  const int pos = q_valid ? first_pos + qi : -1;
  const int block_first = first_pos + q0;             // position of the block's first query
  const int kend = first_pos + min(q0 + kPfQueries, a.num_q);   // keys the block needs
  const int row_elems = a.num_kv_heads * kHeadSize;

  // The block's queries go to LDS once (rows past the last query are zero);
  // each wave reads its Q^T fragments (B operand: lane = query column, dims
  // 16 ks + 8 half .. + 7) from there per tile, which keeps them out of the
  // registers the accumulator needs.
#pragma unroll
  for (int i = 0; i < kPfQueries * kHeadSize / 8 / kPfThreads; ++i) {
    const int piece = threadIdx.x + kPfThreads * i;   // 16-byte piece of the block's rows
    const int row = piece >> 5;
    const int c8 = (piece & 31) * 8;
    const int qrow = q0 + row;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qrow < a.num_q)
      x = *reinterpret_cast<const u32x4*>(a.q + (static_cast<int64_t>(qrow) * hq + h) * kHeadSize + c8);
    *reinterpret_cast<u32x4*>(lds.q + row * kPfKStride + c8) = x;
  }
  const uint16_t* q_frag = lds.q + (kPfCols * w + col) * kPfKStride + 8 * half;

  // Tile staging: thread (row tr, part) moves the 16-byte pieces 64 i + 8 part
  // (i = 0..3) of the head's 256 dims of row tr, for K and for V: every load
  // instruction covers 8 rows x 128 contiguous bytes.
  const int tr = threadIdx.x >> 3;
  const int part = threadIdx.x & 7;
  u32x4 kr[4], vr[4];
  // (logical page, offset) of the thread's row, moved by one tile per fetch
  int lp_r = tr / a.block_size;
  int off_r = tr - lp_r * a.block_size;
  auto fetch = [&](int t0) {
    const int t = t0 + tr;
    const int lp = lp_r, off = off_r;
    off_r += kPfKeys;
    while (off_r >= a.block_size) {
      off_r -= a.block_size;
      ++lp_r;
    }
    if (t < kend) {
      const int64_t page = a.block_table[lp];
      const uint16_t* ks = a.k + page * a.k_page_stride + static_cast<int64_t>(off) * row_elems +
                           g * kHeadSize + 8 * part;
      const uint16_t* vs = a.v + page * a.v_page_stride + static_cast<int64_t>(off) * row_elems +
                           g * kHeadSize + 8 * part;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kr[i] = *reinterpret_cast<const u32x4*>(ks + 64 * i);
        vr[i] = *reinterpret_cast<const u32x4*>(vs + 64 * i);
      }
    } else {   // past the last key: zeros (finite; their weights are 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kr[i] = u32x4{0u, 0u, 0u, 0u};
        vr[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(lds.k + tr * kPfKStride + 64 * i + 8 * part) = kr[i];
      *reinterpret_cast<u32x4*>(lds.v + tr * kPfVStride + 64 * i + 8 * part) = vr[i];
    }
  };

  // transposing-read offsets (elements): 16-lane group G = lane / 16 reads
  // dims 16 (G & 1) + 0..15 of a 32-dim block for keys 4 (G >> 1) + 0..3
  // (+ 8 for the second read) of a 16-key chunk; lane j of the group supplies
  // the address of key j / 4, dims 4 (j % 4) .. + 3
  const int vgrp = lane >> 4;
  const int vj = lane & 15;
  const int v_off = (4 * (vgrp >> 1) + (vj >> 2)) * kPfVStride + 16 * (vgrp & 1) + 4 * (vj & 3);
  const int k_off = col * kPfKStride + 8 * half;   // A-operand read: key row col, 8 dims

  f32x16 acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = f32x16{};
  float m = -INFINITY;   // running max (log2 units) of this lane's query, moved lazily
  float lsum = 0.f;      // this lane's share of the weight sum

  // One tile's scores S^T (scaled to log2 units, causal mask applied);
  // register r holds key t0 + 8 (r / 4) + 4 half + r % 4. Returns the tile max
  // of the lane's query.
  auto scores = [&](int t0, f32x16& s) {
    s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const bf16x8 qf = as_bf16x8(*reinterpret_cast<const u32x4*>(q_frag + 16 * ks));
      const u32x4 kv = *reinterpret_cast<const u32x4*>(lds.k + k_off + 16 * ks);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), qf, s, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] *= a.scale_log2;
    if (t0 + kPfKeys - 1 > block_first) {   // tile reaches past the block's first query
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (t0 + 8 * (r >> 2) + 4 * half + (r & 3) > pos) s[r] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
    return fmaxf(tmax, __shfl_xor(tmax, 32));
  };

  // p = exp2(x - m) rounded to bf16 as the P^T operand (chunk c: keys
  // 16 c .. 16 c + 15 = registers 8 c .. 8 c + 7), then O^T += V^T P^T.
  auto accumulate = [&](const f32x16& s, float m_ref) {
    bf16x8 pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = exp2_fast(s[8 * c + e] - m_ref);
        lsum += p[e];
      }
      const u32x4 packed = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                            pack_bf16(p[6], p[7])};
      pb[c] = as_bf16x8(packed);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint16_t* vp = lds.v + 16 * c * kPfVStride + v_off;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 32 * db));
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 8 * kPfVStride + 32 * db));
        const bf16x8 va = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[c], acc[db], 0, 0, 0);
      }
    }
  };

  fetch(0);
  for (int t0 = 0; t0 < kend; t0 += kPfKeys) {
    __syncthreads();   // the previous tile is consumed
    stash();
    __syncthreads();
    if (t0 + kPfKeys < kend) fetch(t0 + kPfKeys);   // in flight during this tile's math
    f32x16 s;
    const float tmax = scores(t0, s);
    if (__builtin_amdgcn_ballot_w64(tmax > m + kRescaleLog2)) {   // rare after the first tile
      const float m_new = fmaxf(m, tmax);
      const float alpha = m_new == -INFINITY ? 1.f : exp2_fast(m - m_new);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] *= alpha;
      m = m_new;
    }
    accumulate(s, m == -INFINITY ? 0.f : m);   // nothing seen yet: weights 0
  }

  // o = acc / l: register r of block db holds dim 32 db + 8 (r / 4) + 4 half + r % 4
  lsum += __shfl_xor(lsum, 32);
  if (!q_valid) return;
  const float inv = 1.f / lsum;   // lsum >= 1: the maximum key has weight 1
  const int64_t orow = (static_cast<int64_t>(qi) * hq + h) * kHeadSize + 4 * half;
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const f32x4 o = {acc[db][4 * rq] * inv, acc[db][4 * rq + 1] * inv, acc[db][4 * rq + 2] * inv,
                       acc[db][4 * rq + 3] * inv};
      const int64_t idx = orow + 32 * db + 8 * rq;
      if (a.out) {
        u32x2 packed;
        packed.x = f32_to_bf16(o.x) | (f32_to_bf16(o.y) << 16);
        packed.y = f32_to_bf16(o.z) | (f32_to_bf16(o.w) << 16);
        *reinterpret_cast<u32x2*>(a.out + idx) = packed;
      }
      if (a.out_f32) *reinterpret_cast<f32x4*>(a.out_f32 + idx) = o;
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.num_q <= 0) return hipSuccess;
  const int64_t blocks = static_cast<int64_t>(a.num_kv_heads) * kGroup *
                         ((a.num_q + kPfQueries - 1) / kPfQueries);
  hipLaunchKernelGGL(prefill_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kPfThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace pkv
