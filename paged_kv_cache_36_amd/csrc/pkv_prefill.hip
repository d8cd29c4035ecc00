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
// 32 queries, the 32 columns of its MFMA tiles. Per tile of 64 keys:
//  - the workgroup stages the K and V rows of the tile in LDS (rows looked up
//    through the block table one by one, so any page size works); the next
//    tile's rows are loaded into registers while the current one is used,
//  - S^T (64 keys x 32 queries) = K Q^T by 32 v_mfma_f32_32x32x16_bf16, K from
//    LDS as the A operand, the wave's Q^T fragments resident in registers as
//    the B operand; lane l then holds query l % 32 and 16 of its keys per
//    32-key half,
//  - online softmax in log2 units per query (one lane pair), the causal mask
//    only on tiles that reach past the block's first query,
//  - O^T (256 dims x 32 queries) += V^T P^T by 32 MFMAs: p is rounded to bf16
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
constexpr int kPfKeys = 64;                     // keys per tile
// LDS row strides (elements). K: 528 bytes, so the 16 rows one A-operand
// read touches per 16 lanes start 4 banks apart. V: 576 bytes, so the 4 rows x
// 2 dim groups of a transposing read cover distinct banks.
constexpr int kPfKStride = kHeadSize + 8;
constexpr int kPfVStride = kHeadSize + 32;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct PrefillLds {
  uint16_t k[kPfKeys * kPfKStride];
  uint16_t v[kPfKeys * kPfVStride];
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// two fp32 -> packed bf16 pair, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
  const uint32_t ra = (a + 0x7fffu + ((a >> 16) & 1u)) >> 16;
  const uint32_t rb = (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
  return ra | (rb << 16);
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

  // Q^T fragments (B operand): lane = query column, dims 16 ks + 8 half .. + 7
  bf16x8 qf[16];
  {
    const uint16_t* qrow =
        a.q + (static_cast<int64_t>(q_valid ? qi : 0) * hq + h) * kHeadSize + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
      qf[ks] = as_bf16x8(q_valid ? x : u32x4{0u, 0u, 0u, 0u});
    }
  }

  // Tile staging: thread (row tr + 32 rr, part) moves 16-byte pieces
  // 64 i + 8 part of the head's 256 dims, for rr = 0, 1 and i = 0..3: every
  // load instruction covers 8 rows x 128 contiguous bytes.
  const int tr = threadIdx.x >> 3;
  const int part = threadIdx.x & 7;
  u32x4 kr[8], vr[8];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int t = t0 + tr + 32 * rr;
      if (t < kend) {
        const int lp = t / a.block_size;
        const int off = t - lp * a.block_size;
        const int64_t page = a.block_table[lp];
        const uint16_t* ks = a.k + page * a.k_page_stride + static_cast<int64_t>(off) * row_elems +
                             g * kHeadSize + 8 * part;
        const uint16_t* vs = a.v + page * a.v_page_stride + static_cast<int64_t>(off) * row_elems +
                             g * kHeadSize + 8 * part;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kr[4 * rr + i] = *reinterpret_cast<const u32x4*>(ks + 64 * i);
          vr[4 * rr + i] = *reinterpret_cast<const u32x4*>(vs + 64 * i);
        }
      } else {   // past the last key: zeros (finite; their weights are 0)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kr[4 * rr + i] = u32x4{0u, 0u, 0u, 0u};
          vr[4 * rr + i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = tr + 32 * rr;
        *reinterpret_cast<u32x4*>(lds.k + row * kPfKStride + 64 * i + 8 * part) = kr[4 * rr + i];
        *reinterpret_cast<u32x4*>(lds.v + row * kPfVStride + 64 * i + 8 * part) = vr[4 * rr + i];
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
  float m = -INFINITY;   // running max (log2 units) of this lane's query
  float lsum = 0.f;      // this lane's share of the weight sum

  fetch(0);
  for (int t0 = 0; t0 < kend; t0 += kPfKeys) {
    __syncthreads();   // the previous tile is consumed
    stash();
    __syncthreads();
    if (t0 + kPfKeys < kend) fetch(t0 + kPfKeys);   // in flight during this tile's math

    // scores S^T for the two 32-key halves
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const uint16_t* kp = lds.k + kb * 32 * kPfKStride + k_off;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(kp + 16 * ks);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), qf[ks], s[kb], 0, 0, 0);
      }
    }

    // online softmax; register r of half kb holds key t0 + 32 kb + 8 (r / 4) + 4 half + r % 4
    const bool diag = t0 + kPfKeys - 1 > block_first;
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[kb][r] * a.scale_log2;
        if (diag && t0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3) > pos) x = -INFINITY;
        s[kb][r] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m, tmax);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;   // nothing seen yet: weights 0
    if (__builtin_amdgcn_ballot_w64(m_new != m)) {
      const float alpha = exp2_fast(m - m_ref);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] *= alpha;
    }
    m = m_new;

    // P^T fragments: chunk c (keys 16 c .. 16 c + 15) = registers 8 (c % 2) ..
    // + 7 of half c / 2
    bf16x8 pb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = exp2_fast(s[c >> 1][8 * (c & 1) + e] - m_ref);
        lsum += p[e];
      }
      const u32x4 packed = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                            pack_bf16(p[6], p[7])};
      pb[c] = as_bf16x8(packed);
    }

    // O^T += V^T P^T
#pragma unroll
    for (int c = 0; c < 4; ++c) {
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
