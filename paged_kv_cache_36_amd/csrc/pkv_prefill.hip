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
// Work split. One workgroup of 8 waves per (query head, block of 128
// queries): wave (g, k) owns queries 32 g .. 32 g + 31 (the 32 columns of its
// MFMA tiles, their Q^T fragments held in registers) and keys 32 k .. 32 k +
// 31 of every 64-key tile, so the two waves sharing a SIMD interleave their
// matrix and vector phases. Tiles stream through two LDS stages that
// direct-to-LDS loads (global_load_lds_dwordx4) fill one tile ahead: one
// barrier per tile and no register staging. Per wave and tile:
//  - S^T (32 keys x 32 queries) = K Q^T by 16 v_mfma_f32_32x32x16_bf16 (K, the
//    A operand, from LDS); lane l then holds query l % 32 and 16 of the keys,
//  - online softmax in log2 units per query (one lane pair), the causal mask
//    only where the keys reach past the block's first query,
//  - O^T (256 dims x 32 queries) += V^T P^T by 16 MFMAs: p is rounded to bf16
//    straight from the S^T registers (the B operand needs exactly the keys the
//    lane holds, in the order k = keys 4h..4h+3, 8+4h..8+4h+3 of each 16-key
//    chunk, h = l / 32), and V^T comes from LDS through the transposing read
//    in that same key order.
// At the end the two key halves of each query group merge through LDS.
//
// Key splits. When the query blocks are too few to fill the CUs, each block's
// tiles are cut into near-equal ranges, one workgroup each: key_splits ranges,
// or one fewer for the short_blocks shortest query blocks (so the workgroups
// can make whole rounds over the CUs); a workgroup then writes its normalized
// partial output and log2-sum-exp, and prefill_combine_kernel merges the
// splits with the same log-sum-exp weights as decode's partitions (split-KV,
// flash-decoding style).
//
// LDS layout. A direct load writes 64 consecutive 16-byte slots; a tile is
// stored as 1 KiB blocks of 8 rows x 8 pieces (128 contiguous bytes of each
// row, so every load reads whole cache lines):
//  - K: block (piece group pg, row group rg) at pg * 8 + rg; piece p of row r
//    in slot ((p % 8) ^ (rg & 1)) * 8 + r % 8. The A-operand read of step ks
//    (rows 0..31, pieces 2 ks, 2 ks + 1) is then a fixed per-lane offset plus
//    a constant, and each 16 lanes hit 16 distinct slots of 256 bytes.
//  - V: block (key group kb, piece group pb) at kb * 4 + pb; piece p of key
//    r in slot (r % 8) * 8 + ((p % 8) ^ 4 ((r >> 1) & 1)). Each half of a
//    transposing read (4 keys x 64 bytes) hits 16 distinct slots.
//
// Grid order. The workgroups of one KV head read the same keys from position
// 0 upwards; blocks are dealt to XCDs (workgroup b runs on XCD b % 8) so that
// each XCD serves one KV head. Within a head the longest causal ranges go
// first.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pkv_device.h"
#include "pkv_launch.h"
#include "pkv_prefill_common.h"

namespace pkv {
namespace {

constexpr int kPfThreads = 512;                 // 8 waves: 4 query groups x 2 key halves
constexpr int kPfCols = 32;                     // queries per wave
static_assert(kPfQueries == 4 * kPfCols, "four query groups per workgroup");

struct PrefillStage {
  char k[kTileBytes];
  char v[kTileBytes];
};
// the tiles, or after them the merge of the two key halves
union PrefillLds {
  PrefillStage stage[2];
  float merge[4][kPfCols * kHeadSize + 128];
};
static_assert(sizeof(PrefillLds) <= 160 * 1024, "LDS budget of one workgroup");

// kSplit: key_splits > 1 (partials out); with one split the tile range and
// the grid decomposition fold to the plain whole-range form.
template <bool kFold, bool kSplit>
__global__ __launch_bounds__(kPfThreads, 1) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) PrefillLds lds;
  const int hq = a.num_kv_heads * kGroup;
  const int nqb = (a.num_q + kPfQueries - 1) / kPfQueries;
  int h, qb, split, nsplit;
  if (!block_of(blockIdx.x, a.num_kv_heads, nqb, kSplit ? a.key_splits : 1,
                kSplit ? a.short_blocks : 0, h, qb, split, nsplit))
    return;
  const int g = h / kGroup;
  const int lane = lane_id();
  const int wid = wave_id();
  const int w = wid & 3;           // query group
  const int kh = wid >> 2;         // key half of each tile
  const int col = lane & 31;
  const int half = lane >> 5;
  const int q0 = qb * kPfQueries;
  const int qi = q0 + kPfCols * w + col;              // this lane's query
  const bool q_valid = qi < a.num_q;
  const int first_pos = a.seq_len - a.num_q;          // position of query 0
  const int pos = q_valid ? first_pos + qi : -1;
  const int block_first = first_pos + q0;             // position of the block's first query
  const int kend = first_pos + min(q0 + kPfQueries, a.num_q);   // keys the block needs
  const int ntiles = (kend + kPfKeys - 1) / kPfKeys;
  // this workgroup's tiles: split `split` of the block's nsplit near-equal ranges
  const int t_lo = kSplit ? static_cast<int>(static_cast<int64_t>(ntiles) * split / nsplit) : 0;
  const int t_hi =
      kSplit ? static_cast<int>(static_cast<int64_t>(ntiles) * (split + 1) / nsplit) : ntiles;
  const int row_elems = a.num_kv_heads * kHeadSize;
  const int bsz = a.block_size;

  // Q^T fragments (B operand: lane = query column, dims 16 ks + 8 half .. + 7)
  // stay in registers; rows past the last query repeat it (never stored).
  bf16x8 qf[16];
  {
    const uint16_t* qrow =
        a.q + (static_cast<int64_t>(min(qi, a.num_q - 1)) * hq + h) * kHeadSize + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      qf[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 16 * ks));
  }

  // Direct loads: wave wid fills K row group wid (rows 8 wid + s % 8, all
  // four piece groups) and V key group wid (keys 8 wid + s / 8) of each tile.
  // Rows at or past kend read row kend - 1 instead (finite; weight 0).
  const int k_row = 8 * wid + (lane & 7);
  const int v_row = 8 * wid + (lane >> 3);
  const int k_piece = ((lane >> 3) ^ (wid & 1));             // + 8 pg
  const int v_piece = ((lane & 7) ^ (4 * ((lane >> 4) & 1)));   // + 8 pb
  const int last_lp = (kend - 1) / bsz;
  const int last_off = kend - 1 - last_lp * bsz;
  const int nblocks = (a.seq_len + bsz - 1) / bsz;
  const int64_t last_page = a.block_table[last_lp];
  // logical page and offset of row 8 wid of the next tile to load (wave-uniform)
  const int row0 = __builtin_amdgcn_readfirstlane(t_lo * kPfKeys + 8 * wid);
  int lpw = row0 / bsz;
  int offw = row0 - lpw * bsz;
  const int step_pages = kPfKeys / bsz, step_off = kPfKeys % bsz;
  // page ids of logical pages win_base .. win_base + 63, one per lane
  int win_base = lpw;
  int win = a.block_table[min(win_base + lane, nblocks - 1)];

  // Source rows of the next tile's loads and the stage they fill; the eight
  // loads themselves are spread over the S^T products (load()), so no wave
  // stalls on a full memory queue right after the barrier.
  struct NextTile {
    const uint16_t* ksrc;
    const uint16_t* vsrc;
    char* kdst;
    char* vdst;
  };
  // the previous tile's source rows: when this tile's rows sit 64 rows
  // further in the same pages and none is clamped, they just move on
  const uint16_t* k_prev = nullptr;
  const uint16_t* v_prev = nullptr;
  const int64_t tile_elems = static_cast<int64_t>(kPfKeys) * row_elems;
  auto prepare = [&](int tt) {
    const int t0 = tt * kPfKeys;
    char* kdst = lds.stage[tt & 1].k + wid * kBlockBytes;
    char* vdst = lds.stage[tt & 1].v + wid * 4 * kBlockBytes;
    // rows 8 wid .. 8 wid + 7 of tiles tt - 1 and tt in one page, none past kend
    const bool same_page = tt > t_lo && offw >= kPfKeys && offw + 7 < bsz && t0 + kPfKeys <= kend;
    if (same_page) {
      k_prev += tile_elems;
      v_prev += tile_elems;
      offw += kPfKeys;
      if (offw >= bsz) {
        offw -= bsz;
        ++lpw;
      }
      return NextTile{k_prev, v_prev, kdst, vdst};
    }
    if (lpw + 8 - win_base >= 64) {
      win_base = lpw;
      win = a.block_table[min(win_base + lane, nblocks - 1)];
    }
    // every lane takes part in the window lookup (a lane reading from an
    // inactive lane would get nothing), then rows past kend switch to kend - 1
    auto locate = [&](int r, int64_t& page, int& off) {
      int lp = lpw;
      off = offw + (r & 7);
      while (off >= bsz) {
        off -= bsz;
        ++lp;
      }
      const int id = __builtin_amdgcn_ds_bpermute(4 * (lp - win_base), win);
      const bool live = t0 + r < kend;
      page = live ? static_cast<int64_t>(id) : last_page;
      off = live ? off : last_off;
    };
    int64_t kpage, vpage;
    int koff, voff;
    locate(k_row, kpage, koff);
    locate(v_row, vpage, voff);
    const uint16_t* ksrc = a.k + kpage * a.k_page_stride +
                           (static_cast<int64_t>(koff) * row_elems + g * kHeadSize + 8 * k_piece);
    const uint16_t* vsrc = a.v + vpage * a.v_page_stride +
                           (static_cast<int64_t>(voff) * row_elems + g * kHeadSize + 8 * v_piece);
    k_prev = ksrc;
    v_prev = vsrc;
    offw += step_off;
    lpw += step_pages;
    if (offw >= bsz) {
      offw -= bsz;
      ++lpw;
    }
    return NextTile{ksrc, vsrc, kdst, vdst};
  };
  // load i of a tile: K piece group i / 2 (even i) or V piece group i / 2 (odd i)
  auto load = [&](const NextTile& nt, int i) {
    const int pg = i >> 1;
    if (i & 1)
      dma16(nt.vsrc + 64 * pg, nt.vdst + pg * kBlockBytes);
    else
      dma16(nt.ksrc + 64 * pg, nt.kdst + pg * 8 * kBlockBytes);
  };

  // K A-operand read of step ks: row 32 kh + col, pieces 2 ks + half, at
  // block (ks / 4) * 8 + rg, slot (2 (ks % 4) + (half ^ (rg & 1))) * 8 + row % 8
  const int krow = kPfWaveKeys * kh + col;
  const int krg = krow >> 3;
  const int k_lane = krg * kBlockBytes + (((half ^ (krg & 1)) * 8 + (krow & 7)) * 16);
  // V^T transposing reads: 16-lane group G = lane / 16 reads dims 16 (G & 1)
  // + 0..15 of a 32-dim block for keys 4 (G >> 1) + 0..3 (+ 8 for the second
  // read) of a 16-key chunk; lane j of the group supplies the address of key
  // j / 4, dims 4 (j % 4) .. + 3: piece 4 db + 2 (G & 1) + (j % 4) / 2, half
  // j % 2 of it. Within its 8-key group the key is r8 = 4 (G >> 1) + j / 4,
  // whose swizzle flips piece bit 2 when (r8 >> 1) & 1 = (j >> 3) & 1.
  const int vgrp = lane >> 4;
  const int vj = lane & 15;
  const int r8 = 4 * (vgrp >> 1) + (vj >> 2);
  const int vfb = (vj >> 3) & 1;
  const int vp_lo = 2 * (vgrp & 1) + ((vj & 3) >> 1);
  const int v_lane0 = (r8 * 8 + 4 * vfb + vp_lo) * 16 + 8 * (vj & 1);          // even db
  const int v_lane1 = (r8 * 8 + 4 * (vfb ^ 1) + vp_lo) * 16 + 8 * (vj & 1);    // odd db

  f32x16 acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = f32x16{};
  float m = -INFINITY;   // running max (log2 units) of this lane's query, moved lazily
  float lsum = 0.f;      // this lane's share of the weight sum

  // One tile. kMasked: the causal mask may cut the wave's keys (only the
  // tiles that reach past the block's first query). kFold (scale > 0): the
  // scores stay unscaled, their max is scaled once, and each weight is
  // exp2(fma(s, scale, -m)).
  auto step = [&](int tt, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    // this wave's loads of tile tt are done; the barrier makes every wave's
    // rows visible and frees the stage of tile tt - 1
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    // after the last tile these loads fill the free stage with row kend - 1
    // (every row of tile ntiles is past kend): no branch around them
    const NextTile nt = prepare(tt + 1);
    const PrefillStage& st = lds.stage[tt & 1];
    const int t0 = tt * kPfKeys + kPfWaveKeys * kh;   // this wave's first key

    // S^T = K Q^T; register r holds key t0 + 8 (r / 4) + 4 half + r % 4
    f32x16 s = f32x16{};
    const char* kbase = st.k + k_lane;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(kbase + (ks >> 2) * 8 * kBlockBytes +
                                                        (ks & 3) * 256);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), qf[ks], s, 0, 0, 0);
      if (ks & 1) load(nt, ks >> 1);
    }
    if constexpr (!kFold) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] *= a.scale_log2;
    }
    if constexpr (kMasked) {
      if (t0 + kPfWaveKeys - 1 > block_first) {   // keys reach past the block's first query
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (t0 + 8 * (r >> 2) + 4 * half + (r & 3) > pos) s[r] = -INFINITY;
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
    tmax = max_xor32(tmax);
    if constexpr (kFold) tmax *= a.scale_log2;
    if (__builtin_amdgcn_ballot_w64(tmax > m + kRescaleLog2)) {   // rare after the first tile
      const float m_new = fmaxf(m, tmax);
      const float alpha = m_new == -INFINITY ? 1.f : exp2_fast(m - m_new);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] *= alpha;
      m = m_new;
    }
    const float m_ref = m == -INFINITY ? 0.f : m;   // nothing seen yet: weights 0

    // p = exp2(x - m) rounded to bf16 as the P^T operand (chunk c: keys
    // 16 c .. 16 c + 15 = registers 8 c .. 8 c + 7), then O^T += V^T P^T.
    // chunk by chunk (keys 16 c .. 16 c + 15 = registers 8 c .. 8 c + 7): the
    // second chunk's exponentials can run under the first chunk's products
    const char* vbase = st.v + (4 * kh) * 4 * kBlockBytes;
    // V^T fragment of step i = 8 c + db (chunk c, dim block db); each is read
    // two steps ahead of its product (a ring of three), so a product no
    // longer waits on the transposing reads issued right before it
    auto read_vt = [&](int i) {
      // key group of chunk c, read hi: 4 kh + 2 c + hi; piece group db / 2
      const int c = i >> 3, db = i & 7;
      const char* vc = vbase + (db & 1 ? v_lane1 : v_lane0) + (db >> 1) * kBlockBytes +
                       (2 * c) * 4 * kBlockBytes;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vc);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vc + 4 * kBlockBytes));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 vq[3];
    vq[0] = read_vt(0);
    vq[1] = read_vt(1);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (kFold)
          p[e] = exp2_fast(fmaf(s[8 * c + e], a.scale_log2, -m_ref));
        else
          p[e] = exp2_fast(s[8 * c + e] - m_ref);
        lsum += p[e];
      }
      const u32x4 packed = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                            pack_bf16(p[6], p[7])};
      const bf16x8 pb = as_bf16x8(packed);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int i = 8 * c + db;
        if (i + 2 < 16) vq[(i + 2) % 3] = read_vt(i + 2);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vq[i % 3], pb, acc[db], 0, 0, 0);
      }
    }
  };

  // tiles whose 64 keys all precede the block's first query need no mask
  const int n_open = min(t_hi, max(t_lo, (block_first + 1) / kPfKeys));
  {
    const NextTile nt = prepare(t_lo);
#pragma unroll
    for (int i = 0; i < 8; ++i) load(nt, i);
  }
  for (int tt = t_lo; tt < n_open; ++tt) step(tt, std::false_type{});
  for (int tt = n_open; tt < t_hi; ++tt) step(tt, std::true_type{});

  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): the spare loads into LDS are done
  // The two key halves of a query group merge through LDS (the tiles are
  // done): the second half's wave leaves (m, l, acc) there, the first half's
  // wave rescales both to the larger max and writes the output.
  lsum = add_xor32(lsum);
  __syncthreads();
  float* mbuf = lds.merge[w];
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) mbuf[(db * 16 + r) * 64 + lane] = acc[db][r];
    mbuf[kPfCols * kHeadSize + lane] = m;
    mbuf[kPfCols * kHeadSize + 64 + lane] = lsum;
  }
  __syncthreads();
  if (kh == 1 || !q_valid) return;
  // the max of both halves; -inf only when the query sees no key of this
  // workgroup's split (with one split, key 0 is visible to every query)
  const float m2 = mbuf[kPfCols * kHeadSize + lane];
  const float l2 = mbuf[kPfCols * kHeadSize + 64 + lane];
  float mx = fmaxf(m, m2);
  if (mx == -INFINITY) mx = 0.f;   // both halves empty: every weight stays 0
  const float f1 = exp2_fast(m - mx), f2 = exp2_fast(m2 - mx);
  lsum = lsum * f1 + l2 * f2;
  // o = acc / l: register r of block db holds dim 32 db + 8 (r / 4) + 4 half + r % 4.
  // One split: lsum >= 1 (the maximum key has weight 1). Several: the split's
  // normalized partial and its log2-sum-exp, or 0 and -inf for no key.
  // The halves are merged and written one block db at a time (a scheduling
  // barrier per block), so only that block's 16 values from LDS are live
  // next to the accumulator.
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const float w1 = f1 * inv, w2 = f2 * inv;
  float* orow_part = nullptr;
  int64_t orow = 0;
  if constexpr (kSplit) {
    const int64_t prow = (static_cast<int64_t>(split) * a.num_q + qi) * hq + h;
    if (half == 0) a.lse_part[prow] = lsum > 0.f ? mx + __log2f(lsum) : -INFINITY;
    orow_part = a.o_part + prow * kHeadSize + 4 * half;
  } else {
    orow = (static_cast<int64_t>(qi) * hq + h) * kHeadSize + 4 * half;
  }
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    float o[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) o[r] = acc[db][r] * w1 + mbuf[(db * 16 + r) * 64 + lane] * w2;
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const f32x4 v = {o[4 * rq], o[4 * rq + 1], o[4 * rq + 2], o[4 * rq + 3]};
      if constexpr (kSplit) {
        *reinterpret_cast<f32x4*>(orow_part + 32 * db + 8 * rq) = v;
      } else {
        const int64_t idx = orow + 32 * db + 8 * rq;
        if (a.out) {
          u32x2 packed;
          packed.x = f32_to_bf16(v.x) | (f32_to_bf16(v.y) << 16);
          packed.y = f32_to_bf16(v.z) | (f32_to_bf16(v.w) << 16);
          *reinterpret_cast<u32x2*>(a.out + idx) = packed;
        }
        if (a.out_f32) *reinterpret_cast<f32x4*>(a.out_f32 + idx) = v;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Merge of the key splits: one thread per (query, head, 4 dims);
// o = sum_j 2^(lse_j - M) o_j / sum_j 2^(lse_j - M), M = max_j lse_j (split 0
// holds key 0, so M is finite), then the bf16 (RNE) and fp32 outputs.
constexpr int kPfCombineThreads = 256;

__global__ __launch_bounds__(kPfCombineThreads) void prefill_combine_kernel(PrefillArgs a) {
  const int hq = a.num_kv_heads * kGroup;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kPfCombineThreads + threadIdx.x;
  const int64_t row = t / (kHeadSize / 4);   // query * hq + head
  if (row >= static_cast<int64_t>(a.num_q) * hq) return;
  const int d = static_cast<int>(t - row * (kHeadSize / 4)) * 4;
  const int64_t split_rows = static_cast<int64_t>(a.num_q) * hq;
  const int qb = static_cast<int>(row / hq) / kPfQueries;
  const int ns = splits_of(qb, a.key_splits, a.short_blocks);   // this query's block
  float mx = -INFINITY;
  for (int j = 0; j < ns; ++j) mx = fmaxf(mx, a.lse_part[j * split_rows + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int j = 0; j < ns; ++j) {
    const float w = exp2_fast(a.lse_part[j * split_rows + row] - mx);   // 0 for an empty split
    den += w;
    acc += w * *reinterpret_cast<const f32x4*>(a.o_part + (j * split_rows + row) * kHeadSize + d);
  }
  const f32x4 o = acc * (1.f / den);
  const int64_t idx = row * kHeadSize + d;
  if (a.out) {
    u32x2 packed;
    packed.x = f32_to_bf16(o.x) | (f32_to_bf16(o.y) << 16);
    packed.y = f32_to_bf16(o.z) | (f32_to_bf16(o.w) << 16);
    *reinterpret_cast<u32x2*>(a.out + idx) = packed;
  }
  if (a.out_f32) *reinterpret_cast<f32x4*>(a.out_f32 + idx) = o;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.num_q <= 0) return hipSuccess;
  const int64_t blocks = prefill_grid(a.num_q, a.num_kv_heads, a.key_splits, a.short_blocks);
  const bool fold = a.scale_log2 > 0.f, split = a.key_splits > 1;
  auto kernel = fold ? (split ? prefill_kernel<true, true> : prefill_kernel<true, false>)
                     : (split ? prefill_kernel<false, true> : prefill_kernel<false, false>);
  hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kPfThreads), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.key_splits == 1) return e;
  const int64_t threads = static_cast<int64_t>(a.num_q) * a.num_kv_heads * kGroup * (kHeadSize / 4);
  hipLaunchKernelGGL(prefill_combine_kernel,
                     dim3(static_cast<uint32_t>((threads + kPfCombineThreads - 1) / kPfCombineThreads)),
                     dim3(kPfCombineThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
