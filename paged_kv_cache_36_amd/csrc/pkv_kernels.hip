// HIP kernels for single-token decode attention over a paged KV cache, gfx950.
//
// Work split. With fixed partitions one workgroup (4 waves) owns one
// (sequence, partition, KV head) triple, the KV head fastest in the grid so
// the four 512-byte head slices of the same 2 KiB token rows are read
// together. The balanced split instead gives each of 256 workgroups an even
// share of all (sequence, KV head, 64-token tile) units. Inside a workgroup,
// wave w takes the 16-token blocks that start at t_begin + 16 w + 64 k, so the
// workgroup streams 64-token tiles. Each wave keeps its own running softmax
// state for the 6 query heads of the group; the four states are merged once,
// at the end, through LDS.
//
// Per 16-token block a wave
//  - takes the block's physical page from a per-wave list of the page ids
//    (fetched once, one id per lane, read back with v_readlane), so the block
//    table stays out of the loop; block sizes are multiples of 16, so a block
//    never straddles a page and only a run's last block needs a tail mask,
//  - loads K straight into the A-operand layout of v_mfma_f32_16x16x32_bf16
//    (lane = token (lane & 15), 16 contiguous bytes per k-step) and V two
//    512-byte rows per instruction (V nontemporal: every byte is read once),
//    one block ahead of use,
//  - computes the 16 x 6 scores with 8 MFMAs against q read from LDS,
//  - updates (m, l) and rescales the accumulator (online softmax),
//  - accumulates O^T += V^T P^T with 32 v_mfma_f32_16x16x16bf16_1k: V^T is
//    read from LDS with the transposing read, p is split into bf16 hi + lo.
//
// Sources: the attention formula and the decode step ("From Attention to KV
// Cache Compression: Notes from a KernelGen Optimization", "Starting from
// Attention"), the running max / denominator / numerator update (same page,
// "Online Softmax: Streaming Away the Window"), the token -> page map and
// page shape ("海光 DCU 上的长上下文 Attention：从 page784 到 page832 的 KV
// Cache 对齐与访存优化", §1 and §4), one table lookup per page with the tiles
// inside it streamed, for page784 and page832 alike (same page, §7).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kD = kHeadSize;
constexpr int kG = kGroup;
constexpr int kThreads = 64 * kWaves;
constexpr int kProbeBlocks = 16384;   // copy probe: grid-stride over the whole buffer
constexpr int kReadProbeBlocks = 1024;   // read probe: 4 workgroups per CU, one contiguous share each
constexpr int kReadProbeDepth = 16;      // 16-byte nontemporal loads in flight per thread

// ---------------------------------------------------------------------------
// Page walker: the address of a 16-token block of one sequence.
// Token t lives in logical page t / B at offset t % B; its physical page is
// block_table[s, t / B]. The walker keeps (logical page, offset), moves by
// whole blocks (the only division is at the start of a partition) and reads
// physical page ids from a list that lane i of the wave holds for logical
// page `list_base + i`, fetched with one coalesced load per 64 pages.
// ---------------------------------------------------------------------------
struct PageWalker {
  const int32_t* row;  // block_table row of the sequence
  int32_t bsz;
  int32_t lp;          // logical page of the current block
  int32_t off;         // offset of the block's first token inside that page
  int32_t lp_end;      // one past the last logical page the partition touches
  int32_t list_base;   // logical page held by lane 0 of `ids`
  int32_t ids;         // physical page id of logical page list_base + lane

  __device__ __forceinline__ void fetch(int lane) {
    const int32_t j = list_base + lane;
    ids = j < lp_end ? row[j] : 0;
  }
  // `page_end` bounds the logical pages read from the row (one past the last);
  // it only has to cover the blocks that are loaded and stay within the row.
  __device__ __forceinline__ void init(const int32_t* r, int32_t b, int32_t t, int32_t page_end,
                                       int lane) {
    row = r;
    bsz = b;
    lp = t / b;
    off = t - lp * b;
    lp_end = page_end;
    list_base = lp;
    fetch(lane);
  }
  template <bool kRefetch>
  __device__ __forceinline__ void advance(int32_t step, int lane) {
    off += step;
    while (off >= bsz) {
      off -= bsz;
      ++lp;
    }
    if (kRefetch && lp - list_base >= 64) {  // pages smaller than a partition / 64
      list_base = lp;
      fetch(lane);
    }
  }
  __device__ __forceinline__ int32_t page() const {
    return __builtin_amdgcn_readlane(ids, lp - list_base);
  }
  // Element offset of the block's first row for one KV head.
  static __device__ __forceinline__ int32_t pages_for(int32_t t_end, int32_t b) {
    return (t_end + b - 1) / b;
  }
  __device__ __forceinline__ int64_t base(int64_t page_stride, int32_t row_stride,
                                         int32_t head_off) const {
    return static_cast<int64_t>(page()) * page_stride + static_cast<int64_t>(off) * row_stride +
           head_off;
  }
};

// Buffer resource over the 16 rows of a block that start at `rows` (uniform).
// Loads through it carry a VGPR offset per lane and an SGPR offset per row, so
// one block costs one base pointer instead of a 64-bit address per row.
constexpr int kBufferWord3 = 0x00020000;   // raw 32-bit data format (gfx9 family)
// Cache policies of the block loads. A row-layout instruction reads whole
// 512-byte rows (full 128-byte lines) and every byte is read once, so such
// loads stream past the caches (nontemporal). An operand-layout K instruction
// reads 64 of the 128 bytes of each of 16 lines (the MFMA A-operand layout)
// and the next instruction reads the other half, so it keeps the default
// policy and the second half hits in L2.
constexpr int kPolicyOperand = 0;
constexpr int kPolicyRows = 2;             // nontemporal
// With live == false the resource has no records: every load through it
// returns 0 without touching memory (used for the prefetch past a wave's last
// block, so the loop issues the same loads on every path).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint16_t* rows,
                                                             int32_t row_bytes, bool live) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(rows), 0,
                                           live ? kWaveTokens * row_bytes : 0, kBufferWord3);
}

// A block of 16 rows of one KV head in registers, 8 x 16 bytes per lane, in
// one of two layouts (below).
struct RowRegs {
  u32x4 r[8];
};

// Operand layout (K only): the A operand of v_mfma_f32_16x16x32_bf16. Lane l
// holds token (l & 15), and for k-step ks the 8 dims 32 ks + 8 (l >> 4) .. + 7.
// All 16 rows are read even past the last valid token: a block never leaves
// its page, so they are in-bounds page memory, and their scores are masked to
// -inf before use. `voff` is the lane's byte offset, k_lane_offset().
__device__ __forceinline__ int k_lane_offset(int lane, int32_t row_bytes) {
  return (lane & 15) * row_bytes + 16 * (lane >> 4);
}
__device__ __forceinline__ void load_k_operand(const uint16_t* rows, int32_t row_bytes, int voff,
                                               RowRegs& kb, bool live = true) {
  const __amdgpu_buffer_rsrc_t rs = block_rsrc(rows, row_bytes, live);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    kb.r[ks] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 64 * ks, 0, kPolicyOperand);
}

// Row layout (V, and K when it is staged through LDS): two 512-byte rows per
// wave instruction (16 bytes per lane, the widest load, so the block costs 8
// instructions): r[i] of lane l holds dims 8 (l & 31) .. + 7 of row
// block_row(i, l) = 2 i + (l >> 5). Rows after `last` (the block's last valid
// row, 0..15) repeat row `last`: finite data whose softmax weights are exactly
// 0 (rows past the sequence may be NaN, and 0 * NaN is NaN).
__device__ __forceinline__ int block_row(int i, int lane) { return 2 * i + (lane >> 5); }
__device__ __forceinline__ void load_rows(const uint16_t* rows, int32_t row_bytes, int last,
                                          int lane, RowRegs& rb, bool live = true) {
  const __amdgpu_buffer_rsrc_t rs = block_rsrc(rows, row_bytes, live);
#pragma unroll
  for (int i = 0; i < kWaveTokens / 2; ++i) {
    const int rr = min(block_row(i, lane), last);
    rb.r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, rr * row_bytes + 16 * (lane & 31), 0,
                                                    kPolicyRows);
  }
}

// LDS geometry (elements of 16 bits). Rows are padded so that the transposed
// V reads (16 rows x 32 bytes per instruction), the K operand reads (16 rows
// x 16 bytes) and the q fragment reads fall on distinct banks.
constexpr int kQStride = kD + 8;          // q row: 256 dims + 16 bytes pad
constexpr int kKStride = kD + 8;          // K row: 256 dims + 16 bytes pad
constexpr int kVStride = kD + 16;         // V row: 256 dims + 32 bytes pad
constexpr int kKWaveElems = kWaveTokens * kKStride;
constexpr int kVWaveElems = kWaveTokens * kVStride;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Running softmax state of one wave for the 6 query heads of its group.
// Lane l works for head n = l & 15 (lanes with n >= 6 duplicate head 5 and
// are ignored); the output accumulator is the C layout of the 16x16 MFMA for
// O^T[dims][heads]: acc[db][r] is dim 16 db + 4 (l >> 4) + r of head n.
struct WaveState {
  float m;          // running max of scale*log2(e)*score
  float l;          // running sum of weights over this lane's tokens
  f32x4 acc[16];
};

// fp32 -> bf16 round-to-nearest-even bits (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// One 16-token block of one wave:
//  scores S^T[token][head] = K . q by 8 MFMAs (16x16x32, q fragments from
//  LDS; K from registers in the operand layout, or, with kKRows, from its
//  rows staged in LDS), online softmax update, then P.V on MFMA:
//  O^T[dim][head] += V^T[dim][token] . P^T[token][head] with 16x16x16 MFMAs.
//  The P^T operand is the score tile's own layout (lane: head n, tokens
//  4j..4j+3); it is split p = p_hi + p_lo into two bf16 operands so the
//  weights keep ~16 bits. V^T comes from the V rows staged in LDS through the
//  transposing read ds_read_b64_tr_b16: within each 16-lane group, lane i's
//  k-th value is element i % 4 of the 8 bytes addressed by lane i / 4 + 4 k,
//  so lane (j, s) addresses V[4 j + s / 4][16 db + 4 (s % 4)] and receives
//  V[4 j + k][16 db + i].
template <bool kKRows>
__device__ __forceinline__ void process_block(const RowRegs& kb, const RowRegs& vb,
                                              const uint16_t* lds_q, uint16_t* lds_kw,
                                              uint16_t* lds_vw, int t, int t_end,
                                              float scale_log2, int lane, WaveState& st) {
  const int n = lane & 15;   // head column of the score tile
  const int j = lane >> 4;   // row group of the score tile (tokens 4j .. 4j+3)

  // stage this block's V rows (and K rows) into LDS for the reads below
#pragma unroll
  for (int i = 0; i < kWaveTokens / 2; ++i) {
    *reinterpret_cast<u32x4*>(lds_vw + block_row(i, lane) * kVStride + 8 * (lane & 31)) = vb.r[i];
    if (kKRows)
      *reinterpret_cast<u32x4*>(lds_kw + block_row(i, lane) * kKStride + 8 * (lane & 31)) =
          kb.r[i];
  }
  if (kKRows) wave_lds_sync();   // K (and V) rows visible to the whole wave

  // scores
  const uint16_t* qrow = lds_q + min(n, kG - 1) * kQStride + 8 * j;
  const uint16_t* krow = lds_kw + n * kKStride + 8 * j;   // operand of token n, dims 8 j ..
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const u32x4 qv = *reinterpret_cast<const u32x4*>(qrow + 32 * ks);
    const u32x4 kv = kKRows ? *reinterpret_cast<const u32x4*>(krow + 32 * ks) : kb.r[ks];
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv),
                                                __builtin_bit_cast(bf16x8, qv), sc, 0, 0, 0);
  }

  // online softmax update, in log2 units
  float sv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sv[r] = sc[r] * scale_log2;
    if (t + 4 * j + r >= t_end) sv[r] = -INFINITY;
  }
  float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  bm = max_xor32(max_xor16(bm));
  const float m_new = fmaxf(st.m, bm);
  float pv[4];
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pv[r] = exp2_fast(sv[r] - m_new);
    psum += pv[r];
  }
  // rescale only when some head's running max moved (alpha != 1 somewhere)
  if (__builtin_amdgcn_ballot_w64(m_new != st.m)) {
    const float alpha = exp2_fast(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < 16; ++db) st.acc[db] *= alpha;
  }
  st.l += psum;
  st.m = m_new;

  // P^T operands: p = hi + lo, both bf16
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    hi[r] = bf16_rne_bits(pv[r]);
    lo[r] = bf16_rne_bits(pv[r] - __uint_as_float(hi[r] << 16));
  }
  const s16x4 p_hi = __builtin_bit_cast(s16x4, u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)});
  const s16x4 p_lo = __builtin_bit_cast(s16x4, u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)});

  if (!kKRows) wave_lds_sync();   // V rows visible to the whole wave
  const int s = lane & 15;
  const uint16_t* vsrc = lds_vw + (4 * j + (s >> 2)) * kVStride + 4 * (s & 3);
  s16x4 va[16];
#pragma unroll
  for (int db = 0; db < 16; ++db)
    va[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(vsrc + 16 * db));
#pragma unroll
  for (int db = 0; db < 16; ++db)
    st.acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[db], p_hi, st.acc[db], 0, 0, 0);
#pragma unroll
  for (int db = 0; db < 16; ++db)
    st.acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[db], p_lo, st.acc[db], 0, 0, 0);
  wave_lds_sync();   // rows consumed before the next block overwrites them
}

// Block loads of one wave: K and V of tokens [tt, tt + 16) for the walker's
// current block. Past t_end the loads go through an empty resource (no
// memory traffic), so every path of the loop issues the same loads and each
// block waits only for its own data.
template <bool kKRows>
struct BlockLoader {
  const LaunchArgs& a;
  const PageWalker& walker;
  int t_end, row_stride, row_bytes, head_off, voff_k, lane;
  __device__ __forceinline__ void operator()(int tt, RowRegs& kk, RowRegs& vv) const {
    const bool live = tt < t_end;
    // last valid row of the block (select + min only: stays on the scalar unit)
    const int n_left = live ? t_end - tt : kWaveTokens;
    const int last = (n_left < kWaveTokens ? n_left : kWaveTokens) - 1;
    const uint16_t* krows = a.k + walker.base(a.k_page_stride, row_stride, head_off);
    if (kKRows)
      load_rows(krows, row_bytes, last, lane, kk, live);
    else
      load_k_operand(krows, row_bytes, voff_k, kk, live);
    load_rows(a.v + walker.base(a.v_page_stride, row_stride, head_off), row_bytes, last, lane, vv,
              live);
  }
};

// A wave's walk over its blocks t, t + 64, ... < t_end of one partition with
// two register buffers for K and V used alternately: the next block is in
// flight while the current one is consumed. The first block is already in
// (ka, va). kRefetch selects the walker that may refetch the page list inside
// the loop (a refetch makes the wave wait for all of its loads, so the common
// case keeps it out of the loop entirely).
template <bool kKRows, bool kRefetch>
__device__ __forceinline__ void stream_partition(const LaunchArgs& a, PageWalker& walker,
                                                 const BlockLoader<kKRows>& load, RowRegs& ka,
                                                 RowRegs& va, const uint16_t* lds_q,
                                                 uint16_t* lds_kw, uint16_t* lds_vw, int t,
                                                 int t_end, int lane, WaveState& st) {
  RowRegs kb;
  RowRegs vb;
  for (;;) {
    walker.advance<kRefetch>(kTileTokens, lane);
    load(t + kTileTokens, kb, vb);
    process_block<kKRows>(ka, va, lds_q, lds_kw, lds_vw, t, t_end, a.scale_log2, lane, st);
    t += kTileTokens;
    if (t >= t_end) break;
    walker.advance<kRefetch>(kTileTokens, lane);
    load(t + kTileTokens, ka, va);
    process_block<kKRows>(kb, vb, lds_q, lds_kw, lds_vw, t, t_end, a.scale_log2, lane, st);
    t += kTileTokens;
    if (t >= t_end) break;
  }
}

// Workgroup coordinates of a fixed-partition launch: KV head fastest.
struct SplitCoord {
  int s, part, g;
  bool nt;   // stores of this workgroup nontemporal (see run_segment)
};
__device__ __forceinline__ SplitCoord split_coord(const LaunchArgs& a) {
  int bid = blockIdx.x;
  SplitCoord c;
  c.g = bid % a.num_kv_heads;
  bid /= a.num_kv_heads;
  c.part = bid % a.n_parts;
  c.s = bid / a.n_parts;
  c.nt = static_cast<int64_t>(blockIdx.x) + a.resident_wgs < gridDim.x;
  return c;
}

// Workgroup coordinates of a fixed-partition launch in dispatch order (the
// grid is dispatched in workgroup order): first every full partition (s, p),
// (p + 1) P <= L_s, in (s, p) order, then the last, shorter partition of
// every sequence whose length is not a multiple of P, longest first; the
// workgroups after those have no partition and return false. So the grid
// ends with its shortest partitions instead of with whatever partitions the
// last sequences have, and the slots of partitions past a sequence's end are
// not interleaved with live ones. The KV head stays fastest. Wave 0 counts
// the full and the last partitions per sequence from seq_lens (prefix sums in
// LDS, chunks of 64 sequences); every workgroup does this itself. The last
// partitions are ordered by a counting sort over kTailBuckets length buckets
// (bucket 0 the longest; sequence order within a bucket), which only the
// workgroups that take a last partition compute.
constexpr int kTailBuckets = 64;
__device__ __forceinline__ int tail_bucket(int r, int P) {   // 1 <= r < P
  return static_cast<int>(static_cast<int64_t>(P - r) * kTailBuckets / P);
}
__device__ __forceinline__ bool ordered_coord(const LaunchArgs& a, int32_t* full_pref,
                                              int32_t* tail_pref, int32_t* tail_sort,
                                              SplitCoord& c) {
  const int S = a.num_seqs;
  const int P = a.partition_tokens;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry_f = 0, carry_t = 0;
    if (lane == 0) full_pref[0] = tail_pref[0] = 0;
    for (int c0 = 0; c0 < S; c0 += 64) {
      const int si = c0 + lane;
      const int len = si < S ? min(max(a.seq_lens[si], 0), a.max_seq_len) : 0;
      int f = len / P;
      int t = (len - f * P) > 0 ? 1 : 0;
      f = wave_incl_scan(f);
      t = wave_incl_scan(t);
      if (si < S) {
        full_pref[si + 1] = carry_f + f;
        tail_pref[si + 1] = carry_t + t;
      }
      carry_f += __builtin_amdgcn_readlane(f, 63);
      carry_t += __builtin_amdgcn_readlane(t, 63);
    }
  }
  __syncthreads();
  const int bid = blockIdx.x;
  c.g = bid % a.num_kv_heads;
  const int item = bid / a.num_kv_heads;
  const int n_full = full_pref[S];
  c.nt = static_cast<int64_t>(bid) + a.resident_wgs <
         static_cast<int64_t>(n_full + tail_pref[S]) * a.num_kv_heads;
  if (item < n_full) {
    // the last s with full_pref[s] <= item (uniform search)
    int lo = 0, hi = S;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (full_pref[mid] <= item) lo = mid; else hi = mid;
    }
    c.s = lo;
    c.part = item - full_pref[lo];
    return true;
  }
  const int k = item - n_full;   // the k-th longest last partition
  if (k >= tail_pref[S]) return false;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    tail_sort[lane] = 0;   // the bucket counts (kTailBuckets == 64)
    wave_lds_sync();
    for (int c0 = 0; c0 < S; c0 += 64) {
      const int si = c0 + lane;
      const int len = si < S ? min(max(a.seq_lens[si], 0), a.max_seq_len) : 0;
      const int r = len - (len / P) * P;
      if (r > 0) atomicAdd(&tail_sort[tail_bucket(r, P)], 1);
    }
    wave_lds_sync();
    const int cnt = tail_sort[lane];
    const int incl = wave_incl_scan(cnt);
    const int start = incl - cnt;
    // the one bucket holding position k, and k's place inside it
    const uint64_t hit = __builtin_amdgcn_ballot_w64(cnt > 0 && start <= k && k < incl);
    const int b = static_cast<int>(__builtin_ctzll(hit));
    int j = k - __builtin_amdgcn_readlane(start, b);
    for (int c0 = 0; c0 < S; c0 += 64) {
      const int si = c0 + lane;
      const int len = si < S ? min(max(a.seq_lens[si], 0), a.max_seq_len) : 0;
      const int r = len - (len / P) * P;
      const bool in = r > 0 && tail_bucket(r, P) == b;
      const uint64_t m = __builtin_amdgcn_ballot_w64(in);
      const int n = __popcll(m);
      if (j < n) {   // uniform: the j-th member of this chunk
        const int below = static_cast<int>(__builtin_amdgcn_mbcnt_hi(
            static_cast<uint32_t>(m >> 32),
            __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0)));
        if (in && below == j) tail_sort[kTailBuckets] = si;
        break;
      }
      j -= n;
    }
  }
  __syncthreads();
  c.s = tail_sort[kTailBuckets];
  c.part = min(max(a.seq_lens[c.s], 0), a.max_seq_len) / P;   // its full partitions
  return true;
}

// LDS of one split workgroup.
template <bool kKRows>
struct SplitLds {
  uint16_t q[kG * kQStride];
  // per-wave V staging rows; after the loop each wave reuses its own slice
  // for its partial output [kG][kD] fp32
  uint16_t v[kWaves][kVWaveElems];
  // per-wave K staging rows (only with kKRows)
  uint16_t k[kKRows ? kWaves : 1][kKRows ? kKWaveElems : 8];
  alignas(16) float m[kWaves][8];
  alignas(16) float l[kWaves][8];
};
// A wave's partial output in its slice during the merge: fp32 [kG][kAccStride].
// The 4 extra floats per head start the 6 heads' rows 4 banks apart, so the
// 16 lanes of one accumulator write (6 heads x 16 bytes) hit disjoint banks.
constexpr int kAccStride = kD + 4;
static_assert(kVWaveElems * 2 >= kG * kAccStride * 4, "wave slice too small for the merge");

// Where a segment's result goes.
enum SegmentTarget : int {
  kToOutput = 0,       // final bf16 (+ fp32) output: the segment is the whole sequence
  kToPartition = 1,    // o_part[s, h, part, :], lse_part[s, h, part]
  kToSlot = 2,         // o_part[slot, h % 6, :], lse_part[slot, h % 6] (balanced split)
};

// A segment's results with cache policy kPolicy: thread d writes dim d of the
// six heads' rows (bf16 and fp32 outputs, or fp32 partials) and lane 4 h of
// wave 0 the log-sum-exp of head h.
template <int kPolicy>
__device__ __forceinline__ void store_segment(const LaunchArgs& a, SegmentTarget target, int64_t head0,
                                              int64_t index, int d, const float (&ov)[kG],
                                              bool lse_lane, int64_t row0, int lse_off,
                                              float lse) {
  auto rsrc = [](const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferWord3);
  };
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    if (target == kToOutput) {
      const int64_t row = (head0 + h) * kD;
      if (a.out)
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(f32_to_bf16(ov[h])),
                                              rsrc(a.out + row, kD * 2), 2 * d, 0, kPolicy);
      if (a.out_f32)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ov[h]), rsrc(a.out_f32 + row, kD * 4),
                                              4 * d, 0, kPolicy);
    } else {
      const int64_t prow = target == kToPartition ? (head0 + h) * a.n_parts + index : index * kG + h;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ov[h]), rsrc(a.o_part + prow * kD, kD * 4),
                                            4 * d, 0, kPolicy);
    }
  }
  if (lse_lane)
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rsrc(a.lse_part + row0, 0x7fffffff),
                                          lse_off, 0, kPolicy);
}

// The loads a segment starts with: the wave's page list and its 16 bytes of q.
// They depend on the segment's first token and a bound on its pages only, so
// the fixed-partition kernel issues them before its sequence length arrives.
struct SegmentStart {
  PageWalker walker;
  u32x4 qv;
};
// The walker of a segment that starts at token t_begin: wave w begins at
// t_begin + 16 w, with the page ids of logical pages up to page_end listed.
__device__ __forceinline__ void segment_walker(const LaunchArgs& a, int s, int t_begin,
                                               int32_t page_end, PageWalker& walker) {
  walker.init(a.block_table + static_cast<int64_t>(s) * a.max_blocks, a.block_size,
              t_begin + wave_id() * kWaveTokens, page_end, lane_id());
}

// One workgroup's pass over tokens [t_begin, t_end) of sequence s for KV
// head g: the 4 waves stream their blocks, their states are merged through
// LDS and the merged (o, lse) of the 6 query heads is written to `target`.
// Ends with a workgroup barrier so the LDS can be reused right away.
template <bool kKRows, bool kRefetch>
__device__ __forceinline__ void run_segment(const LaunchArgs& a, SplitLds<kKRows>& lds,
                                            SegmentStart& su, int s, int g, int t_begin,
                                            int t_end, SegmentTarget target, int64_t index,
                                            bool nt) {
  const int lane = lane_id();
  const int w = wave_id();
  const int hq = a.num_kv_heads * kG;
  const int64_t head0 = static_cast<int64_t>(s) * hq + g * kG;
  const int row_stride = a.num_kv_heads * kD;
  const int head_off = g * kD;

  // Start-up, ordered so the first K/V loads wait on one memory round trip:
  // the page list and q were fetched together (DecodeOp::begin), the first
  // block is issued as soon as the page list is in, and q goes to LDS while
  // that block is in flight. Every wave issues the same loads (a wave with no
  // block loads through an empty resource), so the waits stay exact.
  uint16_t* lds_vw = lds.v[w];
  uint16_t* lds_kw = lds.k[kKRows ? w : 0];
  int t = t_begin + w * kWaveTokens;
  const bool active = t < t_end;
  PageWalker& walker = su.walker;
  const bool q_thread = threadIdx.x < kG * kD / 8;
  const int qh = min(static_cast<int>(threadIdx.x >> 5), kG - 1), qc = threadIdx.x & 31;
  __builtin_amdgcn_sched_barrier(0);   // keep the q load ahead of the block loads
  const int row_bytes = row_stride * 2;
  const BlockLoader<kKRows> load{a,         walker,   t_end, row_stride,
                                 row_bytes, head_off, k_lane_offset(lane, row_bytes), lane};
  RowRegs ka;
  RowRegs va;
  load(t, ka, va);
  __builtin_amdgcn_sched_barrier(0);   // issue the first block before waiting for q
  if (q_thread) *reinterpret_cast<u32x4*>(lds.q + qh * kQStride + 8 * qc) = su.qv;
  __syncthreads();

  WaveState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int db = 0; db < 16; ++db) st.acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (active)
    stream_partition<kKRows, kRefetch>(a, walker, load, ka, va, lds.q, lds_kw, lds_vw, t, t_end,
                                       lane, st);

  // merge the four waves' states
  const int n = lane & 15;
  const int j = lane >> 4;
  const float l_tot = add_xor32(add_xor16(st.l));
  float* acc_w = reinterpret_cast<float*>(lds_vw);   // this wave's slice, [kG][kAccStride]
  if (n < kG) {
    if (j == 0) {
      lds.m[w][n] = st.m;
      lds.l[w][n] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < 16; ++db)
      *reinterpret_cast<f32x4*>(acc_w + n * kAccStride + 16 * db + 4 * j) = st.acc[db];
  }
  __syncthreads();

  // The weights exp2(m_w - M) / den of the 24 (head, wave) pairs are the same
  // for every thread, so lane 4 h + w of each wave computes the one for head
  // h and wave w (quad reductions give M and den) and every thread takes
  // them with v_readlane: 3 transcendental instructions per wave instead of
  // 36 per thread. Each thread then forms its dim d of the 6 outputs from
  // the waves' partial sums in LDS.
  const int d = threadIdx.x;
  float xv[kG][kWaves];
#pragma unroll
  for (int h = 0; h < kG; ++h)
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww)
      xv[h][ww] = reinterpret_cast<const float*>(lds.v[ww])[h * kAccStride + d];
  const int hk = min(lane >> 2, kG - 1);   // lanes 24.. duplicate head 5
  const int wk = lane & 3;
  const float mk = lds.m[wk][hk];
  const float lk = lds.l[wk][hk];
  float mx = fmaxf(mk, dpp_read<kDppQuadXor1>(mk));
  mx = fmaxf(mx, dpp_read<kDppQuadXor2>(mx));
  const float fk = exp2_fast(mk - mx);   // 0 for a wave without tokens
  float den = fk * lk;
  den += dpp_read<kDppQuadXor1>(den);
  den += dpp_read<kDppQuadXor2>(den);
  // den >= 1: the wave holding the maximum contributes its own weight 1
  const float scale_k = fk * __builtin_amdgcn_rcpf(den);
  const float lse_k = (mx + __log2f(den)) * kLn2;
  // Store policy (nt, uniform): nontemporal while much of the kernel's
  // reads still follow, the default otherwise. Under the split's read stream,
  // results stored with the default (write-back) policy held every later wait,
  // and the end of the workgroup, back: the wide batch's split ran 2.6 % and
  // the 1024-sequence batch's (16 segments per workgroup) 5.3 % slower with
  // them. Stores near the end of the kernel complete sooner with the default
  // policy (one-round grids ran 0.3 to 2 us slower with nontemporal ones).
  float ov[kG];
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    float o = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww)
      o = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(scale_k), 4 * h + ww)),
               xv[h][ww], o);
    ov[h] = o;
  }
  // log-sum-exps: lane 4 h of wave 0 holds head h's
  const bool lse_lane = target != kToOutput && w == 0 && wk == 0 && (lane >> 2) < kG;
  const int64_t row0 = target == kToPartition ? head0 * a.n_parts + index : index * kG;
  const int lse_off = 4 * (target == kToPartition ? min(lane >> 2, kG - 1) * a.n_parts
                                                  : min(lane >> 2, kG - 1));
  // one branch, then stores of a single policy (buffer stores: the policy is
  // an immediate; every base is wave-uniform)
  if (nt)
    store_segment<kPolicyRows>(a, target, head0, index, d, ov, lse_lane, row0, lse_off, lse_k);
  else
    store_segment<0>(a, target, head0, index, d, ov, lse_lane, row0, lse_off, lse_k);
  __syncthreads();   // LDS free for the next segment
}

// Zero output rows of the 6 query heads of (s, g): an empty sequence.
__device__ __forceinline__ void zero_rows(const LaunchArgs& a, int s, int g) {
  const int64_t head0 = static_cast<int64_t>(s) * a.num_kv_heads * kG + g * kG;
  for (int e = threadIdx.x; e < kG * kD; e += kThreads) {
    const int64_t o = head0 * kD + e;
    if (a.out) a.out[o] = 0;
    if (a.out_f32) a.out_f32[o] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// What a split workgroup does with each of its segments. The split kernels
// below decide which segments a workgroup takes (fixed partitions or the
// balanced share) and hand each one to an Op:
//  - DecodeOp runs the attention pass (run_segment);
//  - DebugResolveOp and DebugGatherOp walk the same segment with the same
//    walker instantiation and record what the decode pass would read (the
//    row offsets, or the rows through the decode's own loaders), so the
//    bit-exact address tests cover the code the decode kernels run.
// ---------------------------------------------------------------------------
template <bool kKRows>
struct DecodeOp {
  using Lds = SplitLds<kKRows>;
  static __device__ __forceinline__ SegmentStart begin(const LaunchArgs& a, int s, int g,
                                                       int t_begin, int32_t page_end) {
    SegmentStart su;
    segment_walker(a, s, t_begin, page_end, su.walker);
    // q: 6 rows x 512 bytes, 16 bytes per thread for threads < 192 (the
    // others load a duplicate and do not store it)
    const int64_t head0 = static_cast<int64_t>(s) * a.num_kv_heads * kG + g * kG;
    const int qh = min(static_cast<int>(threadIdx.x >> 5), kG - 1), qc = threadIdx.x & 31;
    su.qv = *reinterpret_cast<const u32x4*>(a.q + (head0 + qh) * kD + 8 * qc);
    return su;
  }
  template <bool kRefetch>
  static __device__ __forceinline__ void segment(const LaunchArgs& a, Lds& lds, SegmentStart& su,
                                                 int s, int g, int t_begin, int t_end,
                                                 SegmentTarget target, int64_t index, bool nt) {
    run_segment<kKRows, kRefetch>(a, lds, su, s, g, t_begin, t_end, target, index, nt);
  }
  static __device__ __forceinline__ void empty(const LaunchArgs& a, int s, int g) {
    zero_rows(a, s, g);
  }
};

struct NoLds {
  int unused;
};

// The blocks of one wave in a segment, in the order stream_partition visits
// them: block t at the walker state reached after (t - first) / 64 advances.
template <bool kRefetch, class F>
__device__ __forceinline__ void walk_blocks(PageWalker& walker, int t_begin, int t_end, F&& f) {
  int t = t_begin + wave_id() * kWaveTokens;
  if (t >= t_end) return;
  for (;;) {
    f(t, walker);
    t += kTileTokens;
    if (t >= t_end) break;
    walker.advance<kRefetch>(kTileTokens, lane_id());
  }
}

struct DebugResolveOp {
  using Lds = NoLds;
  static __device__ __forceinline__ SegmentStart begin(const LaunchArgs& a, int s, int,
                                                       int t_begin, int32_t page_end) {
    SegmentStart su;
    segment_walker(a, s, t_begin, page_end, su.walker);
    return su;
  }
  template <bool kRefetch>
  static __device__ __forceinline__ void segment(const LaunchArgs& a, Lds&, SegmentStart& su,
                                                 int s, int g, int t_begin, int t_end,
                                                 SegmentTarget, int64_t, bool) {
    if (g != a.dbg_kv_head) return;
    const int lane = lane_id();
    const int row_stride = a.num_kv_heads * kD;
    walk_blocks<kRefetch>(su.walker, t_begin, t_end, [&](int t, const PageWalker& wk) {
      const int nv = min(kWaveTokens, t_end - t);
      const int64_t base = wk.base(a.k_page_stride, row_stride, g * kD);
      if (lane < nv)
        a.dbg_offsets[static_cast<int64_t>(s) * a.max_seq_len + t + lane] =
            base + static_cast<int64_t>(lane) * row_stride;
    });
  }
  static __device__ __forceinline__ void empty(const LaunchArgs&, int, int) {}
};

// which == 0: the K loader of this instantiation (operand layout, or rows
// with kKRows); which == 1: the row loader V uses. Reads a.k (the cache under
// test) with the key-cache page stride.
template <bool kKRows>
struct DebugGatherOp {
  using Lds = NoLds;
  static __device__ __forceinline__ SegmentStart begin(const LaunchArgs& a, int s, int,
                                                       int t_begin, int32_t page_end) {
    SegmentStart su;
    segment_walker(a, s, t_begin, page_end, su.walker);
    return su;
  }
  template <bool kRefetch>
  static __device__ __forceinline__ void segment(const LaunchArgs& a, Lds&, SegmentStart& su,
                                                 int s, int g, int t_begin, int t_end,
                                                 SegmentTarget, int64_t, bool) {
    const int lane = lane_id();
    const int row_stride = a.num_kv_heads * kD;
    const int row_bytes = row_stride * 2;
    walk_blocks<kRefetch>(su.walker, t_begin, t_end, [&](int t, const PageWalker& wk) {
      const int nv = min(kWaveTokens, t_end - t);
      const uint16_t* rows = a.k + wk.base(a.k_page_stride, row_stride, g * kD);
      uint16_t* dense = a.dbg_dense +
                        ((static_cast<int64_t>(s) * a.max_seq_len + t) * a.num_kv_heads + g) * kD;
      const int64_t dense_row = static_cast<int64_t>(a.num_kv_heads) * kD;
      RowRegs rb;
      if (a.dbg_which == 0 && !kKRows) {
        load_k_operand(rows, row_bytes, k_lane_offset(lane, row_bytes), rb);
        const int i = lane & 15;
        if (i < nv) {
#pragma unroll
          for (int ks = 0; ks < 8; ++ks)
            *reinterpret_cast<u32x4*>(dense + i * dense_row + 32 * ks + 8 * (lane >> 4)) = rb.r[ks];
        }
      } else {
        load_rows(rows, row_bytes, nv - 1, lane, rb);
#pragma unroll
        for (int i = 0; i < kWaveTokens / 2; ++i) {
          const int rr = block_row(i, lane);
          if (rr < nv) *reinterpret_cast<u32x4*>(dense + rr * dense_row + 8 * (lane & 31)) = rb.r[i];
        }
      }
    });
  }
  static __device__ __forceinline__ void empty(const LaunchArgs&, int, int) {}
};

// ---------------------------------------------------------------------------
// Split-KV partition kernel, fixed partitions of P tokens: one workgroup per
// (sequence, partition, KV head).
// kRefetch: the partition may span more than 64 pages (pages smaller than
// P / 63 tokens), so the page list is refetched inside the loop; chosen on
// the host from P and the block size.
// kOrdered: the workgroups take the partitions in the order of
// ordered_coord (several sequences, several partitions each); otherwise in
// grid order (sequence, partition, KV head), whose page list and q loads go
// out before the sequence length arrives.
// ---------------------------------------------------------------------------
template <class Op, bool kDirect, bool kRefetch, bool kOrdered>
__global__ __launch_bounds__(kThreads, 2) void split_decode_kernel(LaunchArgs a) {
  __shared__ __attribute__((aligned(16))) typename Op::Lds lds;
  SplitCoord c;
  if (kOrdered) {
    __shared__ int32_t full_pref[kMaxOrderedSeqs + 1], tail_pref[kMaxOrderedSeqs + 1];
    __shared__ int32_t tail_sort[kTailBuckets + 1];
    if (!ordered_coord(a, full_pref, tail_pref, tail_sort, c)) return;
  } else {
    c = split_coord(a);
  }
  const int t_begin = c.part * a.partition_tokens;
  // the partition's pages as far as max_seq_len reaches (host-checked to fit
  // the table row), so the page list needs no sequence length
  const int t_cap = min(t_begin + a.partition_tokens, a.max_seq_len);
  SegmentStart su = Op::begin(a, c.s, c.g, t_begin, PageWalker::pages_for(t_cap, a.block_size));
  const int seq_len = min(max(a.seq_lens[c.s], 0), a.max_seq_len);
  if (t_begin >= seq_len) {
    if (kDirect && c.part == 0) Op::empty(a, c.s, c.g);   // empty sequence
    return;
  }
  const int t_end = min(t_cap, seq_len);
  Op::template segment<kRefetch>(a, lds, su, c.s, c.g, t_begin, t_end,
                                 kDirect ? kToOutput : kToPartition, c.part, c.nt);
}

// ---------------------------------------------------------------------------
// Balanced split-KV kernel: the work is cut into 64-token tiles, enumerated
// as (sequence, KV head, tile), and workgroup w of G = min(grid, T) takes
// the tiles [ceil(w T / G), ceil((w + 1) T / G)) of the T in total, so every
// workgroup streams the same number of tiles whatever the length mix; tile u
// belongs to workgroup floor(u G / T). A workgroup
// writes one partial for each (sequence, KV head) run its range touches, at
// slot w + (s * Hkv + g): along the range boundaries the pair (w, s*Hkv + g)
// moves monotonically, so these slots are distinct. Tile prefix sums are
// computed by every workgroup from seq_lens; workgroup 0 also stores them for
// the combine kernel (when a.prefix is set).
// ---------------------------------------------------------------------------
// The balanced split's first tile of workgroup w: equal shares of the T tiles,
// shifted so that odd workgroups (odd XCDs) get 1/kOddShareDiv less and even
// ones 1/kOddShareDiv more, once the shares hold 16 or more tiles (they then
// keep 14 or more, so none is empty).
__device__ __forceinline__ int64_t bal_bound(int64_t w, int64_t T, int64_t G) {
  if (w >= G) return T;
  const int64_t shift = T >= 16 * G ? T / kOddShareDiv : 0;
  return (w * T + (w & 1) * shift + G - 1) / G;
}
// the workgroup whose share holds tile u (the unshifted owner, or a neighbour)
__device__ __forceinline__ int64_t bal_owner(int64_t u, int64_t T, int64_t G) {
  const int64_t q = u * G / T;
  if (q > 0 && u < bal_bound(q, T, G)) return q - 1;
  if (q + 1 < G && u >= bal_bound(q + 1, T, G)) return q + 1;
  return q;
}

constexpr int64_t kNtShareTiles = 64;
__device__ __forceinline__ int tiles_of(int seq_len) {
  return (seq_len + kTileTokens - 1) / kTileTokens;
}

template <class Op, bool kRefetch>
__global__ __launch_bounds__(kThreads, 2) void balanced_split_kernel(LaunchArgs a) {
  __shared__ __attribute__((aligned(16))) typename Op::Lds lds;
  __shared__ int32_t pref[kMaxBalancedSeqs + 1];   // units before sequence s (x Hkv)
  const int S = a.num_seqs;
  const int hkv = a.num_kv_heads;

  // prefix sums of Hkv * tiles, by wave 0 in chunks of 64 sequences
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0;
    if (lane == 0) pref[0] = 0;
    for (int c0 = 0; c0 < S; c0 += 64) {
      const int si = c0 + lane;
      int v = si < S ? hkv * tiles_of(min(max(a.seq_lens[si], 0), a.max_seq_len)) : 0;
      v = wave_incl_scan(v);
      if (si < S) pref[si + 1] = carry + v;
      carry += __builtin_amdgcn_readlane(v, 63);
    }
  }
  __syncthreads();
  if (blockIdx.x == 0 && a.prefix != nullptr)
    for (int i = threadIdx.x; i <= S; i += kThreads) a.prefix[i] = pref[i];

  // G_eff = min(G, T) workgroups take part, so every range is non-empty and
  // the owners floor(u G_eff / T) of consecutive tiles step by 0 or 1.
  const int64_t T = pref[S];
  const int64_t G = min(static_cast<int64_t>(gridDim.x), T);
  const int64_t wg = blockIdx.x;
  if (wg >= G) return;
  const int64_t u0 = bal_bound(wg, T, G);
  const int64_t u1 = bal_bound(wg + 1, T, G);

  // sequence holding unit u0: the last s with pref[s] <= u0 (uniform search)
  int lo = 0, hi = S;   // pref[lo] <= u0 < pref[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pref[mid] <= u0) lo = mid; else hi = mid;
  }
  int s = lo;
  int64_t u = u0;
  while (u < u1) {
    while (u >= pref[s + 1]) ++s;   // skip sequences with no tiles
    const int seq_len = min(max(a.seq_lens[s], 0), a.max_seq_len);
    const int n = tiles_of(seq_len);
    const int64_t base = pref[s];
    const int g = static_cast<int>((u - base) / n);
    const int tile = static_cast<int>((u - base) - static_cast<int64_t>(g) * n);
    const int64_t seg_end = min(u1, base + static_cast<int64_t>(g + 1) * n);
    const int t_begin = tile * kTileTokens;
    const int t_end = min(static_cast<int>(tile + (seg_end - u)) * kTileTokens, seq_len);
    SegmentStart su = Op::begin(a, s, g, t_begin, PageWalker::pages_for(t_end, a.block_size));
    // every workgroup's share ends at about the same time: nontemporal
    // stores for all but its last segment, once shares are long (64 tiles or
    // more; the batched workload's 32-tile shares measured 0.5 us slower with
    // them)
    Op::template segment<kRefetch>(a, lds, su, s, g, t_begin, t_end, kToSlot,
                                   wg + static_cast<int64_t>(s) * hkv + g,
                                   seg_end < u1 && T >= kNtShareTiles * G);
    u = seg_end;
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp combine: o = sum_p exp(lse_p - M) o_p / sum_p exp(lse_p - M),
// M = max_p lse_p. One wave per (sequence, query head, quarter of the 256
// dims): lane l is partition lane l >> 4 (of 4) and dim lane l & 15 (4 dims
// each). The partitions go in chunks of 4 kUnroll (16 or, for rows of at most
// 16 partials, 4 per lane); a chunk's partials and
// log-sum-exps per lane are loaded at once, then folded into a running
// maximum, weight sum and weighted sum that the 4 partition lanes share, so
// the whole reduction stays inside the wave: no LDS, no barrier.
// ---------------------------------------------------------------------------
constexpr int kCombineThreads = 64;
constexpr int kCombinePLanes = 4;
constexpr int kCombineUnroll = 16;

template <bool kBalanced, int kUnroll>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(LaunchArgs a) {
  const int lane = lane_id();
  const int hq = a.num_kv_heads * kG;
  const int quarter = blockIdx.x & 3;
  const int row_id = blockIdx.x >> 2;
  const int s = row_id / hq;
  const int h = row_id - s * hq;
  const int64_t row = static_cast<int64_t>(s) * hq + h;

  // The np partials of this row: partial k at o_part[o_base + k * o_stride]
  // and lse_part[l_base + k * l_stride]. Loads are issued for k < np_load
  // (>= np) and the partials k >= np are dropped by selects afterwards: with
  // fixed partitions np_load = n_parts is known at launch, so the loads do
  // not wait for the sequence length.
  int np_load;
  int np_balanced = 0;   // balanced: the count, known before any partial load
  int len_v = 0;         // fixed: the raw length, in a VGPR
  int64_t o_base, o_stride, l_base, l_stride;
  if (kBalanced) {
    const int g = h / kG;
    const int seq_len = min(max(a.seq_lens[s], 0), a.max_seq_len);
    const int n = tiles_of(seq_len);
    const int64_t T = a.prefix[a.num_seqs];
    const int64_t G = min(static_cast<int64_t>(a.balanced_grid), T);   // as in the split
    const int64_t u_lo = static_cast<int64_t>(a.prefix[s]) + static_cast<int64_t>(g) * n;
    const int64_t w_first = n > 0 ? bal_owner(u_lo, T, G) : 0;
    const int64_t w_last = n > 0 ? bal_owner(u_lo + n - 1, T, G) : -1;
    np_balanced = static_cast<int>(w_last - w_first + 1);
    const int64_t slot0 = w_first + static_cast<int64_t>(s) * a.num_kv_heads + g;
    o_base = (slot0 * kG + (h - g * kG)) * kD;
    o_stride = kG * kD;
    l_base = slot0 * kG + (h - g * kG);
    l_stride = kG;
    np_load = np_balanced;
  } else {
    // The length goes through the vector memory path and stays in a VGPR
    // until the selects: a scalar load would be waited for together with the
    // kernel arguments, ahead of the partial loads.
    const __amdgpu_buffer_rsrc_t lens = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(a.seq_lens), 0, a.num_seqs * 4, kBufferWord3);
    int len_off = s * 4;
    asm("" : "+v"(len_off));   // a per-lane value to the compiler: no early readfirstlane
    len_v = __builtin_amdgcn_raw_buffer_load_b32(lens, len_off, 0, 0);
    np_load = a.n_parts;
    o_base = row * a.n_parts * kD;
    o_stride = kD;
    l_base = row * a.n_parts;
    l_stride = 1;
  }
  const float* lse = a.lse_part + l_base;
  // partials of this row (computed after the first chunk's loads are issued)
  auto count = [&]() {
    if (kBalanced) return np_balanced;
    int lv = len_v;
    asm volatile("" : "+v"(lv));   // first use stays here, not hoisted above the loads
    const int seq_len = min(max(lv, 0), a.max_seq_len);
    return (seq_len + a.partition_tokens - 1) / a.partition_tokens;
  };

  const int pl = lane >> 4;   // partition lane 0..3
  const int dl = lane & 15;   // dims 64 quarter + 4 dl .. + 3
  const float* op = a.o_part + o_base + 64 * quarter + 4 * dl;
  float m_run = -INFINITY;    // running max of the log-sum-exps seen (log2 units)
  float den = 0.f;            // sum of weights exp2(lse2 - m_run), this lane's partitions
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int np = 0;
  for (int c0 = 0; c0 < np_load; c0 += kUnroll * kCombinePLanes) {
    f32x4 x[kUnroll];
    float ls[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {   // straight-line; p >= np_load reads partial 0
      const int p = c0 + pl + u * kCombinePLanes;
      const int pc = p < np_load ? p : 0;
      x[u] = *reinterpret_cast<const f32x4*>(op + pc * o_stride);
      ls[u] = lse[pc * l_stride];
    }
    __builtin_amdgcn_sched_barrier(0);   // all loads issued before the length is used
    np = count();
    float cm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {   // partitions past the length hold stale data
      const bool ok = c0 + pl + u * kCombinePLanes < np;
      ls[u] = ok ? ls[u] * kLog2e : -INFINITY;
      x[u] = ok ? x[u] : f32x4{0.f, 0.f, 0.f, 0.f};
      cm = fmaxf(cm, ls[u]);
    }
    cm = max_xor32(max_xor16(cm));   // over the 4 partition lanes
    const float m_new = fmaxf(m_run, cm);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;   // nothing seen yet: weights 0
    const float rescale = exp2_fast(m_run - m_ref);
    den *= rescale;
    acc *= rescale;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float w = exp2_fast(ls[u] - m_ref);
      den += w;
      acc += w * x[u];
    }
    m_run = m_new;
  }
  // the 4 partition lanes share m_run: plain sums finish the reduction
  den = add_xor32(add_xor16(den));
  acc.x = add_xor32(add_xor16(acc.x));
  acc.y = add_xor32(add_xor16(acc.y));
  acc.z = add_xor32(add_xor16(acc.z));
  acc.w = add_xor32(add_xor16(acc.w));
  if (pl != 0) return;
  const f32x4 r = np > 0 ? acc * (1.f / den) : f32x4{0.f, 0.f, 0.f, 0.f};
  const int64_t idx = row * kD + 64 * quarter + 4 * dl;
  if (a.out) {
    u32x2 packed;
    packed.x = f32_to_bf16(r.x) | (f32_to_bf16(r.y) << 16);
    packed.y = f32_to_bf16(r.z) | (f32_to_bf16(r.w) << 16);
    *reinterpret_cast<u32x2*>(a.out + idx) = packed;
  }
  if (a.out_f32) *reinterpret_cast<f32x4*>(a.out_f32 + idx) = r;
}

// ---------------------------------------------------------------------------
// Balanced combine for batches of many (sequence, KV head) runs: one wave per
// run merges the partials of all 6 of its query heads (a run's partial slots
// are the same for the 6 heads); lane l takes dims 4 l .. 4 l + 3 of each
// head. With many sequences each run has one or two partials, and one wave
// per (sequence, head, quarter) would spend its time starting waves and
// waiting for one load each; here a wave does 6 rows per round trip. The
// partials go in chunks of kGroupChunk, folded into a running maximum, weight
// sum and weighted sum per head (the same update as combine_kernel).
// ---------------------------------------------------------------------------
constexpr int kGroupChunk = 2;

__global__ __launch_bounds__(kCombineThreads) void combine_group_kernel(LaunchArgs a) {
  const int lane = lane_id();
  const int s = blockIdx.x / a.num_kv_heads;
  const int g = blockIdx.x - s * a.num_kv_heads;
  const int seq_len = min(max(a.seq_lens[s], 0), a.max_seq_len);
  const int n = tiles_of(seq_len);
  const int64_t T = a.prefix[a.num_seqs];
  const int64_t G = min(static_cast<int64_t>(a.balanced_grid), T);   // as in the split
  const int64_t u_lo = static_cast<int64_t>(a.prefix[s]) + static_cast<int64_t>(g) * n;
  const int64_t w_first = n > 0 ? bal_owner(u_lo, T, G) : 0;
  const int64_t w_last = n > 0 ? bal_owner(u_lo + n - 1, T, G) : -1;
  const int np = static_cast<int>(w_last - w_first + 1);
  const int64_t slot0 = w_first + static_cast<int64_t>(s) * a.num_kv_heads + g;

  float m_run[kG], den[kG];
  f32x4 acc[kG];
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    m_run[h] = -INFINITY;
    den[h] = 0.f;
    acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int k0 = 0; k0 < np; k0 += kGroupChunk) {
    f32x4 x[kGroupChunk][kG];
    float ls[kGroupChunk][kG];
#pragma unroll
    for (int c = 0; c < kGroupChunk; ++c) {   // straight-line; k >= np reads partial k0
      const int k = k0 + c < np ? k0 + c : k0;
#pragma unroll
      for (int h = 0; h < kG; ++h) {
        const int64_t prow = (slot0 + k) * kG + h;
        x[c][h] = *reinterpret_cast<const f32x4*>(a.o_part + prow * kD + 4 * lane);
        ls[c][h] = a.lse_part[prow];
      }
    }
#pragma unroll
    for (int c = 0; c < kGroupChunk; ++c) {
      const bool ok = k0 + c < np;
#pragma unroll
      for (int h = 0; h < kG; ++h) {
        const float l2 = ok ? ls[c][h] * kLog2e : -INFINITY;
        const float m_new = fmaxf(m_run[h], l2);
        const float m_ref = m_new == -INFINITY ? 0.f : m_new;   // nothing seen yet: weights 0
        const float r = exp2_fast(m_run[h] - m_ref);
        const float w = exp2_fast(l2 - m_ref);
        den[h] = den[h] * r + w;
        acc[h] = acc[h] * r + w * x[c][h];
        m_run[h] = m_new;
      }
    }
  }
  const int64_t head0 = static_cast<int64_t>(s) * a.num_kv_heads * kG + g * kG;
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    const f32x4 r = np > 0 ? acc[h] * (1.f / den[h]) : f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t idx = (head0 + h) * kD + 4 * lane;
    if (a.out) {
      u32x2 packed;
      packed.x = f32_to_bf16(r.x) | (f32_to_bf16(r.y) << 16);
      packed.y = f32_to_bf16(r.z) | (f32_to_bf16(r.w) << 16);
      *reinterpret_cast<u32x2*>(a.out + idx) = packed;
    }
    if (a.out_f32) *reinterpret_cast<f32x4*>(a.out_f32 + idx) = r;
  }
}

// ---------------------------------------------------------------------------
// Debug helper: fill an int64 buffer (the resolve test marks tokens past a
// sequence with -1).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_i64_kernel(int64_t* p, int64_t n, int64_t value) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = value;
}


// ---------------------------------------------------------------------------
// Bandwidth probes.
// ---------------------------------------------------------------------------
// Streaming read: workgroup b reads its own contiguous share of the buffer,
// every wave instruction 1 KiB, 16 nontemporal loads in flight per thread
// (the fastest of the patterns swept: about 7.1 TB/s, against about 6.1 for a
// grid-stride walk with default-policy loads).
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                         float* sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = blockIdx.x * per;
  const int64_t hi = min(n16, lo + per);
  uint32_t x = 0;
  int64_t i = lo + threadIdx.x;
  for (; i + (kReadProbeDepth - 1) * 256 < hi; i += kReadProbeDepth * 256) {
    u32x4 v[kReadProbeDepth];
#pragma unroll
    for (int u = 0; u < kReadProbeDepth; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * 256);
#pragma unroll
    for (int u = 0; u < kReadProbeDepth; ++u) x ^= v[u].x + v[u].y + v[u].z + v[u].w;
  }
  for (; i < hi; i += 256) {
    const u32x4 v = __builtin_nontemporal_load(buf + i);
    x ^= v.x + v.y + v.z + v.w;
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) x ^= __shfl_xor(x, sh);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = __uint_as_float(x);
}

__global__ __launch_bounds__(256) void probe_copy_kernel(u32x4* __restrict__ dst,
                                                         const u32x4* __restrict__ src, int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
bool partition_needs_refetch(int32_t partition_tokens, int32_t block_size) {
  // a wave's blocks start at most 48 tokens into the partition and the walker
  // lists 64 logical pages from its first block's page
  return (partition_tokens + block_size - 1) / block_size + 1 > 64;
}

namespace {

template <class Op>
hipError_t launch_fixed(const LaunchArgs& a, bool direct, bool ordered, hipStream_t stream) {
  const int64_t live = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * a.n_parts;
  if (live == 0) return hipSuccess;
  const bool refetch = partition_needs_refetch(a.partition_tokens, a.block_size);
  // the ordered coordinates only apply to partials (several partitions)
  ordered = ordered && !direct && a.num_seqs <= kMaxOrderedSeqs;
  const int64_t blocks = live;
  auto kern = direct ? (refetch ? split_decode_kernel<Op, true, true, false>
                                : split_decode_kernel<Op, true, false, false>)
            : ordered ? (refetch ? split_decode_kernel<Op, false, true, true>
                                 : split_decode_kernel<Op, false, false, true>)
                      : (refetch ? split_decode_kernel<Op, false, true, false>
                                 : split_decode_kernel<Op, false, false, false>);
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <class Op>
hipError_t launch_balanced(const LaunchArgs& a, bool refetch, hipStream_t stream) {
  if (a.num_seqs == 0 || a.balanced_grid == 0) return hipSuccess;
  auto kern = refetch ? balanced_split_kernel<Op, true> : balanced_split_kernel<Op, false>;
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(a.balanced_grid)), dim3(kThreads), 0, stream,
                     a);
  return hipGetLastError();
}

// The same split (fixed or balanced) with another Op.
template <class Op>
hipError_t launch_walk(const LaunchArgs& a, const SplitChoice& c, hipStream_t stream) {
  return c.balanced ? launch_balanced<Op>(a, c.refetch, stream)
                    : launch_fixed<Op>(a, /*direct=*/false, c.ordered, stream);
}

}  // namespace

hipError_t launch_split(const LaunchArgs& a, bool direct, const SplitChoice& c,
                        hipStream_t stream) {
  return c.k_rows ? launch_fixed<DecodeOp<true>>(a, direct, c.ordered, stream)
                  : launch_fixed<DecodeOp<false>>(a, direct, c.ordered, stream);
}

hipError_t launch_balanced_split(const LaunchArgs& a, bool refetch, bool k_rows,
                                 hipStream_t stream) {
  return k_rows ? launch_balanced<DecodeOp<true>>(a, refetch, stream)
                : launch_balanced<DecodeOp<false>>(a, refetch, stream);
}

hipError_t launch_combine(const LaunchArgs& a, bool balanced, bool per_run, hipStream_t stream) {
  if (balanced && per_run) {
    const int64_t runs = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads;
    if (runs == 0) return hipSuccess;
    hipLaunchKernelGGL(combine_group_kernel, dim3(static_cast<uint32_t>(runs)),
                       dim3(kCombineThreads), 0, stream, a);
    return hipGetLastError();
  }
  const int64_t blocks = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * kG * 4;
  if (blocks == 0) return hipSuccess;
  // fixed partitions: four loads per partition lane when the row has at most
  // 16 partials (the wide batch's 4096-token partitions), else 16 per chunk
  auto kern = balanced               ? combine_kernel<true, kCombineUnroll>
              : a.n_parts <= 4 * kCombinePLanes ? combine_kernel<false, 4>
                                                : combine_kernel<false, kCombineUnroll>;
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)), dim3(kCombineThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_debug_resolve(const LaunchArgs& a, const SplitChoice& c, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(a.num_seqs) * a.max_seq_len;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i64_kernel, dim3(256), dim3(256), 0, stream, a.dbg_offsets, total,
                     static_cast<int64_t>(-1));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_walk<DebugResolveOp>(a, c, stream);
}

hipError_t launch_debug_gather(const LaunchArgs& a, const SplitChoice& c, hipStream_t stream) {
  return c.k_rows ? launch_walk<DebugGatherOp<true>>(a, c, stream)
                  : launch_walk<DebugGatherOp<false>>(a, c, stream);
}

int32_t probe_sink_floats() { return kProbeBlocks * 4; }

hipError_t launch_probe_read(const void* buf, size_t bytes, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(kReadProbeBlocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(buf), static_cast<int64_t>(bytes / 16), sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  hipLaunchKernelGGL(probe_copy_kernel, dim3(kProbeBlocks), dim3(256), 0, stream,
                     static_cast<u32x4*>(dst), static_cast<const u32x4*>(src),
                     static_cast<int64_t>(bytes / 16));
  return hipGetLastError();
}

}  // namespace pkv
