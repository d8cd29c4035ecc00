// HIP kernels for the paged window compression stage, gfx950.
//
// For every boundary token b (request r, position p) the window is positions
// p - C + 1 .. p of request r (cut at 0); each position t reads state row
// block_table[r, t / B] * B + t % B, whose first D = 512 floats are values v
// and next 512 are scores s. Per dimension d the output is
// c_d = sum_i softmax_i(s_{i,d}) v_{i,d} over the window ("From Attention to
// KV Cache Compression: Notes from a KernelGen Optimization", "How One Output
// Is Produced"), computed with the running maximum / denominator / numerator
// of the same page's "Online Softmax: Streaming Away the Window".
//
// Work split. A window is cut into num_splits parts of part_rows rows; one
// workgroup (4 waves) takes one (output, part). Wave w handles dimension half
// w & 1 (lane l: dims 256 (w & 1) + 4 l .. + 3, one 16-byte load of values and
// one of scores per row, so a wave instruction reads 1 KiB contiguous) and the
// part's 8-row batches w >> 1, (w >> 1) + 2, ...; the next batch is loaded
// while the current one is reduced. The part's physical block ids are loaded
// once (lane i: the part's i-th logical block) and each row takes its id with
// v_readlane. The two row phases merge through LDS. A single part writes c
// directly; several write (c_p, log2-sum-exp_p) per dimension and the combine
// kernel merges them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kCmpThreads = 256;
constexpr int kCmpBatch = 8;                  // rows per batch
constexpr int kCmpHalf = kCompressDim / 2;    // dims per wave

struct CmpState {
  float m[4];     // running max, log2 units
  float den[4];
  float num[4];
};

struct CmpLds {
  f32x4 m[2][64];
  f32x4 den[2][64];
  f32x4 num[2][64];
};

__device__ __forceinline__ f32x4 ld4(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}

// ---------------------------------------------------------------------------
// Finalizer ("From Attention to KV Cache Compression: Notes from a KernelGen
// Optimization", "How One Output Is Produced" and "The Finalizer's Sharp
// Edges"). One wave per output; lane l holds dims 8 l .. 8 l + 7.
//  - rho = (mean c^2 + eps)^-1/2 (wave sum), y = (c rho) w;
//  - lanes 0..55 (dims 0..447): z = bf16(y) round trip; group g of 64 dims =
//    lanes 8 g .. 8 g + 7: a = max(max |z|, 1e-4), e = ceil(log2 fl32(a *
//    fl32(1/127))) taken exactly from the fp32 exponent and mantissa,
//    q = trunc(z 2^-e) clipped to [-127, 127], stored as a byte;
//  - lanes 56..63 (dims 448..511): GPT-J pairs (y[448 + 2j], y[449 + 2j])
//    rotated by row (p / C) * C of cos_sin (cos j, sin 32 + j), stored bf16;
//  - the slot's page gets payload [448 INT8][64 bf16] at (slot % 64) * 576
//    and scale bytes [7 x (e + 127)][0] at 64 * 576 + (slot % 64) * 8.
// An output whose boundary index, slot or RoPE row is out of range writes
// nothing.
// ---------------------------------------------------------------------------
constexpr int kFinThreads = 256;
constexpr int kNopeLanes = 56;   // 448 dims / 8

// The sum over the wave, pairs l and l ^ m added for m = 32, 16, ..., 1 in
// turn (every lane ends with the same bits), on the vector ALU.
__device__ __forceinline__ float wave_sum(float x) {
  x = add_xor16(add_xor32(x));
  x += dpp_read<kDppRowRor8>(x);
  x += dpp_read<kDppRowRor4>(x);
  x += dpp_read<kDppRowRor2>(x);
  x += dpp_read<kDppQuadXor1>(x);
  return x;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Where output n goes: its slot and RoPE row, or ok = false when its
// boundary index, slot or RoPE row is out of range. Uniform over the wave
// (and the workgroup).
struct FinIndex {
  bool ok;
  int64_t slot;
  int64_t pc;
};

__device__ __forceinline__ FinIndex fin_index(const FinalizeArgs& a, int n) {
  FinIndex ix = {false, 0, 0};
  const int64_t b = a.boundaries[n];
  if (b < 0 || b >= a.num_tokens) return ix;
  const int64_t slot = a.slots[b];
  const int64_t p = a.positions[b];
  if (slot < 0 || slot >= a.num_kv_pages * kKvBlockSize || p < 0) return ix;
  const int64_t pc = (p / a.compress_ratio) * a.compress_ratio;
  if (pc >= a.cos_sin_rows) return ix;
  return FinIndex{true, slot, pc};
}

// The finalizer of one output whose index checks passed, on its compressed
// values c (lane l: dims 8 l .. 8 l + 7); all 64 lanes of the wave take part.
__device__ __forceinline__ void fin_write(const FinalizeArgs& a, const FinIndex& ix, int lane,
                                          const float (&c)[8]) {
  const f32x4 w0 = *reinterpret_cast<const f32x4*>(a.weight + 8 * lane);
  const f32x4 w1 = *reinterpret_cast<const f32x4*>(a.weight + 8 * lane + 4);
  const float w[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) sq = __builtin_fmaf(c[i], c[i], sq);
  const float mean = wave_sum(sq) * (1.f / kCompressDim);
  const float rho = __builtin_amdgcn_rsqf(mean + a.eps);
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = (c[i] * rho) * w[i];

  uint8_t* page = a.kv + (ix.slot / kKvBlockSize) * a.kv_page_stride;
  const int off = static_cast<int>(ix.slot % kKvBlockSize);
  uint8_t* payload = page + off * kKvTokenStride;

  // NOPE: the group max is taken over all lanes (RoPE lanes join with 0 and
  // their own group result is unused)
  float z[8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    z[i] = __uint_as_float(bf16_bits(y[i]) << 16);
    amax = fmaxf(amax, fabsf(z[i]));
  }
  if (lane >= kNopeLanes) amax = 0.f;
  // max over each group of 8 lanes (pairs l, l ^ 1, then l ^ 2, then l ^ 4)
  amax = fmaxf(amax, dpp_read<kDppQuadXor1>(amax));
  amax = fmaxf(amax, dpp_read<kDppQuadXor2>(amax));
  amax = fmaxf(amax, dpp_read<kDppHalfMirror>(amax));
  const float av = fmaxf(amax, 1.0e-4f);
  const float yq = av * (1.0f / 127.0f);
  int ex;
  const float mant = frexpf(yq, &ex);
  const int e = mant == 0.5f ? ex - 1 : ex;
  if (lane < kNopeLanes) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float q = truncf(ldexpf(z[i], -e));
      q = fminf(fmaxf(q, -127.f), 127.f);
      const uint32_t byte = static_cast<uint32_t>(static_cast<int>(q)) & 0xffu;
      if (i < 4) lo |= byte << (8 * i);
      else hi |= byte << (8 * (i - 4));
    }
    *reinterpret_cast<u32x2*>(payload + 8 * lane) = u32x2{lo, hi};
  } else {
    // pairs j = 4 (lane - 56) + k: (u, w) = (y[2k], y[2k + 1]); each rotated
    // value is one explicit fma over the other rounded product, so every
    // kernel that inlines the finalizer rounds it the same way
    const int j0 = 4 * (lane - kNopeLanes);
    const float* row = a.cos_sin + ix.pc * 64;
    const f32x4 cs = *reinterpret_cast<const f32x4*>(row + j0);
    const f32x4 sn = *reinterpret_cast<const f32x4*>(row + 32 + j0);
    uint32_t packed[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float u = y[2 * k], v = y[2 * k + 1];
      const float ru = __builtin_fmaf(u, cs[k], -(v * sn[k]));
      const float rv = __builtin_fmaf(v, cs[k], u * sn[k]);
      packed[k] = bf16_bits(ru) | (bf16_bits(rv) << 16);
    }
    *reinterpret_cast<u32x4*>(payload + 8 * kNopeLanes + 16 * (lane - kNopeLanes)) =
        u32x4{packed[0], packed[1], packed[2], packed[3]};
  }
  // scale bytes: exponent of group g sits in lane 8 g
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int g = 0; g < 7; ++g) {
    const uint32_t byte = static_cast<uint32_t>(__shfl(e, 8 * g) + 127) & 0xffu;
    if (g < 4) lo |= byte << (8 * g);
    else hi |= byte << (8 * (g - 4));
  }
  if (lane == 0)
    *reinterpret_cast<u32x2*>(page + kKvBlockSize * kKvTokenStride + off * kKvScaleDim) =
        u32x2{lo, hi};
}

// The finalizer of the output whose merged row sits in LDS (512 floats):
// wave-wide, lane l takes dims 8 l .. 8 l + 7.
__device__ __forceinline__ void fin_from_lds(const FinalizeArgs& a, const FinIndex& ix, int lane,
                                             const float* row) {
  const f32x4 c0 = *reinterpret_cast<const f32x4*>(row + 8 * lane);
  const f32x4 c1 = *reinterpret_cast<const f32x4*>(row + 8 * lane + 4);
  const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
  fin_write(a, ix, lane, c);
}

__global__ __launch_bounds__(kFinThreads) void finalize_kernel(FinalizeArgs a) {
  const int lane = lane_id();
  const int n = blockIdx.x * (kFinThreads / 64) + wave_id();
  if (n >= a.num_outputs) return;
  const FinIndex ix = fin_index(a, n);
  if (!ix.ok) return;
  const float* crow = a.compressed + static_cast<int64_t>(n) * kCompressDim + 8 * lane;
  const f32x4 c0 = *reinterpret_cast<const f32x4*>(crow);
  const f32x4 c1 = *reinterpret_cast<const f32x4*>(crow + 4);
  const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
  fin_write(a, ix, lane, c);
}

// kPack: one part per window and the finalizer fused (pkv_compress_pack):
// the two phase-0 waves leave the merged row in LDS and wave 0 packs it.
template <bool kPack>
__global__ __launch_bounds__(kCmpThreads) void compress_split_kernel(CompressArgs a, FinalizeArgs f) {
  __shared__ CmpLds lds;
  __shared__ __attribute__((aligned(16))) float fin_row[kCompressDim];   // kPack only
  const int n = blockIdx.x / a.num_splits;
  const int part = blockIdx.x - n * a.num_splits;
  const int lane = lane_id();
  const int w = wave_id();
  const int half = w & 1;
  const int phase = w >> 1;

  // Boundary token -> (request, position). Indices outside their arrays make
  // the output NaN instead of reading out of bounds.
  const int64_t b = a.boundaries[n];
  bool ok = b >= 0 && b < a.num_tokens;
  const int64_t bs = ok ? b : 0;
  const int r = a.token_to_req[bs];
  const int64_t p = a.positions[bs];
  ok = ok && r >= 0 && r < a.num_reqs && p >= 0 && p / a.block_size < a.max_blocks;
  // the finalizer's slot and RoPE row: scalar loads issued now, used after the loop
  FinIndex fix = {false, 0, 0};
  if constexpr (kPack) fix = fin_index(f, n);

  // The part's positions [ts, ts + nrows): window rows part * R .. part * R +
  // R - 1. A valid p is below max_blocks * B <= INT32_MAX, so 32 bits hold it.
  const int p32 = ok ? static_cast<int>(p) : 0;
  const int lo = p32 - a.compress_ratio + 1 + part * a.part_rows;
  const int hi = min(lo + a.part_rows, p32 + 1);
  const int ts = max(lo, 0);
  const int nrows = ok ? max(hi - ts, 0) : 0;

  // The part's physical block ids: lane i holds logical block lb0 + i. The
  // load is retired here, on every path, so that the waits the compiler
  // places inside the batch loop never hold back a prefetched batch.
  const int lb0 = ts / a.block_size;
  const int o0 = ts - lb0 * a.block_size;
  int blk = 0;
  if (nrows > 0) {
    const int lb_last = (ts + nrows - 1) / a.block_size;
    if (lane <= lb_last - lb0)
      blk = a.block_table[static_cast<int64_t>(r) * a.max_blocks + lb0 + lane];
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): expcnt and lgkmcnt left at their maxima
  const int64_t first = static_cast<int64_t>(__builtin_amdgcn_readlane(blk, 0)) * a.block_stride +
                        static_cast<int64_t>(o0) * a.row_stride;

  const float* base = a.state + kCmpHalf * half + 4 * lane;
  const int nbatch = (nrows + kCmpBatch - 1) / kCmpBatch;

  // (logical block - lb0, offset) of the wave's next row, walked forward: the
  // wave's batches are every other 8-row batch of the part.
  int lb = 0, o = o0;
  auto skip_rows = [&](int rows) {
    o += rows;
    while (o >= a.block_size) {
      o -= a.block_size;
      ++lb;
    }
  };
  skip_rows(kCmpBatch * phase);

  // Row offsets (elements) of batch k, which starts at the walker; rows past
  // the part repeat its first row (their scores are then set to -inf).
  auto row_offsets = [&](int k, int64_t (&off)[kCmpBatch]) {
#pragma unroll
    for (int i = 0; i < kCmpBatch; ++i) {
      const bool valid = k * kCmpBatch + i < nrows;
      const int page = __builtin_amdgcn_readlane(blk, valid ? lb : 0);
      off[i] = valid ? static_cast<int64_t>(page) * a.block_stride +
                           static_cast<int64_t>(o) * a.row_stride
                     : first;
      skip_rows(1);
    }
    skip_rows(kCmpBatch);   // the other phase's batch
  };
  auto load = [&](int k, f32x4 (&v)[kCmpBatch], f32x4 (&s)[kCmpBatch]) {
    int64_t off[kCmpBatch];
    row_offsets(k, off);
#pragma unroll
    for (int i = 0; i < kCmpBatch; ++i) {
      v[i] = ld4(base + off[i]);
      s[i] = ld4(base + off[i] + kCompressDim);
    }
  };

  CmpState st;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    st.m[d] = -INFINITY;
    st.den[d] = 0.f;
    st.num[d] = 0.f;
  }
  auto consume = [&](int k, const f32x4 (&v)[kCmpBatch], f32x4 (&s)[kCmpBatch]) {
    const int valid = nrows - k * kCmpBatch;
    if (valid < kCmpBatch) {   // the part's last batch only
#pragma unroll
      for (int i = 0; i < kCmpBatch; ++i)
        if (i >= valid) s[i] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float bm = s[0][d];
#pragma unroll
      for (int i = 1; i < kCmpBatch; ++i) bm = fmaxf(bm, s[i][d]);
      const float mn = fmaxf(st.m[d], bm * kLog2e);
      const float mref = mn == -INFINITY ? 0.f : mn;   // nothing finite yet: weights 0
      const float alpha = exp2_fast(st.m[d] - mref);
      float ds = 0.f, ns = 0.f;
#pragma unroll
      for (int i = 0; i < kCmpBatch; ++i) {
        const float e = exp2_fast(__builtin_fmaf(s[i][d], kLog2e, -mref));
        ds += e;
        ns = __builtin_fmaf(e, v[i][d], ns);
      }
      st.den[d] = __builtin_fmaf(st.den[d], alpha, ds);
      st.num[d] = __builtin_fmaf(st.num[d], alpha, ns);
      st.m[d] = mn;
    }
  };

  // Batches phase, phase + 2, ...: two in flight. The prefetch is issued
  // unconditionally (past the part it re-reads the part's first row) so that
  // the loop body has one path and its waits count only the batch consumed.
  f32x4 va[kCmpBatch], sa[kCmpBatch], vb[kCmpBatch], sb[kCmpBatch];
  int k = phase;
  if (k < nbatch) {
    load(k, va, sa);
    for (;;) {
      load(k + 2, vb, sb);
      consume(k, va, sa);
      k += 2;
      if (k >= nbatch) break;
      load(k + 2, va, sa);
      consume(k, vb, sb);
      k += 2;
      if (k >= nbatch) break;
    }
  }

  // merge the two row phases of each dimension half
  if (phase == 1) {
    lds.m[half][lane] = f32x4{st.m[0], st.m[1], st.m[2], st.m[3]};
    lds.den[half][lane] = f32x4{st.den[0], st.den[1], st.den[2], st.den[3]};
    lds.num[half][lane] = f32x4{st.num[0], st.num[1], st.num[2], st.num[3]};
  }
  __syncthreads();
  if (phase == 0) {
  const f32x4 m1 = lds.m[half][lane];
  const f32x4 d1 = lds.den[half][lane];
  const f32x4 n1 = lds.num[half][lane];
  f32x4 c, lse;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float mt = fmaxf(st.m[d], m1[d]);
    const float mref = mt == -INFINITY ? 0.f : mt;
    const float w0 = exp2_fast(st.m[d] - mref);
    const float w1 = exp2_fast(m1[d] - mref);
    const float den = st.den[d] * w0 + d1[d] * w1;
    const float num = st.num[d] * w0 + n1[d] * w1;
    c[d] = den > 0.f ? num / den : 0.f;
    lse[d] = den > 0.f ? mt + __log2f(den) : -INFINITY;
    if (!ok) {
      c[d] = __builtin_nanf("");
      lse[d] = INFINITY;
    }
  }
  const int dim = kCmpHalf * half + 4 * lane;
  if (a.num_splits == 1) {
    if (!kPack || a.out)
      *reinterpret_cast<f32x4*>(a.out + static_cast<int64_t>(n) * kCompressDim + dim) = c;
    if constexpr (kPack) *reinterpret_cast<f32x4*>(fin_row + dim) = c;
  } else {
    const int64_t idx = (static_cast<int64_t>(n) * a.num_splits + part) * kCompressDim + dim;
    *reinterpret_cast<f32x4*>(a.o_part + idx) = c;
    *reinterpret_cast<f32x4*>(a.lse_part + idx) = lse;
  }
  }
  if constexpr (kPack) {
    __syncthreads();
    if (w == 0 && fix.ok) fin_from_lds(f, fix, lane, fin_row);
  }
}

// Merge of several (m, weight sum, weighted sum) states of one dimension:
// m is a log2-sum-exp reference; an m of +inf (bad indices) poisons the
// result with NaN, an m of -inf (no finite score) carries no weight.
struct CmbState {
  f32x4 m, tot, acc;
};

__device__ __forceinline__ void cmb_merge(CmbState& x, const f32x4& m2, const f32x4& t2,
                                          const f32x4& a2) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float mt = fmaxf(x.m[d], m2[d]);
    const float mref = mt == -INFINITY ? 0.f : mt;
    const float w1 = exp2_fast(x.m[d] - mref);
    const float w2 = exp2_fast(m2[d] - mref);
    // explicit fma: one rounding order, whatever the compiler contracts
    x.tot[d] = __builtin_fmaf(x.tot[d], w1, t2[d] * w2);
    x.acc[d] = __builtin_fmaf(x.acc[d], w1, a2[d] * w2);
    x.m[d] = mt;
  }
}

__device__ __forceinline__ f32x4 shfl_xor4(const f32x4& v, int mask) {
  return f32x4{__shfl_xor(v[0], mask), __shfl_xor(v[1], mask), __shfl_xor(v[2], mask),
               __shfl_xor(v[3], mask)};
}

// G = a.combine_lanes (a power of two, S <= 8 G) adjacent lanes share one
// (output, 4-dimension group); lane g of them merges parts 8 g .. 8 g + 7, all
// its loads in flight at once, and the G lanes then merge with xor shuffles:
// c = sum_p 2^(lse_p - LSE) c_p / sum_p 2^(lse_p - LSE).
constexpr int kCmbPartsPerLane = 8;
// the fused combine's workgroup: 128 (output dims / 4) x at most 8 lanes
constexpr int kCombinePackMaxThreads = (kCompressDim / 4) * 8;

// Lane g of the combine's merge for one (output, 4 dims): parts 8 g .. 8 g + 7
// in turn (parts past num_splits merge as empty), from base (the output's
// part 0 at these dims).
__device__ __forceinline__ CmbState cmb_lane(const float* lse_part, const float* o_part,
                                             int64_t base, int g, int num_splits) {
  f32x4 l[kCmbPartsPerLane], o[kCmbPartsPerLane];
#pragma unroll
  for (int i = 0; i < kCmbPartsPerLane; ++i) {
    const int j = g * kCmbPartsPerLane + i;
    l[i] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (j < num_splits) {
      l[i] = *reinterpret_cast<const f32x4*>(lse_part + base + static_cast<int64_t>(j) * kCompressDim);
      o[i] = *reinterpret_cast<const f32x4*>(o_part + base + static_cast<int64_t>(j) * kCompressDim);
    }
  }
  CmbState x;
  x.m = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  x.tot = f32x4{0.f, 0.f, 0.f, 0.f};
  x.acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kCmbPartsPerLane; ++i) {
    // a part holds c_p with weight 2^(lse_p - lse_p) = 1; an empty part
    // (lse_p = -inf) holds c_p = 0 and no weight
    f32x4 w = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int d = 0; d < 4; ++d)
      if (l[i][d] == -INFINITY) w[d] = 0.f;
    cmb_merge(x, l[i], w, o[i] * w);
  }
  return x;
}

__device__ __forceinline__ f32x4 cmb_value(const CmbState& x) {
  f32x4 c;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    c[d] = x.tot[d] > 0.f ? x.acc[d] / x.tot[d] : 0.f;
    if (x.tot[d] != x.tot[d] || x.m[d] == INFINITY) c[d] = __builtin_nanf("");
  }
  return c;
}

__global__ __launch_bounds__(kCmpThreads) void compress_combine_kernel(CompressArgs a) {
  const int g_lanes = a.combine_lanes;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kCmpThreads + threadIdx.x;
  const int64_t group = t / g_lanes;                  // (output, 4-dim group)
  const int pg = static_cast<int>(t - group * g_lanes);
  const int groups_per_out = kCompressDim / 4;
  const bool live = group < static_cast<int64_t>(a.num_outputs) * groups_per_out;
  const int64_t n = live ? group / groups_per_out : 0;
  const int dim = static_cast<int>(group - n * groups_per_out) * 4;
  const int64_t base = n * a.num_splits * kCompressDim + dim;
  CmbState x = cmb_lane(a.lse_part, a.o_part, live ? base : 0, live ? pg : a.num_splits,
                        a.num_splits);
  for (int mask = 1; mask < g_lanes; mask <<= 1)   // uniform trip count
    cmb_merge(x, shfl_xor4(x.m, mask), shfl_xor4(x.tot, mask), shfl_xor4(x.acc, mask));
  if (!live || pg != 0) return;
  const f32x4 c = cmb_value(x);
  *reinterpret_cast<f32x4*>(a.out + n * kCompressDim + dim) = c;
}

// The combine with the finalizer fused (pkv_compress_pack, several parts per
// window): one workgroup of 128 G threads per output (G = a.combine_lanes),
// each (4-dimension group, lane) merging the same parts in the same order as
// compress_combine_kernel, so the merged row is bit for bit that kernel's;
// the row goes through LDS to wave 0, which packs it. The finalizer's slot
// and RoPE row are loaded before the parts arrive.
__global__ __launch_bounds__(kCombinePackMaxThreads) void compress_combine_pack_kernel(
    CompressArgs a, FinalizeArgs f) {
  __shared__ __attribute__((aligned(16))) float fin_row[kCompressDim];
  const int g_lanes = a.combine_lanes;
  const int n = blockIdx.x;
  const int t = threadIdx.x;
  const int group = t / g_lanes;
  const int pg = t - group * g_lanes;
  const int dim = 4 * group;
  const FinIndex fix = fin_index(f, n);
  const int64_t base = static_cast<int64_t>(n) * a.num_splits * kCompressDim + dim;
  CmbState x = cmb_lane(a.lse_part, a.o_part, base, pg, a.num_splits);
  for (int mask = 1; mask < g_lanes; mask <<= 1)
    cmb_merge(x, shfl_xor4(x.m, mask), shfl_xor4(x.tot, mask), shfl_xor4(x.acc, mask));
  if (pg == 0) {
    const f32x4 c = cmb_value(x);
    if (a.out) *reinterpret_cast<f32x4*>(a.out + static_cast<int64_t>(n) * kCompressDim + dim) = c;
    *reinterpret_cast<f32x4*>(fin_row + dim) = c;
  }
  __syncthreads();
  if (t < 64 && fix.ok) fin_from_lds(f, fix, t, fin_row);
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, hipStream_t stream) {
  if (a.num_outputs <= 0) return hipSuccess;
  const int64_t blocks = static_cast<int64_t>(a.num_outputs) * a.num_splits;
  hipLaunchKernelGGL(compress_split_kernel<false>, dim3(static_cast<uint32_t>(blocks)),
                     dim3(kCmpThreads), 0, stream, a, FinalizeArgs{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_splits == 1) return e;
  const int64_t threads = static_cast<int64_t>(a.num_outputs) * (kCompressDim / 4) * a.combine_lanes;
  const int64_t cblocks = (threads + kCmpThreads - 1) / kCmpThreads;
  hipLaunchKernelGGL(compress_combine_kernel, dim3(static_cast<uint32_t>(cblocks)),
                     dim3(kCmpThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_compress_pack(const CompressArgs& a, const FinalizeArgs& f,
                                hipStream_t stream) {
  if (a.num_outputs <= 0) return hipSuccess;
  if (a.num_splits == 1) {
    hipLaunchKernelGGL(compress_split_kernel<true>, dim3(static_cast<uint32_t>(a.num_outputs)),
                       dim3(kCmpThreads), 0, stream, a, f);
    return hipGetLastError();
  }
  const int64_t blocks = static_cast<int64_t>(a.num_outputs) * a.num_splits;
  hipLaunchKernelGGL(compress_split_kernel<false>, dim3(static_cast<uint32_t>(blocks)),
                     dim3(kCmpThreads), 0, stream, a, f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compress_combine_pack_kernel, dim3(static_cast<uint32_t>(a.num_outputs)),
                     dim3((kCompressDim / 4) * a.combine_lanes), 0, stream, a, f);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t stream) {
  if (a.num_outputs <= 0) return hipSuccess;
  const int per_block = kFinThreads / 64;
  const int64_t blocks = (static_cast<int64_t>(a.num_outputs) + per_block - 1) / per_block;
  hipLaunchKernelGGL(finalize_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kFinThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace pkv
