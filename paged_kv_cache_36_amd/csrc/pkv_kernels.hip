// HIP kernels for single-token decode attention over a paged KV cache, gfx950.
//
// Work split. One workgroup (4 waves) owns one (sequence, KV head, partition)
// triple; a partition is a run of P consecutive tokens of the sequence. Inside
// it, wave w takes the 16-token blocks that start at t_begin + 16 w + 64 k,
// so the workgroup streams 64-token tiles. Each wave keeps its own running
// softmax state for the 6 query heads of the group and the four states are
// merged once, at the end, through LDS.
//
// Per 16-token block a wave
//  - resolves the block's page once (block sizes are multiples of 16, so a
//    16-token block never straddles a page: one table lookup per block, no
//    per-token division, no tail mask except on the last block of a
//    partition),
//  - loads K straight into the A-operand layout of v_mfma_f32_16x16x32_bf16
//    (lane = token (lane & 15), 16 contiguous bytes per k-step) and V as
//    4 dims per lane (one 512-byte row per wave instruction),
//  - computes the 16 x 6 scores with 8 MFMAs against the resident q fragment,
//  - updates (m, l) and rescales the accumulator (online softmax),
//  - accumulates p * V in fp32 on the VALU (p is broadcast through a
//    wave-private LDS slot).
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

#include "pkv_launch.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = kHeadSize;
constexpr int kG = kGroup;
constexpr int kThreads = 64 * kWaves;
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;
constexpr int kProbeBlocks = 2048;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest, ties to even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Order a wave's own LDS writes before its later LDS reads (and reads before
// later writes). LDS requests of one wave are served in order, so only the
// compiler has to be kept from moving them.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Page walker: the address of a 16-token block of one sequence.
// Token t lives in logical page t / B at offset t % B; its physical page is
// block_table[s, t / B]. The walker keeps (logical page, offset) and moves by
// whole blocks, so the only division is at the start of a partition.
// ---------------------------------------------------------------------------
struct PageWalker {
  const int32_t* row;  // block_table row of the sequence
  int32_t bsz;
  int32_t lp;          // logical page of the current block
  int32_t off;         // offset of the block's first token inside that page

  __device__ __forceinline__ void init(const int32_t* r, int32_t b, int32_t t) {
    row = r;
    bsz = b;
    lp = t / b;
    off = t - lp * b;
  }
  __device__ __forceinline__ void advance(int32_t step) {
    off += step;
    while (off >= bsz) {
      off -= bsz;
      ++lp;
    }
  }
  // Element offset of the block's first row for one KV head.
  __device__ __forceinline__ int64_t base(int64_t page_stride, int32_t row_stride,
                                         int32_t head_off) const {
    return static_cast<int64_t>(row[lp]) * page_stride +
           static_cast<int64_t>(off) * row_stride + head_off;
  }
};

// K block in the A-operand layout of v_mfma_f32_16x16x32_bf16: lane l holds
// token (l & 15), and for k-step ks the 8 dims 32 ks + 8 (l >> 4) .. + 7.
// Rows past the valid count repeat the last valid row (finite data; their
// scores are masked to -inf).
struct KBlock {
  u32x4 r[8];
};
__device__ __forceinline__ void load_k_block(const uint16_t* __restrict__ k, int64_t base,
                                             int32_t row_stride, int n_valid, int lane,
                                             KBlock& kb) {
  const int i = min(lane & 15, n_valid - 1);
  const uint16_t* p = k + base + static_cast<int64_t>(i) * row_stride + 8 * (lane >> 4);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kb.r[ks] = *reinterpret_cast<const u32x4*>(p + 32 * ks);
}

// V block: lane l holds dims 4 l .. 4 l + 3 of each of the 16 tokens (one
// 512-byte row per wave instruction). Rows past the valid count repeat the
// last valid row; their softmax weights are exactly 0.
struct VBlock {
  u32x2 r[16];
};
__device__ __forceinline__ void load_v_block(const uint16_t* __restrict__ v, int64_t base,
                                             int32_t row_stride, int n_valid, int lane,
                                             VBlock& vb) {
  const uint16_t* p = v + base + 4 * lane;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int ii = min(i, n_valid - 1);
    vb.r[i] = *reinterpret_cast<const u32x2*>(p + static_cast<int64_t>(ii) * row_stride);
  }
}

// q of the 6 heads of KV group g in the B-operand layout: lane l holds head
// (l & 15) (zero for heads >= 6) and, for k-step ks, dims 32 ks + 8 (l >> 4).
__device__ __forceinline__ void load_q_frag(const uint16_t* __restrict__ q, int64_t head0,
                                            int lane, bf16x8 (&qf)[8]) {
  const int n = lane & 15;
  if (n < kG) {
    const uint16_t* p = q + (head0 + n) * kD + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p + 32 * ks));
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }
}

// ---------------------------------------------------------------------------
// Split-KV partition kernel.
// ---------------------------------------------------------------------------
template <bool kDirect>
__global__ __launch_bounds__(kThreads) void split_decode_kernel(LaunchArgs a) {
  __shared__ float lds_p[kWaves][kWaveTokens][8];
  __shared__ float lds_alpha[kWaves][8];
  __shared__ float lds_acc[kWaves][kG][kD];
  __shared__ float lds_m[kWaves][8];
  __shared__ float lds_l[kWaves][8];

  const int lane = lane_id();
  const int w = wave_id();
  int bid = blockIdx.x;
  const int part = bid % a.n_parts;
  bid /= a.n_parts;
  const int g = bid % a.num_kv_heads;
  const int s = bid / a.num_kv_heads;
  const int hq = a.num_kv_heads * kG;
  const int64_t head0 = static_cast<int64_t>(s) * hq + g * kG;
  const int seq_len = min(max(a.seq_lens[s], 0), a.max_seq_len);
  const int t_begin = part * a.partition_tokens;

  if (t_begin >= seq_len) {
    if (kDirect && part == 0) {  // empty sequence: zero output rows
      for (int e = threadIdx.x; e < kG * kD; e += kThreads) {
        const int64_t o = head0 * kD + e;
        if (a.out) a.out[o] = 0;
        if (a.out_f32) a.out_f32[o] = 0.f;
      }
    }
    return;
  }
  const int t_end = min(t_begin + a.partition_tokens, seq_len);
  const int row_stride = a.num_kv_heads * kD;
  const int head_off = g * kD;

  bf16x8 qf[8];
  load_q_frag(a.q, head0, lane, qf);

  const int n = lane & 15;   // head column of the score tile
  const int j = lane >> 4;   // row group of the score tile (tokens 4j .. 4j+3)
  float m_run = -INFINITY;
  float l_run = 0.f;
  float acc[kG][4];
#pragma unroll
  for (int h = 0; h < kG; ++h)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[h][c] = 0.f;

  PageWalker walker;
  int t = t_begin + w * kWaveTokens;
  KBlock kc, kn;
  VBlock vc, vn;
  if (t < t_end) {
    walker.init(a.block_table + static_cast<int64_t>(s) * a.max_blocks, a.block_size, t);
    const int nv = min(kWaveTokens, t_end - t);
    load_k_block(a.k, walker.base(a.k_page_stride, row_stride, head_off), row_stride, nv, lane, kc);
    load_v_block(a.v, walker.base(a.v_page_stride, row_stride, head_off), row_stride, nv, lane, vc);
  }

  while (t < t_end) {
    const int t_next = t + kTileTokens;
    if (t_next < t_end) {  // prefetch the wave's next block
      walker.advance(kTileTokens);
      const int nvn = min(kWaveTokens, t_end - t_next);
      load_k_block(a.k, walker.base(a.k_page_stride, row_stride, head_off), row_stride, nvn, lane,
                   kn);
      load_v_block(a.v, walker.base(a.v_page_stride, row_stride, head_off), row_stride, nvn, lane,
                   vn);
    }

    // scores: S^T[token][head] = K[token][:] . q[head][:]
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc.r[ks]), qf[ks],
                                                  sc, 0, 0, 0);

    // online softmax update, in log2 units
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = sc[r] * a.scale_log2;
      if (t + 4 * j + r >= t_end) sv[r] = -INFINITY;
    }
    float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float m_new = fmaxf(m_run, bm);
    const float alpha = exp2_fast(m_run - m_new);
    float pv[4];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pv[r] = exp2_fast(sv[r] - m_new);
      psum += pv[r];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // broadcast p[token][head] and alpha[head] to the whole wave
    if (n < kG) {
#pragma unroll
      for (int r = 0; r < 4; ++r) lds_p[w][4 * j + r][n] = pv[r];
      if (j == 0) lds_alpha[w][n] = alpha;
    }
    wave_lds_sync();

    float al[kG];
#pragma unroll
    for (int h = 0; h < kG; ++h) al[h] = lds_alpha[w][h];
#pragma unroll
    for (int h = 0; h < kG; ++h)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[h][c] *= al[h];

#pragma unroll
    for (int i = 0; i < kWaveTokens; ++i) {
      const float4 pa = *reinterpret_cast<const float4*>(&lds_p[w][i][0]);
      const float2 pb = *reinterpret_cast<const float2*>(&lds_p[w][i][4]);
      const float pw[kG] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y};
      const float vf[4] = {bf16_lo(vc.r[i].x), bf16_hi(vc.r[i].x), bf16_lo(vc.r[i].y),
                           bf16_hi(vc.r[i].y)};
#pragma unroll
      for (int h = 0; h < kG; ++h)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[h][c] = fmaf(pw[h], vf[c], acc[h][c]);
    }
    wave_lds_sync();

    kc = kn;
    vc = vn;
    t = t_next;
  }

  // merge the four waves' states
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (n < kG && j == 0) {
    lds_m[w][n] = m_run;
    lds_l[w][n] = l_tot;
  }
#pragma unroll
  for (int h = 0; h < kG; ++h)
    *reinterpret_cast<float4*>(&lds_acc[w][h][4 * lane]) =
        make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
  __syncthreads();

  const int d = threadIdx.x;
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    float mx = lds_m[0][h];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) mx = fmaxf(mx, lds_m[ww][h]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = exp2_fast(lds_m[ww][h] - mx);
      den = fmaf(f, lds_l[ww][h], den);
      num = fmaf(f, lds_acc[ww][h][d], num);
    }
    const float o = num / den;
    if (kDirect) {
      const int64_t idx = (head0 + h) * kD + d;
      if (a.out) a.out[idx] = static_cast<uint16_t>(f32_to_bf16(o));
      if (a.out_f32) a.out_f32[idx] = o;
    } else {
      const int64_t prow = (head0 + h) * a.n_parts + part;
      a.o_part[prow * kD + d] = o;
      if (d == 0) a.lse_part[prow] = (mx + __log2f(den)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp combine: one wave per (sequence, query head).
// o = sum_p exp(lse_p - M) o_p / sum_p exp(lse_p - M), M = max_p lse_p.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void combine_kernel(LaunchArgs a) {
  const int lane = threadIdx.x;
  const int hq = a.num_kv_heads * kG;
  const int s = blockIdx.x / hq;
  const int h = blockIdx.x - s * hq;
  const int seq_len = min(max(a.seq_lens[s], 0), a.max_seq_len);
  const int np = (seq_len + a.partition_tokens - 1) / a.partition_tokens;
  const int64_t row = static_cast<int64_t>(s) * hq + h;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  if (np > 0) {
    const float* lse = a.lse_part + row * a.n_parts;
    float mx = -INFINITY;
    for (int p = lane; p < np; p += 64) mx = fmaxf(mx, lse[p]);
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) mx = fmaxf(mx, __shfl_xor(mx, sh));
    const float* op = a.o_part + row * a.n_parts * kD + 4 * lane;
    float den = 0.f;
    for (int p = 0; p < np; ++p) {
      const float wgt = exp2_fast((lse[p] - mx) * kLog2e);
      const float4 x = *reinterpret_cast<const float4*>(op + static_cast<int64_t>(p) * kD);
      den += wgt;
      o.x = fmaf(wgt, x.x, o.x);
      o.y = fmaf(wgt, x.y, o.y);
      o.z = fmaf(wgt, x.z, o.z);
      o.w = fmaf(wgt, x.w, o.w);
    }
    const float inv = 1.f / den;
    o.x *= inv;
    o.y *= inv;
    o.z *= inv;
    o.w *= inv;
  }
  const int64_t idx = row * kD + 4 * lane;
  if (a.out) {
    u32x2 packed;
    packed.x = f32_to_bf16(o.x) | (f32_to_bf16(o.y) << 16);
    packed.y = f32_to_bf16(o.z) | (f32_to_bf16(o.w) << 16);
    *reinterpret_cast<u32x2*>(a.out + idx) = packed;
  }
  if (a.out_f32) *reinterpret_cast<float4*>(a.out_f32 + idx) = o;
}

// ---------------------------------------------------------------------------
// Debug kernels: the same partition / wave / block walk as the split kernel.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_i64_kernel(int64_t* p, int64_t n, int64_t value) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = value;
}

__global__ __launch_bounds__(kThreads) void debug_resolve_kernel(LaunchArgs a, int32_t g,
                                                                 int64_t* offs) {
  const int lane = lane_id();
  const int w = wave_id();
  const int part = blockIdx.x % a.n_parts;
  const int s = blockIdx.x / a.n_parts;
  const int seq_len = min(max(a.seq_lens[s], 0), a.max_seq_len);
  const int t_begin = part * a.partition_tokens;
  if (t_begin >= seq_len) return;
  const int t_end = min(t_begin + a.partition_tokens, seq_len);
  const int row_stride = a.num_kv_heads * kD;
  PageWalker walker;
  int t = t_begin + w * kWaveTokens;
  if (t < t_end)
    walker.init(a.block_table + static_cast<int64_t>(s) * a.max_blocks, a.block_size, t);
  while (t < t_end) {
    const int nv = min(kWaveTokens, t_end - t);
    const int64_t base = walker.base(a.k_page_stride, row_stride, g * kD);
    if (lane < nv)
      offs[static_cast<int64_t>(s) * a.max_seq_len + t + lane] =
          base + static_cast<int64_t>(lane) * row_stride;
    t += kTileTokens;
    if (t < t_end) walker.advance(kTileTokens);
  }
}

__global__ __launch_bounds__(kThreads) void debug_gather_kernel(LaunchArgs a, int32_t which,
                                                                uint16_t* dense) {
  const int lane = lane_id();
  const int w = wave_id();
  int bid = blockIdx.x;
  const int part = bid % a.n_parts;
  bid /= a.n_parts;
  const int g = bid % a.num_kv_heads;
  const int s = bid / a.num_kv_heads;
  const int seq_len = min(max(a.seq_lens[s], 0), a.max_seq_len);
  const int t_begin = part * a.partition_tokens;
  if (t_begin >= seq_len) return;
  const int t_end = min(t_begin + a.partition_tokens, seq_len);
  const int row_stride = a.num_kv_heads * kD;
  PageWalker walker;
  int t = t_begin + w * kWaveTokens;
  if (t < t_end)
    walker.init(a.block_table + static_cast<int64_t>(s) * a.max_blocks, a.block_size, t);
  while (t < t_end) {
    const int nv = min(kWaveTokens, t_end - t);
    const int64_t base = walker.base(a.k_page_stride, row_stride, g * kD);
    auto dense_row = [&](int i) {
      return dense + ((static_cast<int64_t>(s) * a.max_seq_len + t + i) * a.num_kv_heads + g) * kD;
    };
    if (which == 0) {
      KBlock kb;
      load_k_block(a.k, base, row_stride, nv, lane, kb);
      const int i = lane & 15;
      if (i < nv) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          *reinterpret_cast<u32x4*>(dense_row(i) + 32 * ks + 8 * (lane >> 4)) = kb.r[ks];
      }
    } else {
      VBlock vb;
      load_v_block(a.k, base, row_stride, nv, lane, vb);
#pragma unroll
      for (int i = 0; i < kWaveTokens; ++i)
        if (i < nv) *reinterpret_cast<u32x2*>(dense_row(i) + 4 * lane) = vb.r[i];
    }
    t += kTileTokens;
    if (t < t_end) walker.advance(kTileTokens);
  }
}

// ---------------------------------------------------------------------------
// Bandwidth probes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                         float* sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  uint32_t x = 0;
  int64_t i = blockIdx.x * 256ll + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a0 = buf[i], a1 = buf[i + stride], a2 = buf[i + 2 * stride], a3 = buf[i + 3 * stride];
    x ^= (a0.x + a0.y + a0.z + a0.w) ^ (a1.x + a1.y + a1.z + a1.w) ^
         (a2.x + a2.y + a2.z + a2.w) ^ (a3.x + a3.y + a3.z + a3.w);
  }
  for (; i < n16; i += stride) {
    const u32x4 a0 = buf[i];
    x ^= a0.x + a0.y + a0.z + a0.w;
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
hipError_t launch_split(const LaunchArgs& a, bool direct, hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * a.n_parts;
  if (blocks == 0) return hipSuccess;
  if (direct)
    hipLaunchKernelGGL(split_decode_kernel<true>, dim3(static_cast<uint32_t>(blocks)),
                       dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(split_decode_kernel<false>, dim3(static_cast<uint32_t>(blocks)),
                       dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(const LaunchArgs& a, hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * kG;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_debug_resolve(const LaunchArgs& a, int32_t kv_head, int64_t* offsets,
                                hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(a.num_seqs) * a.max_seq_len;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i64_kernel, dim3(256), dim3(256), 0, stream, offsets, total,
                     static_cast<int64_t>(-1));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t blocks = static_cast<int64_t>(a.num_seqs) * a.n_parts;
  hipLaunchKernelGGL(debug_resolve_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0,
                     stream, a, kv_head, offsets);
  return hipGetLastError();
}

hipError_t launch_debug_gather(const LaunchArgs& a, int32_t which, uint16_t* dense,
                               hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * a.n_parts;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(debug_gather_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0,
                     stream, a, which, dense);
  return hipGetLastError();
}

int32_t probe_sink_floats() { return kProbeBlocks * 4; }

hipError_t launch_probe_read(const void* buf, size_t bytes, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeBlocks), dim3(256), 0, stream,
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
