/*
 * pkv.h -- single-token decode attention over a paged KV cache, for AMD
 * MI355X (gfx950). C ABI; every call is asynchronous on the caller's stream.
 *
 * What is computed. For every sequence s and query head h (KV head g = h / G,
 * G = num_q_heads / num_kv_heads = 6):
 *     s_t = scale * q[s,h,:] . K_s[t,g,:]            for t < seq_lens[s]
 *     o[s,h,:] = sum_t softmax(s)_t V_s[t,g,:]
 * ("From Attention to KV Cache Compression: Notes from a KernelGen
 * Optimization", "Starting from Attention": dot-product attention and the
 * decode step that attends to every cached token). K_s / V_s row t is read
 * through the block table: logical page t / block_size, offset t %
 * block_size, physical page block_table[s, logical page] ("海光 DCU 上的长上下文
 * Attention：从 page784 到 page832 的 KV Cache 对齐与访存优化", §1; page shape
 * [block_size, 4, 256] per K or V page, §4; both page784 and page832
 * supported, §2 and §7).
 *
 * Conventions for every entry point:
 *  - Pointers named as device pointers must point to device memory (HBM) on
 *    the current HIP device; `params` / `info` are host pointers.
 *  - bf16 values are passed as raw 16-bit storage (`void*` / uint16_t).
 *  - `stream` is a hipStream_t (NULL = the default stream). Nothing here
 *    synchronizes the stream or the device.
 *  - The caller owns and allocates every buffer; the library allocates no
 *    device memory and keeps no state besides an immutable per-process log
 *    flag and each device's compute-unit count (read once, for planning), so
 *    calls are thread-safe. (The one exception, pkv_decode_noalloc, uses a
 *    static device array of its own; see there.)
 *  - Host-side checks run before any launch and return a negative status;
 *    a failed launch returns PKV_ERR_HIP. Nothing is written on error.
 *  - Preconditions that live in device memory are documented, not checked:
 *    0 <= seq_lens[s] <= max_seq_len <= max_blocks_per_seq * block_size;
 *    block_table[s, j] for j < ceil(seq_lens[s] / block_size) is a valid page
 *    index of both caches; outputs alias no input.
 *  - seq_lens[s] == 0 writes a zero output row (lse = -inf in partials).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define PKV_API __attribute__((visibility("default")))
#else
#define PKV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,        /* a required pointer is NULL or misaligned           */
  PKV_ERR_SHAPE = -2,       /* head counts / sizes / table width inconsistent     */
  PKV_ERR_BLOCK_SIZE = -3,  /* block_size not a positive multiple of 16 (decode;
                               prefill and append accept any positive size)       */
  PKV_ERR_PARTITION = -4,   /* partition_tokens not 0 and not a multiple of 64,
                               or a prefill key_splits outside 0..64              */
  PKV_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required         */
  PKV_ERR_UNSUPPORTED = -6, /* head_size != 256, group size != 6, or the call does
                               not apply to this plan                             */
  PKV_ERR_HIP = -7,         /* a HIP launch or runtime call failed                */
  PKV_ERR_STRIDE = -8,      /* page stride too small or not a multiple of 8       */
  PKV_ERR_SCRATCH = -9      /* pkv_decode_noalloc: the call needs more workspace
                               than the static scratch array holds                */
} pkv_status;

/* Geometry of one decode call. All sizes in elements unless noted. */
typedef struct {
  int32_t num_seqs;           /* S >= 0                                             */
  int32_t num_q_heads;        /* Hq = 6 * Hkv (24 for the 24/4 layout)              */
  int32_t num_kv_heads;       /* Hkv >= 1 (4)                                       */
  int32_t head_size;          /* D, must be 256                                     */
  int32_t block_size;         /* B: tokens per physical page, multiple of 16
                                 (784 and 832 are the page sizes of the study)     */
  int32_t max_blocks_per_seq; /* row stride of block_table, in int32 elements       */
  int64_t k_page_stride;      /* elements between consecutive physical K pages:
                                 B*Hkv*D for a [pages,B,Hkv,D] tensor, 2*B*Hkv*D
                                 for the unbind(1) view of [pages,2,B,Hkv,D]        */
  int64_t v_page_stride;      /* same for the V cache                               */
  int32_t max_seq_len;        /* host-known upper bound on seq_lens (grid planning;
                                 with one sequence the partitions are sized from
                                 it, so a tight bound keeps every CU busy)          */
  int32_t partition_tokens;   /* split-KV partition P: 0 = choose automatically,
                                 else a multiple of 64                              */
  float scale;                /* softmax scale (1/sqrt(256) = 1/16 for D = 256)     */
} pkv_decode_params;

/* What a call with these params will launch (host-only query, no GPU work;
 * the grids are sized for the current device's compute units, 256 when no
 * device can be queried).
 * pkv_decode with partition_tokens == 0 and more than one sequence uses the
 * balanced split: a fixed number of workgroups G share the batch's 64-token
 * tiles evenly, whatever the length mix, and each (sequence, KV head) run of
 * a workgroup's range is one partial. A single sequence (which fixed
 * partitions already split evenly), an explicit partition size, batches of
 * more than 4096 sequences, and pkv_split / pkv_decode_partials /
 * pkv_combine always, use partitions of P tokens. */
typedef struct {
  int32_t partition_tokens;      /* P of the fixed partitions (pkv_split,
                                    pkv_decode_partials; pkv_decode when P != 0) */
  int32_t num_partitions;        /* ceil(max_seq_len / P), at least 1              */
  int32_t split_workgroups;      /* workgroups of pkv_decode's split launch: G, or
                                    S * Hkv * num_partitions                       */
  int32_t combine_workgroups;    /* pkv_decode's combine launch: S * Hq * 4 (one
                                    wave per sequence, head and 64 dims), S * Hkv
                                    for a balanced split of 256 or more (sequence,
                                    KV head) runs (one wave per run), or 0 when one
                                    fixed partition covers every sequence         */
  int32_t balanced;              /* 1 when pkv_decode uses the balanced split      */
  int32_t full_groups_per_page;  /* block_size / 64 (12 for 784, 13 for 832)       */
  int32_t tail_tokens_per_page;  /* block_size % 64 (16 for 784, 0 for 832)        */
  int64_t workspace_bytes;       /* what pkv_decode needs in `workspace`           */
  int32_t k_rows;                /* 1: pkv_decode loads K as whole rows and stages
                                    it through LDS (a batch); 0: straight into the
                                    MFMA operand layout (one sequence)             */
  int32_t ordered;               /* 1: pkv_decode's fixed partitions run in the
                                    ordered dispatch (full partitions first, the
                                    shorter last ones at the end)                  */
} pkv_plan_info;

/* Library version string (static storage). */
PKV_API const char* pkv_version(void);

/* Human-readable name of a pkv_status value (static storage). */
PKV_API const char* pkv_status_string(int status);

/* Validate params and report the launch plan. Host only: launches nothing
 * (it may read the current device's compute-unit count once). Returns the
 * same status pkv_decode would return for these params. */
PKV_API pkv_status pkv_plan(const pkv_decode_params* params, pkv_plan_info* info);

/* Bytes of device workspace pkv_decode needs for these params (0 when one
 * partition covers every sequence, or when params are invalid). The
 * workspace holds fp32 per-partition outputs and log-sum-exps. */
PKV_API size_t pkv_decode_workspace_bytes(const pkv_decode_params* params);

/* Decode attention. Device inputs:
 *   q            bf16 [S, Hq, D], contiguous, 16-byte aligned
 *   key_cache    bf16 pages: page p starts at key_cache + p * k_page_stride and
 *                holds [B, Hkv, D] contiguous; 16-byte aligned
 *   value_cache  same with v_page_stride
 *   block_table  int32 [S, max_blocks_per_seq]
 *   seq_lens     int32 [S]
 * Device outputs:
 *   out          bf16 [S, Hq, D], round-to-nearest-even from fp32
 *   out_f32      fp32 [S, Hq, D] before the cast, or NULL
 * Workspace: device memory of at least pkv_decode_workspace_bytes(params)
 * bytes, 256-byte aligned (may be NULL when that is 0); contents on entry are
 * ignored and clobbered. Launches the split kernel (balanced or fixed
 * partitions, see pkv_plan_info) and, unless one fixed partition covers every
 * sequence, the log-sum-exp combine kernel. */
PKV_API pkv_status pkv_decode(const pkv_decode_params* params, const void* q,
                      const void* key_cache, const void* value_cache,
                      const int32_t* block_table, const int32_t* seq_lens,
                      void* out, float* out_f32, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Same computation with the intermediate fp32 results exposed (for checks):
 *   o_partial   fp32 [S, Hq, num_partitions, D]: partition p of sequence s is
 *               softmax attention over tokens [p*P, min((p+1)*P, L_s)),
 *               written for p < ceil(L_s / P) only
 *   lse_partial fp32 [S, Hq, num_partitions]: natural-log log-sum-exp of the
 *               scaled scores of that partition
 *   out_f32     fp32 [S, Hq, D]: the combined output before the bf16 cast
 *   out         bf16 [S, Hq, D] (may be NULL)
 * num_partitions comes from pkv_plan. Always runs split + combine. */
PKV_API pkv_status pkv_decode_partials(const pkv_decode_params* params, const void* q,
                               const void* key_cache, const void* value_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               float* o_partial, float* lse_partial,
                               float* out_f32, void* out, void* stream);

/* The split-KV partition kernel on its own: writes o_partial / lse_partial
 * (layout as in pkv_decode_partials, P and num_partitions from pkv_plan) for
 * every p < ceil(L_s / P); pkv_split followed by pkv_combine computes what
 * pkv_decode computes. */
PKV_API pkv_status pkv_split(const pkv_decode_params* params, const void* q, const void* key_cache,
                     const void* value_cache, const int32_t* block_table,
                     const int32_t* seq_lens, float* o_partial, float* lse_partial,
                     void* stream);

/* The two launches of pkv_decode when it uses the balanced split
 * (pkv_plan_info.balanced == 1), separately: pkv_split_balanced writes
 * the partials and tile prefix sums into `workspace` (at least
 * pkv_decode_workspace_bytes(params) bytes, 256-byte aligned; the layout is
 * internal), and pkv_combine_balanced turns that workspace into out (bf16,
 * may be NULL) and out_f32 (fp32, may be NULL). Returns PKV_ERR_UNSUPPORTED
 * when these params do not select the balanced split. */
PKV_API pkv_status pkv_split_balanced(const pkv_decode_params* params, const void* q,
                              const void* key_cache, const void* value_cache,
                              const int32_t* block_table, const int32_t* seq_lens,
                              void* workspace, size_t workspace_bytes, void* stream);
PKV_API pkv_status pkv_combine_balanced(const pkv_decode_params* params, const int32_t* seq_lens,
                                const void* workspace, size_t workspace_bytes, void* out,
                                float* out_f32, void* stream);

/* The log-sum-exp combine on its own: merges partitions of size P (from
 * pkv_plan(params)) laid out as in pkv_decode_partials into out (bf16,
 * may be NULL) and out_f32 (may be NULL). */
PKV_API pkv_status pkv_combine(const pkv_decode_params* params, const float* o_partial,
                       const float* lse_partial, const int32_t* seq_lens,
                       void* out, float* out_f32, void* stream);

/* Test/debug: the element offset that the decode kernel's page walker computes
 * for every token of KV head kv_head, through the key-cache geometry
 * (k_page_stride). row_offsets int64 [S, max_seq_len]; entries at t >=
 * seq_lens[s] are set to -1. Runs the split launch pkv_decode would run for
 * these params (balanced or fixed partitions, the same page-list bounds and
 * walker instantiation), recording each block's rows instead of reading them. */
PKV_API pkv_status pkv_debug_resolve(const pkv_decode_params* params, int32_t kv_head,
                             const int32_t* block_table, const int32_t* seq_lens,
                             int64_t* row_offsets, void* stream);

/* Test/debug: copy every valid token row of `cache` (key-cache geometry,
 * k_page_stride) into dense bf16 [S, max_seq_len, Hkv, D] through the split
 * walk pkv_decode would run for these params and its block loaders: which = 0
 * uses the K loader of that plan (the MFMA operand layout for one sequence,
 * whole rows for a batch), 1 the V loader (whole rows). Rows at t >=
 * seq_lens[s] are left untouched. */
PKV_API pkv_status pkv_debug_gather(const pkv_decode_params* params, int32_t which,
                            const void* cache, const int32_t* block_table,
                            const int32_t* seq_lens, void* dense, void* stream);

/* Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Computes exactly what pkv_decode computes, with the same plan
 * and kernels (bit-identical outputs), but takes no workspace: the partials
 * (and the balanced split's tile prefix sums) go to a file-scope device array
 * of PKV_NOALLOC_SCRATCH_BYTES bytes in the library, one per GPU, held from
 * the first call on that GPU until the process ends. The call allocates
 * nothing and needs no zeroed memory (everything it reads there it wrote in
 * the same call). A call whose plan needs more workspace than the array
 * holds (pkv_decode_workspace_bytes(params) > PKV_NOALLOC_SCRATCH_BYTES)
 * returns PKV_ERR_SCRATCH before any GPU call; other errors are pkv_decode's.
 * Every call on one GPU shares that GPU's array: calls that may overlap in
 * time on one GPU (other streams, other host threads) race and must be
 * serialised by the caller; calls on one stream are ordered. */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
PKV_API size_t pkv_noalloc_scratch_bytes(void);
PKV_API pkv_status pkv_decode_noalloc(const pkv_decode_params* params, const void* q,
                              const void* key_cache, const void* value_cache,
                              const int32_t* block_table, const int32_t* seq_lens,
                              void* out, float* out_f32, void* stream);

/* Bandwidth probes (used to calibrate measurements, not part of decode):
 * pkv_probe_read streams `bytes` (multiple of 16, 16-byte aligned) from `buf`
 * and writes one float per workgroup sum into `sink` (device, at least
 * pkv_probe_sink_floats() floats); pkv_probe_copy copies `bytes` (multiple
 * of 16, both 16-byte aligned). */
PKV_API int32_t pkv_probe_sink_floats(void);
PKV_API pkv_status pkv_probe_read(const void* buf, size_t bytes, float* sink, void* stream);
PKV_API pkv_status pkv_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

/* ------------------------------------------------------------------------
 * KV append: write new tokens' K and V rows into the paged caches by slot.
 * A slot names one token row of the cache: page = slot / block_size, offset =
 * slot % block_size ("From Attention to KV Cache Compression: Notes from a
 * KernelGen Optimization", sections "Gather and Scatter" and "How One Output
 * Is Produced"); the row is [num_kv_heads, head_size] inside page `page` of a
 * [pages, block_size, num_kv_heads, head_size] cache ("海光 DCU 上的长上下文
 * Attention：从 page784 到 page832 的 KV Cache 对齐与访存优化", §4). For a token
 * at position t of a sequence, slot = block_table[t / B] * B + t % B (§1).
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t num_tokens;     /* N new tokens (0 is a no-op)                           */
  int32_t num_kv_heads;   /* Hkv                                                   */
  int32_t head_size;      /* D; Hkv * D must be a multiple of 8                    */
  int32_t block_size;     /* tokens per page, > 0                                  */
  int64_t num_pages;      /* pages in each cache; slots >= num_pages * block_size
                             are outside the cache and write nothing               */
  int64_t k_page_stride;  /* elements between consecutive K pages (>= B*Hkv*D)     */
  int64_t v_page_stride;  /* same for V (2*B*Hkv*D for the unbind view)            */
  int64_t k_new_stride;   /* elements between consecutive new K rows (>= Hkv*D),
                             e.g. the K slice of a fused QKV projection output      */
  int64_t v_new_stride;   /* same for the new V rows                               */
} pkv_append_params;

/* Device inputs: k_new, v_new bf16 rows [N][Hkv*D] at the given row strides;
 * slot_mapping int64 [N]. A negative slot marks a padding token and writes
 * nothing. Non-negative slots must be distinct (two tokens aimed at one slot
 * leave either row there). Device outputs: key_cache / value_cache rows at
 * the slots, byte-exact copies. All pointers 16-byte aligned (slot_mapping
 * 8-byte), strides multiples of 8 elements. Asynchronous on `stream`;
 * allocates nothing; returns before any launch on a bad argument. */
PKV_API pkv_status pkv_append(const pkv_append_params* params, const void* k_new,
                              const void* v_new, const int64_t* slot_mapping, void* key_cache,
                              void* value_cache, void* stream);

/* Page-size rule ("海光 DCU 上的长上下文 Attention：从 page784 到 page832 的 KV Cache
 * 对齐与访存优化", §3): the tokens per page that hold one state page of
 * `state_page_bytes`, rounded up to a multiple of `alignment_tokens`:
 * ceil(state_page_bytes / (alignment_tokens * attn_bytes_per_token)) *
 * alignment_tokens. Host only. Returns -1 for a non-positive argument or a
 * result beyond INT32_MAX. */
PKV_API int32_t pkv_page_tokens(int64_t state_page_bytes, int64_t attn_bytes_per_token,
                                int32_t alignment_tokens);

/* ------------------------------------------------------------------------
 * Tail-Q chunked prefill of one sequence ("海光 DCU 上的长上下文 Attention：从
 * page784 到 page832 的 KV Cache 对齐与访存优化", §6): the num_q_tokens new
 * tokens are the last num_q_tokens of the sequence's seq_len cached tokens
 * (their K/V rows are already in the cache, e.g. written by pkv_append).
 * Query i sits at position seq_len - num_q_tokens + i and attends every key
 * t <= that position (causal), query head h reading KV head h / 6:
 * o = softmax(scale * q.K^T) . V ("From Attention to KV Cache Compression:
 * Notes from a KernelGen Optimization", "Starting from Attention").
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t num_q_tokens;       /* Q >= 1 new tokens (the pages route Q = 1 to decode;
                                 it is accepted here too)                          */
  int32_t num_q_heads;        /* Hq = 6 * Hkv                                      */
  int32_t num_kv_heads;       /* Hkv                                               */
  int32_t head_size;          /* 256                                               */
  int32_t block_size;         /* B tokens per page, > 0 (any size: rows are looked
                                 up one by one)                                    */
  int32_t max_blocks;         /* entries of block_table                            */
  int64_t k_page_stride;      /* elements between K pages (>= B*Hkv*D)             */
  int64_t v_page_stride;      /* same for V                                        */
  int32_t seq_len;            /* L: cached tokens incl. the new ones,
                                 Q <= L <= max_blocks * B                          */
  float scale;                /* softmax scale (1/16 for D = 256)                  */
  int32_t key_splits;         /* 0: chosen by the library (pkv_prefill_key_splits);
                                 1..64: each query block's keys cut into this many
                                 ranges, merged by a second kernel (split-KV, the
                                 same log-sum-exp merge as decode's partitions)    */
} pkv_prefill_params;

/* The key splits a pkv_prefill call with these params makes per query block
 * (the most; see below), or a negative pkv_status for invalid params. Host
 * only. With key_splits = 0: one split while the launch has two or more
 * workgroups per CU (128 queries x 1 head per workgroup, 256 CUs); else the
 * smallest count S that gives three, at most 16, keeping every split of the
 * shortest query block at 16 or more 64-key tiles; and then, if giving the n
 * shortest query blocks S - 1 splits (for some n below the block count) makes
 * the workgroups a whole number of rounds over the CUs, the fewest such n
 * blocks take S - 1. A caller's key_splits applies to every block. */
PKV_API int32_t pkv_prefill_key_splits(const pkv_prefill_params* params);
/* How many of the shortest query blocks take one key split fewer than
 * pkv_prefill_key_splits in a pkv_prefill call with these params (0 when all
 * take the same count), or a negative pkv_status for invalid params. Host
 * only. */
PKV_API int32_t pkv_prefill_short_blocks(const pkv_prefill_params* params);
/* Workspace pkv_prefill needs: 0 for one split, else splits * Q * Hq * (D + 1)
 * * 4 bytes (fp32 partials and their log-sum-exps). 0 for invalid params. */
PKV_API size_t pkv_prefill_workspace_bytes(const pkv_prefill_params* params);

/* Device inputs: q bf16 [Q, Hq, D] contiguous; key_cache / value_cache as for
 * pkv_decode; block_table int32 [max_blocks] (this sequence's row). Device
 * outputs: out bf16 [Q, Hq, D] (RNE from fp32), out_f32 fp32 [Q, Hq, D] or
 * NULL (at least one of the two). p is rounded to bf16 for the P.V product
 * (fp32 accumulation). workspace: caller-owned device memory of at least
 * pkv_prefill_workspace_bytes(params) bytes, 16-byte aligned (may be NULL
 * when that is 0); its contents need no initialization and are scratch after
 * the call. 16-byte aligned pointers; asynchronous on `stream`; allocates
 * nothing; host checks return an error before any launch (PKV_ERR_PARTITION
 * for key_splits outside 0..64, PKV_ERR_WORKSPACE for a missing or short
 * workspace). */
PKV_API pkv_status pkv_prefill(const pkv_prefill_params* params, const void* q,
                               const void* key_cache, const void* value_cache,
                               const int32_t* block_table, void* out, float* out_f32,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Paged window compression ("From Attention to KV Cache Compression: Notes
 * from a KernelGen Optimization", "The Compression Operator", "How One Output
 * Is Produced"): for every boundary token b, with request r = token_to_req[b]
 * and position p = positions[b], the window is positions t = p - C + 1 .. p of
 * request r (cut at 0; the page's workloads have p >= C - 1). Position t reads
 * state row o = t % B of block block_table[r, t / B]; its first D = 512 floats
 * are values v_t and the next 512 scores s_t. The output, per dimension d:
 *   compressed[n, d] = sum_t softmax_t(s_{t,d}) v_{t,d}   (over the window).
 * A dimension whose window scores are all -inf gives 0. The page's finalizer
 * (RMSNorm, INT8 quantisation, RoPE, byte scatter) is pkv_compress_finalize.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t num_outputs;     /* N boundary tokens (0 is a no-op)                     */
  int32_t num_tokens;      /* T entries of token_to_req and positions (>= 1 when
                              N > 0)                                               */
  int32_t num_reqs;        /* R rows of block_table                                */
  int32_t max_blocks;      /* entries per block_table row; max_blocks * B must not
                              exceed INT32_MAX                                     */
  int32_t head_dim;        /* D: 512 (a state row holds 2 D floats)               */
  int32_t block_size;      /* B state rows per block, > 0 (8 on the page)          */
  int32_t compress_ratio;  /* C window length, >= 1 (128, 256, 512 on the page)    */
  int32_t num_splits;      /* 0: the library chooses; else S window parts per
                              output, 1 <= S <= min(C, 64), each touching at most
                              64 blocks (ceil((ceil(C/S) - 1) / B) + 1 <= 64)      */
  int64_t block_stride;    /* elements between state blocks (>= B * row_stride)    */
  int64_t row_stride;      /* elements between rows of a block (>= 2 D), multiple
                              of 4                                                 */
} pkv_compress_params;

/* Window parts per output the library would use (num_splits resolved), or a
 * negative pkv_status for invalid params. Host only. With num_splits = 0: the
 * smallest power of two giving num_outputs * S >= 256 workgroups (one per CU)
 * while parts keep 16 or more rows, raised as needed to the 64-block limit. */
PKV_API int32_t pkv_compress_splits(const pkv_compress_params* params);

/* Device workspace bytes pkv_compress needs (0 when one part covers each
 * window; else N * S * D * 8 bytes of fp32 partials). Host only; 0 for invalid
 * params. */
PKV_API size_t pkv_compress_workspace_bytes(const pkv_compress_params* params);

/* Device inputs: state_cache fp32 at the given strides (16-byte aligned);
 * token_to_req int32 [T]; positions int64 [T]; boundary_token_indices int64
 * [N]; block_table int32 [R, max_blocks]. Device output: compressed fp32
 * [N, D] (16-byte aligned). Workspace: pkv_compress_workspace_bytes(params)
 * bytes, 256-byte aligned, or NULL when that is 0. A boundary index outside
 * [0, T), a request outside [0, R), a negative position or one whose block
 * lies past max_blocks gives a NaN row and reads nothing else; block-table
 * entries are trusted. Asynchronous on `stream`; allocates nothing; host
 * checks return an error before any launch. */
PKV_API pkv_status pkv_compress(const pkv_compress_params* params, const float* state_cache,
                                const int32_t* token_to_req, const int64_t* positions,
                                const int64_t* boundary_token_indices, const int32_t* block_table,
                                float* compressed, void* workspace, size_t workspace_bytes,
                                void* stream);

/* The compression finalizer ("From Attention to KV Cache Compression: Notes
 * from a KernelGen Optimization", "How One Output Is Produced" and "The
 * Finalizer's Sharp Edges"), applied to pkv_compress's output. For output n
 * with boundary token b, position p = positions[b] and slot =
 * kv_slot_mapping[b]:
 *   y = c * rho * w with rho = (mean(c^2) + eps)^-1/2     (fp32)
 *   dims 0..447: z = bf16(y) read back as fp32; per group g of 64 dims,
 *     a = max(max|z|, 1e-4), e = ceil(log2(a * (1/127))) (exact for the fp32
 *     product), code q = trunc(z * 2^-e) clipped to [-127, 127]
 *   dims 448..511: GPT-J pairs (y[448+2j], y[449+2j]) rotated by cos_j =
 *     cos_sin_cache[pc, j], sin_j = cos_sin_cache[pc, 32 + j], pc = (p / C) * C,
 *     rounded to bf16
 *   KV page slot / 64, slot offset o = slot % 64: bytes o*576 .. +575 get
 *   [448 int8 codes][64 bf16], bytes 64*576 + o*8 .. +7 get [7 x (e + 127)][0].
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t num_outputs;     /* N (0 is a no-op)                                      */
  int32_t num_tokens;      /* T entries of positions and kv_slot_mapping (>= 1 when
                              N > 0)                                                */
  int32_t compress_ratio;  /* C >= 1                                                */
  int32_t cos_sin_rows;    /* rows of cos_sin_cache                                 */
  int64_t num_kv_pages;    /* pages of kv_cache                                     */
  int64_t kv_page_stride;  /* bytes between KV pages: >= 64 * 584, multiple of 16   */
  float rms_norm_eps;      /* eps >= 0, finite (1e-6 on the page)                   */
} pkv_finalize_params;

/* Device inputs: compressed fp32 [N, 512]; positions and kv_slot_mapping int64
 * [T]; boundary_token_indices int64 [N]; rms_norm_weight fp32 [512];
 * cos_sin_cache fp32 [cos_sin_rows, 64]. Device output: kv_cache bytes
 * [num_kv_pages, kv_page_stride]; only the written slots' 576 + 8 bytes
 * change. An output whose boundary index is outside [0, T), whose slot is
 * negative or past the cache, whose position is negative or whose RoPE row is
 * past cos_sin_cache writes nothing; non-finite compressed values give
 * unspecified bytes. Two outputs aimed at one slot leave either's bytes.
 * 16-byte aligned float and byte pointers, 8-byte aligned index pointers.
 * Asynchronous on `stream`; allocates nothing; host checks return an error
 * before any launch. */
PKV_API pkv_status pkv_compress_finalize(const pkv_finalize_params* params,
                                         const float* compressed, const int64_t* positions,
                                         const int64_t* boundary_token_indices,
                                         const float* rms_norm_weight, const float* cos_sin_cache,
                                         const int64_t* kv_slot_mapping, void* kv_cache,
                                         void* stream);

/* The whole compression operator in one call: pkv_compress followed by
 * pkv_compress_finalize ("From Attention to KV Cache Compression: Notes from
 * a KernelGen Optimization", "Our Decomposition": the window reduction, then
 * the packing of its fp32 rows into KV-cache bytes), with the finalizer run
 * inside the last kernel on the row that kernel just merged: one launch when
 * one part covers each window, else the split kernel and a combine that also
 * packs. Arguments are those of the two calls. params and fparams must agree
 * on num_outputs, num_tokens and compress_ratio (else PKV_ERR_SHAPE).
 * `compressed` (fp32 [N, 512], 16-byte aligned) may be NULL; when given it
 * receives exactly what pkv_compress writes. The kv_cache bytes are exactly
 * those of pkv_compress then pkv_compress_finalize: an output with a bad
 * boundary index, request or position packs a NaN row, as it would there, and
 * one whose slot or RoPE row is out of range writes nothing. Workspace as for
 * pkv_compress. Asynchronous on `stream`; allocates nothing; host checks
 * return an error before any launch. */
PKV_API pkv_status pkv_compress_pack(const pkv_compress_params* params,
                                     const pkv_finalize_params* fparams,
                                     const float* state_cache, const int32_t* token_to_req,
                                     const int64_t* positions,
                                     const int64_t* boundary_token_indices,
                                     const int32_t* block_table, const float* rms_norm_weight,
                                     const float* cos_sin_cache, const int64_t* kv_slot_mapping,
                                     void* kv_cache, float* compressed, void* workspace,
                                     size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
