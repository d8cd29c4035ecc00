"""Plain fp64 CPU oracle for single-token decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product path.

Sources (cited by page title and section; the pages are web articles):

* [Attn→KV notes] "From Attention to KV Cache Compression: Notes from a
  KernelGen Optimization" -- sections "Starting from Attention" (the
  dot-product attention formula and the decode step), "The KV Cache Bill",
  "How One Output Is Produced" (the paged row map) and "Online Softmax:
  Streaming Away the Window" (the running max / denominator / numerator).
* [DCU page832] "海光 DCU 上的长上下文 Attention：从 page784 到 page832 的
  KV Cache 对齐与访存优化" (long-context attention on Hygon DCU, KV-cache
  alignment from page784 to page832) -- §1 (logical page, page offset and
  physical page of a token), §4 (24 Q heads over 4 KV heads, head size 256,
  the [pages, BLOCK_SIZE, 4, 256] cache after unbind), §5 and §7 (the paged
  decode loop and its online softmax update), §9 (nothing skipped, causal
  range unchanged).

Readings where the pages leave a step open (each is also listed in the
design notes):

* GQA mapping: query head h reads KV head h // G with G = Hq / Hkv (contiguous
  groups); the pages only say "GQA ratio 6".
* Decode attends to every cached token t < seq_len of its own sequence (the
  current token's K/V is already in the cache); no window, ALiBi, sinks or
  softcap.
* seq_len == 0 gives a zero output row and lse = -inf.
* The softmax scale is a parameter (1/sqrt(d) in the formula; every workload
  here uses 1/16 for d = 256).
* bf16 rounding is round-to-nearest-even, taken directly from fp64.

Parity status: every function below is pinned by ``tests/test_oracle_pins.py``
against closed forms, brute force at high precision, an independent library
routine, hand-derived address fixtures or algebraic identities.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "attention_decode",
    "decode_batch",
    "decode_partials",
    "combine_partials",
    "online_decode",
    "resolve_offsets",
    "gather_rows",
    "bf16_bits_to_f64",
    "f64_to_bf16_bits",
]


# --------------------------------------------------------------------------
# bf16 <-> fp64
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly.

    A bf16 value is the upper half of an IEEE binary32 word, so widening the
    bits by 16 zero bits gives the same number as a float32, which float64
    holds exactly.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """float64 -> bf16 bits by round-to-nearest, ties-to-even, in one step.

    bf16 keeps 8 significant bits, exponent range of binary32 (normal down to
    2^-126, subnormal spacing 2^-133). The value is scaled by a power of two so
    that one unit in the last bf16 place becomes 1.0, rounded with ``rint``
    (ties to even), and scaled back; every step is exact in fp64. Results of
    2^128 or more overflow to infinity. NaN maps to the canonical 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    sign = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(x)
    inf = np.isinf(x)
    fin = ~(nan | inf) & (a > 0)
    if np.any(fin):
        af = a[fin]
        _, e2 = np.frexp(af)              # af = f * 2**e2, f in [0.5, 1)
        e = e2.astype(np.int64) - 1       # af in [2**e, 2**(e+1))
        ulp_exp = np.maximum(e, -126) - 7
        r = np.ldexp(np.rint(np.ldexp(af, -ulp_exp)), ulp_exp)
        over = r >= 2.0 ** 128
        r32 = np.where(over, 0.0, r).astype(np.float32)   # exact: 8 significant bits
        hi = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        hi[over] = 0x7F80
        out[fin] = hi
    out[inf] = 0x7F80
    out[nan] = 0x7FC0
    out = np.where(sign & ~nan, out | np.uint16(0x8000), out).astype(np.uint16)
    return out


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def attention_decode(q, keys, values, scale):
    """One query token per head attending to every cached token of a sequence.

    [Attn→KV notes, "Starting from Attention"]: o = sum_j a_j v_j with
    a_j = exp(s_j) / sum_k exp(s_k) and s_j = q.k_j * scale; the decode step
    attends to all cached tokens. Written two-pass: the maximum score first,
    then the weights, their sum and the weighted sum of values, all in fp64.

    q:      [Hq, D] float64
    keys:   [L, Hkv, D] float64 (logical, unpaged)
    values: [L, Hkv, D] float64
    returns (o [Hq, D], lse [Hq]) with lse = m + ln(sum_t exp(s_t - m)).
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    hq, d = q.shape
    length, hkv, dk = keys.shape
    assert dk == d and values.shape == keys.shape and hq % hkv == 0
    group = hq // hkv
    o = np.zeros((hq, d), dtype=np.float64)
    lse = np.full((hq,), -np.inf, dtype=np.float64)
    if length == 0:
        return o, lse
    for h in range(hq):
        g = h // group                                   # GQA: contiguous groups
        s = scale * (keys[:, g, :] @ q[h])               # [L]
        m = np.max(s)                                    # pass 1
        w = np.exp(s - m)                                # pass 2
        l_sum = np.sum(w)
        o[h] = (w @ values[:, g, :]) / l_sum
        lse[h] = m + np.log(l_sum)
    return o, lse


def decode_batch(q, keys_list, values_list, scale):
    """Batched decode: sequence s uses only its own cached tokens.

    [DCU page832, §9]: no cross-request KV reuse and no tokens skipped.
    q: [S, Hq, D]; keys_list[s], values_list[s]: [L_s, Hkv, D].
    returns (o [S, Hq, D], lse [S, Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    n = q.shape[0]
    o = np.zeros(q.shape, dtype=np.float64)
    lse = np.zeros(q.shape[:2], dtype=np.float64)
    for s in range(n):
        o[s], lse[s] = attention_decode(q[s], keys_list[s], values_list[s], scale)
    return o, lse


def decode_partials(q, keys, values, scale, partition_tokens):
    """Attention restricted to consecutive token partitions of one sequence.

    Partition p covers tokens [p*P, min((p+1)*P, L)); each partition's
    (o_p, lse_p) is ``attention_decode`` on that slice. (Split-KV is not on
    the pages; this is the plain restriction of the definition to a slice.)
    returns (o_p [Hq, n, D], lse_p [Hq, n]) with n = ceil(L / P).
    """
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    length = keys.shape[0]
    p_tok = int(partition_tokens)
    n = -(-length // p_tok)
    hq, d = q.shape
    o_p = np.zeros((hq, n, d), dtype=np.float64)
    lse_p = np.zeros((hq, n), dtype=np.float64)
    for p in range(n):
        lo, hi = p * p_tok, min((p + 1) * p_tok, length)
        o_p[:, p, :], lse_p[:, p] = attention_decode(q, keys[lo:hi], values[lo:hi], scale)
    return o_p, lse_p


def combine_partials(o_p, lse_p):
    """Merge per-partition results by their log-sum-exp weights.

    Splitting the token sum of the softmax into partitions gives
    sum_t exp(s_t) v_t = sum_p exp(lse_p) o_p and sum_t exp(s_t) = sum_p exp(lse_p),
    so o = sum_p exp(lse_p - M) o_p / sum_p exp(lse_p - M) for any shift M
    (the maximum is used) and lse = M + ln(sum_p exp(lse_p - M)).
    o_p: [Hq, n, D], lse_p: [Hq, n] -> (o [Hq, D], lse [Hq]).
    """
    o_p = np.asarray(o_p, dtype=np.float64)
    lse_p = np.asarray(lse_p, dtype=np.float64)
    hq, n, d = o_p.shape
    if n == 0:
        return np.zeros((hq, d)), np.full((hq,), -np.inf)
    m = np.max(lse_p, axis=1, keepdims=True)
    w = np.exp(lse_p - m)                                # [Hq, n]
    den = np.sum(w, axis=1)
    o = np.einsum("hn,hnd->hd", w, o_p) / den[:, None]
    return o, m[:, 0] + np.log(den)


def online_decode(q, keys, values, scale, tile):
    """The streaming form: one pass over token tiles with a running state.

    [Attn→KV notes, "Online Softmax: Streaming Away the Window"] keeps the
    current maximum m, the denominator den and the numerator num; for each
    tile: m' = max(m, max(scores)), old = exp(m - m'), w = exp(scores - m'),
    num' = num * old + sum(w * v), den' = den * old + sum(w); the result is
    num / den. [DCU page832, §5, §7] apply the same update per 64-token tile
    of the paged decode loop. Here the score is per token (shared by all
    dimensions of a head), so m and den are per head and num is a vector.
    returns (o [Hq, D], lse [Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    hq, d = q.shape
    length, hkv, _ = keys.shape
    group = hq // hkv
    o = np.zeros((hq, d))
    lse = np.full((hq,), -np.inf)
    if length == 0:
        return o, lse
    for h in range(hq):
        g = h // group
        m, den, num = -np.inf, 0.0, np.zeros(d)
        for t0 in range(0, length, tile):
            k_t = keys[t0:t0 + tile, g, :]
            v_t = values[t0:t0 + tile, g, :]
            scores = scale * (k_t @ q[h])
            m_next = max(m, float(np.max(scores)))
            old = np.exp(m - m_next)
            w = np.exp(scores - m_next)
            num = num * old + w @ v_t
            den = den * old + float(np.sum(w))
            m = m_next
        o[h] = num / den
        lse[h] = m + np.log(den)
    return o, lse


# --------------------------------------------------------------------------
# paged addressing
# --------------------------------------------------------------------------

def resolve_offsets(block_table, seq_lens, block_size, page_stride, kv_heads,
                    head_size, kv_head, max_len):
    """Element offset of every cached token's row for one KV head.

    [DCU page832, §1]: logical_page = t // BLOCK_SIZE, page_offset =
    t % BLOCK_SIZE, physical_page = block_table[logical_page], then the cache
    strides. [DCU page832, §4]: one K (or V) cache is [pages, BLOCK_SIZE,
    Hkv, D], so the row of (page, offset, head) starts at
    physical_page * page_stride + page_offset * Hkv * D + kv_head * D
    (page_stride = BLOCK_SIZE * Hkv * D when contiguous, twice that for the
    unbind view of a joint K/V tensor).

    returns int64 [S, max_len]; entries at t >= seq_len are -1.
    """
    bt = np.asarray(block_table, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    out = np.full((bt.shape[0], int(max_len)), -1, dtype=np.int64)
    for s in range(bt.shape[0]):
        t = np.arange(int(lens[s]), dtype=np.int64)
        logical_page = t // block_size
        page_offset = t % block_size
        physical_page = bt[s, logical_page]
        out[s, : t.size] = (physical_page * int(page_stride)
                            + page_offset * (kv_heads * head_size)
                            + kv_head * head_size)
    return out


def gather_rows(pool, block_table, seq_lens, block_size):
    """Read back every sequence's cached rows through its block table.

    pool: [pages, BLOCK_SIZE, Hkv, D] (any dtype; bf16 bits as uint16 for
    bit-exact checks). Token t of sequence s lives at
    pool[block_table[s, t // B], t % B] ([DCU page832, §1]).
    returns a list of [L_s, Hkv, D] arrays.
    """
    pool = np.asarray(pool)
    bt = np.asarray(block_table, dtype=np.int64)
    out = []
    for s, length in enumerate(np.asarray(seq_lens, dtype=np.int64)):
        t = np.arange(int(length), dtype=np.int64)
        out.append(pool[bt[s, t // block_size], t % block_size])
    return out
