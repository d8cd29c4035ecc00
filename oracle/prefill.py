"""Plain fp64 CPU oracle for tail-Q chunked prefill over a paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and ``bench.py``'s
``cpu_baseline`` leg, never by the product path.

Sources (cited by page title and section):

* [DCU page832] "海光 DCU 上的长上下文 Attention：从 page784 到 page832 的
  KV Cache 对齐与访存优化" -- §6 (the Tail-Q prefill shape: one sequence,
  1 < q <= 4096 new tokens, causal decoder attention, bf16, 24 Q heads over
  4 KV heads of size 256, page 832, no sliding window, ALiBi, sinks or
  softcap; the call takes the query tokens, the paged K/V, the used key
  length and the block table), §5 (the causal range is kept whole), §9
  (nothing skipped).
* [Attn→KV notes] "From Attention to KV Cache Compression: Notes from a
  KernelGen Optimization" -- "Starting from Attention" (o = softmax(q.K^T *
  scale) . V over the keys a query may see).

Readings where the pages leave a step open (also listed in the design notes):

* The q new tokens are the last q of the sequence's L cached tokens (their
  K/V rows are already in the cache): query i sits at position L - q + i and
  sees keys 0 .. L - q + i (bottom-right causal alignment).
* GQA: query head h reads KV head h // (Hq / Hkv), as for decode.
* The scale is a parameter (1/16 for head size 256 in every workload).
* q = 1 is the decode step; the pages route it elsewhere, but the
  definition covers it and the oracle accepts it.

Parity status: pinned by ``tests/test_oracle_prefill_pins.py`` against the
decode oracle row by row (each query is a decode over its causal prefix),
torch's fp64 scaled-dot-product attention with an explicit mask, a 50-digit
brute force on tiny inputs, the q = 1 reduction and planted mistakes.
"""

from __future__ import annotations

import numpy as np

__all__ = ["query_positions", "attention_prefill"]


def query_positions(num_q, seq_len):
    """Position of each new token: the last num_q of seq_len ([DCU page832, §6])."""
    if not 1 <= num_q <= seq_len:
        raise ValueError("need 1 <= num_q <= seq_len")
    return np.arange(seq_len - num_q, seq_len, dtype=np.int64)


def attention_prefill(q, keys, values, scale, rows=None, block=256):
    """Causal attention of the new tokens over the whole cached sequence.

    q:      [Q, Hq, D] float64 (the new tokens' queries)
    keys:   [L, Hkv, D] float64 (logical, unpaged; the new tokens' rows last)
    values: [L, Hkv, D] float64
    rows:   optional iterable of query indices to compute (others stay 0)
    returns (o [Q, Hq, D], lse [Q, Hq]).

    For query i at position p = L - Q + i and head h (KV head g = h // G):
    s_t = scale * q[i,h] . K[t,g] for t <= p, o = sum_t softmax(s)_t V[t,g],
    lse = max s + ln sum exp(s - max s), two passes in fp64. Queries are taken
    in blocks of `block` rows with the causal limit as an explicit mask.
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    nq, hq, d = q.shape
    length, hkv, dk = keys.shape
    assert dk == d and values.shape == keys.shape and hq % hkv == 0
    group = hq // hkv
    pos = query_positions(nq, length)
    sel = np.arange(nq) if rows is None else np.asarray(sorted(set(int(r) for r in rows)))
    o = np.zeros((nq, hq, d), dtype=np.float64)
    lse = np.zeros((nq, hq), dtype=np.float64)
    t = np.arange(length, dtype=np.int64)
    for b0 in range(0, sel.size, block):
        idx = sel[b0:b0 + block]
        visible = t[None, :] <= pos[idx][:, None]                  # [b, L] causal mask
        for h in range(hq):
            g = h // group
            s = scale * (q[idx, h, :] @ keys[:, g, :].T)           # [b, L]
            s = np.where(visible, s, -np.inf)
            m = np.max(s, axis=1, keepdims=True)                    # pass 1
            w = np.exp(s - m)                                       # pass 2 (0 where masked)
            l_sum = np.sum(w, axis=1, keepdims=True)
            o[idx, h, :] = (w @ values[:, g, :]) / l_sum
            lse[idx, h] = m[:, 0] + np.log(l_sum[:, 0])
    return o, lse
