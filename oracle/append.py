"""Plain CPU oracle for the two steps either side of paged decode: writing new
tokens' K/V rows into the paged cache, and the page-size rule.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and ``bench.py``'s
``cpu_baseline`` leg, never by the product path.

Sources (cited by page title and section):

* [Attn→KV notes] "From Attention to KV Cache Compression: Notes from a
  KernelGen Optimization" -- "Gather and Scatter" (scatter writes computed
  rows back into the paged KV cache at their target slot) and "How One
  Output Is Produced" (a slot splits into page = slot // block size and
  offset = slot % block size).
* [DCU page832] "海光 DCU 上的长上下文 Attention：从 page784 到 page832 的
  KV Cache 对齐与访存优化" -- §1 (token t of a sequence lives at page
  block_table[t // B], offset t % B), §4 (one cache is [pages, B, Hkv, D]:
  a token row holds every KV head), §3 (the page size is the state page
  divided by alignment x per-token attention bytes, rounded up, times the
  alignment; alignment 16 gives 784 and alignment 64 gives 832 on the
  page's shape).

Readings where the pages leave a step open (also listed in the design notes):

* A negative slot marks a padding token: nothing is written for it.
* A slot at or past pages * B is outside the cache: nothing is written (a
  device kernel has no cheap way to raise an error).
* Non-negative slots are distinct; two tokens aimed at one slot are a caller
  error (this oracle would keep the later one; the GPU order is undefined).
* The page-size rule is the bare formula; the page says it leaves out a
  minimum comparison and a later padding branch of the full configuration
  logic, and so does this.

Parity status: pinned by ``tests/test_oracle_append_pins.py`` (hand-derived
slot fixtures, a scatter-then-gather round trip through the decode oracle's
independent address map, the page's 784/832 outcome, closed forms of the
rounding, and planted mistakes).
"""

from __future__ import annotations

import numpy as np

__all__ = ["split_slot", "slots_for_positions", "append_rows", "page_tokens"]


def split_slot(slot, block_size):
    """[Attn→KV notes, "How One Output Is Produced"]: (page, offset) of a slot."""
    slot = int(slot)
    return slot // int(block_size), slot % int(block_size)


def slots_for_positions(block_table_row, positions, block_size):
    """Slot of each token position of one sequence.

    [DCU page832, §1]: position t is at page block_table[t // B], offset
    t % B, i.e. slot = block_table[t // B] * B + t % B.
    """
    bt = np.asarray(block_table_row, dtype=np.int64)
    t = np.asarray(positions, dtype=np.int64)
    return bt[t // block_size] * block_size + t % block_size


def append_rows(pool, new_rows, slots, block_size):
    """Scatter new token rows into a paged cache ([Attn→KV notes, "Gather and
    Scatter"]); returns a new pool, the input is left unchanged.

    pool:     [pages, B, Hkv, D] (any dtype; bf16 bits as uint16 for exact checks)
    new_rows: [N, Hkv, D], row b is written at slot slots[b]
    slots:    [N] integers; negative = padding, >= pages * B = outside
    """
    out = np.array(pool, copy=True)
    rows = np.asarray(new_rows)
    pages = out.shape[0]
    for b, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        if slot < 0 or slot >= pages * block_size:
            continue
        page, offset = split_slot(slot, block_size)
        out[page, offset] = rows[b]
    return out


def page_tokens(state_page_bytes, attn_bytes_per_token, alignment_tokens):
    """[DCU page832, §3]: tokens per page that hold one state page, rounded up
    to a multiple of the alignment:
    ceil(state_page_bytes / (alignment_tokens * attn_bytes_per_token)) * alignment_tokens.
    Exact integer arithmetic; returns -1 for a non-positive argument."""
    s, a, k = int(state_page_bytes), int(attn_bytes_per_token), int(alignment_tokens)
    if s <= 0 or a <= 0 or k <= 0:
        return -1
    unit = k * a
    return -(-s // unit) * k
