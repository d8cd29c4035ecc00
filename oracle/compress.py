"""Plain fp64 CPU oracle for the paged window compression stage: for each
boundary token, a per-dimension softmax over the window of state rows before
it, weighted over the values.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and ``bench.py``'s
``cpu_baseline`` leg, never by the product path.

Sources (cited by page title and section):

* [Attn→KV notes] "From Attention to KV Cache Compression: Notes from a
  KernelGen Optimization" --
  "Competition Background and Problem Statement" (the 12 shapes: num_reqs,
  total_tokens and compress ratio C in {128, 256, 512});
  "The Compression Operator" (every boundary token compresses the window of
  C tokens that ends at it);
  "Gather and Scatter" (request id, position and block table locate the
  window's state rows);
  "How One Output Is Produced" (the window positions, the block-table row
  map with B = 8, values in the first D = 512 columns of a state row and
  scores in the next 512, and the per-dimension softmax over the window
  followed by the weighted sum);
  "The Baseline" (the state cache is float: one C = 512 window moves about
  2 MiB);
  "Online Softmax: Streaming Away the Window" (the running maximum,
  denominator and numerator per dimension, updated tile by tile).

Readings where the pages leave a step open (also listed in the design notes):

* The state cache holds fp32 rows [values(D) | scores(D)]; the output
  ``compressed`` is fp32 [N, D].
* The window of a boundary token at position p is positions p - C + 1 .. p
  of its own request. Positions below 0 do not exist: the window is cut at
  the request's start (the pages' workloads always have p >= C - 1, where
  this never applies).
* The block table maps every window position's logical block to a physical
  block; consecutive logical blocks need not be physically consecutive (the
  page's shortcut of deriving later blocks from the first one relies on how
  its benchmark allocates blocks, and is not assumed here).
* A dimension whose window scores are all -inf gives 0 (no finite weight);
  with any finite score the usual softmax applies and -inf scores get weight
  exactly 0.

Parity status: pinned by ``tests/test_oracle_compress_pins.py`` against
closed forms (equal scores give the window mean; a single finite score per
dimension selects that row exactly; C = 1 returns the row), a 40-digit
brute force on tiny windows, torch's fp64 softmax as an independent library
routine, the online recurrence of the page, the split/combine identity,
hand-derived row fixtures (``tests/golden/compress_rows.txt``), invariance
under score shifts, dimension permutations and physical block shuffles, and
planted mistakes.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "window_positions",
    "window_rows",
    "gather_window",
    "compress_window",
    "compress_outputs",
    "online_compress_window",
    "window_partials",
    "combine_window_partials",
]


def window_positions(p, compress_ratio):
    """[Attn→KV notes, "How One Output Is Produced"]: t_i = p - C + 1 + i for
    0 <= i < C, cut at position 0 (reading above)."""
    p, c = int(p), int(compress_ratio)
    if c < 1 or p < 0:
        raise ValueError("need C >= 1 and p >= 0")
    return np.arange(max(p - c + 1, 0), p + 1, dtype=np.int64)


def window_rows(block_table_row, positions, block_size):
    """Physical state rows of the given positions of one request
    ([Attn→KV notes, "How One Output Is Produced"]): logical block
    l = t // B, offset o = t % B, physical block g = block_table[r, l],
    row = g * B + o."""
    bsz = int(block_size)
    rows = []
    for t in positions:
        t = int(t)
        lb, off = t // bsz, t % bsz
        g = int(block_table_row[lb])
        rows.append(g * bsz + off)
    return np.asarray(rows, dtype=np.int64)


def gather_window(state_cache, block_table_row, p, compress_ratio, block_size):
    """The window's rows of a paged state cache [num_blocks, B, 2D], in window
    order: [n, 2D] (n = C unless the window is cut at 0)."""
    flat = np.asarray(state_cache).reshape(-1, np.asarray(state_cache).shape[-1])
    rows = window_rows(block_table_row, window_positions(p, compress_ratio), block_size)
    return flat[rows]


def compress_window(rows, head_dim=512):
    """[Attn→KV notes, "How One Output Is Produced"]: rows [n, 2D] holding
    values v (first D columns) and scores s (next D). For every dimension d,
    alpha_{i,d} = exp(s_{i,d}) / sum_j exp(s_{j,d}) over the window, and
    c_d = sum_i alpha_{i,d} v_{i,d}. Two passes in fp64 (the maximum first,
    then the shifted exponentials). Returns (c [D], lse [D]) with
    lse_d = ln sum_i exp(s_{i,d}) (-inf where every score is -inf, c = 0)."""
    rows = np.asarray(rows, dtype=np.float64)
    d = int(head_dim)
    v = rows[:, :d]
    s = rows[:, d:2 * d]
    c = np.zeros(d)
    lse = np.full(d, -np.inf)
    if rows.shape[0] == 0:
        return c, lse
    m = s.max(axis=0)
    live = np.isfinite(m)
    with np.errstate(invalid="ignore"):
        w = np.where(live[None, :], np.exp(s - np.where(live, m, 0.0)[None, :]), 0.0)
    den = w.sum(axis=0)
    num = (w * v).sum(axis=0)
    c[live] = num[live] / den[live]
    lse[live] = m[live] + np.log(den[live])
    return c, lse


def compress_outputs(states, token_to_req, positions, boundary_token_indices,
                     compress_ratio, head_dim=512):
    """Every output of the stage from logical (unpaged) per-request state rows.

    states: list of [len_r, 2D] float64 arrays (request r's rows by position)
    token_to_req, positions: per-token request id and position
    boundary_token_indices: the tokens that produce an output
    returns (compressed [N, D], lse [N, D])."""
    n = len(boundary_token_indices)
    out = np.zeros((n, int(head_dim)))
    lse = np.zeros((n, int(head_dim)))
    for j, b in enumerate(boundary_token_indices):
        r = int(token_to_req[int(b)])
        p = int(positions[int(b)])
        t = window_positions(p, compress_ratio)
        out[j], lse[j] = compress_window(np.asarray(states[r])[t], head_dim)
    return out, lse


def online_compress_window(rows, tile, head_dim=512):
    """[Attn→KV notes, "Online Softmax: Streaming Away the Window"]: the same
    result streamed over tiles of `tile` rows. Per dimension: m' = max(m,
    tile max), old = exp(m - m'), w = exp(s - m'), num' = num * old +
    sum(w * v), den' = den * old + sum(w); finally c = num / den."""
    rows = np.asarray(rows, dtype=np.float64)
    d = int(head_dim)
    m = np.full(d, -np.inf)
    den = np.zeros(d)
    num = np.zeros(d)
    for start in range(0, rows.shape[0], int(tile)):
        v = rows[start:start + tile, :d]
        s = rows[start:start + tile, d:2 * d]
        m_next = np.maximum(m, s.max(axis=0))
        live = np.isfinite(m_next)
        safe = np.where(live, m_next, 0.0)
        with np.errstate(invalid="ignore"):
            old = np.where(live, np.exp(m - safe), 1.0)
            w = np.where(live[None, :], np.exp(s - safe[None, :]), 0.0)
        num = num * old + (w * v).sum(axis=0)
        den = den * old + w.sum(axis=0)
        m = m_next
    c = np.zeros(d)
    live = den > 0
    c[live] = num[live] / den[live]
    return c


def window_partials(rows, rows_per_part, head_dim=512):
    """Split the window into consecutive parts of `rows_per_part` rows and
    compress each on its own: returns (c_p [P, D], lse_p [P, D])."""
    rows = np.asarray(rows, dtype=np.float64)
    parts = [rows[i:i + rows_per_part] for i in range(0, rows.shape[0], int(rows_per_part))]
    cs, ls = zip(*(compress_window(p, head_dim) for p in parts)) if parts else ((), ())
    return np.asarray(cs), np.asarray(ls)


def combine_window_partials(c_p, lse_p):
    """Merge per-part results: LSE = ln sum_p exp(lse_p) (max-shifted) and
    c = sum_p exp(lse_p - LSE) c_p, per dimension."""
    c_p = np.asarray(c_p, dtype=np.float64)
    lse_p = np.asarray(lse_p, dtype=np.float64)
    top = lse_p.max(axis=0)
    live = np.isfinite(top)
    safe = np.where(live, top, 0.0)
    with np.errstate(invalid="ignore"):
        w = np.where(live[None, :], np.exp(lse_p - safe[None, :]), 0.0)
    tot = w.sum(axis=0)
    c = np.zeros(c_p.shape[1])
    c[live] = (w * c_p).sum(axis=0)[live] / tot[live]
    lse = np.full(c_p.shape[1], -np.inf)
    lse[live] = top[live] + np.log(tot[live])
    return c, lse
