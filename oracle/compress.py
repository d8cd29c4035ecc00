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
  denominator and numerator per dimension, updated tile by tile);
  "The Finalizer's Sharp Edges" and "How One Output Is Produced" again for
  the finalizer: RMSNorm with weight w, the bf16 round trip of the first 448
  dims, a power-of-two scale per group of 64 (exponent byte e + 127), int8
  codes truncated toward zero, GPT-J interleaved RoPE of the last 64 dims at
  the compressed position (p // C) * C stored as bf16, and the slot's payload
  (576 bytes) and scale (8 bytes) inside a 64-slot KV page.

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
* Finalizer dtypes: rms_norm_weight and cos_sin_cache are fp32 (cos in the
  first 32 columns of a row, sin in the next 32, as the page's code reads
  them); the KV cache is bytes [pages, 64 * (576 + 8)].
* The scale exponent is ceil(log2 y) taken exactly for the fp32 value
  y = fl32(a * fl32(1/127)) (see quant_exponent).
* The scale region's pad byte is written as 0; a negative slot, or one past
  the cache, writes nothing.
* The pages compute y = c rho w in fp32 with an unspecified summation order;
  the oracle computes it in fp64, so a byte whose value hinges on the last
  fp32 bits (a bf16 rounding tie within the fp32 error band) may take either
  neighbour. The parity tests accept exactly those, and count them.

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
    "rms_norm",
    "bf16_round",
    "quant_exponent",
    "quantize_nope",
    "rope_gptj",
    "rope_position",
    "slot_byte_offsets",
    "finalize_output",
    "finalize_outputs",
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


# --------------------------------------------------------------------------
# The finalizer: RMSNorm, NOPE INT8 quantisation, GPT-J RoPE and the byte
# scatter into a packed KV page ([Attn→KV notes, "How One Output Is
# Produced", "The Finalizer's Sharp Edges"]).
# --------------------------------------------------------------------------

HEAD_DIM = 512
NOPE_DIM = 448          # first 448 dims: INT8 with a power-of-two scale per 64
ROPE_DIM = 64           # last 64 dims: GPT-J interleaved pairs, stored as bf16
QUANT_GROUP = 64
KV_BLOCK_SIZE = 64      # slots per KV page
TOKEN_STRIDE = 576      # payload bytes per slot: 448 INT8 + 64 bf16
SCALE_DIM = 8           # scale bytes per slot: 7 exponents + 1 pad byte
KV_PAGE_BYTES = KV_BLOCK_SIZE * (TOKEN_STRIDE + SCALE_DIM)


def rms_norm(c, weight, eps):
    """rho = (mean_d c_d^2 + eps)^(-1/2), y_d = c_d rho w_d (fp64)."""
    c = np.asarray(c, dtype=np.float64)
    rho = 1.0 / np.sqrt(np.mean(c * c) + float(eps))
    return c * rho * np.asarray(weight, dtype=np.float64)


def bf16_round(x):
    """fp64 -> the nearest bf16 value (ties to even), as fp64."""
    from .decode import bf16_bits_to_f64, f64_to_bf16_bits
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


def quant_exponent(amax):
    """e = ceil(log2(a / 127)) for a = max(amax, 1e-4), taken exactly for the
    fp32 value y = fl32(a * fl32(1/127)) that the page's fp32 code forms (a
    reading: the page leaves the log2's own rounding open). With
    y = m 2^E, m in [0.5, 1): ceil(log2 y) = E - 1 when m == 0.5, else E."""
    a = max(np.float32(amax), np.float32(1.0e-4))
    y = np.float32(a) * np.float32(1.0 / 127.0)
    m, e = np.frexp(y)
    return int(e) - 1 if m == 0.5 else int(e)


def quantize_nope(y):
    """The first 448 dims of y: z = bf16(y) (the round trip), per group of 64
    a_g = max(max |z|, 1e-4), e_g = quant_exponent(a_g), q = int8(clip(z 2^-e,
    -127, 127)) with the int8 conversion truncating toward zero. Returns
    (q bytes uint8 [448] in two's complement, scale bytes uint8 [7] = e + 127,
    e [7], z [448])."""
    z = bf16_round(np.asarray(y, dtype=np.float64)[:NOPE_DIM])
    groups = NOPE_DIM // QUANT_GROUP
    q = np.zeros(NOPE_DIM, dtype=np.int64)
    e = np.zeros(groups, dtype=np.int64)
    for g in range(groups):
        zg = z[g * QUANT_GROUP:(g + 1) * QUANT_GROUP]
        e[g] = quant_exponent(np.abs(zg).max())
        scaled = zg * 2.0 ** (-int(e[g]))          # exact: a power-of-two scale
        q[g * QUANT_GROUP:(g + 1) * QUANT_GROUP] = np.clip(np.trunc(scaled), -127, 127)
    return (q % 256).astype(np.uint8), (e + 127).astype(np.uint8), e, z


def rope_gptj(y, cos, sin):
    """GPT-J interleaved rotation of the last 64 dims of y: pair j is
    (u, w) = (y[448 + 2j], y[449 + 2j]); u' = u cos_j - w sin_j,
    w' = w cos_j + u sin_j. Returns the 64 rotated values (fp64)."""
    r = np.asarray(y, dtype=np.float64)[NOPE_DIM:NOPE_DIM + ROPE_DIM]
    u, w = r[0::2], r[1::2]
    cos = np.asarray(cos, dtype=np.float64)
    sin = np.asarray(sin, dtype=np.float64)
    out = np.empty(ROPE_DIM)
    out[0::2] = u * cos - w * sin
    out[1::2] = w * cos + u * sin
    return out


def rope_position(p, compress_ratio):
    """The cos/sin cache row of an output whose boundary token sits at
    position p: the compressed position p_c = floor(p / C) * C, the start of
    the C-token chunk holding p ([Attn→KV notes, "How One Output Is
    Produced", the RoPE step])."""
    c = int(compress_ratio)
    return (int(p) // c) * c


def slot_byte_offsets(slot):
    """(page, payload byte offset, scale byte offset) of a KV slot inside its
    page: page = slot // 64, payload at (slot % 64) * 576, scale at
    64 * 576 + (slot % 64) * 8."""
    slot = int(slot)
    page, off = slot // KV_BLOCK_SIZE, slot % KV_BLOCK_SIZE
    return page, off * TOKEN_STRIDE, KV_BLOCK_SIZE * TOKEN_STRIDE + off * SCALE_DIM


def finalize_output(c, weight, eps, cos_sin_row):
    """One output's bytes: (payload uint8 [576], scale uint8 [8]) plus the
    intermediates (y, z, e) that the parity tests use. cos_sin_row is the
    cache row of the compressed position p_c = (p // C) * C: cos in its
    first 32 entries, sin in the next 32."""
    from .decode import f64_to_bf16_bits
    y = rms_norm(c, weight, eps)
    qb, sb, e, z = quantize_nope(y)
    cs = np.asarray(cos_sin_row, dtype=np.float64)
    rot = rope_gptj(y, cs[:ROPE_DIM // 2], cs[ROPE_DIM // 2:ROPE_DIM])
    rope_bits = f64_to_bf16_bits(rot).astype("<u2")
    payload = np.concatenate([qb, rope_bits.view(np.uint8)])
    scale = np.concatenate([sb, np.zeros(1, dtype=np.uint8)])
    return payload, scale, (y, z, e, rot)


def finalize_outputs(compressed, weight, eps, cos_sin_cache, positions, compress_ratio, slots,
                     kv_cache):
    """Write every output's packed bytes into a copy of kv_cache (uint8
    [pages, page_bytes]): payload and scale at the slot's offsets. A negative
    slot, or one past the cache, writes nothing. positions[j] is output j's
    boundary position p; its RoPE row is cos_sin_cache[rope_position(p, C)]."""
    kv = np.array(kv_cache, dtype=np.uint8, copy=True)
    pages = kv.shape[0]
    for j, slot in enumerate(slots):
        slot = int(slot)
        if slot < 0 or slot >= pages * KV_BLOCK_SIZE:
            continue
        pc = rope_position(positions[j], compress_ratio)
        payload, scale, _ = finalize_output(compressed[j], weight, eps, cos_sin_cache[pc])
        page, po, so = slot_byte_offsets(slot)
        kv[page, po:po + TOKEN_STRIDE] = payload
        kv[page, so:so + SCALE_DIM] = scale
    return kv
