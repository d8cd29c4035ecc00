"""Seeded synthetic inputs for paged single-token decode attention.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic and none of the kernels' address code. It serves both the
HIP path (as device tensors) and the CPU oracle (whose inputs are the logical,
unpaged K/V drawn here).

Recipe (fixed draw order on one ``torch.Generator`` seeded per workload):
  1. seq_lens (when the workload draws them),
  2. q [S, 24, 256], 3. logical K [sum L, 4, 256], 4. logical V,
  5. a permutation of the physical page pool.
Values are fp32 N(0, 1) rounded to bf16 (round-to-nearest-even), times an
exact power-of-two factor where the workload says so. Sequence s owns the next
ceil(L_s / B) ids of the permutation, so sequences interleave physically.
Every pool slot that holds no valid token is NaN (bf16 0x7FC0), and block-table
entries past a sequence's last page point at one extra all-NaN page.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

HQ, HKV, HEAD = 24, 4, 256
NAN_BF16 = 0x7FC0


@dataclass
class Case:
    name: str
    seed: int
    q: torch.Tensor              # [S, HQ, HEAD] bf16
    k_logical: torch.Tensor      # [sum L, HKV, HEAD] bf16 (sequences back to back)
    v_logical: torch.Tensor
    lens: list                   # host copy of seq_lens
    seq_lens: torch.Tensor       # [S] int32
    block_table: torch.Tensor    # [S, max_blocks] int32
    k_cache: torch.Tensor        # [pool + 1, B, HKV, HEAD] bf16; page `pool` is the NaN pad
    v_cache: torch.Tensor
    block_size: int
    scale: float
    partition_tokens: int = 0    # 0 = let the library choose
    pool_pages: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return len(self.lens)

    @property
    def max_seq_len(self) -> int:
        return max(self.lens) if self.lens else 0

    def cu(self, s: int) -> tuple:
        lo = sum(self.lens[:s])
        return lo, lo + self.lens[s]

    def keys(self, s: int) -> torch.Tensor:
        lo, hi = self.cu(s)
        return self.k_logical[lo:hi]

    def values(self, s: int) -> torch.Tensor:
        lo, hi = self.cu(s)
        return self.v_logical[lo:hi]

    def algorithmic_bytes(self) -> int:
        """K and V rows of every valid token plus Q, in bytes."""
        return sum(self.lens) * HKV * HEAD * 2 * 2 + self.num_seqs * HQ * HEAD * 2


# name -> (description, builder kwargs). Sizes follow the five workloads of the
# decode microbenchmark study: tiny, single long sequence at page832, the
# page784/page832 A/B, a batched long-context mix and a wide serving batch.
WORKLOADS = {
    "tiny_l1024_b64": dict(lens=[1024], block_size=64, pool_pages=32, seed=1),
    "long_l8192_b832": dict(lens=[8192], block_size=832, pool_pages=64, seed=2),
    "long_l16384_b832": dict(lens=[16384], block_size=832, pool_pages=64, seed=2),
    "long_l32768_b832": dict(lens=[32768], block_size=832, pool_pages=64, seed=2),
    "ab_l32768_b784": dict(lens=[32768], block_size=784, pool_pages=64, seed=3),
    "ab_l32768_b832": dict(lens=[32768], block_size=832, pool_pages=64, seed=3),
    "batched_8seq_t131072_b832": dict(lens="split131072", block_size=832,
                                      pool_pages=200, seed=4, value_scale=0.5),
    "wide_64seq_b832_p4096": dict(lens="uniform2048_65536", block_size=832,
                                  pool_pages="fit110", seed=5, partition_tokens=4096),
    # the wide batch with the partition size left to the library (its
    # balanced split): the same draw, the library's own plan
    "wide_64seq_b832_auto": dict(lens="uniform2048_65536", block_size=832,
                                 pool_pages="fit110", seed=5),
    # a many-sequence serving batch (beyond the five workloads above): 1024
    # sequences of 256 to 4096 tokens, the partition size left to the library
    "serving_1024seq_b832": dict(lens="uniform256_4096x1024", block_size=832,
                                 pool_pages="fit110", seed=6),
}


def _draw_lens(spec, gen, device):
    if spec == "split131072":
        # 8 sequences, each 4096 + one gap of 7 sorted uniform cut points over
        # 131072 - 8 * 4096 tokens, so the lengths add up to 131072.
        free = 131072 - 8 * 4096
        cuts = torch.randint(0, free + 1, (7,), generator=gen, device=device)
        cuts = sorted(int(c) for c in cuts.cpu())
        edges = [0] + cuts + [free]
        return [4096 + edges[i + 1] - edges[i] for i in range(8)]
    if spec == "uniform2048_65536":
        lens = torch.randint(2048, 65536 + 1, (64,), generator=gen, device=device)
        return [int(x) for x in lens.cpu()]
    if spec == "uniform256_4096x1024":
        lens = torch.randint(256, 4096 + 1, (1024,), generator=gen, device=device)
        return [int(x) for x in lens.cpu()]
    return list(spec)


def _normal_bf16(shape, gen, device, value_scale):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    x = x.to(torch.bfloat16)
    if value_scale != 1.0:
        x = x * value_scale          # power of two: exact in bf16
    return x


def build_case(name, lens, block_size, pool_pages=None, seed=0, value_scale=1.0,
               partition_tokens=0, scale=1.0 / 16.0, gen_device="cpu",
               device="cpu", joint_kv=False):
    """Draw one workload and lay it out in a NaN-poisoned paged pool.

    joint_kv=True stores K and V in one [pool + 1, 2, B, HKV, HEAD] tensor and
    returns the two unbind views (page stride 2 * B * HKV * HEAD).
    """
    gen = torch.Generator(device=gen_device)
    gen.manual_seed(seed)
    lens = _draw_lens(lens, gen, gen_device)
    n_seq = len(lens)
    bsz = int(block_size)
    pages_per_seq = [-(-length // bsz) for length in lens]
    if pool_pages == "fit110":
        pool_pages = math.ceil(1.1 * sum(pages_per_seq))
    if pool_pages is None:
        pool_pages = sum(pages_per_seq) + 3
    assert pool_pages >= sum(pages_per_seq), "pool too small"

    q = _normal_bf16((n_seq, HQ, HEAD), gen, gen_device, value_scale)
    total = sum(lens)
    k_log = _normal_bf16((total, HKV, HEAD), gen, gen_device, value_scale)
    v_log = _normal_bf16((total, HKV, HEAD), gen, gen_device, value_scale)
    perm = torch.randperm(pool_pages, generator=gen, device=gen_device).cpu().tolist()

    max_blocks = max(1, max(pages_per_seq) if pages_per_seq else 1)
    pad_page = pool_pages
    table = torch.full((n_seq, max_blocks), pad_page, dtype=torch.int32)
    nxt = 0
    for s, n in enumerate(pages_per_seq):
        table[s, :n] = torch.tensor(perm[nxt:nxt + n], dtype=torch.int32)
        nxt += n

    shape = (pool_pages + 1, bsz, HKV, HEAD)
    nan = torch.tensor(NAN_BF16, dtype=torch.int16).view(torch.bfloat16)
    if joint_kv:
        joint = torch.empty((pool_pages + 1, 2, bsz, HKV, HEAD), dtype=torch.bfloat16,
                            device=device)
        joint.fill_(float(nan))
        k_cache, v_cache = joint.unbind(1)
    else:
        k_cache = torch.empty(shape, dtype=torch.bfloat16, device=device)
        v_cache = torch.empty(shape, dtype=torch.bfloat16, device=device)
        k_cache.fill_(float(nan))
        v_cache.fill_(float(nan))

    k_dev = k_log.to(device)
    v_dev = v_log.to(device)
    base = 0
    for s, length in enumerate(lens):
        for lp in range(pages_per_seq[s]):
            lo = lp * bsz
            hi = min(lo + bsz, length)
            pp = int(table[s, lp])
            k_cache[pp, : hi - lo] = k_dev[base + lo: base + hi]
            v_cache[pp, : hi - lo] = v_dev[base + lo: base + hi]
        base += length

    return Case(
        name=name, seed=seed, q=q.to(device), k_logical=k_dev, v_logical=v_dev,
        lens=lens, seq_lens=torch.tensor(lens, dtype=torch.int32, device=device),
        block_table=table.to(device), k_cache=k_cache, v_cache=v_cache,
        block_size=bsz, scale=scale, partition_tokens=partition_tokens,
        pool_pages=pool_pages,
    )


def make_case(name, device="cpu", gen_device=None, seed=None, **over):
    """Build a named workload. The wide and serving batches draw on the device
    generator (about 2 x 2.2 G values each); all others draw on the CPU
    generator."""
    spec = dict(WORKLOADS[name])
    if seed is not None:
        spec["seed"] = seed
    if gen_device is None:
        gen_device = device if name.startswith(("wide", "serving")) else "cpu"
    spec.update(over)
    return build_case(name, gen_device=gen_device, device=device, **spec)


def replicate(case: Case, copies: int):
    """Cold-cache replicas: ``copies`` disjoint copies of every used page in one
    pool, with one block table per copy ([copies, S, max_blocks]).

    Replica r's pages are r * pool + the original ids; the last page of the
    new pool is the NaN pad target. Each copy holds the same tokens, so every
    replica gives the same attention result.
    """
    pool = case.pool_pages
    bsz = case.block_size
    dev = case.k_cache.device
    shape = (copies * pool + 1, bsz, HKV, HEAD)
    k_big = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    v_big = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    nan = torch.tensor(NAN_BF16, dtype=torch.int16).view(torch.bfloat16)
    k_big.fill_(float(nan))
    v_big.fill_(float(nan))
    table = case.block_table.cpu()
    used = sorted({int(x) for s in range(case.num_seqs)
                   for x in table[s, : -(-case.lens[s] // bsz)].tolist()})
    used_t = torch.tensor(used, dtype=torch.long, device=dev)
    tables = []
    for r in range(copies):
        k_big[used_t + r * pool] = case.k_cache[used_t]
        v_big[used_t + r * pool] = case.v_cache[used_t]
        t = table.clone()
        for s in range(case.num_seqs):
            n = -(-case.lens[s] // bsz)
            t[s, :n] += r * pool
            t[s, n:] = copies * pool
        tables.append(t)
    return k_big, v_big, torch.stack(tables).to(dev)


def append_inputs(num_tokens, block_size, num_pages, seed, *, pad_every=0, outside=0,
                  hkv=HKV, head=HEAD, device="cpu"):
    """Seeded inputs for the KV-append tests: a pool of random bf16 bits
    [num_pages, B, Hkv, D], new rows [N, Hkv, D] and distinct slots drawn from
    the pool's num_pages * B rows. Every pad_every-th token gets slot -1 and
    the last `outside` tokens get slots past the pool. Draw order: pool,
    rows, slot permutation. Returns (pool, rows, slots) on `device`."""
    gen = torch.Generator().manual_seed(seed)
    pool = torch.randint(-32768, 32768, (num_pages, block_size, hkv, head), generator=gen,
                         dtype=torch.int32).to(torch.int16)
    rows = torch.randint(-32768, 32768, (num_tokens, hkv, head), generator=gen,
                         dtype=torch.int32).to(torch.int16)
    total = num_pages * block_size
    assert num_tokens <= total
    slots = torch.randperm(total, generator=gen)[:num_tokens].to(torch.int64)
    if pad_every:
        slots[::pad_every] = -1
    if outside:
        slots[num_tokens - outside:] = total + torch.arange(outside, dtype=torch.int64) * 7
    return (pool.view(torch.bfloat16).to(device), rows.view(torch.bfloat16).to(device),
            slots.to(device))


def append_bench_inputs(num_tokens, block_size, copies, seed, *, hkv=HKV, head=HEAD,
                        device="cuda"):
    """Seeded inputs for timing KV appends on cold data: `copies` independent
    sets of new rows [copies, N, Hkv, D] (random bf16 bits, drawn on the
    device) and slots [copies, N] laying each copy's N tokens out as one
    sequence over its own shuffled pages of a shared pool. Returns (rows_k,
    rows_v, slots, num_pages)."""
    pages_per_copy = -(-num_tokens // block_size)
    num_pages = copies * pages_per_copy
    gen = torch.Generator(device=device).manual_seed(seed)
    rows_k = torch.randint(-32768, 32768, (copies, num_tokens, hkv, head), generator=gen,
                           dtype=torch.int32, device=device).to(torch.int16).view(torch.bfloat16)
    rows_v = torch.randint(-32768, 32768, (copies, num_tokens, hkv, head), generator=gen,
                           dtype=torch.int32, device=device).to(torch.int16).view(torch.bfloat16)
    cpu_gen = torch.Generator().manual_seed(seed)
    pages = torch.randperm(num_pages, generator=cpu_gen).view(copies, pages_per_copy)
    t = torch.arange(num_tokens, dtype=torch.int64)
    slots = pages[:, t // block_size].to(torch.int64) * block_size + (t % block_size)
    return rows_k, rows_v, slots.to(device), num_pages


# Tail-Q prefill workloads: (new tokens q, cached length L incl. them, page size).
# q = 4096 is the pages' full prefill chunk at the three serving context tiers;
# the last one is a shorter tail chunk.
PREFILL_WORKLOADS = {
    "prefill_q4096_l8192_b832": (4096, 8192, 832),
    "prefill_q4096_l16384_b832": (4096, 16384, 832),
    "prefill_q4096_l32768_b832": (4096, 32768, 832),
    "prefill_q1500_l20000_b832": (1500, 20000, 832),
}


def build_prefill_case(name, num_q, seq_len, block_size, seed=0, device="cpu",
                       gen_device="cpu", pool_pages=None):
    """One sequence of seq_len cached tokens in a shuffled NaN-poisoned pool
    (build_case) plus the queries of its last num_q tokens, q_new [Q, 24, 256]
    bf16 N(0,1), drawn from a second generator seeded with seed + 1.
    Returns (case, q_new)."""
    case = build_case(name, lens=[seq_len], block_size=block_size, pool_pages=pool_pages,
                      seed=seed, gen_device=gen_device, device=device)
    gen = torch.Generator(device=gen_device)
    gen.manual_seed(seed + 1)
    q_new = _normal_bf16((num_q, HQ, HEAD), gen, gen_device, 1.0).to(device)
    return case, q_new


def make_prefill_case(name, device="cpu", gen_device=None, seed=None):
    num_q, seq_len, bsz = PREFILL_WORKLOADS[name]
    if seed is None:
        seed = 40 + sorted(PREFILL_WORKLOADS).index(name)
    return build_prefill_case(name, num_q, seq_len, bsz, seed=seed, device=device,
                              gen_device=gen_device or "cpu")



# ---------------------------------------------------------------------------
# Paged window compression: state rows [values(D) | scores(D)] in fp32 blocks.
# ---------------------------------------------------------------------------

COMPRESS_HEAD = 512

# The 12 shapes of the compression stage: (num_reqs, total_tokens, compress ratio).
COMPRESS_WORKLOADS = {
    f"compress_r{r}_t{t}_c{c}": (r, t, c)
    for c in (128, 256, 512)
    for r, t in ((1, 8192), (4, 32768), (8, 65536), (8, 131072))
}


@dataclass
class CompressCase:
    name: str
    seed: int
    states: torch.Tensor           # [T, 2D] fp32, requests back to back, rows by position
    lens: list                     # tokens per request
    token_to_req: torch.Tensor     # [T] int32
    positions: torch.Tensor        # [T] int64
    boundaries: torch.Tensor       # [N] int64 token indices
    block_table: torch.Tensor      # [R, max_blocks] int32; padding -> the NaN block
    state_cache: torch.Tensor      # [pool + 1, B, 2D] fp32; block `pool` is all NaN
    block_size: int
    compress_ratio: int
    head_dim: int
    pool_blocks: int

    def req_range(self, r):
        lo = sum(self.lens[:r])
        return lo, lo + self.lens[r]

    def boundaries_of(self, r):
        lo, hi = self.req_range(r)
        return [int(b) for b in self.boundaries.cpu().tolist() if lo <= b < hi]

    @property
    def num_outputs(self):
        return int(self.boundaries.shape[0])


def build_compress_case(name, num_reqs, total_tokens, compress_ratio, block_size=8, seed=0,
                        head_dim=COMPRESS_HEAD, lens=None, boundaries="chunk_ends",
                        gen_device="cpu", device="cpu", states_fn=None):
    """Draw one compression workload and lay it out in a NaN-poisoned paged
    state cache.

    Requests get total_tokens / num_reqs tokens each (the last one the
    remainder) unless `lens` is given; every token of a request has its
    position 0 .. len - 1. Boundary tokens: "chunk_ends" takes every token with
    (p + 1) % C == 0 (the windows tile each request exactly); "all" takes
    every token (windows overlap and are cut at position 0); a list gives
    explicit token indices. Draw order: state rows [T, 2D] fp32 N(0, 1)
    (values then scores in each row), then a permutation of the block pool
    (sum of ceil(len / B) plus 10 %). Request r owns the next ceil(len_r / B)
    ids of the permutation; every other row, and one extra padding block that
    unused table entries point to, is NaN. `states_fn(states, positions)`, if
    given, may rewrite the drawn rows in place before they are laid out."""
    if lens is None:
        base = total_tokens // num_reqs
        lens = [base] * (num_reqs - 1) + [total_tokens - base * (num_reqs - 1)]
    lens = [int(x) for x in lens]
    total = sum(lens)
    bsz, c, d = int(block_size), int(compress_ratio), int(head_dim)
    gen = torch.Generator(device=gen_device)
    gen.manual_seed(seed)
    states = torch.randn((total, 2 * d), generator=gen, device=gen_device, dtype=torch.float32)
    if states_fn is not None:
        states_fn(states, torch.cat([torch.arange(n, dtype=torch.int64) for n in lens]))
    blocks_per_req = [-(-n // bsz) for n in lens]
    pool = math.ceil(1.1 * sum(blocks_per_req))
    perm = torch.randperm(pool, generator=gen, device=gen_device).cpu()
    max_blocks = max(max(blocks_per_req), 1)
    table = torch.full((len(lens), max_blocks), pool, dtype=torch.int32)
    nxt = 0
    for r, nb in enumerate(blocks_per_req):
        table[r, :nb] = perm[nxt:nxt + nb].to(torch.int32)
        nxt += nb
    cache = torch.full((pool + 1, bsz, 2 * d), float("nan"), dtype=torch.float32,
                       device=gen_device)
    flat = cache.view(-1, 2 * d)
    tok_req, pos = [], []
    lo = 0
    for r, n in enumerate(lens):
        t = torch.arange(n, dtype=torch.int64)
        rows = table[r, (t // bsz)].to(torch.int64) * bsz + t % bsz
        flat[rows.to(gen_device)] = states[lo:lo + n]
        tok_req.append(torch.full((n,), r, dtype=torch.int32))
        pos.append(t)
        lo += n
    token_to_req = torch.cat(tok_req) if tok_req else torch.zeros(0, dtype=torch.int32)
    positions = torch.cat(pos) if pos else torch.zeros(0, dtype=torch.int64)
    if isinstance(boundaries, str):
        if boundaries == "chunk_ends":
            bnd = torch.nonzero((positions + 1) % c == 0).flatten()
        elif boundaries == "all":
            bnd = torch.arange(total, dtype=torch.int64)
        else:
            raise ValueError(boundaries)
    else:
        bnd = torch.as_tensor(boundaries, dtype=torch.int64)
    return CompressCase(name=name, seed=seed, states=states.to(device), lens=lens,
                        token_to_req=token_to_req.to(device), positions=positions.to(device),
                        boundaries=bnd.to(torch.int64).to(device), block_table=table.to(device),
                        state_cache=cache.to(device), block_size=bsz, compress_ratio=c,
                        head_dim=d, pool_blocks=pool)


def make_compress_case(name, device="cpu", gen_device=None, seed=None):
    num_reqs, total, c = COMPRESS_WORKLOADS[name]
    if seed is None:
        seed = 60 + sorted(COMPRESS_WORKLOADS).index(name)
    return build_compress_case(name, num_reqs, total, c, block_size=8, seed=seed,
                               gen_device=gen_device or "cpu", device=device)
