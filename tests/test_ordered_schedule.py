"""The ordered dispatch of fixed partitions, replayed on the host (no GPU).

With several sequences of several P-token partitions each, workgroup b of the
fixed split takes KV head b % Hkv and item b // Hkv: every full partition
(s, p) first, in (s, p) order, then the last, shorter partition of every
sequence whose length is not a multiple of P, longest first by buckets of
P / 64 tokens (sequence order within a bucket), then nothing. This replays
that arithmetic in Python for many batches and checks that every partition
of every sequence is taken exactly once, that no item is taken twice, and
that the last partitions come in non-increasing bucket order.
"""

import numpy as np
import pytest

TAIL_BUCKETS = 64


def bucket(r, p):
    return (p - r) * TAIL_BUCKETS // p


def ordered_item(lens, p, item):
    """(s, part) of an item, or None: the kernel's prefix sums, binary search
    and bucket counting, written out."""
    full = [n // p for n in lens]
    tail = [1 if n % p else 0 for n in lens]
    full_pref = np.concatenate([[0], np.cumsum(full)])
    n_full = int(full_pref[-1])
    if item < n_full:
        s = int(np.searchsorted(full_pref, item, side="right") - 1)
        return s, item - int(full_pref[s])
    k = item - n_full
    if k >= sum(tail):
        return None
    counts = [0] * TAIL_BUCKETS
    for n in lens:
        if n % p:
            counts[bucket(n % p, p)] += 1
    start = np.concatenate([[0], np.cumsum(counts)])
    b = next(i for i in range(TAIL_BUCKETS) if counts[i] and start[i] <= k < start[i + 1])
    j = k - int(start[b])
    members = [s for s, n in enumerate(lens) if n % p and bucket(n % p, p) == b]
    s = members[j]
    return s, lens[s] // p


def draw(rng):
    nseq = int(rng.integers(2, 300))
    p = int(rng.choice([64, 128, 512, 4096]))
    kinds = rng.random(nseq)
    lens = np.where(kinds < 0.1, 0,
                    np.where(kinds < 0.3, p * rng.integers(1, 6, nseq),
                             rng.integers(1, 20 * p, nseq)))
    return [int(x) for x in lens], p


@pytest.mark.parametrize("seed", range(40))
def test_ordered_dispatch_covers_every_partition_once(seed):
    rng = np.random.default_rng(seed)
    lens, p = draw(rng)
    n_parts = max(-(-max(lens) // p), 1)
    items = len(lens) * n_parts                     # grid = S * n_parts (x Hkv)
    got = [ordered_item(lens, p, i) for i in range(items)]
    live = [x for x in got if x is not None]
    want = {(s, q) for s, n in enumerate(lens) for q in range(-(-n // p))}
    assert len(live) == len(set(live)) == len(want)
    assert set(live) == want
    # live items first, then only empty ones
    first_none = next((i for i, x in enumerate(got) if x is None), len(got))
    assert all(x is None for x in got[first_none:])
    # full partitions before last partitions, last ones longest-bucket first
    kinds = [(lens[s] - q * p) >= p for s, q in live]
    assert kinds == sorted(kinds, reverse=True)
    tails = [bucket(lens[s] % p, p) for (s, q), full in zip(live, kinds) if not full]
    assert tails == sorted(tails)


def test_tail_buckets_span_the_partition():
    # the longest last partition lands in bucket 0 (1 when P = 64: one token
    # per bucket), the shortest in bucket 63
    for p in (64, 128, 4096, 65536):
        assert bucket(p - 1, p) == (1 if p == 64 else 0)
        assert bucket(1, p) == TAIL_BUCKETS - 1
        assert all(0 <= bucket(r, p) < TAIL_BUCKETS for r in range(1, p, max(1, p // 97)))
