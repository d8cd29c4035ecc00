"""The prefill grid with key splits, replayed on the host (no GPU).

Workgroup b of the prefill kernel takes a (query head, query block, key split)
item: with S splits per block and the n shortest (lowest) query blocks taking
S - 1, the items of one KV head are the short blocks' splits first, then the
other blocks' S splits, each group from its longest block down; workgroups
are dealt so that XCD x (of 8, round robin) serves KV head x % Hkv when Hkv
divides 8. This replays that arithmetic and checks that every item is taken
exactly once and nothing else is, and that the combine's split count for a
query matches the splits its block was cut into. It also replays the host's
choice of n (the library's own choice is checked through
pkv_prefill_short_blocks in tests/test_abi_cpu.py).
"""

from __future__ import annotations

import pytest

KXCDS = 8
KGROUP = 6
QUERIES = 128


def splits_of(qb, nsplit, short):
    return nsplit - 1 if qb < short else nsplit


def block_of(b, hkv, nqb, nsplit, short):
    per_kv = KGROUP * (nqb * nsplit - short)
    if KXCDS % hkv == 0:
        x = b % KXCDS
        j = (b // KXCDS) * (KXCDS // hkv) + x // hkv
        if j >= per_kv:
            return None
        h = (x % hkv) * KGROUP + j % KGROUP
    else:
        hq = hkv * KGROUP
        h = b % hq
        j = (b // hq) * KGROUP
    t = j // KGROUP
    short_items = short * (nsplit - 1)
    if t < short_items:
        qb = short - 1 - t // (nsplit - 1)
        split = t % (nsplit - 1)
        ns = nsplit - 1
    else:
        u = t - short_items
        qb = nqb - 1 - u // nsplit
        split = u % nsplit
        ns = nsplit
    return h, qb, split, ns


def grid(hkv, nqb, nsplit, short):
    per_kv = KGROUP * (nqb * nsplit - short)
    blocks = hkv * per_kv
    if KXCDS % hkv == 0:
        per_xcd = -(-per_kv // (KXCDS // hkv))
        blocks = per_xcd * KXCDS
    return blocks


def short_blocks(nq, nsplit, hq, cus=256, forced=False):
    if forced or nsplit < 2:
        return 0
    nqb = -(-nq // QUERIES)
    for n in range(nqb):
        if (hq * (nqb * nsplit - n)) % cus == 0:
            return n
    return 0


@pytest.mark.parametrize("hkv", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("nqb,nsplit,short", [
    (12, 3, 4), (12, 3, 0), (1, 16, 0), (5, 2, 3), (32, 1, 0), (7, 5, 6), (12, 2, 11)])
def test_every_item_once(hkv, nqb, nsplit, short):
    seen = set()
    live = 0
    for b in range(grid(hkv, nqb, nsplit, short)):
        it = block_of(b, hkv, nqb, nsplit, short)
        if it is None:
            continue
        live += 1
        h, qb, split, ns = it
        assert 0 <= h < hkv * KGROUP and 0 <= qb < nqb
        assert ns == splits_of(qb, nsplit, short), "the kernel and the combine disagree"
        assert 0 <= split < ns
        seen.add((h, qb, split))
    want = {(h, qb, sp) for h in range(hkv * KGROUP) for qb in range(nqb)
            for sp in range(splits_of(qb, nsplit, short))}
    assert live == len(seen) == len(want) and seen == want


def test_host_choice_of_short_blocks():
    # Q = 1500 (12 blocks), 24 heads, 3 splits: 864 workgroups are 3.375
    # rounds over 256 CUs; 2 splits for the 4 shortest blocks make 768
    assert short_blocks(1500, 3, 24) == 4
    assert 24 * (12 * 3 - 4) == 3 * 256
    # already whole rounds, one split, or the caller's count: none
    assert short_blocks(4096, 1, 24) == 0
    assert short_blocks(1500, 3, 24, forced=True) == 0
    # no n below the block count gives whole rounds: none
    assert short_blocks(700, 2, 24) == 0
