"""Host-side replay of the balanced split's work assignment (no GPU).

The balanced split cuts every (sequence, KV head) into 64-token tiles,
enumerated as (sequence, head, tile); workgroup w of G = min(grid, T) takes
tiles [B(w), B(w + 1)) with B(w) = ceil((w T + (w mod 2) d) / G), where
d = floor(T / 24) once T >= 16 G and 0 below (odd workgroups, which run on the
odd XCDs, get a share 1/24 smaller, even ones 1/24 larger), and writes one
partial per (sequence, head) run, at slot w + s * Hkv + g. The combine kernel
finds the partials of (s, g) as the owners of its first and last tile: the
unshifted owner floor(u G / T) or its neighbour. This test replays those
formulas on random length mixes and checks that every token is covered
exactly once, that no share is empty, that slots never collide and that the
combine's workgroup range is exactly the set of writers.
"""

import random

import pytest

TILE = 64


def tiles(n):
    return (n + TILE - 1) // TILE


ODD_SHARE_DIV = 24


def bound(w, T, G):
    if w >= G:
        return T
    shift = T // ODD_SHARE_DIV if T >= 16 * G else 0
    return (w * T + (w & 1) * shift + G - 1) // G


def owner(u, T, G):
    q = u * G // T
    if q > 0 and u < bound(q, T, G):
        return q - 1
    if q + 1 < G and u >= bound(q + 1, T, G):
        return q + 1
    return q


def split_schedule(lens, hkv, grid):
    pref = [0]
    for n in lens:
        pref.append(pref[-1] + hkv * tiles(n))
    T = pref[-1]
    G = min(grid, T)
    writes = []          # (w, s, g, t_begin, t_end, slot)
    for w in range(G):
        u0 = bound(w, T, G)
        u1 = bound(w + 1, T, G)
        assert u0 < u1, "empty range"
        lo, hi = 0, len(lens)
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if pref[mid] <= u0:
                lo = mid
            else:
                hi = mid
        s, u = lo, u0
        while u < u1:
            while u >= pref[s + 1]:
                s += 1
            n = tiles(lens[s])
            base = pref[s]
            g = (u - base) // n
            tile = (u - base) - g * n
            seg_end = min(u1, base + (g + 1) * n)
            t_begin = tile * TILE
            t_end = min((tile + seg_end - u) * TILE, lens[s])
            writes.append((w, s, g, t_begin, t_end, w + s * hkv + g))
            u = seg_end
    return pref, T, G, writes


def combine_ranges(lens, hkv, grid, pref, T):
    G = min(grid, T)
    out = {}
    for s, n_tok in enumerate(lens):
        n = tiles(n_tok)
        for g in range(hkv):
            if n == 0:
                out[(s, g)] = []
                continue
            u_lo = pref[s] + g * n
            w_first = owner(u_lo, T, G)
            w_last = owner(u_lo + n - 1, T, G)
            out[(s, g)] = [w + s * hkv + g for w in range(w_first, w_last + 1)]
    return out


CASES = [
    ([8192], 4, 256),
    ([32768], 4, 256),
    ([1024], 4, 64),
    ([5, 1, 0, 70, 64, 65, 3000], 4, 512),
    ([0, 0, 0], 4, 256),
    ([1], 4, 256),                       # T = 4 < G
]


def random_cases(n=40, seed=5):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        s = rng.choice([1, 2, 3, 8, 17, 64, 130])
        lens = [rng.choice([0, 1, 63, 64, 65, rng.randint(1, 70000)]) for _ in range(s)]
        out.append((lens, rng.choice([1, 4, 8]), rng.choice([1, 7, 64, 256, 512, 999])))
    return out


@pytest.mark.parametrize("lens,hkv,grid", CASES + random_cases())
def test_balanced_schedule_covers_each_token_once(lens, hkv, grid):
    pref, T, G, writes = split_schedule(lens, hkv, grid)
    if T == 0:
        assert writes == []
        return
    slots = [w[5] for w in writes]
    assert len(slots) == len(set(slots)), "slot collision"
    assert max(slots) < grid + len(lens) * hkv
    covered = {}
    for w, s, g, tb, te, slot in writes:
        assert 0 <= tb < te <= lens[s] and tb % TILE == 0
        covered.setdefault((s, g), []).append((tb, te, slot))
    ranges = combine_ranges(lens, hkv, grid, pref, T)
    for (s, g), slot_list in ranges.items():
        segs = sorted(covered.get((s, g), []))
        # tokens 0..L-1 covered exactly once, in order
        pos = 0
        for tb, te, _ in segs:
            assert tb == pos
            pos = te
        assert pos == lens[s]
        # the combine reads exactly the slots the split wrote for (s, g)
        assert sorted(x[2] for x in segs) == slot_list


def test_balanced_schedule_is_even():
    lens = [4096 + random.Random(1).randint(0, 30000) for _ in range(8)]
    pref, T, G, writes = split_schedule(lens, 4, 512)
    per_wg = {}
    for w, s, g, tb, te, _ in writes:
        per_wg[w] = per_wg.get(w, 0) + tiles(te - tb)
    assert max(per_wg.values()) - min(per_wg.values()) <= 2
