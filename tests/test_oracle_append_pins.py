"""Pins for oracle/append.py (KV append scatter and the page-size rule).

Each check ties the oracle to something other than itself: hand-derived slot
splits, the decode oracle's independent gather map, the page's 784 -> 832
outcome and closed forms of the rounding. The mutation tests at the end plant
plausible mistakes in copies of the oracle functions and require a pin to fail.
"""

import numpy as np
import pytest

from oracle import append as oa
from oracle import decode as od
from tests.conftest import read_golden

NAN_BITS = 0x7FC0


def slot_rows():
    return [(int(r[0]), int(r[1]), int(r[3]), int(r[4])) for r in read_golden("append_slots.txt")]


def pin_slot_fixture(split_slot, append_rows):
    for bsz, slot, page, offset in slot_rows():
        assert split_slot(slot, bsz) == (page, offset), (bsz, slot)
        pages = max(page + 1, 2)
        pool = np.zeros((pages, bsz, 2, 8), dtype=np.uint16)
        marker = np.full((1, 2, 8), 0xBEEF, dtype=np.uint16)
        out = append_rows(pool, marker, [slot], bsz)
        assert np.all(out[page, offset] == 0xBEEF), (bsz, slot)
        assert np.count_nonzero(out) == 16, (bsz, slot)   # nothing else written


def pin_round_trip(slots_for_positions, append_rows):
    # scatter a sequence through its block table, read it back with the decode
    # oracle's gather (an independent statement of the same map)
    rng = np.random.default_rng(7)
    for bsz, length, pages in ((16, 200, 20), (64, 1000, 24), (784, 2000, 6), (832, 2500, 5)):
        logical = rng.integers(0, 0x7F00, size=(length, 4, 8), dtype=np.uint16)
        n_used = -(-length // bsz)
        table = rng.permutation(pages)[:n_used]
        pool = np.full((pages, bsz, 4, 8), NAN_BITS, dtype=np.uint16)
        slots = slots_for_positions(table, np.arange(length), bsz)
        order = rng.permutation(length)            # append order must not matter
        out = append_rows(pool, logical[order], np.asarray(slots)[order], bsz)
        back = od.gather_rows(out, table[None, :], [length], bsz)[0]
        assert np.array_equal(back, logical), bsz
        written = np.zeros((pages, bsz), dtype=bool)
        for t in range(length):
            written[table[t // bsz], t % bsz] = True
        assert np.all(out[~written] == NAN_BITS), bsz


def pin_padding(append_rows):
    pool = np.arange(3 * 16 * 2 * 8, dtype=np.uint16).reshape(3, 16, 2, 8)
    rows = np.full((4, 2, 8), 0xBEEF, dtype=np.uint16)
    out = append_rows(pool, rows, [-1, -5, 3 * 16, 1000], 16)
    assert np.array_equal(out, pool)


def pin_page_rule_fixture(page_tokens):
    for r in read_golden("page_size_rule.txt"):
        assert page_tokens(int(r[0]), int(r[1]), int(r[2])) == int(r[4]), r


def pin_page_rule_closed_forms(page_tokens):
    rng = np.random.default_rng(3)
    for _ in range(500):
        a = int(rng.integers(1, 10000))
        k = int(rng.choice([1, 16, 64, 128]))
        s = int(rng.integers(1, 10 ** 9))
        n = page_tokens(s, a, k)
        assert n % k == 0 and n > 0
        assert n * a >= s                  # the page holds the state
        assert (n - k) * a < s             # and is the smallest such multiple
        x = int(rng.integers(1, 100))
        assert page_tokens(x * k * a, a, k) == x * k
    assert page_tokens(0, 4096, 16) == -1 and page_tokens(5, 0, 16) == -1
    assert page_tokens(5, 4096, 0) == -1


def test_slot_fixture():
    pin_slot_fixture(oa.split_slot, oa.append_rows)


def test_round_trip_through_gather():
    pin_round_trip(oa.slots_for_positions, oa.append_rows)


def test_padding_and_outside_slots_write_nothing():
    pin_padding(oa.append_rows)


def test_page_rule_fixture():
    pin_page_rule_fixture(oa.page_tokens)


def test_page_rule_closed_forms():
    pin_page_rule_closed_forms(oa.page_tokens)


def test_input_pool_left_unchanged():
    pool = np.zeros((2, 16, 1, 8), dtype=np.uint16)
    oa.append_rows(pool, np.ones((1, 1, 8), dtype=np.uint16), [3], 16)
    assert not pool.any()


# ---------------------------------------------------------------- mutation tests

def _split_swapped(slot, bsz):
    return int(slot) % bsz, int(slot) // bsz


def _slots_page_from_mod(table, t, bsz):
    t = np.asarray(t, dtype=np.int64)
    return np.asarray(table, dtype=np.int64)[t % len(table)] * bsz + t % bsz


def _slots_no_table(table, t, bsz):
    return np.asarray(t, dtype=np.int64)


def _append_transposed(pool, rows, slots, bsz):
    out = np.array(pool, copy=True)
    for b, slot in enumerate(slots):
        if slot < 0 or slot >= out.shape[0] * bsz:
            continue
        out[slot % out.shape[0], slot // out.shape[0]] = rows[b]
    return out


def _append_keeps_negative(pool, rows, slots, bsz):
    out = np.array(pool, copy=True)
    for b, slot in enumerate(slots):
        if slot >= out.shape[0] * bsz:
            continue
        out[slot // bsz, slot % bsz] = rows[b]
    return out


def _page_floor(s, a, k):
    return (int(s) // (k * a)) * k if s > 0 and a > 0 and k > 0 else -1


def _page_no_alignment(s, a, k):
    return -(-int(s) // int(a)) if s > 0 and a > 0 and k > 0 else -1


@pytest.mark.parametrize("pin,args", [
    (pin_slot_fixture, (_split_swapped, oa.append_rows)),
    (pin_slot_fixture, (oa.split_slot, _append_transposed)),
    (pin_round_trip, (_slots_page_from_mod, oa.append_rows)),
    (pin_round_trip, (_slots_no_table, oa.append_rows)),
    (pin_round_trip, (oa.slots_for_positions, _append_transposed)),
    (pin_padding, (_append_keeps_negative,)),
    (pin_page_rule_fixture, (_page_floor,)),
    (pin_page_rule_fixture, (_page_no_alignment,)),
    (pin_page_rule_closed_forms, (_page_floor,)),
])
def test_planted_mistake_is_caught(pin, args):
    with pytest.raises((AssertionError, IndexError)):
        pin(*args)
