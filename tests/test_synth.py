"""The seeded generator against the oracle's gather: bit-exact layout checks."""

import numpy as np
import pytest
import torch

from oracle import decode as od
from paged_kv_cache_36_amd import synth


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("name", ["tiny_l1024_b64", "long_l8192_b832", "ab_l32768_b784",
                                  "ab_l32768_b832"])
def test_scatter_then_gather_is_identity(name):
    case = synth.make_case(name)
    for cache, logical in ((case.k_cache, case.k_logical), (case.v_cache, case.v_logical)):
        rows = od.gather_rows(bits(cache), case.block_table.numpy(), case.lens, case.block_size)
        for s in range(case.num_seqs):
            lo, hi = case.cu(s)
            assert np.array_equal(rows[s], bits(logical[lo:hi]))


def test_unused_slots_are_nan_and_pad_page_is_nan():
    case = synth.build_case("t", lens=[70, 3, 200], block_size=64, pool_pages=12, seed=9)
    kb = bits(case.k_cache)
    used = np.zeros(kb.shape[:2], dtype=bool)
    table = case.block_table.numpy()
    for s, length in enumerate(case.lens):
        t = np.arange(length)
        used[table[s, t // 64], t % 64] = True
    assert np.all(kb[~used] == synth.NAN_BF16)
    assert not np.any(kb[used] == synth.NAN_BF16)
    pad = case.pool_pages
    n_pages = [-(-n // 64) for n in case.lens]
    for s, n in enumerate(n_pages):
        assert np.all(table[s, n:] == pad)
    assert np.all(kb[pad] == synth.NAN_BF16)


def test_pages_are_a_permutation_and_interleave():
    case = synth.make_case("batched_8seq_t131072_b832")
    assert sum(case.lens) == 131072 and min(case.lens) >= 4096 and len(case.lens) == 8
    table = case.block_table.numpy()
    ids = np.concatenate([table[s, : -(-n // 832)] for s, n in enumerate(case.lens)])
    assert len(set(ids.tolist())) == ids.size and ids.max() < 200
    # the largest page id any sequence uses is spread across the pool, not a run
    assert not np.array_equal(np.sort(ids), np.arange(ids.size))


def test_seeded_draws_repeat():
    a = synth.make_case("tiny_l1024_b64")
    b = synth.make_case("tiny_l1024_b64")
    assert torch.equal(a.k_cache.view(torch.int16), b.k_cache.view(torch.int16))
    assert torch.equal(a.block_table, b.block_table)
    c = synth.make_case("tiny_l1024_b64", seed=99)
    assert not torch.equal(a.q.view(torch.int16), c.q.view(torch.int16))


def test_ab_pair_shares_logical_tokens():
    a = synth.make_case("ab_l32768_b784")
    b = synth.make_case("ab_l32768_b832")
    assert torch.equal(a.k_logical.view(torch.int16), b.k_logical.view(torch.int16))
    assert torch.equal(a.v_logical.view(torch.int16), b.v_logical.view(torch.int16))
    assert a.block_table.shape[1] == 42 and b.block_table.shape[1] == 40
    # same pool permutation, first n ids
    assert torch.equal(a.block_table[0, :40], b.block_table[0, :40])


def test_joint_kv_unbind_layout():
    case = synth.build_case("j", lens=[100], block_size=64, pool_pages=4, seed=2, joint_kv=True)
    assert case.k_cache.stride(0) == 2 * 64 * 4 * 256
    rows = od.gather_rows(bits(case.k_cache), case.block_table.numpy(), case.lens, 64)
    assert np.array_equal(rows[0], bits(case.k_logical))


def test_replicas_hold_the_same_tokens():
    case = synth.build_case("r", lens=[100, 40], block_size=64, pool_pages=5, seed=2)
    kb, vb, tables = synth.replicate(case, 3)
    for r in range(3):
        rows = od.gather_rows(bits(kb), tables[r].numpy(), case.lens, 64)
        for s in range(2):
            assert np.array_equal(rows[s], bits(case.keys(s)))
    assert np.all(bits(kb)[-1] == synth.NAN_BF16)


def test_algorithmic_bytes_of_the_workloads():
    # K+V rows of every valid token (4 KV heads x 256 x 2 B x 2) plus Q (24 x 256 x 2 B).
    assert synth.make_case("tiny_l1024_b64").algorithmic_bytes() == 4206592
    assert synth.make_case("long_l8192_b832").algorithmic_bytes() == 33566720
    assert synth.make_case("batched_8seq_t131072_b832").algorithmic_bytes() == 536969216


def test_append_inputs_are_seeded_distinct_and_in_range():
    pool, rows, slots = synth.append_inputs(500, 64, 10, seed=4, pad_every=7, outside=3)
    pool2, rows2, slots2 = synth.append_inputs(500, 64, 10, seed=4, pad_every=7, outside=3)
    assert torch.equal(slots, slots2) and torch.equal(rows.view(torch.int16), rows2.view(torch.int16))
    assert pool.shape == (10, 64, 4, 256) and rows.shape == (500, 4, 256)
    s = slots.tolist()
    assert all(x == -1 for x in s[:-3][::7])   # the last 3 are then moved outside
    assert all(x >= 640 for x in s[-3:])
    inside = [x for x in s if 0 <= x < 640]
    assert len(inside) == len(set(inside))


def test_append_bench_inputs_give_each_copy_its_own_pages():
    rk, rv, slots, pages = synth.append_bench_inputs(2000, 832, 3, seed=7, device="cpu")
    assert rk.shape == (3, 2000, 4, 256) and pages == 9
    flat = slots.flatten().tolist()
    assert len(set(flat)) == len(flat) and min(flat) >= 0 and max(flat) < pages * 832
    for c in range(3):
        used = {x // 832 for x in slots[c].tolist()}
        assert len(used) == 3
        others = {x // 832 for k in range(3) if k != c for x in slots[k].tolist()}
        assert not (used & others)
