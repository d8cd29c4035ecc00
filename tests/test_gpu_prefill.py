"""Tail-Q chunked prefill through the C ABI against the fp64 oracle.

bf16 output: |out - ref| <= 1e-2 + 1e-2 |ref| elementwise. fp32 output: p is
rounded to bf16 (unit roundoff 2^-9) for the P.V product while the
denominator sums the fp32 weights, so each output element is within
2^-9 * max|v| of the exact result (v over the row's visible keys); the test
allows 2^-8 * max|v|.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_36_amd as pkv
from oracle import prefill as opf
from paged_kv_cache_36_amd import synth
from tests.parity_util import assert_bf16_close, bits, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a GPU")
    pkv.load()


def run_prefill(case, q_new, key_splits=0):
    out32 = torch.empty(q_new.shape, dtype=torch.float32, device="cuda")
    out, _ = pkv.prefill(q_new, case.k_cache, case.v_cache, case.block_table[0],
                         case.lens[0], case.block_size, case.scale, out_f32=out32,
                         key_splits=key_splits)
    torch.cuda.synchronize()
    return out, out32


def check(case, q_new, out, out32, rows=None):
    q = f64(q_new)
    k = f64(case.keys(0))
    v = f64(case.values(0))
    ref, _ = opf.attention_prefill(q, k, v, case.scale, rows=rows)
    sel = list(range(q.shape[0])) if rows is None else sorted(set(rows))
    got32 = f64(out32)
    nq, length = q.shape[0], k.shape[0]
    # max |v| over keys 0 .. t, for every t
    vmax_upto = np.maximum.accumulate(np.abs(v).max(axis=(1, 2)))
    for i in sel:
        vmax = vmax_upto[length - nq + i]
        err = np.abs(got32[i] - ref[i]).max()
        assert err <= 2.0 ** -8 * vmax, f"query {i}: fp32 error {err:.3e} > {2.0 ** -8 * vmax:.3e}"
    assert_bf16_close(out, ref, rows=sel, what=f"prefill Q={nq} L={length}")
    assert torch.isfinite(out32).all()


@pytest.mark.parametrize("nq,length,bsz", [
    (2, 2, 64), (17, 40, 16), (128, 128, 832), (129, 300, 784), (200, 1000, 832),
    (1, 500, 64), (333, 333, 64), (64, 4097, 784),
    # pages of 1, 5 and 100 tokens: page crossings inside a wave's rows and
    # page-id window reloads (more than 64 pages per workgroup)
    (70, 150, 1), (130, 1000, 5), (300, 2000, 100),
])
def test_prefill_small_full_check(nq, length, bsz):
    print(f"[gpu] prefill Q={nq} L={length} B={bsz}", flush=True)
    case, q_new = synth.build_prefill_case("pf", nq, length, bsz, seed=nq + length, device="cuda")
    out, out32 = run_prefill(case, q_new)
    check(case, q_new, out, out32)


def test_prefill_medium_full_check():
    print("[gpu] prefill Q=1000 L=5000 B=784", flush=True)
    case, q_new = synth.build_prefill_case("pfm", 1000, 5000, 784, seed=3, device="cuda")
    out, out32 = run_prefill(case, q_new)
    check(case, q_new, out, out32)


def test_prefill_short_blocks_take_one_split_fewer():
    # Q = 1500 over L = 4600 keys: 3 key splits per query block, and the 4
    # shortest of the 12 blocks take 2, so the 768 workgroups make three whole
    # rounds over 256 CUs; every query row against the oracle
    print("[gpu] prefill Q=1500 L=4600 B=784, short blocks", flush=True)
    case, q_new = synth.build_prefill_case("pfs", 1500, 4600, 784, seed=61, device="cuda")
    prm = pkv.prefill_params(q_new, case.k_cache, case.v_cache, case.block_table[0],
                             case.lens[0], case.block_size, case.scale)
    assert pkv.prefill_key_splits(prm) == 3 and pkv.prefill_short_blocks(prm) == 4
    out, out32 = run_prefill(case, q_new)
    check(case, q_new, out, out32)
    # the same queries with 3 splits everywhere agree within the same bounds
    out3, out32_3 = run_prefill(case, q_new, key_splits=3)
    check(case, q_new, out3, out32_3)


def stratified_rows(nq, per_block, seed):
    """per_block query rows from every 128-query block of the kernel (its
    first, last and 32-query group edges, the rest drawn from the seed); each
    oracle row covers all 24 heads."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b0 in range(0, nq, 128):
        b1 = min(b0 + 128, nq)
        edges = [r for r in (b0, b0 + 31, b0 + 32, b0 + 63, b0 + 64, b0 + 95, b0 + 96, b1 - 1)
                 if r < b1]
        rows.update(edges)
        extra = max(0, min(per_block, b1 - b0) - len(edges))
        rows.update(int(x) for x in rng.choice(np.arange(b0, b1), size=extra, replace=False))
    return sorted(rows)


@pytest.mark.parametrize("name,per_block", [
    ("prefill_q4096_l8192_b832", None),      # every query row
    ("prefill_q4096_l16384_b832", 16),       # 512 of 4096 rows, 16 per 128-query block
    ("prefill_q4096_l32768_b832", 16),
    ("prefill_q1500_l20000_b832", 43),       # 512 of 1500 rows
])
def test_prefill_workloads(name, per_block):
    print(f"[gpu] prefill workload {name}", flush=True)
    case, q_new = synth.make_prefill_case(name, device="cuda")
    out, out32 = run_prefill(case, q_new)
    nq = q_new.shape[0]
    rows = None if per_block is None else stratified_rows(nq, per_block, seed=nq)
    check(case, q_new, out, out32, rows=rows)
    assert torch.isfinite(out32).all()
    print(f"[gpu] {name}: checked {nq if rows is None else len(rows)} of {nq} query rows "
          f"(all 24 heads each)", flush=True)


def test_prefill_page_size_invariant_and_repeatable():
    outs = []
    for bsz in (64, 784, 832):
        case, q_new = synth.build_prefill_case("pfi", 300, 2500, bsz, seed=8, device="cuda")
        out, _ = run_prefill(case, q_new)
        outs.append(bits(out))
        again, _ = run_prefill(case, q_new)
        assert np.array_equal(bits(again), outs[-1])
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_prefill_score_jump_rescales_the_accumulator():
    # one key of a later tile scores about 60 log2 units above everything in
    # the first tile for one query: weights relative to the first tile's max
    # would pass 2^40, so the running max must move and the accumulator and
    # the weight sum be rescaled
    print("[gpu] prefill score jump", flush=True)
    nq, length, bsz = 64, 300, 64
    case, q_new = synth.build_prefill_case("pfj", nq, length, bsz, seed=12, device="cuda")
    i, t = 10, 100                                  # query 10 sits at position 246
    q = q_new[i, 0].float()
    k = q * (60.0 * 16.0 / (1.4426950408889634 * float((q * q).sum())))
    k = k.to(torch.bfloat16)
    case.k_logical[t, 0] = k                        # KV head 0 of the one sequence
    page = int(case.block_table[0, t // bsz])
    case.k_cache[page, t % bsz, 0] = k
    out, out32 = run_prefill(case, q_new)
    s = float((q * k.float()).sum()) / 16.0 * 1.4426950408889634
    assert s > 50.0, s
    check(case, q_new, out, out32)


@pytest.mark.parametrize("scale", [0.0, -1.0 / 16.0, 1.0 / 64.0])
def test_prefill_other_scales(scale):
    # a positive scale folds into the exponent's fma; zero and negative scales
    # take the kernel's other instantiation (scores scaled before the max)
    print(f"[gpu] prefill scale {scale}", flush=True)
    nq, length, bsz = 300, 2100, 784
    case, q_new = synth.build_prefill_case("pfs", nq, length, bsz, seed=21, device="cuda")
    case.scale = scale
    out, out32 = run_prefill(case, q_new)
    check(case, q_new, out, out32)


@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("hkv", [1, 2, 3])
def test_prefill_other_kv_head_counts(hkv, splits):
    # 6 query heads per KV head for 1, 2 and 3 KV heads: the grid deals
    # workgroups to XCDs by KV head when the head count divides 8, and in
    # plain order otherwise (3); with one split and with three
    print(f"[gpu] prefill Hkv={hkv} splits={splits}", flush=True)
    nq, length, bsz = 300, 1500, 784
    case, q_new = synth.build_prefill_case("pfh", nq, length, bsz, seed=50 + hkv, device="cuda")
    kc = case.k_cache[:, :, :hkv].contiguous()
    vc = case.v_cache[:, :, :hkv].contiguous()
    q = q_new[:, : 6 * hkv].contiguous()
    out32 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    out, _ = pkv.prefill(q, kc, vc, case.block_table[0], length, bsz, case.scale, out_f32=out32,
                         key_splits=splits)
    torch.cuda.synchronize()
    k = f64(case.keys(0))[:, :hkv]
    v = f64(case.values(0))[:, :hkv]
    ref, _ = opf.attention_prefill(f64(q), k, v, case.scale)
    got32 = f64(out32)
    for i in range(nq):
        vmax = np.abs(v[: length - nq + i + 1]).max()
        assert np.abs(got32[i] - ref[i]).max() <= 2.0 ** -8 * vmax, f"query {i}"
    assert_bf16_close(out, ref, what=f"prefill Hkv={hkv}")


@pytest.mark.parametrize("nq,length,bsz,splits,scale", [
    # 11 tiles per query block: 2 and 3 splits; 7 puts the diagonal tiles in
    # splits of their own (queries that see no key of a split); 64 leaves
    # most splits empty
    (130, 700, 64, 2, 1.0 / 16), (130, 700, 64, 3, 1.0 / 16), (130, 700, 64, 7, 1.0 / 16),
    (130, 700, 64, 64, 1.0 / 16),
    # the unfolded-scale instantiation, pages of 5 tokens
    (200, 1500, 5, 5, -1.0 / 16),
    # one query (the decode shape through prefill), 16 splits
    (1, 5000, 832, 16, 1.0 / 16),
])
def test_prefill_forced_key_splits(nq, length, bsz, splits, scale):
    print(f"[gpu] prefill Q={nq} L={length} B={bsz} splits={splits}", flush=True)
    case, q_new = synth.build_prefill_case("pfk", nq, length, bsz, seed=7 * splits + nq,
                                           device="cuda")
    case.scale = scale
    out, out32 = run_prefill(case, q_new, key_splits=splits)
    check(case, q_new, out, out32)


def test_prefill_auto_splits_match_one_split():
    # the library's own choice (5 splits here) against one split: both within
    # the oracle's tolerance, and close to each other at fp32
    print("[gpu] prefill auto splits vs one split", flush=True)
    case, q_new = synth.build_prefill_case("pfa", 600, 6000, 832, seed=77, device="cuda")
    p = pkv.prefill_params(q_new, case.k_cache, case.v_cache, case.block_table[0], case.lens[0],
                           case.block_size, case.scale)
    assert pkv.prefill_key_splits(p) > 1
    out_a, out32_a = run_prefill(case, q_new)
    out_1, out32_1 = run_prefill(case, q_new, key_splits=1)
    check(case, q_new, out_a, out32_a)
    check(case, q_new, out_1, out32_1)
    vmax = float(case.values(0).float().abs().max())
    assert float((out32_a - out32_1).abs().max()) <= 2.0 ** -8 * vmax


def test_prefill_unbind_view_matches_separate_caches():
    # K and V as the two halves of one [pages, 2, B, Hkv, D] tensor (page
    # strides of 2 B Hkv D elements): the same result, bit for bit
    print("[gpu] prefill unbind view", flush=True)
    case, q_new = synth.build_prefill_case("pfu", 200, 2600, 832, seed=91, device="cuda")
    joint = torch.stack([case.k_cache, case.v_cache], dim=1)
    kc, vc = joint.unbind(1)
    assert kc.stride(0) == 2 * case.k_cache.stride(0)
    out_a, out32_a = run_prefill(case, q_new)
    out32_b = torch.empty_like(out32_a)
    out_b, _ = pkv.prefill(q_new, kc, vc, case.block_table[0], case.lens[0], case.block_size,
                           case.scale, out_f32=out32_b)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_b), bits(out_a))
    assert torch.equal(out32_b.view(torch.int32), out32_a.view(torch.int32))
