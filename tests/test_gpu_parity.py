"""HIP path vs the fp64 CPU oracle, through the C ABI (needs an MI355X)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_36_amd as pkv
from oracle import decode as od
from paged_kv_cache_36_amd import synth
from tests.parity_util import (assert_bf16_close, assert_rows_rel, bits, f64, oracle_case,
                               oracle_case_parallel)

pytestmark = pytest.mark.gpu

SWEEP_LENS = [1, 2, 63, 64, 65, 783, 784, 785, 831, 832, 833, 4095, 4096, 4097]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    pkv.load()   # raises if the HIP library is not built
    print(f"\n[gpu] {torch.cuda.get_device_name(0)}", flush=True)


def run_decode(case, partition_tokens=None, **kw):
    p_tok = case.partition_tokens if partition_tokens is None else partition_tokens
    out = pkv.decode(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                     case.block_size, case.scale, partition_tokens=p_tok,
                     max_seq_len=max(case.max_seq_len, 1), **kw)
    torch.cuda.synchronize()
    return out


def params_of(case, partition_tokens=0):
    return pkv.make_params(case.q, case.k_cache, case.v_cache, case.block_table,
                           case.block_size, case.scale, max(case.max_seq_len, 1),
                           partition_tokens)


# ------------------------------------------------------------ addressing (bit-exact)

def check_resolve(case, prm, heads=range(4)):
    table = case.block_table.cpu().numpy()
    for g in heads:
        got = pkv.debug_resolve(prm, g, case.block_table, case.seq_lens).cpu().numpy()
        ref = od.resolve_offsets(table, case.lens, case.block_size, case.k_cache.stride(0), 4,
                                 256, g, prm.max_seq_len)
        assert np.array_equal(got, ref), (case.name, prm.partition_tokens, g)
        yield got


# The debug walks run the split pkv_decode would run for the same params:
# fixed partitions for P != 0 or one sequence, the balanced split for P = 0
# with several sequences.
@pytest.mark.parametrize("bsz", [16, 64, 784, 832])
@pytest.mark.parametrize("ptok", [64, 256, 0])
def test_resolver_offsets_bit_exact(bsz, ptok):
    case = synth.build_case(f"res{bsz}", lens=[1, 63, 65, 785, 1700, 833], block_size=bsz,
                            seed=11, device="cuda")
    prm = params_of(case, ptok)
    assert pkv.plan(prm)["balanced"] == (1 if ptok == 0 else 0)
    for _ in check_resolve(case, prm):
        pass
    one = synth.build_case(f"res1_{bsz}", lens=[1700], block_size=bsz, seed=14, device="cuda")
    for _ in check_resolve(one, params_of(one, ptok)):
        pass


def test_resolver_balanced_page_list_refetch():
    # 16-token pages and runs longer than 64 pages: the balanced walker
    # refetches its page list inside the loop
    case = synth.build_case("resrf", lens=[150000, 70000, 333], block_size=16, seed=15,
                            device="cuda")
    prm = params_of(case, 0)
    assert pkv.plan(prm)["balanced"] == 1
    for _ in check_resolve(case, prm, heads=[0, 3]):
        pass


def test_resolver_wide_pool_past_2_31_elements():
    # The wide batch's pool holds about 2.4e9 elements per cache, so row
    # offsets pass 2^31: every token's offset for all 4 KV heads, through the
    # split pkv_decode runs for this workload (fixed 4096-token partitions)
    case = synth.make_case("wide_64seq_b832_p4096", device="cuda")
    prm = params_of(case, case.partition_tokens)
    top = 0
    for got in check_resolve(case, prm):
        top = max(top, int(got.max()))
    assert top > 2 ** 31, top
    print(f"[gpu] wide pool: largest row offset {top} elements (2^31 = {2 ** 31})", flush=True)


def check_gather(case, prm, which):
    sentinel = 0x1234
    dense = pkv.debug_gather(prm, which, case.k_cache, case.block_table, case.seq_lens,
                             fill=sentinel)
    torch.cuda.synchronize()
    d = bits(dense)
    for s in range(case.num_seqs):
        n = case.lens[s]
        assert np.array_equal(d[s, :n], bits(case.keys(s))), (which, case.block_size, s)
        assert np.all(d[s, n:] == sentinel)


@pytest.mark.parametrize("which", [0, 1])
@pytest.mark.parametrize("bsz", [16, 64, 784, 832])
def test_tile_loaders_gather_bit_exact(which, bsz):
    # a batch (K as whole rows), with fixed partitions and with the balanced
    # split, and one sequence (K in the MFMA operand layout)
    case = synth.build_case(f"gat{bsz}", lens=[70, 1, 1600, 832], block_size=bsz, seed=12,
                            device="cuda")
    for ptok in (256, 0):
        check_gather(case, params_of(case, ptok), which)
    one = synth.build_case(f"gat1_{bsz}", lens=[1601], block_size=bsz, seed=13, device="cuda")
    for ptok in (256, 0):
        check_gather(one, params_of(one, ptok), which)


def test_joint_kv_unbind_view_addressing():
    case = synth.build_case("joint", lens=[900, 33], block_size=832, seed=13, device="cuda",
                            joint_kv=True)
    assert case.k_cache.stride(0) == 2 * 832 * 1024
    prm = params_of(case, 128)
    dense = pkv.debug_gather(prm, 0, case.v_cache, case.block_table, case.seq_lens)
    torch.cuda.synchronize()
    for s in range(2):
        assert np.array_equal(bits(dense)[s, :case.lens[s]], bits(case.values(s)))
    out = run_decode(case, 128)
    assert_bf16_close(out, oracle_case(case)[0], what="unbind view")


# ------------------------------------------------------------ decode vs oracle

def test_tiny_workload():
    case = synth.make_case("tiny_l1024_b64", device="cuda")
    ref, _ = oracle_case(case)
    for ptok in (0, 64, 256, 1024):
        print(f"[gpu] tiny P={ptok}", flush=True)
        assert_bf16_close(run_decode(case, ptok), ref, what=f"tiny P={ptok}")


# page sizes of the study (784, 832), the smallest (16), and other multiples of
# 16 whose pages split the 64-token tiles differently (48, 80, 1024)
@pytest.mark.parametrize("bsz", [16, 48, 64, 80, 784, 832, 1024])
def test_length_sweep(bsz):
    case = synth.build_case(f"sweep{bsz}", lens=SWEEP_LENS, block_size=bsz, seed=21,
                            device="cuda")
    ref, _ = oracle_case(case)
    for ptok in (0, 128, 4096):
        print(f"[gpu] sweep B={bsz} P={ptok}", flush=True)
        assert_bf16_close(run_decode(case, ptok), ref, what=f"sweep B={bsz} P={ptok}")


def test_one_sequence_in_a_thousand_partitions():
    # 64-token partitions of a 65 553-token sequence: 1025 partials per
    # (head) row, the last of 17 tokens, so the combine runs 17 chunks of 64
    lens = [65536 + 17]
    case = synth.build_case("parts1025", lens=lens, block_size=832, seed=71, device="cuda")
    ref, _ = oracle_case(case)
    prm = params_of(case, 64)
    assert pkv.plan(prm)["num_partitions"] == 1025
    out32 = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    print("[gpu] one sequence, P=64, 1025 partitions", flush=True)
    out = run_decode(case, 64, out_f32=out32)
    assert_rows_rel(f64(out32), ref, what="1025 partitions fp32")
    assert_bf16_close(out, ref, what="1025 partitions")


@pytest.mark.parametrize("bsz", [4096, 16384])
def test_pages_larger_than_any_partition(bsz):
    # a page holds several partitions (and, at 16384, a whole sequence or
    # more): the walkers stay inside one page for many blocks, and the page
    # stride is 16 M elements at 16384 tokens per page
    lens = [1, 4095, 4097, 20000, 16384]
    case = synth.build_case(f"bigpage{bsz}", lens=lens, block_size=bsz, seed=72, device="cuda")
    ref, _ = oracle_case(case)
    for ptok in (0, 256, 4096):
        print(f"[gpu] B={bsz} P={ptok}", flush=True)
        assert_bf16_close(run_decode(case, ptok), ref, what=f"B={bsz} P={ptok}")


def test_partials_and_fp32_output():
    case = synth.build_case("parts", lens=[1, 300, 4097, 5000, 64], block_size=784, seed=31,
                            device="cuda")
    ptok = 1024
    o_p, lse_p, out32, out = pkv.decode_partials(
        case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens, case.block_size,
        case.scale, partition_tokens=ptok, max_seq_len=case.max_seq_len)
    torch.cuda.synchronize()
    o_p, lse_p, out32 = f64(o_p), f64(lse_p), f64(out32)
    q = f64(case.q)
    worst = 0.0
    for s in range(case.num_seqs):
        k, v = f64(case.keys(s)), f64(case.values(s))
        ref_p, ref_lse = od.decode_partials(q[s], k, v, case.scale, ptok)
        n = ref_p.shape[1]
        worst = max(worst, assert_rows_rel(o_p[s, :, :n], ref_p, what=f"o_partial s={s}"))
        assert np.all(np.abs(lse_p[s, :, :n] - ref_lse) <= 1e-4 * np.maximum(1, np.abs(ref_lse)))
        # partitions past the sequence are not written
        assert np.all(o_p[s, :, n:] == 0) and np.all(np.isnan(lse_p[s, :, n:]))
        ref_o, _ = od.attention_decode(q[s], k, v, case.scale)
        assert_rows_rel(out32[s], ref_o, what=f"out_f32 s={s}")
    assert_bf16_close(out, oracle_case(case)[0], what="partials bf16")
    print(f"[gpu] worst fp32 partial row rel err {worst:.2e}", flush=True)


def test_combine_entry_point_on_oracle_partials():
    # The combine kernel alone, fed partials computed by the oracle.
    case = synth.build_case("comb", lens=[700, 4097, 1], block_size=832, seed=32, device="cuda")
    ptok = 512
    prm = params_of(case, ptok)
    n_max = pkv.plan(prm)["num_partitions"]
    q = f64(case.q)
    o_p = np.zeros((3, 24, n_max, 256))
    lse_p = np.zeros((3, 24, n_max))
    for s in range(3):
        a, b = od.decode_partials(q[s], f64(case.keys(s)), f64(case.values(s)), case.scale, ptok)
        o_p[s, :, :a.shape[1]] = a
        lse_p[s, :, :a.shape[1]] = b
    o_dev = torch.from_numpy(o_p).float().cuda()
    lse_dev = torch.from_numpy(lse_p).float().cuda()
    out = torch.empty_like(case.q)
    out32 = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    pkv.combine(prm, o_dev, lse_dev, case.seq_lens, out=out, out_f32=out32)
    torch.cuda.synchronize()
    ref = oracle_case(case)[0]
    for s in range(3):
        assert_rows_rel(f64(out32)[s], ref[s], what=f"combine s={s}")
    assert_bf16_close(out, ref, what="combine bf16")


def test_invariant_to_page_size_and_permutation_bitwise():
    outs = []
    for bsz in (64, 784, 832):
        for seed in (41, 42, 43):
            # same logical tokens (drawn from seed 40), different pool permutations
            base = synth.build_case("inv", lens=[3000, 1234], block_size=bsz, seed=40)
            g = torch.Generator().manual_seed(seed)
            pool = base.pool_pages
            perm = torch.randperm(pool, generator=g)
            k = base.k_cache.clone()
            v = base.v_cache.clone()
            k[perm] = base.k_cache[:pool]
            v[perm] = base.v_cache[:pool]
            tbl = base.block_table.clone()
            real = tbl < pool
            tbl[real] = perm[tbl[real].long()].int()
            out = pkv.decode(base.q.cuda(), k.cuda(), v.cuda(), tbl.cuda(), base.seq_lens.cuda(),
                             bsz, base.scale, partition_tokens=256, max_seq_len=base.max_seq_len)
            torch.cuda.synchronize()
            outs.append(bits(out))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    assert_bf16_close(torch.from_numpy(outs[0].view(np.int16)).view(torch.bfloat16),
                      oracle_case(base)[0], what="invariance")


def test_repeat_runs_bitwise_and_direct_path():
    case = synth.build_case("rep", lens=[2000, 65, 1], block_size=832, seed=51, device="cuda")
    a = bits(run_decode(case, 192))
    b = bits(run_decode(case, 192))
    assert np.array_equal(a, b)
    ref = oracle_case(case)[0]
    direct = run_decode(case, 2048)          # one partition: the split kernel writes out itself
    assert pkv.plan(params_of(case, 2048))["num_partitions"] == 1
    assert_bf16_close(direct, ref, what="direct path")


def test_empty_sequences_give_zero_rows():
    case = synth.build_case("empty", lens=[0, 100, 0], block_size=64, seed=52, device="cuda")
    ref = oracle_case(case, seqs=[1])[0]
    for ptok in (64, 4096):
        out = run_decode(case, ptok)
        o = f64(out)
        assert np.all(o[0] == 0) and np.all(o[2] == 0)
        assert_bf16_close(out, ref, rows=[1], what=f"empty P={ptok}")


# ------------------------------------------------------------ the five workloads

@pytest.mark.parametrize("name", ["long_l8192_b832", "long_l16384_b832", "long_l32768_b832"])
def test_long_sequence_workloads(name):
    case = synth.make_case(name, device="cuda")
    ref, _ = oracle_case(case)
    for ptok in (0, 512):
        print(f"[gpu] {name} P={ptok}", flush=True)
        assert_bf16_close(run_decode(case, ptok), ref, what=f"{name} P={ptok}")


def test_page784_vs_page832_ab():
    a = synth.make_case("ab_l32768_b784", device="cuda")
    b = synth.make_case("ab_l32768_b832", device="cuda")
    oa, ob = run_decode(a), run_decode(b)
    assert np.array_equal(bits(oa), bits(ob)), "page784 and page832 outputs differ"
    ref, _ = oracle_case(a)
    assert_bf16_close(oa, ref, what="ab784")


def test_batched_long_context_workload():
    case = synth.make_case("batched_8seq_t131072_b832", device="cuda")
    out32 = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    out = run_decode(case, out_f32=out32)
    print(f"[gpu] batched plan {pkv.plan(params_of(case))}", flush=True)
    ref, _ = oracle_case_parallel(case)
    assert_bf16_close(out, ref, what="batched")
    assert_rows_rel(f64(out32), ref, what="batched fp32")


def test_wide_serving_batch_every_sequence():
    # all 64 sequences (about 2.2 M tokens) against the oracle, which runs on
    # the host's cores; bf16 output elementwise and the fp32 output per row
    case = synth.make_case("wide_64seq_b832_p4096", device="cuda")
    assert case.partition_tokens == 4096
    out32 = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    out = run_decode(case, out_f32=out32)
    print(f"[gpu] wide: {case.num_seqs} sequences, {sum(case.lens)} tokens, oracle on host",
          flush=True)
    ref, _ = oracle_case_parallel(case)
    assert_bf16_close(out, ref, what="wide")
    worst = assert_rows_rel(f64(out32), ref, what="wide fp32")
    print(f"[gpu] wide: worst fp32 row rel err {worst:.2e}", flush=True)
    # the same batch with the partition size left to the library: its balanced
    # split, whose page offsets also pass 2^31 elements
    prm = params_of(case, 0)
    assert pkv.plan(prm)["balanced"] == 1
    out32b = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    outb = run_decode(case, 0, out_f32=out32b)
    assert_bf16_close(outb, ref, what="wide, balanced")
    worst = assert_rows_rel(f64(out32b), ref, what="wide, balanced fp32")
    print(f"[gpu] wide, balanced: worst fp32 row rel err {worst:.2e}", flush=True)


# ------------------------------------------------------------ other KV head counts

# finite, different heads made from the case's 4: the rows themselves, their
# dims reversed, rotated by one, and reversed then rotated by three
HEAD_TRANSFORMS = [lambda t: t, lambda t: t.flip(-1), lambda t: t.roll(1, -1),
                   lambda t: t.flip(-1).roll(3, -1)]


def heads_variant(case, hkv):
    """The case's pages with hkv KV heads (6 query heads each): the first hkv
    heads for hkv <= 4; for 8 and 16, the 4 heads followed by transformed
    copies (HEAD_TRANSFORMS), with q's head groups transformed alike. Returns
    (q, k_cache, v_cache, keys(s), values(s)) with the same block table."""
    def widen(t):
        if hkv <= 4:
            return t[..., :hkv, :].contiguous()
        return torch.cat([f(t) for f in HEAD_TRANSFORMS[:hkv // 4]], dim=-2).contiguous()
    q = case.q[:, :6 * hkv].contiguous() if hkv <= 4 else torch.cat(
        [f(case.q) for f in HEAD_TRANSFORMS[:hkv // 4]], dim=1).contiguous()
    return (q, widen(case.k_cache), widen(case.v_cache), lambda s: widen(case.keys(s)),
            lambda s: widen(case.values(s)))


@pytest.mark.parametrize("hkv", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("ptok", [0, 256])
def test_other_kv_head_counts(hkv, ptok):
    # the balanced split (P = 0) and ordered fixed partitions, Hq = 6 Hkv
    case = synth.build_case(f"hkv{hkv}", lens=[3000, 1, 833, 0, 2500], block_size=784,
                            seed=85, device="cuda")
    q, kc, vc, keys, values = heads_variant(case, hkv)
    assert q.shape[1] == 6 * hkv and kc.shape[2] == hkv
    out32 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    out = pkv.decode(q, kc, vc, case.block_table, case.seq_lens, case.block_size, case.scale,
                     partition_tokens=ptok, max_seq_len=case.max_seq_len, out_f32=out32)
    torch.cuda.synchronize()
    prm = pkv.make_params(q, kc, vc, case.block_table, case.block_size, case.scale,
                          case.max_seq_len, ptok)
    info = pkv.plan(prm)
    assert info["balanced"] == (1 if ptok == 0 else 0)
    qd = f64(q)
    for s, n in enumerate(case.lens):
        if n == 0:
            assert np.all(f64(out)[s] == 0)
            continue
        ref, _ = od.attention_decode(qd[s], f64(keys(s)), f64(values(s)), case.scale)
        assert_bf16_close(out[s], ref, what=f"Hkv={hkv} P={ptok} s={s}")
        assert_rows_rel(f64(out32)[s], ref, what=f"Hkv={hkv} P={ptok} s={s} fp32")
    # the walker with this row stride, bit-exact
    table = case.block_table.cpu().numpy()
    for g in range(hkv):
        got = pkv.debug_resolve(prm, g, case.block_table, case.seq_lens).cpu().numpy()
        ref = od.resolve_offsets(table, case.lens, case.block_size, kc.stride(0), hkv, 256, g,
                                 case.max_seq_len)
        assert np.array_equal(got, ref), (hkv, ptok, g)


# ------------------------------------------------------------ fixed partitions, ordered

def test_fixed_partitions_ordered_dispatch_edge_cases():
    # More than 64 sequences (the per-workgroup prefix sums take several
    # chunks), lengths that are exact multiples of P (no last partition),
    # shorter than P (no full partition), empty, and one token.
    rng = np.random.default_rng(81)
    lens = [int(x) for x in rng.integers(0, 3000, size=300)]
    lens[:8] = [0, 1, 512, 1024, 511, 513, 2048, 0]
    case = synth.build_case("ord300", lens=lens, block_size=784, seed=81, device="cuda")
    prm = params_of(case, 512)
    info = pkv.plan(prm)
    assert info["ordered"] == 1 and info["k_rows"] == 1 and info["balanced"] == 0
    out32 = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    out = run_decode(case, 512, out_f32=out32)
    live = [s for s, n in enumerate(lens) if n > 0]
    ref, _ = oracle_case_parallel(case, seqs=live)
    assert_bf16_close(out, ref, rows=live, what="ordered 300 seqs")
    assert_rows_rel(f64(out32)[live], ref[live], what="ordered 300 seqs fp32")
    for s, n in enumerate(lens):
        if n == 0:
            assert np.all(f64(out)[s] == 0)
    # the ordered walk, bit-exact
    for _ in check_resolve(case, prm, heads=[1, 2]):
        pass


def test_fixed_partitions_ordered_at_the_batch_limit():
    # 1024 sequences, the most the ordered dispatch takes: every thread of a
    # workgroup scans four lengths
    rng = np.random.default_rng(83)
    lens = [int(x) for x in rng.integers(0, 900, size=1024)]
    case = synth.build_case("ord1024", lens=lens, block_size=832, seed=83, device="cuda")
    prm = params_of(case, 256)
    assert pkv.plan(prm)["ordered"] == 1
    out = run_decode(case, 256)
    live = [s for s, n in enumerate(lens) if n > 0]
    ref, _ = oracle_case_parallel(case, seqs=live)
    assert_bf16_close(out, ref, rows=live, what="ordered 1024 seqs")
    assert all(np.all(f64(out)[s] == 0) for s, n in enumerate(lens) if n == 0)


def test_balanced_split_at_the_batch_limit():
    # 4096 sequences, the most the balanced split takes (sixteen lengths per
    # thread in its prefix scan)
    rng = np.random.default_rng(84)
    lens = [int(x) for x in rng.integers(0, 200, size=4096)]
    case = synth.build_case("bal4096", lens=lens, block_size=64, seed=84, device="cuda")
    prm = params_of(case, 0)
    assert pkv.plan(prm)["balanced"] == 1
    out, out32 = run_balanced(case)
    live = [s for s, n in enumerate(lens) if n > 0]
    ref, _ = oracle_case_parallel(case, seqs=live)
    assert_bf16_close(out, ref, rows=live, what="balanced 4096 seqs")
    assert_rows_rel(f64(out32)[live], ref[live], what="balanced 4096 seqs fp32")


def test_serving_batch_every_sequence():
    # 1024 sequences of 256 to 4096 tokens (2.2 M tokens), the partition size
    # left to the library (the balanced split)
    case = synth.make_case("serving_1024seq_b832", device="cuda")
    assert pkv.plan(params_of(case, 0))["balanced"] == 1
    out = run_decode(case)
    ref, _ = oracle_case_parallel(case)
    assert_bf16_close(out, ref, what="serving batch")


def test_fixed_partitions_beyond_the_ordered_limit_use_grid_order():
    rng = np.random.default_rng(82)
    lens = [int(x) for x in rng.integers(1, 700, size=1100)]
    case = synth.build_case("grid1100", lens=lens, block_size=832, seed=82, device="cuda")
    prm = params_of(case, 256)
    assert pkv.plan(prm)["ordered"] == 0
    out = run_decode(case, 256)
    ref, _ = oracle_case_parallel(case)
    assert_bf16_close(out, ref, what="grid order 1100 seqs")


# ------------------------------------------------------------ balanced split

def run_balanced(case, max_seq_len=None):
    """pkv_decode with the partition size left to the library (balanced)."""
    out32 = torch.empty(case.q.shape, dtype=torch.float32, device=case.q.device)
    out = pkv.decode(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                     case.block_size, case.scale, partition_tokens=0,
                     max_seq_len=max_seq_len or max(case.max_seq_len, 1), out_f32=out32)
    torch.cuda.synchronize()
    return out, out32


@pytest.mark.parametrize("lens,bsz", [
    ([3000, 1234, 64, 65, 1], 832),
    ([2000, 1, 1, 1], 64),          # far fewer tiles than planned workgroups
    ([5000, 0, 777, 0], 784),       # empty sequences inside the batch
])
def test_balanced_split_fp32_and_bf16(lens, bsz):
    case = synth.build_case("bal", lens=lens, block_size=bsz, seed=61, device="cuda")
    prm = params_of(case, 0)
    assert pkv.plan(prm)["balanced"] == 1
    out, out32 = run_balanced(case)
    ref, _ = oracle_case(case)
    got32 = f64(out32)
    for s, n in enumerate(lens):
        if n == 0:
            assert np.all(got32[s] == 0) and np.all(f64(out)[s] == 0)
        else:
            assert_rows_rel(got32[s], ref[s], what=f"balanced fp32 s={s}")
    assert_bf16_close(out, ref, rows=[s for s, n in enumerate(lens) if n > 0],
                      what=f"balanced {lens}")


def test_balanced_split_many_sequences():
    rng = np.random.default_rng(62)
    lens = [int(x) for x in rng.integers(1, 700, size=300)]
    case = synth.build_case("bal300", lens=lens, block_size=832, seed=62, device="cuda")
    out, out32 = run_balanced(case)
    ref, _ = oracle_case(case)
    assert_rows_rel(f64(out32), ref, what="balanced 300 seqs fp32")
    assert_bf16_close(out, ref, what="balanced 300 seqs")


def test_balanced_split_page_list_refetch():
    # 16-token pages and long sequences: a workgroup's run spans more than 64
    # pages, so the walker refetches its page list inside the loop
    case = synth.build_case("balrf", lens=[150000, 150000], block_size=16, seed=63, device="cuda")
    prm = params_of(case, 0)
    assert pkv.plan(prm)["balanced"] == 1
    out, out32 = run_balanced(case)
    ref, _ = oracle_case(case)
    assert_rows_rel(f64(out32), ref, what="balanced refetch fp32")
    assert_bf16_close(out, ref, what="balanced refetch")


def test_balanced_split_page_size_invariant_bitwise():
    outs = []
    for bsz in (64, 784, 832):
        case = synth.build_case("balinv", lens=[3000, 1234, 700], block_size=bsz, seed=64,
                                device="cuda")
        out, _ = run_balanced(case, max_seq_len=3000)
        outs.append(bits(out))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("nseq", [3, 70])
def test_balanced_split_and_combine_entry_points_match_decode(nseq):
    # the two halves of pkv_decode, called on their own, give its exact bits;
    # 70 sequences (280 runs) take the combine with one wave per run
    lens = [3000, 1234, 64] if nseq == 3 else [int(x) for x in
                                               np.random.default_rng(66).integers(1, 2000, nseq)]
    case = synth.build_case("balhalves", lens=lens, block_size=832, seed=65, device="cuda")
    prm = params_of(case, 0)
    info = pkv.plan(prm)
    assert info["balanced"] == 1
    assert info["combine_workgroups"] == (nseq * 4 if nseq * 4 >= 256 else nseq * 24 * 4)
    if nseq > 3:
        ref, _ = oracle_case_parallel(case)
        out_ref, _ = run_balanced(case)
        assert_bf16_close(out_ref, ref, what="balanced 70 seqs")
    out, out32 = run_balanced(case)
    ws = torch.empty(pkv.workspace_bytes(prm), dtype=torch.uint8, device="cuda")
    pkv.split_balanced(prm, case.q, case.k_cache, case.v_cache, case.block_table,
                       case.seq_lens, ws)
    o2 = torch.empty_like(case.q)
    o2_32 = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    pkv.combine_balanced(prm, case.seq_lens, ws, out=o2, out_f32=o2_32)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o2), bits(out))
    assert torch.equal(o2_32, out32)
