"""Pins for the CPU oracle: closed forms, brute force, a library routine, fixtures.

Each check below pins the oracle to something other than itself. The mutation
tests at the end plant plausible mistakes in copies of the oracle and show that
at least one pin fails for each.
"""

import math

import mpmath
import numpy as np
import pytest
import torch

import oracle
from oracle import decode as od
from tests.conftest import read_golden

RNG = np.random.default_rng(12345)


def bf16_round(x):
    """Random test data on the bf16 grid (so it matches what the kernels see)."""
    return od.bf16_bits_to_f64(od.f64_to_bf16_bits(x))


def rand_case(length, hq=24, hkv=4, d=256, rng=RNG, scale_v=1.0):
    q = bf16_round(rng.standard_normal((hq, d)) * scale_v)
    k = bf16_round(rng.standard_normal((length, hkv, d)) * scale_v)
    v = bf16_round(rng.standard_normal((length, hkv, d)) * scale_v)
    return q, k, v


# ---------------------------------------------------------------- pin helpers
# Each helper takes a decode function fn(q, keys, values, scale) -> (o, lse)
# and raises AssertionError when fn disagrees with the closed form.

def pin_all_equal_keys(fn):
    # Identical keys give identical scores, so the weights are uniform and the
    # output is the arithmetic mean of the values (any scale).
    q, k, v = rand_case(37)
    k[:] = k[0:1]
    o, _ = fn(q, k, v, 1.0 / 16)
    for h in range(24):
        g = h // 6
        mean = np.array([math.fsum(v[:, g, d]) / 37 for d in range(256)])
        np.testing.assert_allclose(o[h], mean, rtol=0, atol=1e-12)


def pin_scale_zero(fn):
    q, k, v = rand_case(19)
    o, lse = fn(q, k, v, 0.0)
    for h in range(24):
        np.testing.assert_allclose(o[h], v[:, h // 6, :].sum(0) / 19, atol=1e-12)
        assert abs(lse[h] - math.log(19)) < 1e-12


def pin_all_equal_values(fn):
    q, k, v = rand_case(23)
    v[:] = v[0:1]
    o, _ = fn(q, k, v, 1.0 / 16)
    for h in range(24):
        np.testing.assert_allclose(o[h], v[0, h // 6], atol=1e-12)


def pin_one_hot(fn):
    # Make the 6 query rows of each group equal to u_g and key j = 8 u_g: that
    # score is 8 |u_g|^2 / 16, about 128, while every other is a few units,
    # so the softmax puts all but ~L e^-100 of its mass on token j.
    q, k, v = rand_case(50)
    j = 29
    for g in range(4):
        u = q[6 * g]
        q[6 * g: 6 * g + 6] = u
        k[j, g] = 8.0 * u
    o, lse = fn(q, k, v, 1.0 / 16)
    for h in range(24):
        g = h // 6
        np.testing.assert_allclose(o[h], v[j, g], atol=1e-30 + 50 * math.exp(-60))
        s_j = math.fsum(q[h] * k[j, g]) / 16
        assert abs(lse[h] - s_j) < 1e-9


def pin_single_token(fn):
    q, k, v = rand_case(1)
    o, lse = fn(q, k, v, 1.0 / 16)
    for h in range(24):
        g = h // 6
        assert np.array_equal(o[h], v[0, g])
        assert abs(lse[h] - math.fsum(q[h] * k[0, g]) / 16) < 1e-13


def pin_gqa_mapping(fn):
    # Equal keys (uniform weights) and a constant value per KV head: query head
    # h must return the constant of KV head h // 6.
    q, k, v = rand_case(9)
    k[:] = k[0:1]
    for g in range(4):
        v[:, g, :] = 10.0 * (g + 1)
    o, _ = fn(q, k, v, 1.0 / 16)
    for h in range(24):
        np.testing.assert_allclose(o[h], 10.0 * (h // 6 + 1), atol=1e-12)


def brute_force_mp(q, k, v, scale, heads):
    """Direct one-pass evaluation at 50 decimal digits (no max shift)."""
    mpmath.mp.dps = 50
    hq, d = q.shape
    length, hkv, _ = k.shape
    group = hq // hkv
    res = {}
    for h in heads:
        g = h // group
        qs = [mpmath.mpf(float(x)) for x in q[h]]
        w = []
        for t in range(length):
            s = mpmath.fsum(qs[i] * mpmath.mpf(float(k[t, g, i])) for i in range(d))
            w.append(mpmath.exp(s * mpmath.mpf(scale)))
        den = mpmath.fsum(w)
        o = [mpmath.fsum(w[t] * mpmath.mpf(float(v[t, g, i])) for t in range(length)) / den
             for i in range(d)]
        res[h] = (np.array([float(x) for x in o]), float(mpmath.log(den)))
    return res


def pin_brute_force(fn, lengths=(1, 2, 3, 5, 17, 63, 64, 65)):
    rng = np.random.default_rng(7)
    for length in lengths:
        q, k, v = rand_case(length, d=32, rng=rng)     # small d keeps mpmath fast
        o, lse = fn(q, k, v, 0.25)
        ref = brute_force_mp(q, k, v, 0.25, heads=(0, 5, 6, 13, 23))
        for h, (o_ref, lse_ref) in ref.items():
            np.testing.assert_allclose(o[h], o_ref, rtol=1e-12, atol=1e-13)
            assert abs(lse[h] - lse_ref) < 1e-12 * max(1.0, abs(lse_ref))


def pin_torch_sdpa(fn):
    # Library routine: torch's scaled_dot_product_attention in float64 on the
    # CPU, with K/V repeated to 24 heads (contiguous groups of 6).
    for length in (1, 64, 333):
        q, k, v = rand_case(length)
        o, _ = fn(q, k, v, 1.0 / 16)
        qt = torch.from_numpy(q)[:, None, :]                       # [24, 1, 256]
        kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(6, 0).contiguous()
        vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(6, 0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, scale=1.0 / 16)[:, 0, :].numpy()
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


ALL_PINS = [pin_all_equal_keys, pin_scale_zero, pin_all_equal_values, pin_one_hot,
            pin_single_token, pin_gqa_mapping, pin_brute_force, pin_torch_sdpa]


# ------------------------------------------------------------------ tests

@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_attention_decode_pins(pin):
    pin(od.attention_decode)


@pytest.mark.parametrize("pin", [pin_all_equal_keys, pin_one_hot, pin_gqa_mapping,
                                 pin_single_token], ids=lambda p: p.__name__)
def test_online_decode_pins(pin):
    pin(lambda q, k, v, s: od.online_decode(q, k, v, s, tile=64))


@pytest.mark.parametrize("tile", [1, 16, 64, 100])
def test_online_matches_brute_force(tile):
    pin_brute_force(lambda q, k, v, s: od.online_decode(q, k, v, s, tile=tile),
                    lengths=(1, 17, 65))


def test_online_equals_two_pass_random():
    q, k, v = rand_case(1000)
    a = od.attention_decode(q, k, v, 1.0 / 16)
    b = od.online_decode(q, k, v, 1.0 / 16, tile=64)
    np.testing.assert_allclose(b[0], a[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(b[1], a[1], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("ptok", [64, 100, 4096])
def test_split_combine_algebra(ptok):
    q, k, v = rand_case(1500)
    o_ref, lse_ref = od.attention_decode(q, k, v, 1.0 / 16)
    o_p, lse_p = od.decode_partials(q, k, v, 1.0 / 16, ptok)
    assert o_p.shape == (24, -(-1500 // ptok), 256)
    o, lse = od.combine_partials(o_p, lse_p)
    np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, atol=1e-13)
    # each partition is the definition on its slice
    o1, l1 = od.attention_decode(q, k[ptok:2 * ptok], v[ptok:2 * ptok], 1.0 / 16) \
        if 1500 > ptok else od.attention_decode(q, k, v, 1.0 / 16)
    idx = 1 if 1500 > ptok else 0
    np.testing.assert_allclose(o_p[:, idx], o1, rtol=1e-13, atol=1e-14)


def test_zero_length():
    q, k, v = rand_case(0)
    o, lse = od.attention_decode(q, k, v, 1.0 / 16)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o_b, lse_b = od.decode_batch(q[None], [k], [v], 1.0 / 16)
    assert np.all(o_b == 0)


def test_decode_batch_sequences_independent():
    rng = np.random.default_rng(3)
    cases = [rand_case(n, rng=rng) for n in (5, 70, 1)]
    q = np.stack([c[0] for c in cases])
    o, lse = od.decode_batch(q, [c[1] for c in cases], [c[2] for c in cases], 1.0 / 16)
    for s, c in enumerate(cases):
        o_s, lse_s = od.attention_decode(c[0], c[1], c[2], 1.0 / 16)
        assert np.array_equal(o[s], o_s) and np.array_equal(lse[s], lse_s)


def test_large_scores_stable():
    # Scores around 1e3 overflow exp() unless the maximum is subtracted first.
    q, k, v = rand_case(40)
    o, lse = od.attention_decode(q * 64, k * 64, v, 1.0 / 16)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    ref = brute_force_mp(q[:, :32] * 64, k[:, :, :32] * 64, v[:, :, :32], 1.0 / 16, heads=(0,))
    o2, lse2 = od.attention_decode(q[:, :32] * 64, k[:, :, :32] * 64, v[:, :, :32], 1.0 / 16)
    np.testing.assert_allclose(o2[0], ref[0][0], rtol=1e-11, atol=1e-12)


# ---- bf16 conversions

def test_bf16_rounding_fixture():
    for val, bits in read_golden("bf16_rounding.txt"):
        x = float.fromhex(val) if val.lower().startswith(("0x", "-0x")) else float(val)
        got = int(od.f64_to_bf16_bits(np.array([x]))[0])
        assert got == int(bits, 16), (val, hex(got), bits)


def test_bf16_rounding_matches_torch_on_fp32_inputs():
    # For values that are exact in fp32, one RNE step from fp64 equals torch's
    # fp32 -> bf16 RNE cast.
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(20000) * 1e38).astype(np.float32),
        rng.integers(0, 2**32, 50000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = od.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_widen_matches_torch():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = od.bf16_bits_to_f64(bits)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    assert od.bf16_bits_to_f64(np.array([0x3F80]))[0] == 1.0
    assert od.bf16_bits_to_f64(np.array([0x0001]))[0] == 2.0 ** -133


def test_bf16_roundtrip_identity():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    vals = od.bf16_bits_to_f64(bits)
    ok = ~np.isnan(vals)
    assert np.array_equal(od.f64_to_bf16_bits(vals[ok]), bits[ok])


# ---- addressing

def test_resolve_offsets_fixture():
    for row in read_golden("address_examples.txt"):
        bsz, stride, table, tok, g, arrow, lp, off, pp, expect = row
        assert arrow == "->"
        table = [int(x) for x in table.split(",")]
        bsz, stride, tok, g = int(bsz), int(stride), int(tok), int(g)
        # the fixture's intermediate columns restate the page's token map
        assert tok // bsz == int(lp) and tok % bsz == int(off) and table[int(lp)] == int(pp)
        offs = od.resolve_offsets(np.array([table]), np.array([tok + 1]), bsz, stride,
                                  4, 256, g, tok + 1)
        assert offs[0, tok] == int(expect), row


def test_resolve_offsets_past_length_is_minus_one():
    offs = od.resolve_offsets(np.array([[2, 0, 1]]), np.array([70]), 64, 65536, 4, 256, 1, 200)
    assert np.all(offs[0, 70:] == -1)
    assert offs[0, 64] == 0 * 65536 + 0 + 256
    assert offs[0, 69] == 5 * 1024 + 256


def test_gather_rows_reads_through_table():
    pool = np.arange(5 * 4 * 2 * 3).reshape(5, 4, 2, 3)      # 5 pages, B=4, Hkv=2, D=3
    rows = od.gather_rows(pool, np.array([[3, 0, 4]]), np.array([10]), 4)[0]
    assert rows.shape == (10, 2, 3)
    assert np.array_equal(rows[0], pool[3, 0])
    assert np.array_equal(rows[5], pool[0, 1])
    assert np.array_equal(rows[9], pool[4, 1])


# ---------------------------------------------------------------- mutants
# Plausible mistakes planted in copies of the oracle: each must fail a pin.

def _mutant(kind):
    def fn(q, keys, values, scale):
        hq, d = q.shape
        length, hkv, _ = keys.shape
        group = hq // hkv
        o = np.zeros((hq, d))
        lse = np.full((hq,), -np.inf)
        for h in range(hq):
            g = h % hkv if kind == "gqa_interleaved" else h // group
            sc = 1.0 if kind == "no_scale" else scale
            s = sc * (keys[:, g, :] @ q[h])
            m = np.max(s)
            w = np.exp(s - m)
            if kind == "drop_last_token":
                w = w.copy()
                w[-1] = 0.0 if length > 1 else w[-1]
            l_sum = np.sum(w)
            vv = values[:, g, :]
            if kind == "values_transposed_head":
                vv = values[:, (g + 1) % hkv, :]
            o[h] = (w @ vv) / l_sum
            lse[h] = (np.log(l_sum) if kind == "lse_no_max" else m + np.log(l_sum))
        return o, lse
    return fn


@pytest.mark.parametrize("kind", ["gqa_interleaved", "no_scale", "drop_last_token",
                                  "values_transposed_head", "lse_no_max"])
def test_pins_catch_planted_mistakes(kind):
    fn = _mutant(kind)
    failures = 0
    for pin in ALL_PINS:
        try:
            pin(fn)
        except AssertionError:
            failures += 1
    assert failures >= 1, f"no pin caught mutant {kind}"


def test_mutant_harness_is_faithful():
    # The unmutated copy passes every pin, so the failures above come from the
    # planted mistakes and not from the copy itself.
    fn = _mutant("none")
    for pin in ALL_PINS:
        pin(fn)
