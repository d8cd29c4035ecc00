"""Pins for oracle/prefill.py (tail-Q causal prefill).

Each check ties the oracle to something other than itself: the decode oracle
(pinned on its own) applied to each query's causal prefix, torch's fp64
scaled-dot-product attention with an explicit mask, a 50-digit brute force,
closed forms of the causal mean, and planted mistakes that must fail.
"""

import numpy as np
import pytest
import torch

from oracle import decode as od
from oracle import prefill as op


def rand_case(rng, nq, length, hkv=2, d=32, group=6):
    q = rng.standard_normal((nq, hkv * group, d))
    k = rng.standard_normal((length, hkv, d))
    v = rng.standard_normal((length, hkv, d))
    return q, k, v


def pin_row_by_row_decode(fn):
    rng = np.random.default_rng(1)
    for nq, length in ((1, 1), (2, 2), (5, 9), (64, 64), (7, 200)):
        q, k, v = rand_case(rng, nq, length)
        o, lse = fn(q, k, v, 0.25)
        for i in range(nq):
            p = length - nq + i
            ro, rl = od.attention_decode(q[i], k[: p + 1], v[: p + 1], 0.25)
            np.testing.assert_allclose(o[i], ro, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[i], rl, rtol=1e-12, atol=1e-12)


def pin_torch_sdpa(fn):
    rng = np.random.default_rng(2)
    for nq, length in ((3, 3), (16, 40), (33, 33)):
        q, k, v = rand_case(rng, nq, length)
        o, _ = fn(q, k, v, 0.125)
        tq = torch.from_numpy(q).permute(1, 0, 2)                        # [Hq, Q, D]
        tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(6, 0)
        tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(6, 0)
        pos = torch.arange(length - nq, length)
        mask = torch.arange(length)[None, :] <= pos[:, None]             # bottom-right causal
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                               scale=0.125)
        np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def pin_causal_mean(fn):
    # all keys equal: every visible token gets the same weight, so query i
    # returns the mean of V over its prefix 0 .. L - Q + i
    rng = np.random.default_rng(3)
    nq, length = 6, 11
    q = rng.standard_normal((nq, 6, 8))
    k = np.ones((length, 1, 8))
    v = rng.standard_normal((length, 1, 8))
    o, lse = fn(q, k, v, 0.5)
    for i in range(nq):
        p = length - nq + i
        np.testing.assert_allclose(o[i], np.repeat(v[: p + 1, 0].mean(0)[None], 6, 0), atol=1e-13)
        np.testing.assert_allclose(lse[i], 0.5 * q[i].sum(1) + np.log(p + 1), atol=1e-12)


def pin_brute_force(fn):
    import mpmath
    mpmath.mp.dps = 50
    rng = np.random.default_rng(4)
    nq, length, d = 3, 5, 4
    q, k, v = rand_case(rng, nq, length, hkv=1, d=d)
    o, lse = fn(q, k, v, 0.7)
    for i in range(nq):
        p = length - nq + i
        for h in range(6):
            s = [mpmath.mpf(0.7) * mpmath.fsum(mpmath.mpf(q[i, h, j]) * mpmath.mpf(k[t, 0, j])
                                              for j in range(d)) for t in range(p + 1)]
            z = mpmath.fsum(mpmath.e ** x for x in s)
            for j in range(d):
                ref = mpmath.fsum(mpmath.e ** s[t] * mpmath.mpf(v[t, 0, j]) for t in range(p + 1)) / z
                assert abs(o[i, h, j] - float(ref)) < 1e-13
            assert abs(lse[i, h] - float(mpmath.log(z))) < 1e-13


ALL_PINS = [pin_row_by_row_decode, pin_torch_sdpa, pin_causal_mean, pin_brute_force]


@pytest.mark.parametrize("pin", ALL_PINS)
def test_oracle_pin(pin):
    pin(op.attention_prefill)


def test_q1_is_decode_over_the_whole_sequence():
    rng = np.random.default_rng(5)
    q, k, v = rand_case(rng, 1, 300, hkv=4, d=64)
    o, lse = op.attention_prefill(q, k, v, 1 / 8)
    ro, rl = od.attention_decode(q[0], k, v, 1 / 8)
    np.testing.assert_allclose(o[0], ro, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse[0], rl, rtol=1e-13, atol=1e-13)


def test_selected_rows_match_full_computation():
    rng = np.random.default_rng(6)
    q, k, v = rand_case(rng, 40, 100)
    full, full_lse = op.attention_prefill(q, k, v, 0.3, block=7)
    part, part_lse = op.attention_prefill(q, k, v, 0.3, rows=[0, 13, 39])
    for i in range(40):
        if i in (0, 13, 39):
            np.testing.assert_array_equal(part[i], full[i])
            np.testing.assert_array_equal(part_lse[i], full_lse[i])
        else:
            assert not part[i].any()


def test_query_positions():
    assert op.query_positions(3, 10).tolist() == [7, 8, 9]
    assert op.query_positions(1, 1).tolist() == [0]
    with pytest.raises(ValueError):
        op.query_positions(5, 4)


# ---------------------------------------------------------------- mutation tests

def _mutant(kind):
    def fn(q, keys, values, scale, rows=None, block=256):
        nq, hq, d = q.shape
        length, hkv, _ = keys.shape
        group = hq // hkv
        o = np.zeros((nq, hq, d))
        lse = np.zeros((nq, hq))
        t = np.arange(length)
        for i in range(nq):
            p = length - nq + i
            if kind == "top_left":
                limit = i
            elif kind == "exclusive":
                limit = p - 1
            elif kind == "one_more":
                limit = min(p + 1, length - 1)
            elif kind == "no_mask":
                limit = length - 1
            else:
                limit = p
            vis = t <= limit
            for h in range(hq):
                g = (h % hkv) if kind == "gqa_interleaved" else h // group
                s = scale * (keys[:, g, :] @ q[i, h])
                s = np.where(vis, s, -np.inf)
                m = s.max()
                w = np.exp(s - m)
                o[i, h] = (w @ values[:, g, :]) / w.sum()
                lse[i, h] = m + np.log(w.sum())
        return o, lse
    return fn


@pytest.mark.parametrize("kind", ["top_left", "exclusive", "one_more", "no_mask",
                                  "gqa_interleaved"])
def test_planted_mistake_is_caught(kind):
    fn = _mutant(kind)
    failed = 0
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed >= 1, kind


def test_mutant_harness_is_faithful():
    fn = _mutant("none")
    for pin in ALL_PINS:
        pin(fn)
