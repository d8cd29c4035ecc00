"""Pins for the finalizer part of oracle/compress.py (RMSNorm, NOPE INT8
quantisation, GPT-J RoPE, the byte scatter into a packed KV page).

Each check ties the oracle to something other than itself: hand-derived
quantisation, slot and RoPE-row fixtures, closed forms (a vector whose normalised values
are all +-1, quarter-turn rotations), torch's fp64 RMSNorm, rotation norms and
a full closed-form output. The mutation tests at the end plant plausible
mistakes in copies of the oracle functions and require a pin to fail.
"""

from types import SimpleNamespace

import numpy as np
import pytest
import torch

from oracle import compress as oc
from tests.conftest import read_golden


def impl(**over):
    ns = SimpleNamespace(rms_norm=oc.rms_norm, quant_exponent=oc.quant_exponent,
                         quantize_nope=oc.quantize_nope, rope_gptj=oc.rope_gptj,
                         slot_byte_offsets=oc.slot_byte_offsets,
                         rope_position=oc.rope_position,
                         finalize_output=oc.finalize_output,
                         finalize_outputs=oc.finalize_outputs)
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


def pin_quant_fixture(f):
    for r in read_golden("nope_quant.txt"):
        if r[0] == "exp":
            assert f.quant_exponent(float(r[1])) == int(r[3]), r
            group = np.zeros(448)
            group[5] = float(r[1])                         # this group's amax
            _, scale, e, _ = f.quantize_nope(group)
            assert int(e[0]) == int(r[3]) and int(scale[0]) == int(r[4]), r
        else:
            z, e = float(r[1]), int(r[2])
            group = np.zeros(448)
            group[0] = z
            big = 127 * 2.0 ** e                            # fixes the group's exponent at e
            group[1] = big                                  # 127 * 2^e * fl32(1/127) -> 2^e
            q, _, eg, _ = f.quantize_nope(group)
            assert int(eg[0]) == e, r
            assert int(q[0]) == int(r[5]), r


def pin_slot_fixture(f):
    for r in read_golden("kv_slots.txt"):
        assert f.slot_byte_offsets(int(r[0])) == (int(r[2]), int(r[3]), int(r[4])), r


def pin_rms_norm(f):
    rng = np.random.default_rng(1)
    for _ in range(5):
        c = rng.standard_normal(512) * rng.uniform(0.01, 10)
        w = rng.uniform(0.5, 2.0, 512)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(c)[None], (512,),
                                           torch.from_numpy(w), eps=1e-6)[0].numpy()
        np.testing.assert_allclose(f.rms_norm(c, w, 1e-6), ref, rtol=1e-14, atol=0)
    c = np.full(512, 3.0)                                   # closed form: 3 / sqrt(9 + eps)
    np.testing.assert_allclose(f.rms_norm(c, np.ones(512), 0.25), np.full(512, 3 / np.sqrt(9.25)),
                               rtol=1e-15)


def pin_rope(f):
    rng = np.random.default_rng(2)
    y = np.zeros(512)
    y[448:] = rng.standard_normal(64)
    u, w = y[448::2], y[449::2]
    out = f.rope_gptj(y, np.ones(32), np.zeros(32))         # no rotation
    np.testing.assert_array_equal(out, y[448:])
    out = f.rope_gptj(y, np.zeros(32), np.ones(32))         # a quarter turn: (u, w) -> (-w, u)
    np.testing.assert_array_equal(out[0::2], -w)
    np.testing.assert_array_equal(out[1::2], u)
    th = rng.uniform(-np.pi, np.pi, 32)
    out = f.rope_gptj(y, np.cos(th), np.sin(th))            # lengths of the pairs are kept
    np.testing.assert_allclose(out[0::2] ** 2 + out[1::2] ** 2, u ** 2 + w ** 2, rtol=1e-13)
    one = np.zeros(512)
    one[448 + 2 * 7] = 1.0                                  # pair 7 only: interleaved, not halves
    out = f.rope_gptj(one, np.cos(th), np.sin(th))
    assert np.count_nonzero(out) == 2 and out[14] == np.cos(th[7]) and out[15] == np.sin(th[7])


def pin_closed_form_output(f):
    # c = +-2^3 everywhere: mean c^2 = 64, rho = 1/8 (eps = 0), y = +-1 exactly;
    # every group has amax 1 -> e = -6, q = +-64; the rotation with cos = 0.6,
    # sin = 0.8 gives +-0.6 -+ 0.8 combinations, rounded to bf16
    rng = np.random.default_rng(3)
    sign = rng.choice([-1.0, 1.0], 512)
    c = 8.0 * sign
    cs = np.concatenate([np.full(32, 0.6), np.full(32, 0.8)])
    payload, scale, _ = f.finalize_output(c, np.ones(512), 0.0, cs)
    q = np.where(sign[:448] > 0, 64, 256 - 64)
    assert np.array_equal(payload[:448], q.astype(np.uint8))
    assert np.array_equal(scale, np.array([121] * 7 + [0], dtype=np.uint8))
    u, w = sign[448::2], sign[449::2]
    rot = np.empty(64)
    rot[0::2] = u * 0.6 - w * 0.8
    rot[1::2] = w * 0.6 + u * 0.8
    bits = payload[448:].view("<u2")
    got = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    # |rot| is 1.4 or 0.2; their nearest bf16 values, by hand: 1.4 =
    # 1.0110011|0011..b -> 1.0110011b = 1.3984375 (rounds down); 0.2 =
    # 1.1001100|1100..b * 2^-3 -> 1.1001101b * 2^-3 = 0.2001953125 (rounds up)
    want = np.where(np.abs(rot) > 1, 1.3984375, 0.2001953125) * np.sign(rot)
    assert np.array_equal(got, want)


def pin_rope_rows(f):
    for r in read_golden("rope_rows.txt"):
        assert f.rope_position(int(r[0]), int(r[1])) == int(r[3]), r


def pin_scatter(f):
    rng = np.random.default_rng(4)
    pages = 3
    kv = rng.integers(0, 256, size=(pages, oc.KV_PAGE_BYTES), dtype=np.uint8)
    comp = rng.standard_normal((5, 512))
    cs = rng.standard_normal((300, 64))
    slots = [5, -1, 130, 3 * 64, 63]                      # padding and outside slots write nothing
    pos = [127, 255, 200, 299, 150]
    rows = [0, 128, 128, 256, 128]                        # their RoPE rows at C = 128, by hand
    out = f.finalize_outputs(comp, np.ones(512), 1e-6, cs, pos, 128, slots, kv)
    touched = np.zeros_like(kv, dtype=bool)
    for j, s in enumerate(slots):
        if s < 0 or s >= pages * 64:
            continue
        page, po, so = f.slot_byte_offsets(s)
        payload, scale, _ = f.finalize_output(comp[j], np.ones(512), 1e-6, cs[rows[j]])
        assert np.array_equal(out[page, po:po + 576], payload)
        assert np.array_equal(out[page, so:so + 8], scale)
        touched[page, po:po + 576] = True
        touched[page, so:so + 8] = True
    assert np.array_equal(out[~touched], kv[~touched])


ALL_PINS = [pin_quant_fixture, pin_slot_fixture, pin_rms_norm, pin_rope, pin_closed_form_output,
            pin_rope_rows, pin_scatter]


@pytest.mark.parametrize("pin", ALL_PINS)
def test_oracle_pin(pin):
    pin(impl())


def test_quantised_values_round_trip():
    # q * 2^e reproduces z within one code step, and every code fits int8
    rng = np.random.default_rng(5)
    for scale in (1e-5, 1e-2, 1.0, 300.0):
        y = rng.standard_normal(512) * scale
        q, sb, e, z = oc.quantize_nope(y)
        qi = q.astype(np.int64)
        qi = np.where(qi > 127, qi - 256, qi)
        assert np.all(np.abs(qi) <= 127)
        step = 2.0 ** np.repeat(e, 64)
        assert np.all(np.abs(z - qi * step) < step)
        assert np.all(sb == (e + 127))


# ---------------------------------------------------------------- mutation tests

def _m_floor(y):
    q, sb, e, z = oc.quantize_nope(y)
    qq = np.zeros(448, dtype=np.int64)
    for g in range(7):
        zz = z[g * 64:(g + 1) * 64] * 2.0 ** (-int(e[g]))
        qq[g * 64:(g + 1) * 64] = np.clip(np.floor(zz), -127, 127)
    return (qq % 256).astype(np.uint8), sb, e, z


def _m_no_round_trip(y):
    y = np.asarray(y, dtype=np.float64)
    real = oc.bf16_round
    try:
        oc.bf16_round = lambda x: np.asarray(x, dtype=np.float64)
        return oc.quantize_nope(y)
    finally:
        oc.bf16_round = real


def _m_scale_128(y):
    q, sb, e, z = oc.quantize_nope(y)
    return q, (e + 128).astype(np.uint8), e, z


def _m_exp_floor(a):
    a = max(np.float32(a), np.float32(1e-4))
    return int(np.floor(np.log2(np.float32(a) * np.float32(1 / 127))))


def _m_no_amax_floor(a):
    if a == 0:
        return -1000
    return oc.quant_exponent(a)


def _m_rope_halves(y, cos, sin):
    r = np.asarray(y, dtype=np.float64)[448:512]
    u, w = r[:32], r[32:]
    return np.concatenate([u * cos - w * sin, w * cos + u * sin])


def _m_rope_sign(y, cos, sin):
    return oc.rope_gptj(y, cos, -np.asarray(sin))


def _m_scale_no_base(slot):
    page, po, so = oc.slot_byte_offsets(slot)
    return page, po, so - 64 * 576


def _m_payload_stride(slot):
    page, po, so = oc.slot_byte_offsets(slot)
    return page, (slot % 64) * 584, so


def _m_rms_no_mean(c, w, eps):
    c = np.asarray(c, dtype=np.float64)
    return c / np.sqrt(np.sum(c * c) + eps) * w


MUTANTS = {
    "floor_not_trunc": dict(quantize_nope=_m_floor),
    "no_bf16_round_trip": dict(quantize_nope=_m_no_round_trip),
    "scale_byte_plus_128": dict(quantize_nope=_m_scale_128),
    "exponent_floor": dict(quant_exponent=_m_exp_floor),
    "no_amax_floor": dict(quant_exponent=_m_no_amax_floor),
    "rope_rotate_halves": dict(rope_gptj=_m_rope_halves),
    "rope_sign": dict(rope_gptj=_m_rope_sign),
    "scale_without_payload_base": dict(slot_byte_offsets=_m_scale_no_base),
    "payload_stride_584": dict(slot_byte_offsets=_m_payload_stride),
    "rms_sum_not_mean": dict(rms_norm=_m_rms_no_mean),
}


# Mistakes in the RoPE row are planted in the module itself, so that the
# oracle's own finalize_outputs (which looks the row up per output) uses them.
MODULE_MUTANTS = {
    "rope_row_is_position": dict(rope_position=lambda p, c: int(p)),
    "rope_row_is_chunk_index": dict(rope_position=lambda p, c: int(p) // int(c)),
    "rope_row_is_chunk_end": dict(rope_position=lambda p, c: (int(p) // int(c) + 1) * int(c) - 1),
}


def _count_failing_pins(f):
    failed = 0
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(f)
        except (AssertionError, ValueError, IndexError, OverflowError):
            failed += 1
    return failed


@pytest.mark.parametrize("kind", sorted(MUTANTS))
def test_planted_mistake_is_caught(kind):
    assert _count_failing_pins(impl(**MUTANTS[kind])) >= 1, kind


@pytest.mark.parametrize("kind", sorted(MODULE_MUTANTS))
def test_planted_rope_row_mistake_is_caught(kind, monkeypatch):
    for name, fn in MODULE_MUTANTS[kind].items():
        monkeypatch.setattr(oc, name, fn)
    failed = _count_failing_pins(impl())
    # both the fixture pin and the scatter pin (through finalize_outputs) see it
    assert failed >= 2, (kind, failed)


def test_mutant_harness_is_faithful():
    for pin in ALL_PINS:
        pin(impl())
