"""Pins of the oracle's FP4 (E2M1 elements, E8M0 per-32 scale) packer and
unpacker against the format's own definition, not against the oracle itself."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def e2m1_from_bits(code: int) -> float:
    """E2M1 from its bit fields: sign, 2-bit exponent (bias 1), 1-bit mantissa."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = (m * 0.5) if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1)
    return -mag if s else mag


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, np.float32))


def nibbles(codes):
    c = np.asarray(codes, np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = c & 15
    out[..., 1::2] = c >> 4
    return out


def test_decode_matches_bit_fields_for_every_code_and_scale():
    # every code in one row of 32 per scale byte; bytes 0..254 (255 is NaN in E8M0)
    codes_row = np.array([c | (c2 << 4) for c, c2 in zip(range(0, 16, 2), range(1, 16, 2))] * 2,
                         np.uint8)
    for byte in range(0, 255):
        out = oracle.fp4_unpack(codes_row[None, :], np.array([[byte]], np.uint8))[0]
        for i in range(32):
            code = i % 16
            want = math.ldexp(e2m1_from_bits(code), byte - 127)
            assert out[i] == want and math.copysign(1, out[i]) == math.copysign(1, want), (byte, code)


def test_midpoints_and_grid_from_fixture():
    g = json.load(open(os.path.join(GOLD, "e2m1_ties.json")))
    anchor = 4.0  # puts the block's largest magnitude in [4, 8): scale exponent 0

    def code_of(y):
        blk = np.zeros(32, np.float32)
        blk[0] = anchor
        blk[1] = y
        blk[2] = -y
        codes, scales = oracle.fp4_pack(bf16(blk)[None, :])
        assert scales[0, 0] == 127
        n = nibbles(codes)[0]
        assert n[2] == (n[1] | 8)  # sign is the only difference
        return int(n[1])

    for y, want in g["grid"]:
        assert code_of(y) == want, y
    for tie, below, at, above in g["midpoints"]:
        t = np.float32(tie)
        assert bf16(t) == f32_to_bf16_bits(np.array([t]))[0]
        lo = float(bf16_bits_to_f32(bf16(t) - np.uint16(1)).reshape(-1)[0])
        hi = float(bf16_bits_to_f32(bf16(t) + np.uint16(1)).reshape(-1)[0])
        assert code_of(lo) == below, tie
        assert code_of(float(tie)) == at, tie
        assert code_of(hi) == above, tie


def _random_blocks(n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 32)).astype(np.float32)
    x *= np.exp2(rng.integers(-140, 120, size=(n, 1))).astype(np.float32)
    x[::17] = 0.0
    x[::19, ::3] = -0.0
    x[5::23, :31] = 0.0  # blocks with a single non-zero element
    return bf16(x)


def test_scale_puts_block_max_in_top_binade():
    """The microscaling rule for E2M1: the block's largest magnitude, divided
    by the power-of-two scale, lands in [4, 8) (the binade of 4 and 6), unless
    the exponent is clamped at -127 (then it is below 8)."""
    xb = _random_blocks(4000, 1)
    codes, scales = oracle.fp4_pack(xb)
    amax = np.abs(bf16_bits_to_f32(xb).astype(np.float64)).max(axis=1)
    E = scales[:, 0].astype(np.int64) - 127
    y = amax * np.exp2(-E.astype(np.float64))
    zero = amax == 0
    assert np.all(scales[zero, 0] == 0)
    clamped = (E == -127) & ~zero
    ok = (y >= 4) & (y < 8)
    assert np.all(ok | clamped | zero)
    assert np.all(y[clamped] < 8)


def test_each_element_is_a_nearest_grid_value():
    xb = _random_blocks(3000, 2)
    codes, scales = oracle.fp4_pack(xb)
    x = bf16_bits_to_f32(xb).astype(np.float64)
    deq = oracle.fp4_unpack(codes, scales)
    grid = np.array([abs(e2m1_from_bits(c)) for c in range(8)])
    scale = np.exp2(scales.astype(np.float64) - 127)
    y = np.abs(x) / scale
    err = np.abs(np.abs(deq) / scale - y)
    best = np.min(np.abs(y[..., None] - grid), axis=-1)
    assert np.all(err == best)
    # sign bit of every element is kept, including -0
    assert np.all((nibbles(codes) >> 3) == np.signbit(x))


def test_round_trip_on_the_representable_grid():
    rng = np.random.default_rng(3)
    n = 2000
    codes = rng.integers(0, 256, size=(n, 16), dtype=np.uint8)
    scales = rng.integers(1, 253, size=(n, 1), dtype=np.uint8)
    deq = oracle.fp4_unpack(codes, scales)
    x = bf16(deq.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f32(x).astype(np.float64), deq)  # exact in bf16
    c2, s2 = oracle.fp4_pack(x)
    deq2 = oracle.fp4_unpack(c2, s2)
    assert np.array_equal(deq2, deq)
    # byte-exact when the block's largest magnitude code is 6 (=4) or 7 (=6)
    top = (nibbles(codes) & 7).max(axis=1)
    sel = top >= 6
    assert sel.sum() > 100
    # -0 and +0 both pack back as given only through the sign bit; compare codes
    assert np.array_equal(c2[sel], codes[sel])
    assert np.array_equal(s2[sel], scales[sel])


def test_every_bf16_pattern_against_fixed_scale():
    """All 65,536 bf16 patterns (finite ones whose magnitude does not exceed
    the anchor), each in a block whose largest element fixes the scale."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        vals = bf16_bits_to_f32(pats).astype(np.float64)
    finite = np.isfinite(vals)
    for E0 in (-130, -20, 0, 9, 100):
        anchor = math.ldexp(6.0, E0)
        sel = finite & (np.abs(vals) <= anchor)
        p = pats[sel]
        blocks = np.zeros((p.size, 32), np.uint16)
        blocks[:, 0] = bf16(np.float32(anchor))
        blocks[:, 1] = p
        codes, scales = oracle.fp4_pack(blocks)
        Ew = max(E0, -127)
        assert np.all(scales[:, 0] == Ew + 127)
        y = np.abs(vals[sel]) * 2.0 ** (-Ew)
        # decision thresholds of round-to-nearest-even on the E2M1 grid
        want = ((y > 0.25).astype(int) + (y >= 0.75) + (y > 1.25) + (y >= 1.75)
                + (y > 2.5) + (y >= 3.5) + (y > 5.0))
        got = nibbles(codes)[:, 1]
        assert np.array_equal(got & 7, want), E0
        assert np.array_equal(got >> 3, np.signbit(vals[sel]).astype(np.uint8))


def test_pack_rejects_bad_dim():
    with pytest.raises(ValueError):
        oracle.fp4_pack(np.zeros((2, 48), np.uint16))
