"""Pins of the oracle's FP4 cache with one E4M3 scale per 16 channels (the
pages' own form: "DeepSeek-V4.1 Flash Pushes KV Cache Compression for Agent
Workloads", summary and closing paragraph).  E4M3 decoding and the scale
rounding are checked against torch's float8_e4m3fn (a library routine); the
element rounding against the already-pinned E8M0 packer on blocks whose scale
is a power of two, exact round trips, tie points and monotonicity."""
import numpy as np
import torch

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, np.float32))


def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in codes])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.all((ref == got) | both_nan)
    assert set(np.flatnonzero(np.isnan(got)).tolist()) == {0x7F, 0xFF}
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0


def _scale_of_block(amax):
    blk = np.zeros((1, 16), np.uint16)
    blk[0, 0] = bf16([amax])[0]
    _, sc = oracle.fp4e_pack(blk)
    return int(sc[0, 0])


def test_scale_is_amax_over_6_rounded_like_torch():
    rng = np.random.default_rng(1)
    amax = bf16_bits_to_f32(bf16(np.abs(rng.standard_normal(3000)) *
                                 np.exp2(rng.integers(-14, 11, 3000))))
    amax = np.concatenate([amax, bf16_bits_to_f32(bf16([6.375, 6.75, 6 * 2.0 ** -10,
                                                        6 * 1.5 * 2.0 ** -10, 2688.0, 1.0]))])
    for a in amax:
        want = torch.tensor([float(a) / 6.0], dtype=torch.float32).to(torch.float8_e4m3fn)
        want = int(want.view(torch.uint8)[0])
        assert _scale_of_block(float(a)) == want, a
    # exact ties go to the even code: 6.375 / 6 = 1.0625 lies halfway between 1 and 1.125
    assert _scale_of_block(6.375) == 0x38
    # beyond 6 * 448 the scale saturates at 448; below 6 * 2^-10 it is 0
    assert _scale_of_block(3000.0) == 0x7E
    assert _scale_of_block(1e30) == 0x7E and _scale_of_block(3.0e38) == 0x7E
    # and the elements of such a block saturate at 6 * 448
    blk = np.zeros((1, 16), np.uint16)
    blk[0, :3] = bf16([1e30, -5000.0, 1000.0])
    c, sc = oracle.fp4e_pack(blk)
    assert np.array_equal(oracle.fp4e_unpack(c, sc)[0, :3], [2688.0, -2688.0, 896.0])
    assert _scale_of_block(6 * 2.0 ** -11) == 0


def test_power_of_two_scales_reduce_to_the_e8m0_packer():
    """When amax = 6 * 2^k the E4M3 scale is 2^k, the scale the E8M0 packer
    picks for the same block, so both must give the same element codes."""
    rng = np.random.default_rng(2)
    n = 4000
    x = rng.standard_normal((n, 32)).astype(np.float32)
    k = rng.integers(-6, 8, size=(n, 1))
    x = np.clip(x, -5.9, 5.9) * np.exp2(k)
    x[:, 0] = 6.0 * np.exp2(k[:, 0])       # amax of the first half
    x[:, 16] = -6.0 * np.exp2(k[:, 0])     # amax of the second half
    x[::7, 5] = 0.0
    x[::11, 9] = -0.0
    xb = bf16(x)
    c8, _ = oracle.fp4_pack(xb)
    ce, se = oracle.fp4e_pack(xb)
    assert np.array_equal(ce, c8)
    sv = np.array([oracle.e4m3_value(v) for v in se.reshape(-1)]).reshape(se.shape)
    assert np.array_equal(sv, np.exp2(np.repeat(k, 2, axis=1)).astype(np.float64))


def test_round_trip_ties_and_monotonicity():
    rng = np.random.default_rng(3)
    # exactly representable blocks: a scale code and 16 E2M1 values, with the
    # block maximum 6 s so the packer picks that scale back
    blocks, want = [], []
    for sc in rng.integers(0x08, 0x7E, 200):
        s = oracle.e4m3_value(int(sc))
        v = E2M1[rng.integers(0, 8, 16)] * np.where(rng.random(16) < 0.5, -1, 1)
        v[0] = 6.0
        blocks.append(v * s)
        want.append(v * s)
    xb = bf16(np.array(blocks))
    assert np.array_equal(bf16_bits_to_f32(xb).astype(np.float64), np.array(want))
    c, s = oracle.fp4e_pack(xb)
    assert np.array_equal(oracle.fp4e_unpack(c, s), np.array(want))
    # midpoints between neighbouring E2M1 values go to the even code
    mids = (E2M1[:-1] + E2M1[1:]) / 2
    even = [0, 2, 2, 4, 4, 6, 6]
    for m, e in zip(mids, even):
        blk = np.zeros(16)
        blk[0] = 6.0
        blk[1] = m
        c, s = oracle.fp4e_pack(bf16(blk[None]))
        assert s[0, 0] == 0x38 and (c[0, 0] >> 4) == e, (m, c[0, 0] >> 4)
    # larger magnitudes never get a smaller code under one scale
    blk = np.linspace(0, 6.5, 16)
    c, _ = oracle.fp4e_pack(bf16(blk[None]))
    codes = np.array([(c[0, i // 2] >> (4 * (i & 1))) & 7 for i in range(16)])
    assert np.all(np.diff(codes) >= 0) and codes[-1] == 7


def test_dequantised_error_within_half_a_step():
    rng = np.random.default_rng(4)
    x = bf16(rng.standard_normal((500, 64)) * np.exp2(rng.integers(-8, 8, (500, 1))))
    c, s = oracle.fp4e_pack(x)
    d = oracle.fp4e_unpack(c, s)
    xf = bf16_bits_to_f32(x).astype(np.float64).reshape(-1, 16)
    sv = np.array([oracle.e4m3_value(v) for v in s.reshape(-1)])
    # inside [0, 6 s] the nearest grid value is at most half the widest gap
    # (2 s, between 4 s and 6 s) away; beyond 6 s it is 6 s
    err = np.abs(d.reshape(-1, 16) - xf)
    lim = np.maximum(sv[:, None] * 1.0, np.abs(xf) - 6 * sv[:, None])
    assert np.all(err <= lim + 1e-300)
    assert np.array_equal(np.signbit(d), np.signbit(xf.reshape(d.shape)))
