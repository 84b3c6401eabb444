"""The seeded input generator: determinism, shapes and planted needles."""
import numpy as np

import synth


def test_streams_are_deterministic_and_distinct():
    sp = synth.Spec("t", n_seq=2, t_cap=100, q_pos=[99, 50], q_seq=[0, 1], kv_format="fp4",
                    k=8, window=4, schedule=synth.repeating_schedule(3), needles=3, seed=5)
    a = synth.make_inputs(sp)
    b = synth.make_inputs(sp)
    for f in ("kv", "k_idx", "q", "q_idx", "local_k", "local_v"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert not np.array_equal(a.kv[0], a.kv[1])
    assert not np.array_equal(a.q[0], a.q[1])
    assert not np.array_equal(a.local_k, a.local_v)


def test_needles_scale_main_k_and_indexer_key_by_four():
    sp = synth.Spec("t", n_seq=1, t_cap=64, q_pos=[63], q_seq=[0], kv_format="bf16", k=8,
                    window=4, needles=5, seed=9)
    x = synth.make_inputs(sp)
    plain = synth.make_inputs(synth.Spec(**{**sp.__dict__, "needles": 0}))
    pos = x.needle_pos[0]
    assert pos.size == 5 and np.unique(pos).size == 5
    f = synth.bf16_bits_to_f32
    np.testing.assert_array_equal(f(x.kv[0, pos, :128]), 4 * f(plain.kv[0, pos, :128]))
    np.testing.assert_array_equal(f(x.kv[0, pos, 128:]), f(plain.kv[0, pos, 128:]))
    np.testing.assert_array_equal(f(x.k_idx[0, pos]), 4 * f(plain.k_idx[0, pos]))
    rest = np.setdiff1d(np.arange(64), pos)
    np.testing.assert_array_equal(x.kv[0, rest], plain.kv[0, rest])


def test_named_configs_shapes():
    assert synth.config(3).schedule.count(synth.FULL) == 1
    assert synth.config(3).n_layers == 20
    c5 = synth.config(5)
    assert c5.nq == 4096 and c5.q_pos[0] == 126976 and c5.q_pos[-1] == 131071
    assert c5.local_cap >= 131071 - (126976 - 127) + 1
    assert synth.config(4).pool == 16384


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e38], np.float32)
    b = synth.f32_to_bf16_bits(x)
    assert b[0] == 0x3F80
    assert b[1] == 0x3F80          # exact tie -> even
    assert b[2] == 0x3F81          # above the tie
    assert b[3] == 0xC020
