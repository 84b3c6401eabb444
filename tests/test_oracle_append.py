"""Pins of the oracle's decode append ("CED", section "Why Prefill Recomputes
a Recent Segment": the chosen token's global KV is appended and each layer
updates its local state), through closed forms of the stack that reads it:
a query whose own new key dominates every other key attends (almost) only to
its own position, once through the global selection and once through the
local window, so each layer's output is the mean of the appended global V
and that layer's appended local V."""
import numpy as np

import oracle
import synth
from synth import bf16_bits_to_f32, f32_to_bf16_bits

SCALE = 128 ** -0.5


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, np.float32))


def f64(b):
    return bf16_bits_to_f32(b).astype(np.float64)


def _setup(fp4=False):
    sp = synth.Spec("append", n_seq=3, t_cap=300, q_pos=[299, 150, 17], q_seq=[0, 1, 2],
                    kv_format="fp4" if fp4 else "bf16", k=16, window=8, local_cap=12,
                    schedule=[synth.FULL, synth.REUSE, synth.REUSE], seed=91)
    x = synth.make_inputs(sp)
    rng = np.random.default_rng(3)
    S, L = sp.n_seq, sp.n_layers
    u = bf16(rng.standard_normal((S, 128)))
    # every head of every layer asks the same question u[b]
    q = np.broadcast_to(u[None, :, None, :], (L, S, 16, 128)).copy()
    # exact bf16 products by 4: the new keys dominate by ~45 logits
    k4 = bf16(4.0 * f64(u))
    vg = bf16(rng.standard_normal((S, 128)))
    kv_new = np.concatenate([k4, vg], axis=1)
    kidx_new = bf16(4.0 * f64(x.q_idx[0]))
    k_new = np.broadcast_to(k4[None], (L, S, 128)).copy()
    v_new = bf16(rng.standard_normal((L, S, 128)))
    return sp, x, q, kv_new, kidx_new, k_new, v_new


def _run(sp, x, q, kv, k_idx, lk, lv, fp4):
    c = oracle.Cache(kv, k_idx, fp4=fp4)
    return oracle.stack(c, sp.schedule, x.q_pos, q, x.q_idx, lk, lv, sp.window, sp.lo, sp.k,
                        sp.pool)


def test_append_closed_form_bf16():
    sp, x, q, kv_new, kidx_new, k_new, v_new = _setup()
    kv, k_idx, lk, lv = oracle.append(x.kv, x.k_idx, x.local_k, x.local_v, x.q_pos, kv_new,
                                      kidx_new, k_new, v_new)
    out, sel, _ = _run(sp, x, q, kv, k_idx, lk, lv, False)
    for b, t in enumerate(sp.q_pos):
        assert t in sel[0, b], "the appended key must win the layer-0 scan"
        for l in range(sp.n_layers):
            want = 0.5 * (f64(kv_new[b, 128:]) + f64(v_new[l, b]))
            np.testing.assert_allclose(out[l, b], np.broadcast_to(want, (16, 128)), rtol=0,
                                       atol=1e-12)
    # without the append the same queries do not reduce to that mean
    out0, _, _ = _run(sp, x, q, x.kv, x.k_idx, x.local_k, x.local_v, False)
    assert np.abs(out0[0, 0] - 0.5 * (f64(kv_new[0, 128:]) + f64(v_new[0, 0]))).max() > 1e-2


def test_append_closed_form_fp4():
    """With an FP4 cache the global V is the dequantised appended row."""
    sp, x, q, kv_new, kidx_new, k_new, v_new = _setup(fp4=True)
    kv, k_idx, lk, lv = oracle.append(x.kv, x.k_idx, x.local_k, x.local_v, x.q_pos, kv_new,
                                      kidx_new, k_new, v_new)
    out, sel, _ = _run(sp, x, q, kv, k_idx, lk, lv, True)
    codes, scales = oracle.fp4_pack(kv_new)
    deq = oracle.fp4_unpack(codes, scales)
    for b, t in enumerate(sp.q_pos):
        assert t in sel[0, b]
        for l in range(sp.n_layers):
            # the FP4 key row is 4u rounded to E2M1: still dominant, but its
            # logit differs from the local entry's, so the two share the
            # weight as a two-entry softmax
            qk_g = f64(q[l, b, 0]) @ deq[b, :128] * SCALE
            qk_l = f64(q[l, b, 0]) @ f64(k_new[l, b]) * SCALE
            w = 1.0 / (1.0 + np.exp(qk_l - qk_g))  # weight of the global entry
            want = w * deq[b, 128:] + (1 - w) * f64(v_new[l, b])
            np.testing.assert_allclose(out[l, b], np.broadcast_to(want, (16, 128)), rtol=0,
                                       atol=1e-9)


def test_append_skips_out_of_range_and_writes_ring_slot():
    sp, x, q, kv_new, kidx_new, k_new, v_new = _setup()
    pos = np.array([sp.t_cap, -1, 17], np.int32)  # only sequence 2 is written
    kv, k_idx, lk, lv = oracle.append(x.kv, x.k_idx, x.local_k, x.local_v, pos, kv_new,
                                      kidx_new, k_new, v_new)
    assert np.array_equal(kv[:2], x.kv[:2]) and np.array_equal(k_idx[:2], x.k_idx[:2])
    assert np.array_equal(lk[:, :2], x.local_k[:, :2])
    assert np.array_equal(kv[2, 17], kv_new[2])
    rows = np.ones(sp.t_cap, bool)
    rows[17] = False
    assert np.array_equal(kv[2, rows], x.kv[2, rows])
    slot = 17 % sp.local_cap
    assert np.array_equal(lk[:, 2, slot], k_new[:, 2])
    assert np.array_equal(lv[:, 2, slot], v_new[:, 2])
    others = np.arange(sp.local_cap) != slot
    assert np.array_equal(lk[:, 2, others], x.local_k[:, 2, others])
    # the window of a query at 17 now reads the new local row at its own slot:
    # the closed form above holds for sequence 2 alone
    out, _, _ = _run(sp, x, q, kv, k_idx, lk, lv, False)
    want = 0.5 * (f64(kv_new[2, 128:]) + f64(v_new[1, 2]))
    np.testing.assert_allclose(out[1, 2], np.broadcast_to(want, (16, 128)), rtol=0, atol=1e-12)
