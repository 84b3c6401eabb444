"""Pins of the oracle's bounded replay ("CED", section "Why Prefill Recomputes
a Recent Segment", Fig. 6): the recent segment of a prompt passes through every
decoder layer again to rebuild each layer's local state, and window references
before the segment are cut off."""
import numpy as np

import oracle
import synth
from synth import bf16_bits_to_f32, f32_to_bf16_bits

SCALE = 128 ** -0.5


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, np.float32))


def f64(b):
    return bf16_bits_to_f32(b).astype(np.float64)


def _rows(L, n, seed):
    rng = np.random.default_rng(seed)
    return bf16(rng.standard_normal((L, n, 128))), bf16(rng.standard_normal((L, n, 128)))


def test_fig6_segment_and_truncation_closed_form():
    """Fig. 6: six prompt positions p0..p5, two decoder layers, replay segment
    {p4, p5} with a two-position window.  With every query zero all logits are
    0, so a layer's output is the plain mean of the V rows it attends: the
    global rows p0..t (k covers every causal position) and the window, which
    for p4 is {p4} only (p3 lies before the segment) and for p5 is {p4, p5},
    both from the rows the replay itself wrote."""
    for fp4 in (False, True):
        sp = synth.Spec("fig6", n_seq=1, t_cap=6, q_pos=[4, 5], q_seq=[0, 0],
                        kv_format="fp4" if fp4 else "bf16", k=6, window=2, local_cap=4,
                        schedule=[synth.FULL, synth.FULL], seed=5)
        x = synth.make_inputs(sp)
        c = oracle.Cache(x.kv, x.k_idx, fp4=fp4)
        L, n = 2, 2
        q = np.zeros((L, n, 16, 128), np.uint16)
        k_new, v_new = _rows(L, n, 6)
        out, sel, _, lk, lv = oracle.replay(c, sp.schedule, 0, [4, 5], q, x.q_idx[:, :2],
                                            x.local_k, x.local_v, 2, 4, 6, 0, k_new, v_new)
        if fp4:
            gv = oracle.fp4_unpack(*oracle.fp4_pack(x.kv[0]))[:, 128:]
        else:
            gv = f64(x.kv[0, :, 128:])
        for l in range(L):
            assert sel[l, 0].tolist() == [0, 1, 2, 3, 4, -1]
            assert sel[l, 1].tolist() == [0, 1, 2, 3, 4, 5]
            want4 = np.vstack([gv[:5], f64(v_new[l, 0])[None]]).mean(0)
            want5 = np.vstack([gv[:6], f64(v_new[l, :2])]).mean(0)
            np.testing.assert_allclose(out[l, 0], np.broadcast_to(want4, (16, 128)), atol=1e-12)
            np.testing.assert_allclose(out[l, 1], np.broadcast_to(want5, (16, 128)), atol=1e-12)
            # the ring now holds the segment's rows in slots 4 % 4 and 5 % 4
            assert np.array_equal(lk[l, 0, 0], k_new[l, 0]) and np.array_equal(lk[l, 0, 1], k_new[l, 1])
            assert np.array_equal(lv[l, 0, 2:], x.local_v[l, 0, 2:])
        # without the cut-off p4 also reads the old ring row of p3
        out_full, _, _, _, _ = oracle.replay(c, sp.schedule, 0, [4, 5], q, x.q_idx[:, :2],
                                             x.local_k, x.local_v, 2, 0, 6, 0, k_new, v_new)
        want4 = np.vstack([gv[:5], f64(x.local_v[0, 0, 3])[None], f64(v_new[0, 0])[None]]).mean(0)
        np.testing.assert_allclose(out_full[0, 0], np.broadcast_to(want4, (16, 128)), atol=1e-12)


def test_single_position_replay_is_the_decode_step():
    """Replaying only the last position with no cut-off is one decode step:
    the append of that position's local rows followed by the stack."""
    sp = synth.Spec("replay1", n_seq=2, t_cap=700, q_pos=[650, 650], q_seq=[0, 1],
                    kv_format="fp4", k=32, window=16, pool=128, local_cap=32,
                    schedule=synth.repeating_schedule(6), seed=17)
    x = synth.make_inputs(sp)
    c = oracle.Cache(x.kv, x.k_idx, fp4=True)
    L = sp.n_layers
    k_new, v_new = _rows(L, 1, 18)
    seq, t = 1, 650
    out, sel, pool, lk, lv = oracle.replay(c, sp.schedule, seq, [t], x.q[:, 1:2], x.q_idx[:, 1:2],
                                           x.local_k, x.local_v, sp.window, 0, sp.k, sp.pool,
                                           k_new, v_new)
    # the same through the decode path on a one-sequence copy
    c1 = oracle.Cache(x.kv[seq:seq + 1], x.k_idx[seq:seq + 1], fp4=True)
    _, _, lk1, lv1 = oracle.append(x.kv[seq:seq + 1], x.k_idx[seq:seq + 1],
                                   x.local_k[:, seq:seq + 1], x.local_v[:, seq:seq + 1], [t],
                                   x.kv[seq, t][None], None, k_new, v_new)
    out1, sel1, pool1 = oracle.stack(c1, sp.schedule, [t], x.q[:, 1:2], x.q_idx[:, 1:2], lk1, lv1,
                                     sp.window, 0, sp.k, sp.pool)
    assert np.array_equal(sel, sel1) and np.array_equal(pool, pool1)
    assert np.array_equal(out, out1)
    assert np.array_equal(lk[:, seq], lk1[:, 0]) and np.array_equal(lv[:, seq], lv1[:, 0])
    assert np.array_equal(lk[:, 0], x.local_k[:, 0])


def test_replay_modes_per_query():
    """Each query of the segment follows the schedule on its own: Full picks
    the top-k of its causal scores (and its pool), Reindex the top-k of its
    own pool, Reuse the previous layer's picks."""
    start, n = 900, 24
    sp = synth.Spec("replay-modes", n_seq=2, t_cap=1000, q_pos=list(range(start, start + n)),
                    q_seq=[1] * n, kv_format="bf16", k=40, window=8, pool=160, local_cap=32,
                    schedule=[synth.FULL, synth.REINDEX, synth.REUSE, synth.REINDEX], seed=23)
    x = synth.make_inputs(sp)
    c = oracle.Cache(x.kv, x.k_idx, fp4=False)
    k_new, v_new = _rows(sp.n_layers, n, 24)
    out, sel, pool, _, _ = oracle.replay(c, sp.schedule, 1, x.q_pos, x.q, x.q_idx, x.local_k,
                                         x.local_v, sp.window, start, sp.k, sp.pool, k_new, v_new)
    for i, t in enumerate(x.q_pos):
        s = oracle.scores(x.q_idx[0, i], x.k_idx[1, :t + 1])
        assert np.array_equal(sel[0, i], oracle.topk(s, sp.k))
        assert np.array_equal(pool[i], oracle.topk(s, sp.pool))
        ps = oracle.scores(x.q_idx[1, i], x.k_idx[1, pool[i]])
        assert np.array_equal(sel[1, i], oracle.topk(ps, sp.k, pool[i]))
        assert np.array_equal(sel[2, i], sel[1, i])
        ps = oracle.scores(x.q_idx[3, i], x.k_idx[1, pool[i]])
        assert np.array_equal(sel[3, i], oracle.topk(ps, sp.k, pool[i]))
    assert np.isfinite(out).all()
