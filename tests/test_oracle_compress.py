"""Pins of the oracle's sequence compression ("CED", section "What Does the
Sequence Compression Rate Reduce?": with rate m the information of m
positions is combined into one global entry; 8 positions with m = 2 give 4
entries).  The combine rule is a reading (the element-wise mean, rounded
once to bf16), checked against torch's bf16 rounding; the causal rule (a
query reads only entries whose whole group lies at or before it) against
closed forms on the pages' 8-position example."""
import numpy as np
import torch

import oracle
import synth
from synth import bf16_bits_to_f32, f32_to_bf16_bits


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, np.float32))


def f64(b):
    return bf16_bits_to_f32(b).astype(np.float64)


def test_mean_of_pairs_rounds_like_torch():
    rng = np.random.default_rng(1)
    x = bf16(rng.standard_normal((500, 2, 64)) * np.exp2(rng.integers(-30, 30, (500, 2, 1))))
    got = oracle.compress(x, 2)[:, 0]
    mean = (f64(x[:, 0]) + f64(x[:, 1])) / 2   # exact in double
    want = torch.from_numpy(mean.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    assert np.array_equal(got.view(np.int16), want.numpy())


def test_mean_ties_and_exact_cases():
    # 1 and the next bf16 up average to a tie, which goes to the even significand
    a, b = bf16([1.0])[0], np.uint16(bf16([1.0])[0] + 1)
    got = oracle.compress(np.array([[[a], [b]]], np.uint16), 2)
    assert got[0, 0] == a
    # equal rows and opposite rows
    x = bf16([[[3.5, -2.0]], [[3.5, 2.0]]]).reshape(1, 2, 2)
    assert np.array_equal(f64(oracle.compress(x, 2))[0, 0], [3.5, 0.0])
    # signed zeros follow IEEE addition: -0 and -0 give -0, -0 and +0 give +0
    z = np.array([[[0x8000, 0x8000]], [[0x8000, 0x0000]]], np.uint16).reshape(1, 2, 2)
    assert oracle.compress(z, 2)[0, 0].tolist() == [0x8000, 0x0000]
    # m = 1 is the identity; a trailing incomplete group is dropped
    y = bf16(np.arange(24, dtype=np.float32).reshape(1, 3, 8))
    assert np.array_equal(oracle.compress(y, 1), y)
    assert oracle.compress(y, 2).shape == (1, 1, 8)


def _example(m, seed=3):
    """The pages' teaching size: 8 positions -> 8 / m entries of one sequence."""
    sp = synth.Spec("m%d" % m, n_seq=1, t_cap=8, q_pos=[7], q_seq=[0], kv_format="bf16", k=8,
                    window=2, local_cap=8, seed=seed)
    x = synth.make_inputs(sp)
    kv = oracle.compress(x.kv, m)
    kidx = oracle.compress(x.k_idx, m)
    return sp, x, kv, kidx


def test_only_complete_groups_are_visible():
    """Zero queries make every logit 0, so the output is the plain mean of
    the attended V rows: the visible entries (groups wholly at or before t)
    and the window.  With m = 2 the query at 4 reads entries {0, 1} (positions
    0-3), the one at 5 also entry 2 (positions 4, 5)."""
    sp, x, kv, kidx = _example(2)
    assert kv.shape == (1, 4, 256)
    c = oracle.Cache(kv, kidx, fp4=False, m=2)
    q = np.zeros((3, 16, 128), np.uint16)
    pos = np.array([4, 5, 0], np.int32)
    out, sel, _ = oracle.layer(c, pos, [0, 0, 0], oracle.FULL, q, x.q_idx[0, [0, 0, 0]],
                               x.local_k[0], x.local_v[0], 2, 0, 8)
    assert sel[0].tolist()[:3] == [0, 1, -1]
    assert sel[1].tolist()[:4] == [0, 1, 2, -1]
    assert (sel[2] == -1).all()  # position 0 completes no group
    gv = f64(kv[0, :, 128:])
    lv = f64(x.local_v[0, 0])
    for i, (t, ents) in enumerate([(4, 2), (5, 3), (0, 0)]):
        rows = [gv[j] for j in range(ents)] + [lv[p % 8] for p in range(max(t - 1, 0), t + 1)]
        np.testing.assert_allclose(out[i], np.broadcast_to(np.mean(rows, 0), (16, 128)),
                                   atol=1e-12)


def test_rate_one_is_the_uncompressed_cache():
    sp, x, kv, kidx = _example(1)
    c1 = oracle.Cache(kv, kidx, fp4=True, m=1)
    c0 = oracle.Cache(x.kv, x.k_idx, fp4=True)
    a = oracle.layer(c1, [7, 3], [0, 0], oracle.FULL, x.q[0, [0, 0]], x.q_idx[0, [0, 0]],
                     x.local_k[0], x.local_v[0], 2, 0, 4)
    b = oracle.layer(c0, [7, 3], [0, 0], oracle.FULL, x.q[0, [0, 0]], x.q_idx[0, [0, 0]],
                     x.local_k[0], x.local_v[0], 2, 0, 4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_compressed_stack_reads_entries_by_group():
    """A stack on an m = 2 cache: each query's Full selection is the top-k of
    its causal entry scores (entries 0 .. (t + 1) / 2 - 1)."""
    sp = synth.Spec("m2-stack", n_seq=2, t_cap=600, q_pos=[599, 400], q_seq=[0, 1],
                    kv_format="fp4", k=40, window=8, pool=120, local_cap=16,
                    schedule=[synth.FULL, synth.REINDEX, synth.REUSE], seed=7)
    x = synth.make_inputs(sp)
    kv, kidx = oracle.compress(x.kv, 2), oracle.compress(x.k_idx, 2)
    c = oracle.Cache(kv, kidx, fp4=True, m=2)
    t = np.array([599, 400], np.int32)
    out, sel, pool = oracle.stack(c, sp.schedule, t, x.q, x.q_idx, x.local_k, x.local_v,
                                  sp.window, 0, sp.k, sp.pool)
    for b in range(2):
        n = (t[b] + 1) // 2
        s = oracle.scores(x.q_idx[0, b], kidx[b, :n])
        assert np.array_equal(sel[0, b], oracle.topk(s, sp.k))
        assert np.array_equal(pool[b], oracle.topk(s, sp.pool))
        assert sel[0, b].max() <= n - 1
    assert np.isfinite(out).all()
