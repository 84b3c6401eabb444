"""Pins of the oracle's attention, Full / Reindex / Reuse modes and stack
driver: dense-attention equivalence (library routine), closed forms, the
pages' worked examples (Figures 4 and 5) and mode invariants."""
import json
import os

import numpy as np
import torch

import oracle
import synth
from synth import bf16_bits_to_f32, f32_to_bf16_bits

GOLD = os.path.join(os.path.dirname(__file__), "golden")
SCALE = 128 ** -0.5


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, np.float32))


def f64(b):
    return bf16_bits_to_f32(b).astype(np.float64)


def small_spec(**kw):
    base = dict(name="tiny", n_seq=1, t_cap=300, q_pos=[299], q_seq=[0], kv_format="bf16",
                k=300, window=0, local_cap=128, seed=77)
    base.update(kw)
    return synth.Spec(**base)


def sdpa(q, K, V):
    """torch's scaled_dot_product_attention in float64 on the CPU."""
    qt = torch.from_numpy(q)[None, :, None, :]           # [1, 16, 1, 128]
    Kt = torch.from_numpy(K)[None, None].expand(1, 16, -1, -1)
    Vt = torch.from_numpy(V)[None, None].expand(1, 16, -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=SCALE)
    return o[0, :, 0, :].numpy()


def test_full_context_top_k_without_window_is_dense_causal_attention():
    # k = t + 1, bf16 main cache, W = 0: every position <= t is read
    for t in (0, 5, 299):
        sp = small_spec(q_pos=[t], k=t + 1)
        x = synth.make_inputs(sp)
        c = oracle.Cache(x.kv, x.k_idx, fp4=False)
        out, sel, _ = oracle.layer(c, x.q_pos, x.q_seq, oracle.FULL, x.q[0], x.q_idx[0],
                                   x.local_k[0], x.local_v[0], 0, 0, t + 1)
        assert np.array_equal(sel[0], np.arange(t + 1))
        # dense causal attention over the whole cache, read at row t
        K = f64(x.kv[0, :, :128])
        V = f64(x.kv[0, :, 128:])
        qf = f64(x.q[0, 0])
        qt = torch.from_numpy(qf)[None, :, None, :].expand(1, 16, sp.t_cap, 128)
        Kt = torch.from_numpy(K)[None, None].expand(1, 16, -1, -1)
        Vt = torch.from_numpy(V)[None, None].expand(1, 16, -1, -1)
        o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, is_causal=True,
                                                             scale=SCALE)
        np.testing.assert_allclose(out[0], o[0, :, t, :].numpy(), rtol=1e-12, atol=1e-13)


def test_selection_plus_window_is_softmax_over_concatenation():
    sp = small_spec(q_pos=[200], k=37, window=50, local_cap=64)
    x = synth.make_inputs(sp)
    c = oracle.Cache(x.kv, x.k_idx, fp4=False)
    out, sel, _ = oracle.layer(c, x.q_pos, x.q_seq, oracle.FULL, x.q[0], x.q_idx[0],
                               x.local_k[0], x.local_v[0], 50, 0, 37)
    s = sel[0][sel[0] >= 0]
    w = np.arange(151, 201)
    K = np.concatenate([f64(x.kv[0, s, :128]), f64(x.local_k[0, 0, w % 64])])
    V = np.concatenate([f64(x.kv[0, s, 128:]), f64(x.local_v[0, 0, w % 64])])
    np.testing.assert_allclose(out[0], sdpa(f64(x.q[0, 0]), K, V), rtol=1e-12, atol=1e-13)


def test_one_entry_returns_its_value_and_equal_logits_average():
    rng = np.random.default_rng(8)
    V = f64(bf16(rng.standard_normal((5, 128))))
    K = f64(bf16(rng.standard_normal((5, 128))))
    q = bf16(rng.standard_normal((16, 128)))
    o1 = oracle.attention(q, K[:1], V[:1], SCALE)
    assert np.array_equal(o1, np.broadcast_to(V[0], (16, 128)))
    o0 = oracle.attention(np.zeros((16, 128), np.uint16), K, V, SCALE)
    np.testing.assert_allclose(o0, np.broadcast_to(V.mean(0), (16, 128)), rtol=1e-14, atol=1e-15)


def test_fp4_cache_attention_reads_the_dequantised_rows():
    sp = small_spec(q_pos=[120], k=16, window=8, local_cap=16, kv_format="fp4")
    x = synth.make_inputs(sp)
    c = oracle.Cache(x.kv, x.k_idx, fp4=True)
    out, sel, _ = oracle.layer(c, x.q_pos, x.q_seq, oracle.FULL, x.q[0], x.q_idx[0],
                               x.local_k[0], x.local_v[0], 8, 0, 16)
    s = sel[0]
    deq = oracle.fp4_unpack(c.codes[0, s], c.scales[0, s])
    w = np.arange(113, 121)
    K = np.concatenate([deq[:, :128], f64(x.local_k[0, 0, w % 16])])
    V = np.concatenate([deq[:, 128:], f64(x.local_v[0, 0, w % 16])])
    np.testing.assert_allclose(out[0], sdpa(f64(x.q[0, 0]), K, V), rtol=1e-12, atol=1e-13)


def test_attention_does_not_depend_on_selection_order():
    sp = small_spec(q_pos=[250], k=40, window=16, local_cap=32, kv_format="fp4")
    x = synth.make_inputs(sp)
    c = oracle.Cache(x.kv, x.k_idx, fp4=True)
    _, sel, _ = oracle.layer(c, x.q_pos, x.q_seq, oracle.FULL, x.q[0], x.q_idx[0],
                             x.local_k[0], x.local_v[0], 16, 0, 40)
    a = oracle.attend(c, x.q_pos, x.q_seq, x.q[0], sel, x.local_k[0], x.local_v[0], 16, 0)
    perm = sel[:, ::-1].copy()
    b = oracle.attend(c, x.q_pos, x.q_seq, x.q[0], perm, x.local_k[0], x.local_v[0], 16, 0)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------ worked examples

def _one_hot_rows(n, offset=0):
    r = np.zeros((n, 128), np.float32)
    for i in range(n):
        r[i, offset + i] = 1.0
    return r


def test_figure4_worked_example():
    g = json.load(open(os.path.join(GOLD, "fig4_selection.json")))
    t, k, W = g["query_pos"], g["topk"], g["window"]
    T = t + 1
    # indexer keys: one-hot, so the score of p_j is the indexer query's j-th entry
    k_idx = bf16(np.eye(64)[:T] * 1.0)[None]
    q_idx = np.zeros(64, np.float32)
    q_idx[:T] = [5.0, 1.0, 2.0, 4.0, 3.0, 0.5]  # p0 and p3 score highest
    # global V rows carry one-hot channel j, local V rows channel 64 + pos
    kv = np.zeros((1, T, 256), np.float32)
    kv[0, :, 128:] = _one_hot_rows(T)
    lv = np.zeros((1, 8, 128), np.float32)
    for p in range(8):
        lv[0, p, 64 + p] = 1.0
    c = oracle.Cache(bf16(kv), k_idx, fp4=False)
    q = np.zeros((1, 16, 128), np.uint16)  # equal logits: output = mean of the entries' V
    out, sel, _ = oracle.layer(c, [t], [0], oracle.FULL, q, bf16(q_idx)[None],
                               bf16(np.zeros((1, 8, 128))), bf16(lv), W, 0, k)
    assert sel[0].tolist() == g["selected"]
    o = out[0, 0]
    n = g["attention_entries"]
    want = np.zeros(128)
    for j in g["selected"]:
        want[j] = 1.0 / n
    for p in g["window_positions"]:
        want[64 + p] = 1.0 / n
    np.testing.assert_allclose(o, want, atol=1e-15)


def test_figure5_worked_example_full_reindex_reuse():
    g = json.load(open(os.path.join(GOLD, "fig5_modes.json")))
    t, k = g["query_pos"], g["topk"]
    T = t + 1
    k_idx = bf16(np.eye(64)[:T] * 1.0)[None]
    qf = np.zeros(64, np.float32)
    qf[:T] = [6.0, 4.0, 0.0, 5.0, 1.0, 2.0]   # Full: p0, p3; pool of 3: p0, p1, p3
    qr = np.zeros(64, np.float32)
    qr[:T] = [0.0, 6.0, 9.0, 5.0, 7.0, 8.0]   # Reindex: best outside the pool are p2, p4, p5
    q_idx = np.stack([bf16(qf), bf16(qr), bf16(qr)])[:, None, :]
    kv = bf16(np.ones((1, T, 256)))
    c = oracle.Cache(kv, k_idx, fp4=False)
    q = np.zeros((3, 1, 16, 128), np.uint16)
    lk = np.zeros((3, 1, 8, 128), np.uint16)
    modes = [synth.FULL, synth.REINDEX, synth.REUSE]
    out, sel, pool = oracle.stack(c, modes, [t], q, q_idx, lk, lk, 1, 0, k, pool=3)
    assert sorted(pool[0].tolist()) == g["pool_contains"]
    assert sel[0, 0].tolist() == g["full_selected"]
    assert sel[1, 0].tolist() == g["reindex_selected"]
    assert sel[2, 0].tolist() == g["reuse_selected"]


def test_page_schedule_counts():
    g = json.load(open(os.path.join(GOLD, "schedule_20.json")))
    s = synth.page_schedule_20()
    assert len(s) == g["n_layers"]
    assert s.count(synth.FULL) == g["full"]
    assert s.count(synth.REINDEX) == g["reindex"]
    assert s.count(synth.REUSE) == g["reuse"]


# ---------------------------------------------------------- invariants

def _stack_case(block=1, pool=96, fp4=True, T=1500, S=2):
    sched = synth.repeating_schedule(7)
    sp = synth.Spec("stack", n_seq=S, t_cap=T, q_pos=[T - 1 - 311 * s for s in range(S)],
                    q_seq=list(range(S)), kv_format="fp4" if fp4 else "bf16", k=24,
                    window=16, pool=pool, block=block, schedule=sched, local_cap=32, seed=99)
    x = synth.make_inputs(sp)
    c = oracle.Cache(x.kv, x.k_idx, fp4=fp4)
    out, sel, pl = oracle.stack(c, sched, x.q_pos, x.q, x.q_idx, x.local_k, x.local_v,
                                sp.window, 0, sp.k, sp.pool, block=block)
    return sp, x, c, out, sel, pl


def test_stack_mode_invariants():
    sp, x, c, out, sel, pool = _stack_case()
    for s in range(sp.n_seq):
        t = sp.q_pos[s]
        P = set(pool[s].tolist())
        for l, m in enumerate(sp.schedule):
            cur = sel[l, s]
            assert np.all(cur <= t)                       # causal triangle
            assert np.all(np.diff(cur[cur >= 0]) > 0)     # ascending, distinct
            if m == synth.REUSE:
                assert np.array_equal(cur, sel[l - 1, s])  # bit-identical
            else:
                assert set(cur[cur >= 0].tolist()) <= P    # inside the pool
    # Reindex layers recompute: some differ from the Full layer's picks
    assert any(not np.array_equal(sel[l], sel[0]) for l, m in enumerate(sp.schedule)
               if m == synth.REINDEX)


def test_reindex_with_the_full_layers_query_reproduces_full():
    sp, x, c, out, sel, pool = _stack_case()
    for s in range(sp.n_seq):
        o, rsel, _ = oracle.layer(c, x.q_pos[s:s + 1], [s], oracle.REINDEX, x.q[0, s:s + 1],
                                  x.q_idx[0, s:s + 1], x.local_k[0], x.local_v[0], sp.window, 0,
                                  sp.k, pool=sp.pool, pool_io=pool[s:s + 1])
        assert np.array_equal(rsel[0], sel[0, s])
        np.testing.assert_array_equal(o[0], out[0, s])


def test_stack_layer_equals_single_layer_call():
    sp, x, c, out, sel, pool = _stack_case(fp4=False)
    l = 6  # a Reuse layer right after a Reindex layer
    assert sp.schedule[l] == synth.REUSE and sp.schedule[l - 1] == synth.REINDEX
    o, _, _ = oracle.layer(c, x.q_pos, x.q_seq, oracle.REUSE, x.q[l], x.q_idx[l], x.local_k[l],
                           x.local_v[l], sp.window, 0, sp.k, pool=sp.pool, pool_io=pool,
                           sel_io=sel[l - 1])
    np.testing.assert_array_equal(o, out[l])


def test_blockwise_pool_covers_everything_when_blocks_fit():
    # with no more blocks than the pool holds, blockwise selection is tokenwise top-k
    T = 700
    sp = small_spec(t_cap=T, q_pos=[T - 1], k=50, kv_format="fp4", window=4, local_cap=8)
    x = synth.make_inputs(sp)
    c = oracle.Cache(x.kv, x.k_idx, fp4=True)
    args = (c, x.q_pos, x.q_seq, oracle.FULL, x.q[0], x.q_idx[0], x.local_k[0], x.local_v[0], 4, 0, 50)
    ob, sb, pb = oracle.layer(*args, pool=16 * 64, block=64)
    ot, st, _ = oracle.layer(*args)
    assert np.array_equal(sb, st)
    np.testing.assert_array_equal(ob, ot)
    assert sorted(pb[0][pb[0] >= 0].tolist()) == list(range(T))


def test_blockwise_pool_is_made_of_the_best_blocks():
    T, blk, nbsel = 1000, 8, 10
    sp = small_spec(t_cap=T, q_pos=[T - 5], k=20, kv_format="fp4", window=4, local_cap=8)
    x = synth.make_inputs(sp)
    c = oracle.Cache(x.kv, x.k_idx, fp4=True)
    t = T - 5
    _, sel, pool = oracle.layer(c, x.q_pos, x.q_seq, oracle.FULL, x.q[0], x.q_idx[0], x.local_k[0],
                                x.local_v[0], 4, 0, 20, pool=nbsel * blk, block=blk)
    s = oracle.scores(x.q_idx[0, 0], x.k_idx[0, :t + 1])
    bs = np.array([s[b * blk:min((b + 1) * blk, t + 1)].max() for b in range((t + blk) // blk)])
    chosen = sorted(set((pool[0][pool[0] >= 0] // blk).tolist()))
    assert len(chosen) == nbsel
    others = np.setdiff1d(np.arange(bs.size), chosen)
    assert bs[chosen].min() >= bs[others].max()
    # every position of a chosen block up to t is in the pool, nothing past t
    want = [j for b in chosen for j in range(b * blk, (b + 1) * blk) if j <= t]
    assert sorted(pool[0][pool[0] >= 0].tolist()) == want
    # the final top-k is tokenwise inside the pool
    ids = pool[0]
    ps = np.where(ids >= 0, s[np.clip(ids, 0, None)], -np.inf).astype(np.float32)
    ref = sorted(ids[np.argsort(-ps, kind="stable")[:20]].tolist())
    assert sel[0].tolist() == ref


def test_prefill_rows_equal_single_query_calls():
    T = 400
    qp = list(range(360, 400))
    sp = synth.Spec("pf", n_seq=1, t_cap=T, q_pos=qp, q_seq=[0] * len(qp), kv_format="fp4",
                    k=32, window=16, local_cap=128, seed=5)
    x = synth.make_inputs(sp)
    c = oracle.Cache(x.kv, x.k_idx, fp4=True)
    out, sel, _ = oracle.layer(c, x.q_pos, x.q_seq, oracle.FULL, x.q[0], x.q_idx[0], x.local_k[0],
                               x.local_v[0], 16, 0, 32)
    for i in (0, 7, 39):
        o1, s1, _ = oracle.layer(c, x.q_pos[i:i + 1], [0], oracle.FULL, x.q[0, i:i + 1],
                                 x.q_idx[0, i:i + 1], x.local_k[0], x.local_v[0], 16, 0, 32)
        assert np.array_equal(s1[0], sel[i])
        np.testing.assert_array_equal(o1[0], out[i])


def test_window_respects_lower_bound():
    sp = small_spec(q_pos=[100], k=4, window=32, local_cap=64)
    x = synth.make_inputs(sp)
    c = oracle.Cache(x.kv, x.k_idx, fp4=False)
    base = (c, x.q_pos, x.q_seq, x.q[0], None, x.local_k[0], x.local_v[0], 32)
    sel = np.full((1, 4), -1, np.int32)
    o_lo = oracle.attend(c, x.q_pos, x.q_seq, x.q[0], sel, x.local_k[0], x.local_v[0], 32, 90)
    w = np.arange(90, 101)
    K = f64(x.local_k[0, 0, w % 64])
    V = f64(x.local_v[0, 0, w % 64])
    np.testing.assert_allclose(o_lo[0], sdpa(f64(x.q[0, 0]), K, V), rtol=1e-12, atol=1e-13)
