"""GPU parity of the bounded replay (csa2_replay_run: a prompt's recent
segment through every decoder layer, "CED", section "Why Prefill Recomputes a
Recent Segment") against the oracle: the rings the replay writes bit for bit,
and every layer's selections and outputs through the cascade (each oracle step
re-run on the GPU's upstream picks), on small ragged segments (split and
one-workgroup-per-query attention, fused and materialised Full top-k) and on
the 20-layer workload's last 128 positions at full size (every one of the
128 queries through every layer)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_attention_shared_amd as csa2
from gpu_util import DevInputs, attn_check, boundary_check, dev16, host, oracle_cache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.device_check()
    yield
    torch.cuda.synchronize()


def log(*a):
    print(*a, flush=True)


def _segment_spec(name, n_seq, seq, t_cap, start, n, **kw):
    base = dict(kv_format="fp4", k=64, window=32, local_cap=128, seed=71)
    base.update(kw)
    return synth.Spec(name, n_seq=n_seq, t_cap=t_cap, q_pos=list(range(start, start + n)),
                      q_seq=[seq] * n, lo=start, **base)


def _rows(sp, seed):
    rng = np.random.default_rng(seed)
    shape = (sp.n_layers, sp.nq, 128)
    f = synth.f32_to_bf16_bits
    return (f(rng.standard_normal(shape).astype(np.float32)),
            f(rng.standard_normal(shape).astype(np.float32)))


def _run(sp, d, seq, k_new, v_new):
    L = sp.n_layers
    return csa2.replay_run(d.cache, list(sp.schedule), seq, d.q_pos, d.q,
                           [d.q_idx[l] if sp.schedule[l] != synth.REUSE else None
                            for l in range(L)],
                           d.local, sp.k, sp.pool, sp.block,
                           local_k=[dev16(k_new[l]) for l in range(L)],
                           local_v=[dev16(v_new[l]) for l in range(L)])


def _rings_after(sp, x, seq, k_new, v_new):
    """The rings once the segment's rows are in: slot p % cap of each layer."""
    lk, lv = x.local_k.copy(), x.local_v.copy()
    slots = np.asarray(sp.q_pos) % sp.local_cap
    lk[:, seq, slots] = k_new
    lv[:, seq, slots] = v_new
    return lk, lv


def check_replay(sp, x, seq, outs, sels, pool, lk, lv, sample, rate=1):
    """With rate > 1, x.kv / x.k_idx hold entries of `rate` positions and a
    query at t reads entries 0 .. (t + 1) / rate - 1."""
    c = oracle_cache(sp, x.kv, x.k_idx, rate)
    sels = [host(s) for s in sels]
    outs = [host(o) for o in outs]
    pool = host(pool) if pool is not None else None
    worst = 0.0
    for l, m in enumerate(sp.schedule):
        for i in sample:
            t = (sp.q_pos[i] + 1) // rate - 1  # the last readable entry
            g = sels[l][i]
            assert np.all(g <= t), "causal"
            if m == synth.REUSE:
                assert np.array_equal(g, sels[l - 1][i])
            elif m == synth.FULL:
                s = oracle.scores(x.q_idx[l, i], x.k_idx[seq, :t + 1])
                ids = np.arange(t + 1, dtype=np.int32)
                if sp.pool:
                    boundary_check(pool[i], ids, s, sp.pool, "L%d pool q%d" % (l, i))
                    assert set(g[g >= 0].tolist()) <= set(pool[i][pool[i] >= 0].tolist())
                boundary_check(g, ids, s, sp.k, "L%d full q%d" % (l, i))
            else:
                gp = pool[i]
                okp = gp >= 0
                ps = np.zeros(gp.size, np.float32)
                ps[okp] = oracle.scores(x.q_idx[l, i], x.k_idx[seq, gp[okp]])
                boundary_check(g, gp, ps, sp.k, "L%d reindex q%d" % (l, i))
        qi = np.asarray(sample)
        ref = oracle.attend(c, np.asarray(sp.q_pos)[qi], np.full(qi.size, seq, np.int32),
                            x.q[l, qi], sels[l][qi], lk[l], lv[l], sp.window, sp.lo)
        worst = max(worst, attn_check(outs[l][qi], ref, "L%d attention" % l))
    return worst


@pytest.mark.parametrize("n,schedule,pool", [
    (101, "repeat", 256),   # split attention, materialised Full rows (pool)
    (300, "repeat", 256),   # one workgroup per query
    (77, "full", 0),        # fused Full top-k, every layer Full
    (300, "repeat", 1000),  # scoring and selecting launches; score rows padded to whole lines
])
def test_replay_small_segments(n, schedule, pool):
    sched = (synth.repeating_schedule(7) if schedule == "repeat"
             else [synth.FULL, synth.REUSE, synth.FULL])
    sp = _segment_spec("replay-%d" % n, n_seq=2, seq=1, t_cap=3001, start=3001 - n, n=n,
                       pool=pool, schedule=sched, local_cap=max(128, 2 * n))
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    k_new, v_new = _rows(sp, 72)
    log("replay n=%d %s pool=%d" % (n, schedule, pool))
    outs, sels, pl = _run(sp, d, 1, k_new, v_new)
    torch.cuda.synchronize()
    lk, lv = _rings_after(sp, x, 1, k_new, v_new)
    for l in range(sp.n_layers):
        assert np.array_equal(host(d.local[l].k), lk[l]), "ring K layer %d" % l
        assert np.array_equal(host(d.local[l].v), lv[l]), "ring V layer %d" % l
    err = check_replay(sp, x, 1, outs, sels, pl, lk, lv, range(n))
    log("replay max abs err", err)
    # the oracle's own replay agrees on the selections of the first layer
    _, osel, _, olk, olv = oracle.replay(oracle.Cache(x.kv, x.k_idx, fp4=True), sp.schedule, 1,
                                         sp.q_pos, x.q, x.q_idx, x.local_k, x.local_v, sp.window,
                                         sp.lo, sp.k, sp.pool, k_new, v_new)
    assert np.array_equal(olk, lk) and np.array_equal(olv, lv)
    g0 = host(sels[0])
    agree = np.mean([np.array_equal(g0[i], osel[0, i]) for i in range(n)])
    assert agree > 0.9, agree  # the rest differ only at boundary ties (checked above)


def test_replay_without_cut_off_reads_older_slots():
    """lo below the segment: the windows of its first queries reach ring slots
    the segment did not write (the caller's earlier rows)."""
    n, start = 40, 2000
    sp = _segment_spec("replay-nocut", n_seq=1, seq=0, t_cap=2048, start=start, n=n, pool=0,
                       schedule=[synth.FULL, synth.REUSE], local_cap=128)
    sp = synth.Spec(**{**sp.__dict__, "lo": 0})
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    k_new, v_new = _rows(sp, 73)
    outs, sels, pl = _run(sp, d, 0, k_new, v_new)
    torch.cuda.synchronize()
    lk, lv = _rings_after(sp, x, 0, k_new, v_new)
    check_replay(sp, x, 0, outs, sels, pl, lk, lv, range(n))


def test_replay_workload_last_128_positions():
    """The 20-layer workload's stack on one 131072-token sequence, replaying
    its last 128 positions with the window cut off at the segment."""
    base = synth.config(3)
    n, T = 128, base.t_cap
    sp = _segment_spec("replay-workload", n_seq=1, seq=0, t_cap=T, start=T - n, n=n,
                       k=base.k, window=base.window, pool=base.pool, schedule=base.schedule,
                       local_cap=base.local_cap, seed=1006)
    log("replay workload: %d queries, %d layers" % (n, sp.n_layers))
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    k_new, v_new = _rows(sp, 74)
    outs, sels, pl = _run(sp, d, 0, k_new, v_new)
    torch.cuda.synchronize()
    lk, lv = _rings_after(sp, x, 0, k_new, v_new)
    for l in range(sp.n_layers):
        assert np.array_equal(host(d.local[l].k), lk[l])
    # every query of the segment
    sample = list(range(n))
    err = check_replay(sp, x, 0, outs, sels, pl, lk, lv, sample)
    log("replay workload max abs err", err)
