"""GPU parity of sequence compression ("CED", section "What Does the Sequence
Compression Rate Reduce?"): csa2_compress bit-exact against the oracle's mean
of pairs, and a cache of m = 2 entries through attention, the decode stack
(scan, pool, Reindex, blockwise), the append, the prefill-chunk scores and
top-k and the bounded replay, against the oracle with the same rate (a query
reads only entries whose whole group is at or before it)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_attention_shared_amd as csa2
from gpu_util import DevInputs, attn_check, boundary_check, dev16, dev32, host
from test_gpu_parity import check_stack

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


def test_compress_bit_exact():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3000, 2, 256)).astype(np.float32)
    x *= np.exp2(rng.integers(-140, 120, size=(3000, 2, 1))).astype(np.float32)
    xb = synth.f32_to_bf16_bits(x)
    xb[::7, 1] = xb[::7, 0] + 1          # neighbouring values: ties of the mean
    xb[::11, 1] = xb[::11, 0] ^ 0x8000   # opposite values
    xb[::13, :, :8] = 0x0001             # the smallest subnormal
    got = host(csa2.compress(dev16(xb.reshape(3000 * 2, 256)), 2))
    want = oracle.compress(xb.reshape(3000 * 2, 256), 2)
    assert np.array_equal(got, want)
    one = host(csa2.compress(dev16(xb.reshape(6000, 256)), 1))
    assert np.array_equal(one, xb.reshape(6000, 256))


def _m2_inputs(sp_pos, scale="e8m0"):
    """Positions-level inputs of sp_pos, their m = 2 entries, and the device cache."""
    x = synth.make_inputs(sp_pos)
    kv_e = oracle.compress(x.kv, 2)
    ki_e = oracle.compress(x.k_idx, 2)
    d_kv = csa2.compress(dev16(x.kv), 2)
    d_ki = csa2.compress(dev16(x.k_idx), 2)
    assert np.array_equal(host(d_kv), kv_e) and np.array_equal(host(d_ki), ki_e)
    pack = csa2.pack_fp4 if scale == "e8m0" else csa2.pack_fp4_e4m3
    codes, scales = pack(d_kv)
    cache = csa2.Cache(codes, d_ki, scales, m=2)
    xe = synth.Inputs(sp_pos, kv_e, ki_e, x.q, x.q_idx, x.local_k, x.local_v, x.q_pos, x.q_seq,
                      x.needle_pos)
    return x, xe, cache, (codes, scales, d_ki)


def test_attention_reads_complete_groups_only():
    T = 4002  # positions; 2001 entries
    q_pos = [4001, 4000, 2, 1, 0, 3333]
    sp = synth.Spec("m2-attn", n_seq=2, t_cap=T, q_pos=q_pos, q_seq=[0, 1, 0, 1, 0, 1],
                    kv_format="fp4", k=96, window=40, local_cap=64, seed=13)
    x, xe, cache, _ = _m2_inputs(sp)
    c = oracle.Cache(xe.kv, xe.k_idx, fp4=True, m=2)
    _, sel, _ = oracle.layer(c, x.q_pos, x.q_seq, oracle.FULL, x.q[0], x.q_idx[0], x.local_k[0],
                             x.local_v[0], sp.window, 0, sp.k)
    for i, t in enumerate(q_pos):
        g = sel[i][sel[i] >= 0]
        assert g.size == min(sp.k, (t + 1) // 2) and (g.size == 0 or g.max() <= (t + 1) // 2 - 1)
    ref = oracle.attend(c, x.q_pos, x.q_seq, x.q[0], sel, x.local_k[0], x.local_v[0], sp.window, 0)
    local = csa2.Local(dev16(x.local_k[0]), dev16(x.local_v[0]), sp.window)
    out = host(csa2.sparse_attn(cache, dev16(x.q[0]), dev32(x.q_pos), dev32(x.q_seq),
                                dev32(sel), local))
    err = attn_check(out, ref, "m=2 attention")
    log("m=2 attention max abs err", err)
    # a selection reaching past the last complete group must not be read:
    # the GPU skips entry (t + 1) / 2 for an even t, as the oracle would refuse it
    sel2 = sel.copy()
    sel2[1, 0] = 2000   # query at 4000: entries 0..1999 are complete
    out2 = host(csa2.sparse_attn(cache, dev16(x.q[0]), dev32(x.q_pos), dev32(x.q_seq),
                                 dev32(sel2), local))
    sel3 = sel2.copy()
    sel3[1, 0] = -1
    ref3 = oracle.attend(c, x.q_pos, x.q_seq, x.q[0], sel3, x.local_k[0], x.local_v[0],
                         sp.window, 0)
    attn_check(out2, ref3, "m=2 attention, incomplete group skipped")


@pytest.mark.parametrize("block,kv", [(1, "fp4"), (64, "fp4"), (1, "fp4e")])
def test_stack_on_compressed_cache(block, kv):
    T = 2 * 6000
    sp_pos = synth.Spec("m2-stack", n_seq=3, t_cap=T, q_pos=[T - 1, 7000, 5001], q_seq=[0, 1, 2],
                        kv_format=kv, k=64, window=32, pool=64 * 8, block=block,
                        schedule=synth.repeating_schedule(6), local_cap=48, seed=17)
    x, xe, cache, _ = _m2_inputs(sp_pos, "e8m0" if kv == "fp4" else "e4m3")
    L = sp_pos.n_layers
    outs, sels, pool = csa2.stack_run(
        cache, list(sp_pos.schedule), dev32(x.q_pos), [dev16(x.q[l]) for l in range(L)],
        [dev16(x.q_idx[l]) if sp_pos.schedule[l] != synth.REUSE else None for l in range(L)],
        [csa2.Local(dev16(x.local_k[l]), dev16(x.local_v[l]), sp_pos.window) for l in range(L)],
        sp_pos.k, sp_pos.pool, block)
    torch.cuda.synchronize()
    sp_e = synth.Spec(**{**sp_pos.__dict__, "t_cap": T // 2})
    err = check_stack(sp_e, xe, None, outs, sels, pool, rate=2)
    log("m=2 stack block=%d %s max abs err" % (block, kv), err)


def test_append_writes_an_entry_when_a_group_completes():
    T = 200
    sp_pos = synth.Spec("m2-append", n_seq=3, t_cap=T, q_pos=[199, 150, 9], q_seq=[0, 1, 2],
                        kv_format="fp4", k=8, window=8, local_cap=16, seed=19)
    x, xe, cache, (codes, scales, d_ki) = _m2_inputs(sp_pos)
    rng = np.random.default_rng(20)
    f = synth.f32_to_bf16_bits
    kv_new = f(rng.standard_normal((3, 256)).astype(np.float32))
    ki_new = f(rng.standard_normal((3, 64)).astype(np.float32))
    k_new = f(rng.standard_normal((1, 3, 128)).astype(np.float32))
    v_new = f(rng.standard_normal((1, 3, 128)).astype(np.float32))
    local = csa2.Local(dev16(x.local_k[0]), dev16(x.local_v[0]), sp_pos.window)
    pos = np.array([199, 150, 9], np.int32)  # odd: entries 99 and 4; even: no entry
    csa2.append(cache, dev32(pos), dev16(kv_new), dev16(ki_new), [local], [dev16(k_new[0])],
                [dev16(v_new[0])])
    torch.cuda.synchronize()
    kv_e, ki_e = xe.kv.copy(), xe.k_idx.copy()
    for b, p in enumerate(pos):
        if p % 2 == 1:
            kv_e[b, p // 2] = kv_new[b]
            ki_e[b, p // 2] = ki_new[b]
    oc, os_ = oracle.fp4_pack(kv_e)
    assert np.array_equal(host(codes), oc) and np.array_equal(host(scales), os_)
    assert np.array_equal(host(d_ki), ki_e)
    lk = x.local_k[0].copy()
    lk[np.arange(3), pos % 16] = k_new[0]
    assert np.array_equal(host(local.k), lk)


def _m2_prefill_case(T_pos, nq, seed, extra):
    rng = np.random.default_rng(seed)
    pos = np.concatenate([np.asarray(extra, np.int64), rng.integers(0, T_pos, nq - len(extra))])
    sp = synth.Spec("m2-prefill", n_seq=1, t_cap=T_pos, q_pos=[int(p) for p in pos],
                    q_seq=[0] * nq, kv_format="fp4", k=8, window=8, local_cap=16, seed=seed)
    return _m2_inputs(sp)


def test_prefill_score_and_topk_on_compressed_cache():
    """The prefill-chunk calls on m = 2 entries: even and odd positions, the
    first two positions (no complete group at 0), rows shorter than k."""
    T_pos, nq, k = 2 * 20000, 70, 512
    extra = [0, 1, 2, 3, 2 * k - 2, 2 * k - 1, 2 * k, 20001, 20002, T_pos - 2, T_pos - 1]
    x, xe, cache, _ = _m2_prefill_case(T_pos, nq, 23, extra)
    q_idx, q_pos = dev16(x.q_idx[0]), dev32(x.q_pos)
    sc = host(csa2.prefill_score(cache, 0, q_idx, q_pos))
    g = host(csa2.prefill_topk(cache, 0, q_idx, q_pos, k))
    torch.cuda.synchronize()
    k64 = (xe.k_idx[0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q64 = (x.q_idx[0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for i, p in enumerate(x.q_pos):
        te = (int(p) + 1) // 2 - 1  # the last complete entry
        assert np.all(np.isneginf(sc[i, te + 1:])), "row %d: entries past %d must be -inf" % (i, te)
        if te < 0:
            assert (g[i] == -1).all(), "row %d: no complete entry, nothing selected" % i
            continue
        ref = oracle.scores(x.q_idx[0, i], xe.k_idx[0, :te + 1]).astype(np.float64)
        bound = 64 * 2.0 ** -24 * np.abs(k64[:te + 1] * q64[i]).sum(axis=1) + 2.0 ** -24 * np.abs(ref)
        assert np.all(np.abs(sc[i, :te + 1] - ref) <= bound), "row %d scores" % i
        boundary_check(g[i], np.arange(te + 1, dtype=np.int32), ref.astype(np.float32), k,
                       "m=2 prefill q%d t=%d" % (i, p))


@pytest.mark.parametrize("schedule,pool", [("repeat", 256), ("full", 0)])
def test_replay_on_compressed_cache(schedule, pool):
    """The bounded replay over m = 2 entries: materialised Full rows with a
    pool and Reindex, and the fused Full top-k; the window reads positions."""
    from test_gpu_replay import _rings_after, check_replay
    n, T_pos = 70, 2 * 3000
    sched = (synth.repeating_schedule(6) if schedule == "repeat"
             else [synth.FULL, synth.REUSE, synth.FULL])
    sp = synth.Spec("m2-replay", n_seq=2, t_cap=T_pos, q_pos=list(range(T_pos - n, T_pos)),
                    q_seq=[1] * n, kv_format="fp4", k=64, window=32, pool=pool, schedule=sched,
                    local_cap=128, lo=T_pos - n, seed=29)
    x, xe, cache, _ = _m2_inputs(sp)
    L = sp.n_layers
    rng = np.random.default_rng(30)
    f = synth.f32_to_bf16_bits
    k_new = f(rng.standard_normal((L, n, 128)).astype(np.float32))
    v_new = f(rng.standard_normal((L, n, 128)).astype(np.float32))
    local = [csa2.Local(dev16(x.local_k[l]), dev16(x.local_v[l]), sp.window, sp.lo) for l in range(L)]
    outs, sels, pl = csa2.replay_run(cache, list(sched), 1, dev32(x.q_pos),
                                     [dev16(x.q[l]) for l in range(L)],
                                     [dev16(x.q_idx[l]) if sched[l] != synth.REUSE else None
                                      for l in range(L)],
                                     local, sp.k, sp.pool,
                                     local_k=[dev16(k_new[l]) for l in range(L)],
                                     local_v=[dev16(v_new[l]) for l in range(L)])
    torch.cuda.synchronize()
    lk, lv = _rings_after(sp, x, 1, k_new, v_new)
    for l in range(L):
        assert np.array_equal(host(local[l].k), lk[l]), "ring K layer %d" % l
    sp_e = synth.Spec(**{**sp.__dict__, "t_cap": T_pos // 2})
    err = check_replay(sp_e, xe, 1, outs, sels, pl, lk, lv, range(n), rate=2)
    log("m=2 replay %s max abs err" % schedule, err)
