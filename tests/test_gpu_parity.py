"""GPU parity of every C ABI call against the oracle, on seeded synthetic
inputs: small ragged shapes that span several tiles, and the five named
workloads at full size (the prefill chunk on sampled queries)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_attention_shared_amd as csa2
from gpu_util import (DevInputs, attn_check, bf16_to_f64, boundary_check, dev16, dev32, host,
                      oracle_cache)

pytestmark = pytest.mark.gpu

SCALE = 128 ** -0.5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.device_check()  # raises unless gfx950 and the library is built
    yield
    torch.cuda.synchronize()


def log(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ FP4

def _blocks_with_varied_scales(n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 32)).astype(np.float32)
    x *= np.exp2(rng.integers(-140, 120, size=(n, 1))).astype(np.float32)
    x[::17] = 0.0
    x[::19, ::3] = -0.0
    return synth.f32_to_bf16_bits(x)


def test_fp4_pack_and_unpack_bit_exact():
    rows = []
    rows.append(_blocks_with_varied_scales(8192, 1).reshape(-1, 256))
    # every finite bf16 pattern next to an anchor that fixes the block scale
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (pats >> 7) & 0xFF
    pats = pats[exp != 0xFF]
    for anchor in (np.float32(6.0), np.float32(3.0e-39), np.float32(2.0 ** 100)):
        a = synth.f32_to_bf16_bits(np.array([anchor]))[0]
        mag = synth.bf16_bits_to_f32(pats & 0x7FFF)
        p = pats[mag <= anchor]
        p = np.concatenate([p, np.zeros((-p.size) % 31, np.uint16)])
        blk = np.zeros((p.size // 31, 32), np.uint16)
        blk[:, 0] = a
        blk[:, 1:] = p.reshape(-1, 31)
        blk = np.concatenate([blk, np.zeros(((-blk.shape[0]) % 8, 32), np.uint16)])
        rows.append(blk.reshape(-1, 256))
    x = np.concatenate(rows)
    log("fp4 rows", x.shape)
    codes, scales = csa2.pack_fp4(dev16(x))
    oc, os_ = oracle.fp4_pack(x)
    assert np.array_equal(host(codes), oc)
    assert np.array_equal(host(scales), os_)
    deq = host(csa2.unpack_fp4(codes, scales)).astype(np.float64)
    odeq = oracle.fp4_unpack(oc, os_)
    assert np.array_equal(deq, odeq)
    assert np.array_equal(np.signbit(deq), np.signbit(odeq))
    # a single row (decode append) and an empty call
    c1, s1 = csa2.pack_fp4(dev16(x[:1]))
    assert np.array_equal(host(c1), oc[:1]) and np.array_equal(host(s1), os_[:1])
    c0, s0 = csa2.pack_fp4(dev16(x[:0]))
    assert c0.numel() == 0


# --------------------------------------------------------------- scores

def _ragged_spec(kv="fp4", **kw):
    base = dict(name="ragged", n_seq=3, t_cap=5003, q_pos=[5002, 2999, 0, 4100],
                q_seq=[0, 1, 2, 1], kv_format=kv, k=96, window=40, local_cap=64, seed=21)
    base.update(kw)
    return synth.Spec(**base)


def test_index_score_dense_blocks_and_candidates():
    sp = _ragged_spec()
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    s = host(csa2.index_score(d.cache, d.q_idx[0], d.q_pos, d.q_seq))
    assert s.shape == (4, sp.t_cap)
    for i in range(sp.nq):
        t, b = sp.q_pos[i], sp.q_seq[i]
        ref = oracle.scores(x.q_idx[0, i], x.k_idx[b, :t + 1]).astype(np.float64)
        bound = bf16_to_f64(x.k_idx[b, :t + 1]).__abs__() @ np.abs(bf16_to_f64(x.q_idx[0, i]))
        assert np.all(np.abs(s[i, :t + 1] - ref) <= 1e-6 * bound + 1e-30)
        assert np.all(s[i, t + 1:] == -np.inf)
    # block max of the same fp32 token scores
    bs = host(csa2.index_score(d.cache, d.q_idx[0], d.q_pos, d.q_seq, block=64))
    nb = (sp.t_cap + 63) // 64
    assert bs.shape == (4, nb)
    for i in range(sp.nq):
        want = np.array([s[i, 64 * j:64 * (j + 1)].max() for j in range(nb)], np.float32)
        assert np.array_equal(bs[i], want)
    # candidates: -1 slots and positions after the query give -inf
    rng = np.random.default_rng(3)
    cand = rng.integers(-1, sp.t_cap, size=(4, 777)).astype(np.int32)
    cs = host(csa2.index_score(d.cache, d.q_idx[0], d.q_pos, d.q_seq, cand=dev32(cand)))
    for i in range(sp.nq):
        t = sp.q_pos[i]
        ok = (cand[i] >= 0) & (cand[i] <= t)
        assert np.all(cs[i, ~ok] == -np.inf)
        assert np.array_equal(cs[i, ok], s[i, cand[i, ok]])


# ---------------------------------------------------------------- top-k

@pytest.mark.parametrize("n,k,k2", [(100, 7, 30), (5000, 64, 700), (32768, 2048, 8192),
                                    (40000, 256, 0), (131072, 2048, 8192)])
def test_topk_bit_exact_on_identical_scores(n, k, k2):
    rng = np.random.default_rng(n)
    nq = 3
    s = (rng.integers(-40, 41, size=(nq, n)) * 0.25).astype(np.float32)
    s[rng.random((nq, n)) < 0.05] = -0.0
    s[0, rng.random(n) < 0.3] = -np.inf
    s[1] = rng.standard_normal(n).astype(np.float32) * 8
    s[2, : n // 2] = -np.inf  # fewer valid than some k
    ids = None
    g, g2 = csa2.topk(torch.from_numpy(s).cuda(), k, k2=k2)
    g, g2 = host(g), (host(g2) if k2 else None)
    for i in range(nq):
        sv = np.where(np.isneginf(s[i]), np.float32(0), s[i])
        ids_i = np.where(np.isneginf(s[i]), -1, np.arange(n)).astype(np.int32)
        assert np.array_equal(g[i], oracle.topk(sv, k, ids_i)), i
        if k2:
            assert np.array_equal(g2[i], oracle.topk(sv, k2, ids_i)), i
    del ids


def test_topk_one_workgroup_rows_of_32768():
    """64 rows of 32768 slots, one workgroup each (32 slots a thread), both
    targets: ties, -inf, -0."""
    n, nq, k, k2 = 32768, 64, 2048, 4096
    rng = np.random.default_rng(4242)
    s = (rng.integers(-40, 41, size=(nq, n)) * 0.25).astype(np.float32)
    s[rng.random((nq, n)) < 0.05] = -0.0
    s[::3] = (rng.standard_normal((len(range(0, nq, 3)), n)) * 8).astype(np.float32)
    s[1::5, : n // 2] = -np.inf
    g, g2 = csa2.topk(torch.from_numpy(s).cuda(), k, k2=k2)
    g, g2 = host(g), host(g2)
    for i in range(nq):
        sv = np.where(np.isneginf(s[i]), np.float32(0), s[i])
        ids_i = np.where(np.isneginf(s[i]), -1, np.arange(n)).astype(np.int32)
        assert np.array_equal(g[i], oracle.topk(sv, k, ids_i)), i
        assert np.array_equal(g2[i], oracle.topk(sv, k2, ids_i)), i


@pytest.mark.parametrize("k,k2", [(200, 0), (700, 1000)])
def test_topk_one_workgroup_sampled_floor(k, k2):
    """Rows of 16384 slots with k < n / 16 take the sampled floor (a 1/8
    sample's histogram bounds the keys the full pass counts): normal scores
    (the floor holds); every eighth slot -- the sampled ones -- far above
    the rest (the floor is too high and the row is counted whole); ties
    around the k-th key; half the slots -inf."""
    n, nq = 16384, 4
    rng = np.random.default_rng(41 + k)
    s = (rng.standard_normal((nq, n)) * 8).astype(np.float32)
    s[1, ::8] += np.float32(100)
    s[2] = (rng.integers(-20, 21, size=n) * 0.5).astype(np.float32)
    s[3, rng.random(n) < 0.5] = -np.inf
    g, g2 = csa2.topk(torch.from_numpy(s).cuda(), k, k2=k2)
    g, g2 = host(g), (host(g2) if k2 else None)
    for i in range(nq):
        sv = np.where(np.isneginf(s[i]), np.float32(0), s[i])
        ids_i = np.where(np.isneginf(s[i]), -1, np.arange(n)).astype(np.int32)
        assert np.array_equal(g[i], oracle.topk(sv, k, ids_i)), i
        if k2:
            assert np.array_equal(g2[i], oracle.topk(sv, k2, ids_i)), i


@pytest.mark.parametrize("n,k,k2", [(9000, 300, 0), (50000, 500, 3000)])  # one workgroup; long path
def test_topk_through_ascending_ids_with_empty_slots(n, k, k2):
    rng = np.random.default_rng(7)
    nq = 4
    ids = np.sort(rng.choice(10 * n, size=(nq, n), replace=True), axis=1).astype(np.int32)
    ids = np.maximum.accumulate(ids, axis=1)
    ids[:, 1:][ids[:, 1:] == ids[:, :-1]] = -1  # duplicates become empty slots
    ids[rng.random((nq, n)) < 0.05] = -1
    s = (rng.integers(-10, 11, size=(nq, n))).astype(np.float32)
    s[1] = rng.standard_normal(n).astype(np.float32) * 8  # few ties
    g, g2 = csa2.topk(torch.from_numpy(s).cuda(), k, ids=dev32(ids), k2=k2)
    g = host(g)
    for i in range(nq):
        assert np.array_equal(g[i], oracle.topk(s[i], k, ids[i])), i
        if k2:
            assert np.array_equal(host(g2)[i], oracle.topk(s[i], k2, ids[i])), i


# ------------------------------------------------------------ attention

@pytest.mark.parametrize("kv,window,lo,cap", [("fp4", 40, 0, 64), ("bf16", 40, 0, 64),
                                              ("fp4", 0, 0, 64), ("fp4", 64, 4090, 64),
                                              ("fp4", 200, 0, 256)])  # window over 7 chunks
def test_sparse_attn_on_oracle_selection(kv, window, lo, cap):
    sp = _ragged_spec(kv=kv, window=window, lo=lo, local_cap=cap)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    c = oracle.Cache(x.kv, x.k_idx, fp4=(kv == "fp4"))
    _, sel, _ = oracle.layer(c, x.q_pos, x.q_seq, oracle.FULL, x.q[0], x.q_idx[0], x.local_k[0],
                             x.local_v[0], window, lo, sp.k)
    sel[1, ::5] = -1  # empty slots are skipped
    ref = oracle.attend(c, x.q_pos, x.q_seq, x.q[0], sel, x.local_k[0], x.local_v[0], window, lo)
    out = host(csa2.sparse_attn(d.cache, d.q[0], d.q_pos, d.q_seq, dev32(sel), d.local[0]))
    err = attn_check(out, ref, "attn %s W=%d lo=%d" % (kv, window, lo))
    log("attn max abs err", err)


@pytest.mark.parametrize("kv,window,lo,cap,nq", [
    ("fp4", 40, 0, 64, 300), ("bf16", 40, 0, 64, 300), ("fp4", 0, 0, 64, 300),
    ("fp4", 64, 4090, 64, 300),
    ("fp4", 40, 0, 64, 20), ("fp4", 40, 0, 64, 19), ("fp4", 128, 0, 256, 48)])  # around the layout switch
def test_sparse_attn_many_queries(kv, window, lo, cap, nq):
    """From 20 queries on, one workgroup per query (the prefill layout), below
    it split workgroups; k = 96 puts the selection/window boundary inside a
    32-entry tile."""
    rng = np.random.default_rng(77)
    q_pos = [int(v) for v in rng.integers(0, 5003, nq)]
    q_pos[:4] = [5002, 0, 31, 4100]
    q_seq = [int(v) for v in rng.integers(0, 3, nq)]
    sp = _ragged_spec(kv=kv, window=window, lo=lo, local_cap=cap, q_pos=q_pos, q_seq=q_seq, seed=31)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    c = oracle.Cache(x.kv, x.k_idx, fp4=(kv == "fp4"))
    _, sel, _ = oracle.layer(c, x.q_pos, x.q_seq, oracle.FULL, x.q[0], x.q_idx[0], x.local_k[0],
                             x.local_v[0], window, lo, sp.k)
    sel[1::7, ::5] = -1  # empty slots are skipped
    ref = oracle.attend(c, x.q_pos, x.q_seq, x.q[0], sel, x.local_k[0], x.local_v[0], window, lo)
    out = host(csa2.sparse_attn(d.cache, d.q[0], d.q_pos, d.q_seq, dev32(sel), d.local[0]))
    err = attn_check(out, ref, "attn x%d %s W=%d lo=%d" % (nq, kv, window, lo))
    log("many-query attn max abs err", err)


# ---------------------------------------------------------------- stack

def check_stack(sp, x, d, outs, sels, pool, sample=None, rate=1):
    """Layer-by-layer cascade: each oracle step runs on the GPU's upstream picks.
    With rate > 1, x.kv / x.k_idx hold entries of `rate` positions and a
    query at t reads entries 0 .. (t + 1) / rate - 1."""
    c = oracle_cache(sp, x.kv, x.k_idx, rate)
    sels = [host(s) for s in sels]
    outs = [host(o) for o in outs]
    pool = host(pool) if pool is not None else None
    seqs = range(sp.n_seq) if sample is None else sample
    worst = 0.0
    for l, m in enumerate(sp.schedule):
        for b in seqs:
            t = (sp.q_pos[b] + 1) // rate - 1  # the last readable entry
            g = sels[l][b]
            assert np.all(g <= t), "causal"
            if m == synth.REUSE:
                assert np.array_equal(g, sels[l - 1][b])
            elif m == synth.FULL:
                s = oracle.scores(x.q_idx[l, b], x.k_idx[b, :t + 1])
                ids = np.arange(t + 1, dtype=np.int32)
                if sp.block == 1:
                    if sp.pool:
                        boundary_check(pool[b], ids, s, sp.pool, "L%d pool b%d" % (l, b))
                        gp = set(pool[b][pool[b] >= 0].tolist())
                        assert set(g[g >= 0].tolist()) <= gp
                    boundary_check(g, ids, s, sp.k, "L%d full b%d" % (l, b))
                else:
                    nb = t // sp.block + 1
                    bs = oracle.block_scores(s, sp.block)
                    gp = pool[b]
                    gblocks = np.unique(gp[gp >= 0] // sp.block)
                    boundary_check(gblocks, np.arange(nb, dtype=np.int32), bs,
                                   sp.pool // sp.block, "L%d blocks b%d" % (l, b))
                    want = [j for blk in gblocks for j in range(blk * sp.block,
                                                                min((blk + 1) * sp.block, t + 1))]
                    assert sorted(gp[gp >= 0].tolist()) == want
                    ps = np.where(gp >= 0, s[np.clip(gp, 0, None)], np.float32(0)).astype(np.float32)
                    boundary_check(g, gp, ps, sp.k, "L%d pool-topk b%d" % (l, b))
            else:  # Reindex on the GPU's pool
                gp = pool[b]
                ps = np.zeros(gp.size, np.float32)
                okp = gp >= 0
                ps[okp] = oracle.scores(x.q_idx[l, b], x.k_idx[b, gp[okp]])
                boundary_check(g, gp, ps, sp.k, "L%d reindex b%d" % (l, b))
                assert set(g[g >= 0].tolist()) <= set(gp[okp].tolist())
        qi = np.array(list(seqs))
        ref = oracle.attend(c, x.q_pos[qi], qi, x.q[l, qi], sels[l][qi], x.local_k[l], x.local_v[l],
                            sp.window, sp.lo)
        worst = max(worst, attn_check(outs[l][qi], ref, "L%d attention" % l))
    return worst


def run_stack(sp, x, d, want_sel=True):
    return csa2.stack_run(d.cache, list(sp.schedule), d.q_pos, d.q,
                          [d.q_idx[l] if sp.schedule[l] != synth.REUSE else None
                           for l in range(sp.n_layers)],
                          d.local, sp.k, sp.pool, sp.block, want_sel=want_sel)


def test_stack_small_ragged_and_deterministic():
    sp = synth.Spec("stack-small", n_seq=3, t_cap=3001, q_pos=[3000, 1777, 300], q_seq=[0, 1, 2],
                    kv_format="fp4", k=64, window=32, pool=256,
                    schedule=synth.repeating_schedule(7), local_cap=48, seed=31)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    outs, sels, pool = run_stack(sp, x, d)
    err = check_stack(sp, x, d, outs, sels, pool)
    log("stack small max abs err", err)
    outs2, sels2, pool2 = run_stack(sp, x, d)
    for l in range(sp.n_layers):
        assert torch.equal(outs[l].view(torch.int16), outs2[l].view(torch.int16))
        assert torch.equal(sels[l], sels2[l])
    assert torch.equal(pool, pool2)


def test_stack_batch_of_24_runs_one_workgroup_per_query():
    """24 sequences: the stack's attention takes the one-workgroup-per-query
    form (no split, no partials), the selection kernels their few-row forms."""
    rng = np.random.default_rng(43)
    n = 24
    q_pos = [int(v) for v in rng.integers(200, 3001, n)]
    q_pos[0] = 3000
    sp = synth.Spec("stack-b24", n_seq=n, t_cap=3001, q_pos=q_pos, q_seq=list(range(n)),
                    kv_format="fp4", k=256, window=64, pool=512,
                    schedule=synth.repeating_schedule(6), local_cap=96, seed=47)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    outs, sels, pool = run_stack(sp, x, d)
    err = check_stack(sp, x, d, outs, sels, pool)
    log("stack batch 24 max abs err", err)


def test_stack_pool_not_a_multiple_of_32():
    """A pool of 1000: the Reindex scores of consecutive queries do not start on
    cache-line boundaries unless the score rows are padded (the scoring
    workgroups hand their scores over line by line)."""
    sp = synth.Spec("stack-pool1000", n_seq=3, t_cap=3001, q_pos=[3000, 2222, 1500],
                    q_seq=[0, 1, 2], kv_format="fp4", k=64, window=32, pool=1000,
                    schedule=synth.repeating_schedule(6), local_cap=48, seed=37)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    outs, sels, pool = run_stack(sp, x, d)
    err = check_stack(sp, x, d, outs, sels, pool)
    log("stack pool 1000 max abs err", err)
    outs2, sels2, _ = run_stack(sp, x, d)
    for l in range(sp.n_layers):
        assert torch.equal(outs[l].view(torch.int16), outs2[l].view(torch.int16))
        assert torch.equal(sels[l], sels2[l])


def test_stack_blockwise_small():
    """Blocks of 64 positions: the pool is rescored from its block ids, and
    the position list written only for a caller's pool output."""
    sp = synth.Spec("blockwise-small", n_seq=2, t_cap=20000, q_pos=[19999, 12345], q_seq=[0, 1],
                    kv_format="fp4", k=128, window=16, pool=32 * 64, block=64,
                    schedule=[synth.FULL, synth.REINDEX, synth.REUSE], local_cap=16,
                    needle_blocks=4, seed=41)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    outs, sels, pool = run_stack(sp, x, d)
    check_stack(sp, x, d, outs, sels, pool)
    # without the pool output: the same selections and outputs, bit for bit
    outs2, sels2, pool2 = csa2.stack_run(d.cache, list(sp.schedule), d.q_pos, d.q,
                                         [d.q_idx[l] if sp.schedule[l] != synth.REUSE else None
                                          for l in range(sp.n_layers)],
                                         d.local, sp.k, sp.pool, sp.block, want_pool=False)
    assert pool2 is None
    for l in range(sp.n_layers):
        assert torch.equal(sels[l], sels2[l]), "layer %d selection" % l
        assert torch.equal(outs[l].view(torch.int16), outs2[l].view(torch.int16)), "layer %d" % l


def test_page_schedule_small():
    sp = synth.Spec("page-schedule", n_seq=2, t_cap=2500, q_pos=[2499, 1800], q_seq=[0, 1],
                    kv_format="fp4", k=32, window=16, pool=128,
                    schedule=synth.page_schedule_20(), local_cap=16, seed=51)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    outs, sels, pool = run_stack(sp, x, d)
    check_stack(sp, x, d, outs, sels, pool)


@pytest.mark.parametrize("distinct", [20, 40, 120])
def test_reindex_exact_ties(distinct):
    """Key rows drawn from `distinct` rows, so pool scores tie exactly in
    groups of ~20000/distinct: the Reindex selection must be the oracle's,
    lower positions first inside the boundary group.  Small boundary buckets
    are ranked directly, large ones (20 rows: ~1000 ties) go through the radix
    refinement."""
    sp = synth.Spec("reindex-ties", n_seq=2, t_cap=20000, q_pos=[19999, 15000], q_seq=[0, 1],
                    kv_format="fp4", k=2048, window=16, pool=8192,
                    schedule=[synth.FULL, synth.REINDEX], local_cap=16, seed=61)
    x = synth.make_inputs(sp)
    rng = np.random.default_rng(62 + distinct)
    rows = x.k_idx[0, :distinct].copy()
    for b in range(sp.n_seq):
        x.k_idx[b] = rows[rng.integers(0, distinct, sp.t_cap)]
    d = DevInputs(x)
    outs, sels, pool = run_stack(sp, x, d)
    gpool, g = host(pool), host(sels[1])
    for b in range(sp.n_seq):
        gp = gpool[b]
        assert np.all(gp >= 0)
        ps = oracle.scores(x.q_idx[1, b], x.k_idx[b, gp])
        ref = oracle.topk(ps, sp.k, gp)
        assert np.array_equal(g[b], ref), "b%d: Reindex selection differs from the oracle" % b


# ------------------------------------------------------ named workloads

@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_decode_workload_full_size(cid):
    sp = synth.config(cid)
    log("workload", cid, sp.name)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    outs, sels, pool = run_stack(sp, x, d)
    torch.cuda.synchronize()
    err = check_stack(sp, x, d, outs, sels, pool)
    log("workload", cid, "max abs err", err)


def test_prefill_workload_sampled():
    sp = synth.config(5)
    log("workload 5", sp.name)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    nq = sp.nq
    sel = torch.empty((nq, sp.k), dtype=torch.int32, device="cuda")
    out = torch.empty((nq, 16, 128), dtype=torch.bfloat16, device="cuda")
    chunk = 512
    for i0 in range(0, nq, chunk):
        sl = slice(i0, i0 + chunk)
        sc = csa2.index_score(d.cache, d.q_idx[0][sl], d.q_pos[sl], d.q_seq[sl])
        g, _ = csa2.topk(sc, sp.k)
        sel[sl] = g
        del sc
    out = csa2.sparse_attn(d.cache, d.q[0], d.q_pos, d.q_seq, sel, d.local[0])
    torch.cuda.synchronize()
    gsel = host(sel)
    gout = host(out)
    c = oracle.Cache(x.kv, x.k_idx, fp4=True)
    sample = np.unique(np.concatenate([[0, 1, nq - 1], np.random.default_rng(5).choice(nq, 29)]))
    for i in sample:
        t = sp.q_pos[i]
        s = oracle.scores(x.q_idx[0, i], x.k_idx[0, :t + 1])
        boundary_check(gsel[i], np.arange(t + 1, dtype=np.int32), s, sp.k, "prefill q%d" % i)
    ref = oracle.attend(c, x.q_pos[sample], x.q_seq[sample], x.q[0, sample], gsel[sample],
                        x.local_k[0], x.local_v[0], sp.window, sp.lo)
    err = attn_check(gout[sample], ref, "prefill attention")
    log("prefill sampled max abs err", err)
