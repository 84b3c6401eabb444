"""GPU regression tests of workspace reuse: the counters a call leaves in its
workspace sit at addresses that do not depend on the call's shape (attention:
fixed; top-k and the stack: fixed up to 64 rows), so calls of other shapes
sharing one zero-filled workspace must still match the oracle.  Layers of one
stack whose windows differ split their attention into different chunk counts
and share the attention counters."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_attention_shared_amd as csa2
from gpu_util import DevInputs, attn_check, boundary_check, dev16, dev32, host

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


def test_stack_layers_with_different_windows():
    """k = 512 with windows 128, 0, 128, 32: the layers' attention runs 4, 2,
    4 and 2 chunks per query; every layer through the cascade."""
    windows = [128, 0, 128, 32]
    sp = synth.Spec("windows", n_seq=3, t_cap=5003, q_pos=[5002, 3100, 700], q_seq=[0, 1, 2],
                    kv_format="fp4", k=512, window=128, pool=2048,
                    schedule=[synth.FULL, synth.REINDEX, synth.REUSE, synth.REUSE],
                    local_cap=128, seed=81)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    local = [csa2.Local(d.local[l].k, d.local[l].v, windows[l]) for l in range(sp.n_layers)]
    q_idx = [d.q_idx[l] if sp.schedule[l] != synth.REUSE else None for l in range(sp.n_layers)]
    c = oracle.Cache(x.kv, x.k_idx, fp4=True)
    ws = None
    for rep in range(2):  # the second run reuses the first run's workspace
        if ws is None:
            from sparse_attention_shared_amd._lib import _StackArgs, stack_workspace
            outs0 = [torch.empty((3, 16, 128), dtype=torch.bfloat16, device="cuda")
                     for _ in range(sp.n_layers)]
            need = stack_workspace(_StackArgs(d.cache, sp.schedule, d.q_pos, d.q, q_idx, local,
                                              outs0, sp.k, sp.pool, 1, 128 ** -0.5, None, None))
            ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        outs, sels, pool = csa2.stack_run(d.cache, list(sp.schedule), d.q_pos, d.q, q_idx, local,
                                          sp.k, sp.pool, ws=ws)
        torch.cuda.synchronize()
        gsel = [host(s) for s in sels]
        gpool = host(pool)
        for b in range(sp.n_seq):
            t = sp.q_pos[b]
            s = oracle.scores(x.q_idx[0, b], x.k_idx[b, :t + 1])
            ids = np.arange(t + 1, dtype=np.int32)
            boundary_check(gpool[b], ids, s, sp.pool, "pool b%d" % b)
            boundary_check(gsel[0][b], ids, s, sp.k, "full b%d" % b)
            gp = gpool[b]
            ps = oracle.scores(x.q_idx[1, b], x.k_idx[b, gp])
            boundary_check(gsel[1][b], gp, ps, sp.k, "reindex b%d" % b)
        for l in range(sp.n_layers):
            ref = oracle.attend(c, x.q_pos, x.q_seq, x.q[l], gsel[l], x.local_k[l], x.local_v[l],
                                windows[l], 0)
            err = attn_check(host(outs[l]), ref, "run %d layer %d W=%d" % (rep, l, windows[l]))
            log("run", rep, "layer", l, "window", windows[l], "max abs err", err)
    # the workspace's counters are all back to zero
    assert int(ws[:64 * 256 * 2].count_nonzero()) == 0


def test_sparse_attn_calls_sharing_a_workspace():
    """Two calls on one workspace: 8 queries (k = 600, W = 100: 4 chunks),
    then 4 queries (k = 300, W = 40: 2 chunks), then the first again."""
    rng = np.random.default_rng(91)
    shapes = [(8, 600, 100), (4, 300, 40), (8, 600, 100)]
    need = max(csa2.sparse_attn_workspace(nq, k, w) for nq, k, w in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, (nq, k, w) in enumerate(shapes):
        q_pos = [int(v) for v in rng.integers(1000, 5003, nq)]
        q_seq = [int(v) for v in rng.integers(0, 3, nq)]
        sp = synth.Spec("ws-attn", n_seq=3, t_cap=5003, q_pos=q_pos, q_seq=q_seq,
                        kv_format="fp4", k=k, window=w, local_cap=128, seed=92 + i)
        x = synth.make_inputs(sp)
        d = DevInputs(x)
        c = oracle.Cache(x.kv, x.k_idx, fp4=True)
        _, sel, _ = oracle.layer(c, x.q_pos, x.q_seq, oracle.FULL, x.q[0], x.q_idx[0],
                                 x.local_k[0], x.local_v[0], w, 0, k)
        ref = oracle.attend(c, x.q_pos, x.q_seq, x.q[0], sel, x.local_k[0], x.local_v[0], w, 0)
        out = csa2.sparse_attn(d.cache, d.q[0], d.q_pos, d.q_seq, dev32(sel), d.local[0], ws=ws)
        err = attn_check(host(out), ref, "call %d (nq %d, k %d, W %d)" % (i, nq, k, w))
        log("call", i, "max abs err", err)
    torch.cuda.synchronize()
    assert int(ws[:64 * 256].count_nonzero()) == 0


def test_topk_calls_sharing_a_workspace():
    """Long rows (50000 and 70000 slots) on one workspace: 1 row, then 4, then
    2 rows of another length."""
    ws = None
    for i, (nq, n, k, k2) in enumerate([(1, 50000, 300, 3000), (4, 50000, 2048, 0),
                                         (2, 70000, 500, 1000)]):
        rng = np.random.default_rng(100 + i)
        s = (rng.integers(-30, 31, size=(nq, n)) * 0.5).astype(np.float32)
        s[nq - 1] = rng.standard_normal(n).astype(np.float32)
        if ws is None:
            need = max(csa2.topk_workspace(a, b, c, e) for a, b, c, e in
                       [(1, 50000, 300, 3000), (4, 50000, 2048, 0), (2, 70000, 500, 1000)])
            ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        g, g2 = csa2.topk(torch.from_numpy(s).cuda(), k, k2=k2, ws=ws)
        g = host(g)
        for r in range(nq):
            assert np.array_equal(g[r], oracle.topk(s[r], k)), "call %d row %d" % (i, r)
            if k2:
                assert np.array_equal(host(g2)[r], oracle.topk(s[r], k2)), "call %d row %d" % (i, r)
    torch.cuda.synchronize()
