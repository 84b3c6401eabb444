"""GPU test of csa2_sparse_attn_noalloc (the allocation-free attention): its
outputs must be bit-identical to csa2_sparse_attn's with a workspace, on two
calls in a row -- the second smaller, so it runs on what the first left in
the library's fixed scratch -- and both within the oracle's tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_attention_shared_amd as csa2
from gpu_util import DevInputs, attn_check, dev32, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.device_check()
    yield
    torch.cuda.synchronize()


def _case(nq, k, window, seed):
    rng = np.random.default_rng(seed)
    q_pos = [int(v) for v in rng.integers(k, 6000, nq)]
    q_pos[0] = 5999
    q_seq = [int(v) for v in rng.integers(0, 3, nq)]
    sp = synth.Spec("noalloc", n_seq=3, t_cap=6000, q_pos=q_pos, q_seq=q_seq, kv_format="fp4",
                    k=k, window=window, local_cap=256, seed=seed)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    c = oracle.Cache(x.kv, x.k_idx, fp4=True)
    _, sel, _ = oracle.layer(c, x.q_pos, x.q_seq, oracle.FULL, x.q[0], x.q_idx[0], x.local_k[0],
                             x.local_v[0], window, 0, k)
    sel[::3, ::7] = -1  # empty slots are skipped
    ref = oracle.attend(c, x.q_pos, x.q_seq, x.q[0], sel, x.local_k[0], x.local_v[0], window, 0)
    return d, dev32(sel), ref


def test_noalloc_matches_workspace_form_on_two_calls():
    # 12 queries x 8 chunks, then 5 queries x 3 chunks (a smaller call over
    # the scratch the first left), then a one-chunk call (no scratch at all)
    for i, (nq, k, window) in enumerate([(12, 2048, 128), (5, 600, 40), (4, 200, 16)]):
        d, sel, ref = _case(nq, k, window, 200 + i)
        g = csa2.sparse_attn_noalloc(d.cache, d.q[0], d.q_pos, d.q_seq, sel, d.local[0])
        w = csa2.sparse_attn(d.cache, d.q[0], d.q_pos, d.q_seq, sel, d.local[0])
        torch.cuda.synchronize()
        assert torch.equal(g.view(torch.int16), w.view(torch.int16)), \
            "call %d: outputs differ from the workspace form" % i
        err = attn_check(host(g), ref, "noalloc call %d (nq %d, k %d, W %d)" % (i, nq, k, window))
        print("noalloc call", i, "max abs err", err, flush=True)


def test_noalloc_rejects_calls_beyond_its_scratch():
    d, sel, _ = _case(2, 64, 16, 210)
    loc = d.local[0]
    big = torch.zeros((15, 8704), dtype=torch.int32, device="cuda") - 1  # 15 x 34 chunks > 504
    q = torch.zeros((15, 16, 128), dtype=torch.bfloat16, device="cuda")
    pos = torch.full((15,), 100, dtype=torch.int32, device="cuda")
    with pytest.raises(csa2.Csa2Error, match="allocation-free scratch"):
        csa2.sparse_attn_noalloc(d.cache, q, pos, None, big, loc)
