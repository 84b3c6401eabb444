"""GPU tests of the recorded stack (csa2_stack_plan_*, a HIP graph): every
replay must equal an eager csa2_stack_run of the same inputs bit for bit, with
eager work and synchronisations between replays, also after inputs change in
place; and the plan's outputs pass the oracle cascade."""
import numpy as np
import pytest
import torch

import synth
import sparse_attention_shared_amd as csa2
from gpu_util import DevInputs
from test_gpu_parity import check_stack, run_stack

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


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def _plan(sp, d, want_sel=True):
    return csa2.StackPlan(d.cache, list(sp.schedule), d.q_pos, d.q,
                          [d.q_idx[l] if sp.schedule[l] != synth.REUSE else None
                           for l in range(sp.n_layers)],
                          d.local, sp.k, sp.pool, sp.block, want_sel=want_sel)


def _check_replays(sp, x, d, want_sel=True, replays=3):
    plan = _plan(sp, d, want_sel)
    for rep in range(replays):
        plan.launch()
        torch.cuda.synchronize()
        outs, sels, pool = run_stack(sp, x, d, want_sel=want_sel)  # eager, in between
        torch.cuda.synchronize()
        for l in range(sp.n_layers):
            assert _same(plan.out[l], outs[l]), "replay %d layer %d output" % (rep, l)
            if want_sel:
                assert _same(plan.sel[l], sels[l]), "replay %d layer %d selection" % (rep, l)
        if plan.pool is not None:
            assert _same(plan.pool, pool), "replay %d pool" % rep
        # unrelated eager work on the same stream between replays
        junk = torch.randn(1 << 20, device="cuda").sum()
        del junk
    return plan


def test_plan_small_ragged_stack_and_oracle():
    sp = synth.Spec("stack-small", n_seq=3, t_cap=3001, q_pos=[3000, 1777, 300], q_seq=[0, 1, 2],
                    kv_format="fp4", k=64, window=32, pool=256,
                    schedule=synth.repeating_schedule(7), local_cap=48, seed=31)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    plan = _check_replays(sp, x, d)
    err = check_stack(sp, x, d, plan.out, plan.sel, plan.pool)
    log("plan small max abs err", err)
    # new query values in place: the next replay must use them
    rng = np.random.default_rng(5)
    for l in range(sp.n_layers):
        d.q[l].copy_(torch.from_numpy(synth.f32_to_bf16_bits(
            rng.standard_normal(tuple(d.q[l].shape)).astype(np.float32)).view(np.int16)).cuda()
            .view(torch.bfloat16))
    plan.launch()
    torch.cuda.synchronize()
    outs, _, _ = run_stack(sp, x, d)
    for l in range(sp.n_layers):
        assert _same(plan.out[l], outs[l]), "after in-place update, layer %d" % l
    plan.close()


def test_plan_blockwise_stack():
    sp = synth.Spec("blockwise-small", n_seq=2, t_cap=20000, q_pos=[19999, 12345], q_seq=[0, 1],
                    kv_format="fp4", k=128, window=16, pool=32 * 64, block=64,
                    schedule=[synth.FULL, synth.REINDEX, synth.REUSE], local_cap=16,
                    needle_blocks=4, seed=41)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    _check_replays(sp, x, d).close()


def test_plan_decode_workload_full_size():
    sp = synth.config(3)
    log("workload 3 through a plan")
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    _check_replays(sp, x, d, want_sel=False).close()
