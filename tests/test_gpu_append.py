"""GPU parity of the decode append (csa2_append, and the append step of a
stack run or plan) against the oracle's append: the written global rows,
indexer keys and local ring slots bit for bit, every other row untouched, and
the stack that follows reading the new position (oracle cascade)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_attention_shared_amd as csa2
from gpu_util import DevInputs, dev16, dev32, host
from test_gpu_parity import _blocks_with_varied_scales, check_stack, run_stack

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


def _bf16(rng, shape):
    return synth.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def _new_rows(S, L, seed, varied=True):
    """New rows; with `varied` the K | V row spans every FP4 block scale."""
    rng = np.random.default_rng(seed)
    kv_new = (_blocks_with_varied_scales(8 * S, seed).reshape(S, 256) if varied
              else _bf16(rng, (S, 256)))
    return kv_new, _bf16(rng, (S, 64)), _bf16(rng, (L, S, 128)), _bf16(rng, (L, S, 128))


def _check_cache(sp, d, kv, k_idx, what):
    if sp.kv_format in ("fp4", "fp4e"):
        oc, os_ = (oracle.fp4_pack if sp.kv_format == "fp4" else oracle.fp4e_pack)(kv)
        assert np.array_equal(host(d.codes), oc), what + ": FP4 codes"
        assert np.array_equal(host(d.scales), os_), what + ": FP4 scales"
    else:
        assert np.array_equal(host(d.kv), kv), what + ": bf16 rows"
    assert np.array_equal(host(d.k_idx), k_idx), what + ": indexer keys"


@pytest.mark.parametrize("kv", ["fp4", "bf16"])
def test_append_rows_bit_exact(kv):
    sp = synth.Spec("append-rows", n_seq=4, t_cap=1000, q_pos=[999, 0, 517, 3],
                    q_seq=[0, 1, 2, 3], kv_format=kv, k=8, window=8, local_cap=48,
                    schedule=[synth.FULL] * 3, seed=61)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    S, L = sp.n_seq, sp.n_layers
    kv_new, kidx_new, k_new, v_new = _new_rows(S, L, 7)
    # a fourth ring of another capacity, and two sequences that are skipped
    rng = np.random.default_rng(8)
    ek, ev = _bf16(rng, (1, S, 7, 128)), _bf16(rng, (1, S, 7, 128))
    extra = csa2.Local(dev16(ek[0]), dev16(ev[0]), 4)
    ekn, evn = _bf16(rng, (1, S, 128)), _bf16(rng, (1, S, 128))
    pos = np.array([999, 0, -1, 1000], np.int32)
    log("append rows", kv, pos.tolist())
    csa2.append(d.cache, dev32(pos), dev16(kv_new), dev16(kidx_new), d.local + [extra],
                [dev16(k_new[l]) for l in range(L)] + [dev16(ekn[0])],
                [dev16(v_new[l]) for l in range(L)] + [dev16(evn[0])])
    torch.cuda.synchronize()
    kv2, ki2, lk2, lv2 = oracle.append(x.kv, x.k_idx, x.local_k, x.local_v, pos, kv_new,
                                       kidx_new, k_new, v_new)
    _check_cache(sp, d, kv2, ki2, "append")
    for l in range(L):
        assert np.array_equal(host(d.local[l].k), lk2[l]), "ring K layer %d" % l
        assert np.array_equal(host(d.local[l].v), lv2[l]), "ring V layer %d" % l
    _, _, ek2, ev2 = oracle.append(x.kv, x.k_idx, ek, ev, pos, kv_new, None, ekn, evn)
    assert np.array_equal(host(extra.k), ek2[0]) and np.array_equal(host(extra.v), ev2[0])
    # local rings only, no global row
    kv3, kidx3, k3, v3 = _new_rows(S, L, 9)
    pos = np.array([5, 6, 7, 8], np.int32)
    csa2.append(d.cache, dev32(pos), None, None, d.local, [dev16(k3[l]) for l in range(L)],
                [dev16(v3[l]) for l in range(L)])
    torch.cuda.synchronize()
    _check_cache(sp, d, kv2, ki2, "ring-only append")
    _, _, lk3, lv3 = oracle.append(kv2, ki2, lk2, lv2, pos, kv3, None, k3, v3)
    for l in range(L):
        assert np.array_equal(host(d.local[l].k), lk3[l])
        assert np.array_equal(host(d.local[l].v), lv3[l])


def test_append_more_layers_than_one_launch_holds():
    S, L, cap = 2, 70, 4
    rng = np.random.default_rng(12)
    kv = _bf16(rng, (S, 50, 256))
    ki = _bf16(rng, (S, 50, 64))
    lk, lv = _bf16(rng, (L, S, cap, 128)), _bf16(rng, (L, S, cap, 128))
    codes, scales = csa2.pack_fp4(dev16(kv))
    cache = csa2.Cache(codes, dev16(ki), scales)
    local = [csa2.Local(dev16(lk[l]), dev16(lv[l]), cap) for l in range(L)]
    kv_new, kidx_new, k_new, v_new = _new_rows(S, L, 13)
    pos = np.array([49, 22], np.int32)
    csa2.append(cache, dev32(pos), dev16(kv_new), dev16(kidx_new), local,
                [dev16(k_new[l]) for l in range(L)], [dev16(v_new[l]) for l in range(L)])
    torch.cuda.synchronize()
    kv2, ki2, lk2, lv2 = oracle.append(kv, ki, lk, lv, pos, kv_new, kidx_new, k_new, v_new)
    oc, os_ = oracle.fp4_pack(kv2)
    assert np.array_equal(host(codes), oc) and np.array_equal(host(scales), os_)
    assert np.array_equal(host(cache.k_idx), ki2)
    for l in range(L):
        assert np.array_equal(host(local[l].k), lk2[l]), "ring K layer %d" % l
        assert np.array_equal(host(local[l].v), lv2[l]), "ring V layer %d" % l


def _stack_spec():
    return synth.Spec("stack-append", n_seq=3, t_cap=3001, q_pos=[3000, 1777, 300],
                      q_seq=[0, 1, 2], kv_format="fp4", k=64, window=32, pool=256,
                      schedule=synth.repeating_schedule(7), local_cap=48, seed=33)


def _stack_rows(sp, x, seed):
    S, L = sp.n_seq, sp.n_layers
    kv_new, kidx_new, k_new, v_new = _new_rows(S, L, seed, varied=False)
    # sequence 0's new key is 4x its layer-0 indexer query: its own position
    # must win layer 0's scan, which only happens if the scan reads the append
    kidx_new[0] = synth.f32_to_bf16_bits(4.0 * synth.bf16_bits_to_f32(x.q_idx[0, 0]))
    return kv_new, kidx_new, k_new, v_new


def _append_arg(rows):
    kv_new, kidx_new, k_new, v_new = rows
    L = k_new.shape[0]
    return (dev16(kv_new), dev16(kidx_new), [dev16(k_new[l]) for l in range(L)],
            [dev16(v_new[l]) for l in range(L)])


def _appended_inputs(sp, x, rows):
    kv_new, kidx_new, k_new, v_new = rows
    kv2, ki2, lk2, lv2 = oracle.append(x.kv, x.k_idx, x.local_k, x.local_v, x.q_pos, kv_new,
                                       kidx_new, k_new, v_new)
    x2 = synth.Inputs(sp, kv2, ki2, x.q, x.q_idx, lk2, lv2, x.q_pos, x.q_seq, x.needle_pos)
    return x2


def test_stack_with_append_matches_oracle():
    sp = _stack_spec()
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    rows = _stack_rows(sp, x, 21)
    log("stack with append")
    outs, sels, pool = csa2.stack_run(
        d.cache, list(sp.schedule), d.q_pos, d.q,
        [d.q_idx[l] if sp.schedule[l] != synth.REUSE else None for l in range(sp.n_layers)],
        d.local, sp.k, sp.pool, sp.block, append=_append_arg(rows))
    torch.cuda.synchronize()
    x2 = _appended_inputs(sp, x, rows)
    _check_cache(sp, d, x2.kv, x2.k_idx, "stack append")
    assert sp.q_pos[0] in host(sels[0])[0].tolist()
    err = check_stack(sp, x2, d, outs, sels, pool)
    log("stack with append max abs err", err)


def test_plan_with_append_and_in_place_rows():
    sp = _stack_spec()
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    rows = _stack_rows(sp, x, 22)
    app = _append_arg(rows)
    plan = csa2.StackPlan(
        d.cache, list(sp.schedule), d.q_pos, d.q,
        [d.q_idx[l] if sp.schedule[l] != synth.REUSE else None for l in range(sp.n_layers)],
        d.local, sp.k, sp.pool, sp.block, want_sel=True, append=app)
    plan.launch()
    torch.cuda.synchronize()
    x2 = _appended_inputs(sp, x, rows)
    _check_cache(sp, d, x2.kv, x2.k_idx, "plan append")
    check_stack(sp, x2, d, plan.out, plan.sel, plan.pool)
    # new rows written in place into the same buffers: the next launch appends them
    rows2 = _stack_rows(sp, x, 23)
    for dst, src in zip(app[:2], rows2[:2]):
        dst.copy_(dev16(src))
    for l in range(sp.n_layers):
        app[2][l].copy_(dev16(rows2[2][l]))
        app[3][l].copy_(dev16(rows2[3][l]))
    plan.launch()
    torch.cuda.synchronize()
    x3 = _appended_inputs(sp, x2, rows2)
    _check_cache(sp, d, x3.kv, x3.k_idx, "plan append after in-place update")
    err = check_stack(sp, x3, d, plan.out, plan.sel, plan.pool)
    log("plan with append max abs err", err)
    # an eager run with the same rows gives the plan's outputs bit for bit
    outs, sels, pool = run_stack(sp, x3, d)
    for l in range(sp.n_layers):
        assert torch.equal(outs[l].view(torch.int16), plan.out[l].view(torch.int16))
        assert torch.equal(sels[l], plan.sel[l])
    plan.close()
