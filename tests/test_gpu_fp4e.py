"""GPU parity of the FP4 cache with one E4M3 scale per 16 channels (the
pages' own form, "DeepSeek-V4.1 Flash Pushes KV Cache Compression for Agent
Workloads"): pack and unpack bit-exact against the oracle, then attention
(split and one-workgroup-per-query kernels), the decode stack with the append,
and the bounded replay on caches of that form."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_attention_shared_amd as csa2
from gpu_util import DevInputs, attn_check, dev16, dev32, host
from test_gpu_parity import _ragged_spec, check_stack, run_stack

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


def test_pack_and_unpack_bit_exact():
    rng = np.random.default_rng(5)
    rows = []
    x = rng.standard_normal((4096, 16)).astype(np.float32)
    x *= np.exp2(rng.integers(-140, 120, size=(4096, 1))).astype(np.float32)
    x[::13] = 0.0
    x[::17, ::3] = -0.0
    rows.append(synth.f32_to_bf16_bits(x).reshape(-1, 256))
    # every finite bf16 pattern next to an anchor that fixes the block scale:
    # a scale of 1 (anchor 6), a subnormal scale, the saturated scale 448, and
    # an anchor whose scale rounds to 0
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    pats = pats[((pats >> 7) & 0xFF) != 0xFF]
    for anchor in (6.0, 6.0 * 2.0 ** -8, 3000.0, 2.0 ** -12):
        a = synth.f32_to_bf16_bits(np.array([anchor], np.float32))[0]
        mag = synth.bf16_bits_to_f32(pats & 0x7FFF)
        p = pats[mag <= anchor]
        p = np.concatenate([p, np.zeros((-p.size) % 15, np.uint16)])
        blk = np.zeros((p.size // 15, 16), np.uint16)
        blk[:, 0] = a
        blk[:, 1:] = p.reshape(-1, 15)
        blk = np.concatenate([blk, np.zeros(((-blk.shape[0]) % 16, 16), np.uint16)])
        rows.append(blk.reshape(-1, 256))
    x = np.concatenate(rows)
    log("fp4e rows", x.shape)
    codes, scales = csa2.pack_fp4_e4m3(dev16(x))
    oc, os_ = oracle.fp4e_pack(x)
    assert np.array_equal(host(scales), os_)
    assert np.array_equal(host(codes), oc)
    deq = host(csa2.unpack_fp4_e4m3(codes, scales)).astype(np.float64)
    odeq = oracle.fp4e_unpack(oc, os_)
    assert np.array_equal(deq, odeq)
    assert np.array_equal(np.signbit(deq), np.signbit(odeq))


@pytest.mark.parametrize("nq", [4, 100])   # split kernel, one workgroup per query
def test_sparse_attn_on_oracle_selection(nq):
    rng = np.random.default_rng(9)
    q_pos = [int(v) for v in rng.integers(0, 5003, nq)]
    q_pos[:4] = [5002, 0, 31, 4100]
    q_seq = [int(v) for v in rng.integers(0, 3, nq)]
    sp = _ragged_spec(kv="fp4e", q_pos=q_pos, q_seq=q_seq, seed=41)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    c = oracle.Cache(x.kv, x.k_idx, fp4=True, scale="e4m3")
    _, sel, _ = oracle.layer(c, x.q_pos, x.q_seq, oracle.FULL, x.q[0], x.q_idx[0], x.local_k[0],
                             x.local_v[0], sp.window, sp.lo, sp.k)
    sel[1::5, ::3] = -1
    ref = oracle.attend(c, x.q_pos, x.q_seq, x.q[0], sel, x.local_k[0], x.local_v[0], sp.window,
                        sp.lo)
    out = host(csa2.sparse_attn(d.cache, d.q[0], d.q_pos, d.q_seq, dev32(sel), d.local[0]))
    err = attn_check(out, ref, "fp4e attn x%d" % nq)
    log("fp4e attn max abs err", err)


def test_page_configuration_stack_with_append():
    """The pages' own parameters on a small cache: E4M3/16 scales, Top-512
    style selection (k = 64 here), the 1 Full / 4 Reindex / 15 Reuse schedule,
    and the decode append of every sequence's position."""
    sp = synth.Spec("page-e4m3", n_seq=2, t_cap=2600, q_pos=[2599, 1900], q_seq=[0, 1],
                    kv_format="fp4e", k=64, window=16, pool=256,
                    schedule=synth.page_schedule_20(), local_cap=32, seed=57)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    rng = np.random.default_rng(58)
    f = synth.f32_to_bf16_bits
    L, S = sp.n_layers, sp.n_seq
    kv_new = f(rng.standard_normal((S, 256)).astype(np.float32))
    kidx_new = f(rng.standard_normal((S, 64)).astype(np.float32))
    k_new = f(rng.standard_normal((L, S, 128)).astype(np.float32))
    v_new = f(rng.standard_normal((L, S, 128)).astype(np.float32))
    outs, sels, pool = csa2.stack_run(
        d.cache, list(sp.schedule), d.q_pos, d.q,
        [d.q_idx[l] if sp.schedule[l] != synth.REUSE else None for l in range(L)],
        d.local, sp.k, sp.pool, sp.block,
        append=(dev16(kv_new), dev16(kidx_new), [dev16(k_new[l]) for l in range(L)],
                [dev16(v_new[l]) for l in range(L)]))
    torch.cuda.synchronize()
    kv2, ki2, lk2, lv2 = oracle.append(x.kv, x.k_idx, x.local_k, x.local_v, x.q_pos, kv_new,
                                       kidx_new, k_new, v_new)
    oc, os_ = oracle.fp4e_pack(kv2)
    assert np.array_equal(host(d.codes), oc) and np.array_equal(host(d.scales), os_)
    x2 = synth.Inputs(sp, kv2, ki2, x.q, x.q_idx, lk2, lv2, x.q_pos, x.q_seq, x.needle_pos)
    err = check_stack(sp, x2, d, outs, sels, pool)
    log("page-configuration stack max abs err", err)


def test_replay_on_e4m3_cache():
    n, T = 70, 3000
    sp = synth.Spec("replay-e4m3", n_seq=1, t_cap=T, q_pos=list(range(T - n, T)), q_seq=[0] * n,
                    kv_format="fp4e", k=64, window=32, pool=256, lo=T - n,
                    schedule=synth.repeating_schedule(6), local_cap=128, seed=59)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    rng = np.random.default_rng(60)
    f = synth.f32_to_bf16_bits
    k_new = f(rng.standard_normal((sp.n_layers, n, 128)).astype(np.float32))
    v_new = f(rng.standard_normal((sp.n_layers, n, 128)).astype(np.float32))
    L = sp.n_layers
    outs, sels, pl = csa2.replay_run(d.cache, list(sp.schedule), 0, d.q_pos, d.q,
                                     [d.q_idx[l] if sp.schedule[l] != synth.REUSE else None
                                      for l in range(L)],
                                     d.local, sp.k, sp.pool,
                                     local_k=[dev16(k_new[l]) for l in range(L)],
                                     local_v=[dev16(v_new[l]) for l in range(L)])
    torch.cuda.synchronize()
    from test_gpu_replay import _rings_after, check_replay
    lk, lv = _rings_after(sp, x, 0, k_new, v_new)
    err = check_replay(sp, x, 0, outs, sels, pl, lk, lv, range(n))
    log("replay e4m3 max abs err", err)


def test_page_configuration_full_size():
    """The pages' own configuration at the 20-layer workload's full size: FP4
    with E4M3 per 16, top-512, SWA 128, the 1 Full / 4 Reindex / 15 Reuse
    schedule, batch 4 at 131072 tokens with an 8192-position pool, and the
    decode append of every sequence's position; every layer of every
    sequence through the cascade."""
    base = synth.config(3)
    sp = synth.Spec(**{**base.__dict__, "name": "page configuration", "kv_format": "fp4e",
                       "k": 512, "schedule": synth.page_schedule_20(), "seed": 1013})
    log("page configuration:", sp.n_seq, "x", sp.t_cap)
    x = synth.make_inputs(sp)
    d = DevInputs(x)
    rng = np.random.default_rng(1014)
    f = synth.f32_to_bf16_bits
    L, S = sp.n_layers, sp.n_seq
    kv_new = f(rng.standard_normal((S, 256)).astype(np.float32))
    kidx_new = f(rng.standard_normal((S, 64)).astype(np.float32))
    k_new = f(rng.standard_normal((L, S, 128)).astype(np.float32))
    v_new = f(rng.standard_normal((L, S, 128)).astype(np.float32))
    outs, sels, pool = csa2.stack_run(
        d.cache, list(sp.schedule), d.q_pos, d.q,
        [d.q_idx[l] if sp.schedule[l] != synth.REUSE else None for l in range(L)],
        d.local, sp.k, sp.pool, sp.block,
        append=(dev16(kv_new), dev16(kidx_new), [dev16(k_new[l]) for l in range(L)],
                [dev16(v_new[l]) for l in range(L)]))
    torch.cuda.synchronize()
    kv2, ki2, lk2, lv2 = oracle.append(x.kv, x.k_idx, x.local_k, x.local_v, x.q_pos, kv_new,
                                       kidx_new, k_new, v_new)
    bi = np.arange(S)
    t = x.q_pos.astype(np.int64)
    oc, os_ = oracle.fp4e_pack(kv2[bi, t])
    assert np.array_equal(host(d.codes)[bi, t], oc) and np.array_equal(host(d.scales)[bi, t], os_)
    x2 = synth.Inputs(sp, kv2, ki2, x.q, x.q_idx, lk2, lv2, x.q_pos, x.q_seq, x.needle_pos)
    err = check_stack(sp, x2, d, outs, sels, pool)
    log("page configuration full size max abs err", err)
