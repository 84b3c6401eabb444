"""The C ABI library loads, exports every function include/csa2.h declares, and
validates arguments on the host (these cases fail before any device work, so
they run without a GPU)."""
import ctypes
import os
import re

import pytest
import torch

import sparse_attention_shared_amd as csa2
from sparse_attention_shared_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, INVALID, SHAPE, SCHEDULE, WORKSPACE, UNSUPPORTED, NO_DEVICE, HIP, TOO_LARGE = range(9)


def declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for f in os.listdir(inc):
        if f.endswith(".h"):
            src = open(os.path.join(inc, f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(csa2_\w+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_function():
    L = csa2.lib()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert csa2.version() == 100


def test_status_strings():
    L = csa2.lib()
    for s in range(9):
        assert L.csa2_status_str(s) and L.csa2_status_str(s) != b"unknown status"
    assert L.csa2_status_str(99) == b"unknown status"


FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: every call below fails validation
FAKE_ODD = ctypes.c_void_p(0x10004)  # misaligned


def test_pack_validation():
    L = csa2.lib()
    assert L.csa2_pack_fp4(FAKE, 4, 48, FAKE, FAKE, None) == SHAPE
    assert L.csa2_pack_fp4(FAKE, -1, 32, FAKE, FAKE, None) == SHAPE
    assert L.csa2_pack_fp4(None, 4, 32, FAKE, FAKE, None) == INVALID
    assert L.csa2_pack_fp4(FAKE_ODD, 4, 32, FAKE, FAKE, None) == INVALID
    assert L.csa2_unpack_fp4(FAKE, FAKE, 4, 40, FAKE, None) == SHAPE


def _cache(fmt=csa2.KV_FP4, n_seq=2, t_cap=100, data=FAKE, scales=FAKE, k_idx=FAKE):
    return _lib.csa2_cache(fmt, n_seq, t_cap, data, scales, k_idx)


def test_score_topk_attn_validation():
    L = csa2.lib()
    c = _cache()
    bp = ctypes.byref
    # block must be 1 or 64 on the dense path, 1 with candidates
    assert L.csa2_index_score(bp(c), FAKE, FAKE, None, 2, None, 0, 7, FAKE, 100, None) == SHAPE
    assert L.csa2_index_score(bp(c), FAKE, FAKE, None, 2, FAKE, 10, 64, FAKE, 100, None) == SHAPE
    assert L.csa2_index_score(bp(c), FAKE, FAKE, None, 2, None, 0, 1, FAKE, 99, None) == SHAPE
    assert L.csa2_index_score(bp(_cache(fmt=5)), FAKE, FAKE, None, 2, None, 0, 1, FAKE, 100,
                              None) == INVALID
    assert L.csa2_index_score(bp(_cache(k_idx=None)), FAKE, FAKE, None, 2, None, 0, 1, FAKE, 100,
                              None) == INVALID
    # top-k: k >= 1, k2 >= k, ld >= n
    assert L.csa2_topk(FAKE, 2, 100, 100, None, 0, FAKE, 0, None, None, 0, None) == SHAPE
    assert L.csa2_topk(FAKE, 2, 100, 100, None, 8, FAKE, 4, FAKE, None, 0, None) == SHAPE
    assert L.csa2_topk(FAKE, 2, 100, 50, None, 8, FAKE, 0, None, None, 0, None) == SHAPE
    # attention: window <= cap, FP4 cache needs scales
    loc = _lib.csa2_local(FAKE, FAKE, 64, 128, 0)
    assert L.csa2_sparse_attn(bp(c), FAKE, FAKE, None, 2, FAKE, 8, bp(loc), 0.1, FAKE, FAKE,
                              1 << 20, None) == SHAPE
    loc = _lib.csa2_local(FAKE, FAKE, 128, 128, 0)
    assert L.csa2_sparse_attn(bp(_cache(scales=None)), FAKE, FAKE, None, 2, FAKE, 8, bp(loc), 0.1,
                              FAKE, FAKE, 1 << 20, None) == INVALID
    n = _lib._sz()
    # one workgroup per query (k <= 256, window <= 32): no workspace; a wider
    # window is spread over ceil(window / 32) chunks, which need one
    assert L.csa2_sparse_attn_workspace(2, 8, 32, ctypes.byref(n)) == OK and n.value == 0
    assert L.csa2_sparse_attn_workspace(2, 8, 128, ctypes.byref(n)) == OK and n.value > 0
    assert L.csa2_sparse_attn_workspace(2, 2048, 128, ctypes.byref(n)) == OK and n.value > 0
    # from 20 queries on every query has a workgroup of its own
    m = _lib._sz()
    assert L.csa2_sparse_attn_workspace(19, 2048, 128, ctypes.byref(m)) == OK and m.value > 0
    assert L.csa2_sparse_attn_workspace(20, 2048, 128, ctypes.byref(m)) == OK and m.value == 0
    assert L.csa2_sparse_attn(bp(c), FAKE, FAKE, None, 2, FAKE, 2048, bp(loc), 0.1, FAKE, FAKE,
                              n.value - 1, None) == WORKSPACE


def _desc(modes, k=8, pool=16, block=1, cache=None):
    Lr = len(modes)
    keep = {}
    keep["cache"] = cache or _cache()
    keep["modes"] = (ctypes.c_int32 * Lr)(*modes)
    ptrs = (ctypes.c_void_p * Lr)(*([0x10000] * Lr))
    keep["ptrs"] = ptrs
    keep["loc"] = (_lib.csa2_local * Lr)(*[_lib.csa2_local(FAKE, FAKE, 128, 128, 0)] * Lr)
    d = _lib.csa2_stack_desc(Lr, keep["modes"], ctypes.pointer(keep["cache"]), FAKE, k, pool, block,
                             0.1, ptrs, ptrs, keep["loc"], ptrs, None, None)
    return d, keep


@pytest.mark.parametrize("modes,pool,block,k,want", [
    ([2, 0], 16, 1, 8, SCHEDULE),        # Reuse first
    ([1, 2], 16, 1, 8, SCHEDULE),        # Reindex first
    ([0, 1], 0, 1, 8, SCHEDULE),         # Reindex without a pool
    ([0, 7], 16, 1, 8, SCHEDULE),        # unknown mode
    ([0, 1], 4, 1, 8, SHAPE),            # pool smaller than k
    ([0], 100, 64, 8, SHAPE),            # blockwise pool not a multiple of the block
    ([0], 0, 64, 8, SHAPE),              # blockwise without a pool
    ([0], 16, 3, 8, SHAPE),              # unsupported block size
])
def test_stack_schedule_validation(modes, pool, block, k, want):
    d, keep = _desc(modes, k=k, pool=pool, block=block)
    n = _lib._sz()
    assert csa2.lib().csa2_stack_workspace(ctypes.byref(d), ctypes.byref(n)) == want
    assert csa2.lib().csa2_stack_run(ctypes.byref(d), FAKE, 1 << 30, None) == want


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful without a GPU")
def test_valid_arguments_without_a_device_report_no_device():
    L = csa2.lib()
    assert L.csa2_device_check() == NO_DEVICE
    # valid shapes, validation passes, then the device check refuses: nothing is launched
    assert L.csa2_pack_fp4(FAKE, 4, 32, FAKE, FAKE, None) == NO_DEVICE
    d, keep = _desc([0, 1, 2, 2])
    n = _lib._sz()
    assert L.csa2_stack_workspace(ctypes.byref(d), ctypes.byref(n)) == OK
    assert L.csa2_stack_run(ctypes.byref(d), FAKE, n.value, None) == NO_DEVICE


def test_prefill_validation():
    L = csa2.lib()
    c = _cache(t_cap=1000)
    bp = ctypes.byref
    # prefill scores: sequence in range, row stride >= t_cap, non-null operands
    assert L.csa2_prefill_score(bp(c), 2, FAKE, FAKE, 4, FAKE, 1000, None) == SHAPE
    assert L.csa2_prefill_score(bp(c), 0, FAKE, FAKE, 4, FAKE, 999, None) == SHAPE
    assert L.csa2_prefill_score(bp(c), 0, None, FAKE, 4, FAKE, 1000, None) == INVALID
    assert L.csa2_prefill_score(bp(c), 0, FAKE_ODD, FAKE, 4, FAKE, 1000, None) == INVALID
    # fused prefill top-k: 1 <= k <= 2048, t_cap <= 2^18, workspace large enough
    n = _lib._sz()
    assert L.csa2_prefill_topk_workspace(4, 1000, 0, bp(n)) == SHAPE
    assert L.csa2_prefill_topk_workspace(4, 1000, 4096, bp(n)) == SHAPE
    assert L.csa2_prefill_topk_workspace(4, (1 << 18) + 1, 64, bp(n)) == SHAPE
    assert L.csa2_prefill_topk_workspace(4, 1000, 64, bp(n)) == OK and n.value > 0
    assert L.csa2_prefill_topk(bp(c), 0, FAKE, FAKE, 4, 64, FAKE, FAKE, n.value - 1, None) == WORKSPACE
    assert L.csa2_prefill_topk(bp(c), 0, FAKE, FAKE, 4, 3000, FAKE, FAKE, n.value, None) == SHAPE
    assert L.csa2_prefill_topk(bp(c), 5, FAKE, FAKE, 4, 64, FAKE, FAKE, n.value, None) == SHAPE
    big = _cache(t_cap=(1 << 18) + 64)
    assert L.csa2_prefill_topk(bp(big), 0, FAKE, FAKE, 4, 64, FAKE, FAKE, 1 << 30, None) == SHAPE
    assert L.csa2_prefill_topk(bp(c), 0, None, FAKE, 4, 64, FAKE, FAKE, n.value, None) == INVALID
    # nothing to do is not an error
    assert L.csa2_prefill_topk(bp(c), 0, None, None, 0, 64, None, None, 0, None) == OK


def test_topk_workspace_rule():
    """Rows of at most 32768 slots take one workgroup each (no workspace);
    longer rows take the chunked path, which needs one."""
    L = csa2.lib()
    n = _lib._sz()
    def ws(nq, slots):
        assert L.csa2_topk_workspace(nq, slots, 256, 0, ctypes.byref(n)) == OK
        return n.value
    assert ws(1, 16384) == 0 and ws(300, 16384) == 0
    assert ws(1, 32768) == 0 and ws(500, 32768) == 0
    assert ws(1, 32769) > 0 and ws(500, 40000) > 0


def test_stack_plan_validation():
    L = csa2.lib()
    plan = _lib._P()
    d, keep = _desc([2, 0])  # Reuse first
    assert L.csa2_stack_plan_create(ctypes.byref(d), FAKE, 1 << 30, ctypes.byref(plan)) == SCHEDULE
    assert plan.value is None
    d, keep = _desc([0, 1, 2, 2])
    assert L.csa2_stack_plan_create(ctypes.byref(d), FAKE, 1 << 30, None) == INVALID
    assert L.csa2_stack_plan_create(ctypes.byref(d), FAKE, 1, ctypes.byref(plan)) == WORKSPACE
    assert L.csa2_stack_plan_launch(None, None) == INVALID
    assert L.csa2_stack_plan_destroy(None) == OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful without a GPU")
def test_stack_plan_without_a_device_reports_no_device():
    L = csa2.lib()
    d, keep = _desc([0, 1, 2, 2])
    n = _lib._sz()
    assert L.csa2_stack_workspace(ctypes.byref(d), ctypes.byref(n)) == OK
    plan = _lib._P()
    assert L.csa2_stack_plan_create(ctypes.byref(d), FAKE, n.value, ctypes.byref(plan)) == NO_DEVICE


def test_append_validation():
    L = csa2.lib()
    bp = ctypes.byref
    c = _cache()
    loc = (_lib.csa2_local * 2)(_lib.csa2_local(FAKE, FAKE, 16, 8, 0),
                                _lib.csa2_local(FAKE, FAKE, 0, 0, 0))
    rows = (ctypes.c_void_p * 2)(0x10000, 0x10000)
    odd = (ctypes.c_void_p * 2)(0x10000, 0x10004)
    nul = (ctypes.c_void_p * 2)(0x10000, None)
    assert L.csa2_append(bp(c), None, FAKE, FAKE, 0, None, None, None, None) == INVALID
    assert L.csa2_append(bp(c), FAKE, FAKE_ODD, FAKE, 0, None, None, None, None) == INVALID
    assert L.csa2_append(bp(c), FAKE, FAKE, FAKE_ODD, 0, None, None, None, None) == INVALID
    assert L.csa2_append(bp(c), FAKE, FAKE, FAKE, -1, None, None, None, None) == SHAPE
    assert L.csa2_append(bp(c), FAKE, FAKE, FAKE, 1, None, rows, rows, None) == INVALID
    assert L.csa2_append(bp(c), FAKE, FAKE, FAKE, 2, loc, rows, rows, None) == SHAPE  # cap 0
    loc2 = (_lib.csa2_local * 2)(_lib.csa2_local(FAKE, FAKE, 16, 8, 0),
                                 _lib.csa2_local(FAKE, FAKE, 16, 8, 0))
    assert L.csa2_append(bp(c), FAKE, FAKE, FAKE, 2, loc2, rows, odd, None) == INVALID
    assert L.csa2_append(bp(c), FAKE, FAKE, FAKE, 2, loc2, nul, rows, None) == INVALID
    loc2[1].v = FAKE_ODD
    assert L.csa2_append(bp(c), FAKE, FAKE, FAKE, 2, loc2, rows, rows, None) == INVALID
    # a cache whose rows the append needs
    nodata = _cache(data=None)
    assert L.csa2_append(bp(nodata), FAKE, FAKE, None, 0, None, None, None, None) == INVALID
    noidx = _cache(k_idx=None)
    assert L.csa2_append(bp(noidx), FAKE, FAKE, FAKE, 0, None, None, None, None) == INVALID
    # the stack's append fields
    d, keep = _desc([0, 2])
    n = _lib._sz()
    d.append_kidx = 0x10000  # an indexer row without the KV row
    assert L.csa2_stack_workspace(bp(d), bp(n)) == INVALID
    d.append_kv = 0x10004
    assert L.csa2_stack_workspace(bp(d), bp(n)) == INVALID
    d.append_kv = 0x10000
    assert L.csa2_stack_workspace(bp(d), bp(n)) == OK
    d.append_k = rows  # k rows without v rows
    assert L.csa2_stack_workspace(bp(d), bp(n)) == INVALID
    d.append_v = odd
    assert L.csa2_stack_workspace(bp(d), bp(n)) == INVALID
    d.append_v = rows
    assert L.csa2_stack_workspace(bp(d), bp(n)) == OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful without a GPU")
def test_append_without_a_device_reports_no_device():
    L = csa2.lib()
    c = _cache()
    loc = (_lib.csa2_local * 1)(_lib.csa2_local(FAKE, FAKE, 16, 8, 0))
    rows = (ctypes.c_void_p * 1)(0x10000)
    assert L.csa2_append(ctypes.byref(c), FAKE, FAKE, FAKE, 1, loc, rows, rows, None) == NO_DEVICE
    assert L.csa2_append(ctypes.byref(c), FAKE, None, None, 0, None, None, None, None) == NO_DEVICE


def _replay(modes=(0, 2), seq=0, n=8, k=16, pool=0, cap=128, rows=True):
    keep = {}
    Lr = len(modes)
    keep["cache"] = _cache()
    keep["modes"] = (ctypes.c_int32 * Lr)(*modes)
    ptrs = (ctypes.c_void_p * Lr)(*([0x10000] * Lr))
    keep["ptrs"] = ptrs
    keep["loc"] = (_lib.csa2_local * Lr)(*[_lib.csa2_local(FAKE, FAKE, cap, 32, 0)] * Lr)
    lr = ptrs if rows else None
    d = _lib.csa2_replay_desc(Lr, keep["modes"], ctypes.pointer(keep["cache"]), seq, n, FAKE, k,
                              pool, 1, 0.1, ptrs, ptrs, keep["loc"], lr, lr, ptrs, None, None)
    return d, keep


@pytest.mark.parametrize("kw,want", [
    (dict(seq=2), SHAPE),               # sequence out of range (n_seq = 2)
    (dict(seq=-1), SHAPE),
    (dict(n=0), SHAPE),
    (dict(n=200, cap=128), SHAPE),      # segment rows would share ring slots
    (dict(n=200, cap=128, rows=False), OK),  # no rows written: any n
    (dict(modes=(2, 0)), SCHEDULE),     # Reuse first
    (dict(modes=(0, 1)), SCHEDULE),     # Reindex without a pool
    (dict(), OK),
])
def test_replay_validation(kw, want):
    L = csa2.lib()
    d, keep = _replay(**kw)
    n = _lib._sz()
    assert L.csa2_replay_workspace(ctypes.byref(d), ctypes.byref(n)) == want
    if want != OK:
        assert L.csa2_replay_run(ctypes.byref(d), FAKE, 1 << 30, None) == want
    else:
        assert n.value > 0
        assert L.csa2_replay_run(ctypes.byref(d), FAKE, n.value - 1, None) == WORKSPACE


def test_replay_null_operands():
    L = csa2.lib()
    d, keep = _replay()
    d.q_pos = None
    n = _lib._sz()
    assert L.csa2_replay_workspace(ctypes.byref(d), ctypes.byref(n)) == INVALID
    d, keep = _replay()
    odd = (ctypes.c_void_p * 2)(0x10000, 0x10004)
    d.local_v = odd
    assert L.csa2_replay_workspace(ctypes.byref(d), ctypes.byref(n)) == INVALID


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful without a GPU")
def test_replay_without_a_device_reports_no_device():
    L = csa2.lib()
    d, keep = _replay()
    n = _lib._sz()
    assert L.csa2_replay_workspace(ctypes.byref(d), ctypes.byref(n)) == OK
    assert L.csa2_replay_run(ctypes.byref(d), FAKE, n.value, None) == NO_DEVICE


def test_compression_rate_validation():
    L = csa2.lib()
    bp = ctypes.byref
    c = _cache()
    c.m = 3
    n = _lib._sz()
    assert L.csa2_index_score(bp(c), FAKE, FAKE, None, 2, None, 0, 1, FAKE, 100, None) == SHAPE
    c.m = 2  # the prefill-chunk calls and the replay take entries of two positions
    assert L.csa2_prefill_score(bp(c), 0, FAKE, FAKE, 4, FAKE, 100, None) in (OK, NO_DEVICE)
    assert L.csa2_prefill_topk(bp(c), 0, FAKE, FAKE, 4, 64, FAKE, FAKE, 1 << 30, None) in (
        OK, NO_DEVICE)
    if not torch.cuda.is_available():
        assert L.csa2_prefill_topk(bp(c), 0, FAKE, FAKE, 4, 64, FAKE, FAKE, 1 << 30,
                                   None) == NO_DEVICE
    d, keep = _replay()
    keep["cache"].m = 2
    assert L.csa2_replay_workspace(bp(d), bp(n)) == OK
    # csa2_compress: m in {1, 2}, dim % 8 == 0, aligned operands
    assert L.csa2_compress(FAKE, 4, 3, 256, FAKE, None) == SHAPE
    assert L.csa2_compress(FAKE, 4, 2, 250, FAKE, None) == SHAPE
    assert L.csa2_compress(FAKE, -1, 2, 256, FAKE, None) == SHAPE
    assert L.csa2_compress(None, 4, 2, 256, FAKE, None) == INVALID
    assert L.csa2_compress(FAKE_ODD, 4, 2, 256, FAKE, None) == INVALID


def test_noalloc_attention_limit():
    """The allocation-free attention refuses, before any device work, calls
    whose partials exceed its fixed 4 MiB: nq * chunks <= 504 below 20
    queries, any size from 20 queries on (no scratch is used)."""
    L = csa2.lib()
    c = _cache(n_seq=64, t_cap=5000)
    loc = _lib.csa2_local(FAKE, FAKE, 128, 128, 0)
    bp = ctypes.byref
    # 15 queries x 34 chunks (k = 8704) = 510 > 504
    assert L.csa2_sparse_attn_noalloc(bp(c), FAKE, FAKE, None, 15, FAKE, 8704, bp(loc), 0.1,
                                      FAKE, None) == TOO_LARGE
    # 15 queries x 32 chunks fits; so does any call from 20 queries on
    for nq, k in ((15, 8192), (20, 8704), (2, 2048)):
        st = L.csa2_sparse_attn_noalloc(bp(c), FAKE, FAKE, None, nq, FAKE, k, bp(loc), 0.1, FAKE,
                                        None)
        assert st in (OK, NO_DEVICE) and st != TOO_LARGE
        if not torch.cuda.is_available():
            assert st == NO_DEVICE
    # the usual validation comes first
    assert L.csa2_sparse_attn_noalloc(bp(c), None, FAKE, None, 2, FAKE, 8, bp(loc), 0.1, FAKE,
                                      None) == INVALID
