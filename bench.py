"""CSA2 decode benchmark on one MI355X.

Workload: a 20-layer decoder stack sharing one FP4 global KV cache; batch 4,
context 131072 tokens per sequence, 16 query heads over one KV head
(head_dim 128); layer 0 Full builds an 8192-position candidate pool and keeps
top-2048, then [Reindex, Reuse, Reuse, Reuse] repeats; every layer attends to
its 2048 selected entries plus a 128-position local window.

One step = one decode token for every sequence: the append of its position
(global K | V row packed to FP4, indexer key, and the 20 layers' local ring
slots; --no-append leaves it out), then all 20 layers (index scoring, top-k,
gather + FP4 dequant, attention) through the C ABI: by default every kernel
launched from the host (csa2_stack_run); --graph replays a stack recorded once
per cache copy (csa2_stack_plan_create) as a HIP graph.  Inputs are resident
in HBM before the timed region; the timed steps rotate over several copies of
the cache so that consecutive steps do not find it in the 256 MB Infinity
Cache.

The default line also measures the other named workloads as extra keys
(--no-extra leaves them out): one Full layer at batch 1 over 2048 bf16
entries, one Full layer at batch 8 over 32768 FP4 entries, the blockwise
Full layer over 2^20 entries, and the 4096-query prefill chunk.

With --workload prefill it times the prefill chunk alone: 4096 queries at
positions 126976..131071 of one 131072-token sequence, each selecting its
top-2048 positions (csa2_prefill_topk) and attending to them plus its window
(csa2_sparse_attn), reported as query positions per second.  With --workload
replay it times the bounded replay of the last 128 positions of one
131072-token sequence through the same 20-layer stack (csa2_replay_run).
With --workload config1, config2 or config4 it times that single-layer
decode workload alone (the record the default line carries for it).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA2 decode tokens/s + achieved HBM GB/s (% peak) at 128k ctx, FP4 shared KV"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "sparse_attention_shared_amd", "csrc")


# ----------------------------------------------------------------- accounting

def algorithmic_bytes(schedule, B, T, k, P, W, append=True, row=136, block=1):
    """Bytes the method must move per step (the append, selected rows, the
    scans the indexer needs, window, queries, outputs and index lists); the
    dense attention it avoids and intermediates such as score rows are not
    counted.  row: bytes of one global K+V entry (136 with E8M0 per 32, 144
    with E4M3 per 16, 512 in bf16).  block > 1: the Full layer scores
    64-token blocks, then regathers the pool's keys (P of them) tokenwise."""
    kidx = 128           # bf16 indexer key
    win = W * 2 * 128 * 2
    qio = 16 * 128 * 2 * 2  # main Q in + output
    total = 0
    if append:           # read bf16 K|V, key, local K/V; write FP4 row, key, ring slots
        total += 512 + kidx + row + kidx + len(schedule) * 2 * (2 * 128 * 2)
    for m in schedule:
        b = attn_bytes_per_query(k, W, row)
        if m == 0:
            b += T * kidx + 64 * 2 + (P + k) * 4  # full scan, q_I, write pool + sel
            if block > 1:
                nb = (T + block - 1) // block
                b += 2 * nb * 4 + P * kidx + P * 4  # block scores out + in, pool keys, read pool
        elif m == 1:
            b += P * kidx + 64 * 2 + (P + k) * 4  # pool rescore, q_I, read pool, write sel
        total += b
    return total * B


def attn_bytes_per_query(k, W, row=136):
    """Algorithmic bytes of one query's attention: the k gathered global
    entries, the window's bf16 local K and V, main Q in and output out, and
    the selection list read."""
    return k * row + W * 2 * 128 * 2 + 16 * 128 * 2 * 2 + k * 4


def src_hash(names):
    """Fingerprint of kernel sources (the files the kernel is built from)."""
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(CSRC, n), "rb").read())
    return h.hexdigest()[:16]


ATTN_SRC = ("k_attn.hip", "csa2_dev.h", "csa2_kernels.h")


def traffic_from_profile(name, srcs):
    """HBM bytes per launch of a kernel from a committed counter summary
    (profiles/<name>.json), or None when it is missing or the kernel's sources
    changed since it was taken."""
    p = os.path.join(ROOT, "profiles", name + ".json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_src_sha256_16") != src_hash(srcs):
        return None
    return d.get("hbm_bytes_per_launch")


def pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def oracle_threads():
    # the box grants one GPU's share of its CPUs (16)
    return max(1, min(16, host_cores()))


# ------------------------------------------------------------- CPU baseline

def _rate(fn, units_per_call, budget_s, threads, max_calls):
    """Calls fn(i) (each a plain C oracle call that releases the GIL) on
    `threads` threads until the budget; returns (units/s, calls, seconds)."""
    t0 = time.perf_counter()
    n = 0
    if threads == 1:
        while True:
            fn(n)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s or n >= max_calls:
                break
        return n * units_per_call / el, n, el
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        pending = set()
        i = 0
        while True:
            while len(pending) < 2 * threads and i < max_calls and time.perf_counter() - t0 < budget_s:
                pending.add(ex.submit(fn, i))
                i += 1
            if not pending:
                break
            done, pending = cf.wait(pending, return_when=cf.FIRST_COMPLETED)
            for f in done:
                f.result()
                n += 1
        el = time.perf_counter() - t0
    return n * units_per_call / el, n, el


def cpu_baseline_stack(sp, x, budget_s=6.0, what="decode steps", unit="tokens/s"):
    """The oracle (plain C, unchanged) on whole single-sequence stacks of the
    same workload (sequence 0 of the inputs x): one thread, then one thread
    per host core given to this process (independent steps in parallel)."""
    import numpy as np
    import oracle
    c = oracle.Cache(x.kv[:1], x.k_idx[:1], fp4=sp.kv_format != "bf16",
                     scale="e4m3" if sp.kv_format == "fp4e" else "e8m0")
    q_pos = np.ascontiguousarray(x.q_pos[:1])
    q, q_idx = np.ascontiguousarray(x.q[:, :1]), np.ascontiguousarray(x.q_idx[:, :1])
    lk, lv = np.ascontiguousarray(x.local_k[:, :1]), np.ascontiguousarray(x.local_v[:, :1])

    def one(_):
        oracle.stack(c, sp.schedule, q_pos, q, q_idx, lk, lv, sp.window, sp.lo, sp.k, sp.pool,
                     sp.block)

    v1, n1, e1 = _rate(one, 1, budget_s / 2, 1, 64)
    nt = oracle_threads()
    vn, nn, en = _rate(one, 1, budget_s / 2, nt, 4096)
    return {"value": vn, "unit": unit, "cores": nt, "host_cores": host_cores(),
            "value_1thread": v1, "kind": "oracle",
            "sample": "single-sequence %s of the same workload (%s): %d on one thread in "
                      "%.1f s, %d on %d threads in %.1f s; the oracle code is unchanged, the "
                      "threads run independent steps (ctypes releases the GIL); the append's "
                      "few-KB row writes are not in the sample" % (what, sp.name, n1, e1, nn,
                                                                   nt, en)}


def cpu_baseline_prefill(x, sp, budget_s=6.0):
    """The oracle on single queries of the prefill chunk (scores over ~129k
    positions, top-2048, attention): one thread, then one per core."""
    import oracle
    c = oracle.Cache(x.kv, x.k_idx, fp4=True)

    def one(n):
        i = (n * 997) % sp.nq
        t = int(sp.q_pos[i])
        s = oracle.scores(x.q_idx[0, i], x.k_idx[0, :t + 1])
        sel = oracle.topk(s, sp.k)
        oracle.attend(c, x.q_pos[i:i + 1], x.q_seq[i:i + 1], x.q[0, i:i + 1], sel[None],
                      x.local_k[0], x.local_v[0], sp.window, sp.lo)

    v1, n1, e1 = _rate(one, 1, budget_s / 2, 1, 512)
    nt = oracle_threads()
    vn, nn, en = _rate(one, 1, budget_s / 2, nt, 4096)
    return {"value": vn, "unit": "query positions/s", "cores": nt, "host_cores": host_cores(),
            "value_1thread": v1, "kind": "oracle",
            "sample": "queries of the prefill chunk: %d on one thread in %.1f s, %d on %d "
                      "threads in %.1f s" % (n1, e1, nn, nt, en)}


# ------------------------------------------------------------------ devices

def _d16(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


class Timer:
    """HIP events around each timed step (per-step times) and around the whole
    timed region (the mean), on the current stream."""

    def __init__(self, steps):
        import torch
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(steps)]
        self.t0 = torch.cuda.Event(enable_timing=True)
        self.t1 = torch.cuda.Event(enable_timing=True)

    def run(self, step, steps):
        import torch
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        self.t0.record()
        for i in range(steps):
            self.ev[i][0].record()
            step(i)
            self.ev[i][1].record()
        self.t1.record()
        torch.cuda.synchronize()
        self.wall = time.perf_counter() - wall0
        self.ms = self.t0.elapsed_time(self.t1) / steps
        self.per = [a.elapsed_time(b) for a, b in self.ev[:steps]]
        return self.ms

    def stats(self):
        return {"ms_per_step": self.ms, "ms_median": pct(self.per, 50), "ms_p10": pct(self.per, 10),
                "ms_p90": pct(self.per, 90)}


def _events(n):
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:  # create the underlying HIP events
        e.record()
    torch.cuda.synchronize()
    return ev


_HIP = None


def _hip_runtime():
    """The HIP runtime this process runs on (the one torch loaded, which the
    library links against), for the two event calls torch does not expose."""
    global _HIP
    if _HIP is None:
        import ctypes
        import torch
        torch.cuda.init()
        path = next((ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln), None)
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        _HIP = ctypes.CDLL(path)
    return _HIP


class KernelEvent:
    """A HIP event for the start or end of one kernel, created with
    hipEventDisableSystemFence: recording it does no system-scope cache
    write-back and invalidate.  A kernel bracketed by torch's default events
    ran ~1.8 us longer in the profiler's own trace (11.7 vs 9.9 us for the
    decode attention) because that fence becomes part of its end; with these
    it runs as unbracketed launches do (9.9 vs 9.8 us).  Read only after a
    device synchronisation."""
    _FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        self._c = ctypes
        h = ctypes.c_void_p()
        rc = _hip_runtime().hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(self._FLAGS))
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags: %d" % rc)
        self.cuda_event = h.value

    def elapsed_time(self, end):
        ms = self._c.c_float()
        rc = _hip_runtime().hipEventElapsedTime(self._c.byref(ms), self._c.c_void_p(self.cuda_event),
                                                self._c.c_void_p(end.cuda_event))
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime: %d" % rc)
        return ms.value

    def __del__(self):
        if getattr(self, "cuda_event", None) and _HIP is not None:
            _HIP.hipEventDestroy(self._c.c_void_p(self.cuda_event))


def _kernel_events(n):
    return [KernelEvent() for _ in range(n)]


class DecodeSetup:
    """Device inputs of a decode workload: `copies` copies of the cache (rotated
    across steps), per-layer queries and rings, optional append rows."""

    def __init__(self, sp, copies, append, kv_fmt="fp4"):
        import numpy as np
        import torch
        import synth
        import sparse_attention_shared_amd as csa2
        self.sp = sp
        B, L = sp.n_seq, sp.n_layers
        x = synth.make_inputs(sp)
        self.x = x
        kv = _d16(x.kv)
        k_idx0 = _d16(x.k_idx)
        if sp.kv_format == "bf16":
            data0, scales0 = kv, None
        else:
            data0, scales0 = (csa2.pack_fp4 if sp.kv_format == "fp4" else csa2.pack_fp4_e4m3)(kv)
            del kv
        self.caches = []
        for i in range(copies):
            if i == 0:
                d, s, ki = data0, scales0, k_idx0
            else:
                d, s, ki = data0.clone(), (scales0.clone() if scales0 is not None else None), \
                    k_idx0.clone()
            self.caches.append(csa2.Cache(d, ki, s))
        self.q_pos = torch.from_numpy(x.q_pos).cuda()
        self.q = [_d16(x.q[l]) for l in range(L)]
        self.q_idx = [_d16(x.q_idx[l]) if sp.schedule[l] != synth.REUSE else None for l in range(L)]
        self.local = [csa2.Local(_d16(x.local_k[l]), _d16(x.local_v[l]), sp.window) for l in range(L)]
        self.out = [torch.empty((B, 16, 128), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
        # the appended rows are the ones the inputs already hold at q_pos, so
        # every step rewrites the same values and the cache stays what the
        # oracle sees
        self.app = None
        if append:
            bi = np.arange(B)
            t = x.q_pos.astype(np.int64)
            self.app = (_d16(x.kv[bi, t]), _d16(x.k_idx[bi, t]),
                        [_d16(x.local_k[l][bi, t % sp.local_cap]) for l in range(L)],
                        [_d16(x.local_v[l][bi, t % sp.local_cap]) for l in range(L)])
        from sparse_attention_shared_amd._lib import _StackArgs, stack_workspace
        need = stack_workspace(_StackArgs(self.caches[0], sp.schedule, self.q_pos, self.q,
                                          self.q_idx, self.local, self.out, sp.k, sp.pool,
                                          sp.block, 128 ** -0.5, None, None))
        self.ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()

    def step(self, i, scan_ev=None, attn_ev=None):
        import sparse_attention_shared_amd as csa2
        sp = self.sp
        csa2.stack_run(self.caches[i % len(self.caches)], sp.schedule, self.q_pos, self.q,
                       self.q_idx, self.local, sp.k, sp.pool, sp.block, want_sel=False,
                       want_pool=False, ws=self.ws, out=self.out, scan_events=scan_ev,
                       attn_events=attn_ev, append=self.app)


def time_decode(setup, steps, warmup, kernel_events=True, graph=False):
    """Times `steps` decode steps after `warmup` (the value: no event inside a
    step), then, with kernel_events, the same number of steps again in which
    each step times the scan and ONE layer's attention launch (layer i % L at
    step i) with the kernel's own start and end events (KernelEvent: no
    system-scope fence, so the bracketed launch runs as the others do).  Each
    bracketed launch costs the host time (with every launch of a step
    bracketed the GPU waited for the host: 0.68 vs 0.30 ms per step), so the
    timed steps carry none and each kernel-timing step brackets one launch.  Returns (Timer, attention launch durations
    in ms, scan durations in ms, Timer of the kernel-timing steps or None)."""
    import torch
    import sparse_attention_shared_amd as csa2
    sp = setup.sp
    L = sp.n_layers
    tm = Timer(steps)
    attn_ms, scan_ms, tk = [], [], None

    def one_layer(i):
        e = [None] * (2 * L)
        e[2 * (i % L)], e[2 * (i % L) + 1] = _kernel_events(2)
        return e

    if not graph:
        for i in range(warmup):
            setup.step(i)
        tm.run(setup.step, steps)
    else:
        plans = [csa2.StackPlan(c, sp.schedule, setup.q_pos, setup.q, setup.q_idx, setup.local,
                                sp.k, sp.pool, sp.block, out=setup.out, append=setup.app)
                 for c in setup.caches]
        for i in range(warmup):
            plans[i % len(plans)].launch()
        tm.run(lambda i: plans[i % len(plans)].launch(), steps)
        for pl in plans:
            pl.close()
    if kernel_events:
        # events recorded inside a graph do not bracket its kernels, so the
        # kernels are always timed on host-launched steps of the same stack
        n = max(steps, L)
        aev = [one_layer(i) for i in range(n)]
        sev = [_kernel_events(2) for _ in range(n)]
        tk = Timer(n)
        tk.run(lambda i: setup.step(i, sev[i], aev[i]), n)
        for i in range(n):
            l = i % L
            attn_ms.append(aev[i][2 * l].elapsed_time(aev[i][2 * l + 1]))
            scan_ms.append(sev[i][0].elapsed_time(sev[i][1]))
    return tm, attn_ms, scan_ms, tk


def decode_record(setup, tm, attn_ms, scan_ms, row):
    """Throughput, step bandwidth and per-kernel rooflines of a decode run."""
    sp = setup.sp
    B, T = sp.n_seq, sp.t_cap
    step_bytes = algorithmic_bytes(sp.schedule, B, T, sp.k, sp.pool, sp.window,
                                   append=setup.app is not None, row=row, block=sp.block)
    rec = dict(tm.stats())
    rec["value"] = B / (tm.ms * 1e-3)
    rec["step_algorithmic_bytes"] = step_bytes
    rec["hbm_gbps"] = step_bytes / (tm.ms * 1e-3) / 1e9
    rec["hbm_frac_of_peak"] = rec["hbm_gbps"] / PEAK_HBM_GBPS
    kern = {}
    if attn_ms:
        a_ms = sum(attn_ms) / len(attn_ms)
        a_bytes = B * attn_bytes_per_query(sp.k, sp.window, row)
        kern["attention"] = {
            "launches_per_step": sp.n_layers, "launch_ms_mean": a_ms,
            "launch_ms_median": pct(attn_ms, 50), "algorithmic_bytes_per_launch": a_bytes,
            "achieved_gbps": a_bytes / (a_ms * 1e-3) / 1e9,
            "ms_per_step": a_ms * sp.n_layers}
    if scan_ms:
        s_ms = sum(scan_ms) / len(scan_ms)
        s_bytes = B * T * 128
        kern["scan"] = {"launches_per_step": 1, "launch_ms_mean": s_ms,
                        "algorithmic_bytes_per_launch": s_bytes,
                        "achieved_gbps": s_bytes / (s_ms * 1e-3) / 1e9, "ms_per_step": s_ms}
    rec["kernels"] = kern
    return rec


# ----------------------------------------------------------------- workloads

def bench_prefill_run(steps, warmup):
    """The 4096-query prefill chunk: fused indexer top-k then attention, both
    through the C ABI, inputs resident in HBM.  Returns (record, x, sp)."""
    import numpy as np
    import torch
    import synth
    import sparse_attention_shared_amd as csa2

    sp = synth.config(5)
    x = synth.make_inputs(sp)
    codes, scales = csa2.pack_fp4(_d16(x.kv))
    cache = csa2.Cache(codes, _d16(x.k_idx), scales)
    nq = sp.nq
    q_pos = torch.from_numpy(x.q_pos).cuda()
    q_seq = torch.from_numpy(x.q_seq).cuda()
    q = _d16(x.q[0])
    q_idx = _d16(x.q_idx[0])
    local = csa2.Local(_d16(x.local_k[0]), _d16(x.local_v[0]), sp.window)
    sel = torch.empty((nq, sp.k), dtype=torch.int32, device="cuda")
    out = torch.empty((nq, 16, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(csa2.prefill_topk_workspace(nq, sp.t_cap, sp.k), dtype=torch.uint8,
                     device="cuda")
    ev = [_events(3) for _ in range(steps)]

    def step(i, e=None):
        if e:
            e[0].record()
        csa2.prefill_topk(cache, 0, q_idx, q_pos, sp.k, out=sel, ws=ws)
        if e:
            e[1].record()
        csa2.sparse_attn(cache, q, q_pos, q_seq, sel, local, out=out)
        if e:
            e[2].record()

    for i in range(warmup):
        step(i)
    tm = Timer(steps)
    tm.run(lambda i: step(i, ev[i]), steps)
    topk_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / len(ev)
    attn_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / len(ev)
    # algorithmic work: the causal indexer product once, and QK + PV over the
    # selection and window for 16 heads
    pos = np.asarray(sp.q_pos, dtype=np.int64)
    idx_flop = float(2 * 64 * (pos + 1).sum())
    ent = sp.k + np.minimum(pos + 1, sp.window)
    attn_flop = float((2 * 2 * 16 * 128 * ent).sum())
    parts = {
        "csa2_prefill_topk": {"ms": topk_ms, "tflops": idx_flop / (topk_ms * 1e-3) / 1e12,
                              "algorithmic_flop": idx_flop},
        "csa2_sparse_attn": {"ms": attn_ms, "tflops": attn_flop / (attn_ms * 1e-3) / 1e12,
                             "algorithmic_flop": attn_flop},
    }
    dom = max(parts, key=lambda n: parts[n]["ms"])
    rec = dict(tm.stats())
    rec.update({
        "value": nq / (tm.ms * 1e-3), "unit": "query positions/s",
        "tflops": (idx_flop + attn_flop) / (tm.ms * 1e-3) / 1e12,
        "mfma_frac_of_peak": (idx_flop + attn_flop) / (tm.ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "parts": parts,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": parts[dom]["tflops"],
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": parts[dom]["tflops"] / PEAK_BF16_TFLOPS, "traffic": None},
        "wall_s_timed_region": tm.wall,
    })
    return rec, x, sp


def extra_decode(cid, steps, warmup, oracle_budget):
    """One of the single-layer decode workloads (1, 2, 4) as an extra key."""
    import torch
    import synth
    sp = synth.config(cid)
    row = {"bf16": 512, "fp4": 136, "fp4e": 144}[sp.kv_format]
    st = DecodeSetup(sp, copies=2 if cid == 4 else 4, append=False)
    tm, attn_ms, scan_ms, _ = time_decode(st, steps, warmup)
    rec = decode_record(st, tm, attn_ms, scan_ms, row)
    rec["unit"] = "tokens/s"
    rec["workload"] = sp.name
    rec["append"] = False
    if oracle_budget > 0:
        rec["cpu_baseline"] = cpu_baseline_stack(sp, st.x, oracle_budget, "one-layer decode steps")
    del st
    torch.cuda.empty_cache()
    return rec


def bench_replay(args):
    """One step = csa2_replay_run of the last 128 positions of a 131072-token
    sequence through the 20-layer stack (ring rows, Full / Reindex / Reuse
    selections, attention), inputs resident in HBM."""
    import ctypes
    import numpy as np
    import torch
    import oracle
    import synth
    import sparse_attention_shared_amd as csa2
    from sparse_attention_shared_amd import _lib

    base = synth.config(3)
    n, T = 128, base.t_cap
    sp = synth.Spec("replay", n_seq=1, t_cap=T, q_pos=list(range(T - n, T)), q_seq=[0] * n,
                    kv_format="fp4", k=base.k, window=base.window, pool=base.pool,
                    schedule=base.schedule, local_cap=128, lo=T - n, seed=1007)
    L = sp.n_layers
    print("generating inputs ...", file=sys.stderr, flush=True)
    x = synth.make_inputs(sp)
    rng = np.random.default_rng(7)
    k_new = synth.f32_to_bf16_bits(rng.standard_normal((L, n, 128)).astype(np.float32))
    v_new = synth.f32_to_bf16_bits(rng.standard_normal((L, n, 128)).astype(np.float32))
    codes, scales = csa2.pack_fp4(_d16(x.kv))
    cache = csa2.Cache(codes, _d16(x.k_idx), scales)
    q_pos = torch.from_numpy(x.q_pos).cuda()
    q = [_d16(x.q[l]) for l in range(L)]
    q_idx = [_d16(x.q_idx[l]) if sp.schedule[l] != synth.REUSE else None for l in range(L)]
    local = [csa2.Local(_d16(x.local_k[l]), _d16(x.local_v[l]), sp.window, sp.lo) for l in range(L)]
    lk = [_d16(k_new[l]) for l in range(L)]
    lv = [_d16(v_new[l]) for l in range(L)]
    out = [torch.empty((n, 16, 128), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    args_c = _lib._ReplayArgs(cache, sp.schedule, 0, q_pos, q, q_idx, local, out, sp.k, sp.pool,
                              1, 128 ** -0.5, lk, lv)
    ws = torch.zeros(_lib.replay_workspace(args_c), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    L_ = csa2.lib()

    def step(i):
        st = L_.csa2_replay_run(ctypes.byref(args_c.desc), _lib._ptr(ws), ws.numel(),
                                _lib._stream())
        if st:
            raise RuntimeError("csa2_replay_run status %d" % st)

    for i in range(args.warmup):
        step(i)
    tm = Timer(args.steps)
    tm.run(step, args.steps)
    result = {
        "metric": "CSA2 bounded-replay query positions/s (last 128 positions, 20 layers) "
                  "at 128k ctx",
        "value": n / (tm.ms * 1e-3), "unit": "query positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": "bounded replay: the last 128 positions of one 131072-token sequence "
                        "through the 20-layer CSA2 stack (Full pool 8192 then [Reindex, Reuse "
                        "x3]*, top-k 2048, SWA 128 cut off at the segment), FP4 (E2M1 + E8M0/32) "
                        "shared KV, 16 q heads / 1 KV head, head_dim 128, indexer dim 64",
            "queries": n, "context": sp.t_cap, "layers": L, "k": sp.k, "pool": sp.pool,
            "window": sp.window},
        "wall_s_timed_region": tm.wall,
    }
    result.update(tm.stats())
    if not args.no_cpu_baseline:
        print("timing the oracle on the host ...", file=sys.stderr, flush=True)
        c = oracle.Cache(x.kv, x.k_idx, fp4=True)

        def one(i):
            j = (i * 4) % n
            sl = slice(j, j + 4)
            oracle.replay(c, sp.schedule, 0, x.q_pos[sl], x.q[:, sl], x.q_idx[:, sl], x.local_k,
                          x.local_v, sp.window, sp.lo, sp.k, sp.pool, k_new[:, sl], v_new[:, sl])

        v1, n1, e1 = _rate(one, 4, 6.0, 1, 32)
        nt = oracle_threads()
        vn, nn, en = _rate(one, 4, 6.0, nt, 4096)
        result["cpu_baseline"] = {
            "value": vn, "unit": "query positions/s", "cores": nt, "host_cores": host_cores(),
            "value_1thread": v1, "kind": "oracle",
            "sample": "4-position sub-segments through the 20 layers: %d on one thread in %.1f "
                      "s, %d on %d threads in %.1f s" % (n1, e1, nn, nt, en)}
    print(json.dumps(result), flush=True)


def bench_prefill(args):
    rec, x, sp = bench_prefill_run(args.steps, args.warmup)
    result = {
        "metric": "CSA2 prefill-chunk query positions/s at 128k ctx, FP4 shared KV",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": "CSA2 prefill chunk: 4096 queries at positions 126976..131071 of one "
                        "131072-token sequence, FP4 (E2M1 + E8M0/32) shared KV, indexer dim 64, "
                        "top-k 2048, SWA 128, 16 q heads / 1 KV head, head_dim 128",
            "queries": sp.nq, "context": sp.t_cap, "k": sp.k, "window": sp.window},
    }
    result.update(rec)
    if not args.no_cpu_baseline:
        print("timing the oracle on the host ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline_prefill(x, sp)
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=4, help="cache copies rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="leave the other named workloads out of the default line")
    ap.add_argument("--schedule", choices=["repeat", "page"], default="repeat")
    ap.add_argument("--kv", choices=["fp4", "fp4e"], default="fp4",
                    help="fp4: one E8M0 scale per 32 channels; fp4e: one E4M3 scale per 16")
    ap.add_argument("--topk", type=int, default=0, help="selected entries per layer (default 2048)")
    ap.add_argument("--workload", choices=["decode", "prefill", "replay", "config1", "config2",
                                           "config4"], default="decode",
                    help="decode: the 20-layer stack (the metric); configN: one of the "
                         "single-layer decode workloads alone (its record, as in "
                         "extra_workloads, for profiling)")
    ap.add_argument("--graph", action="store_true",
                    help="replay a recorded stack (HIP graph) per step instead of host launches")
    ap.add_argument("--no-append", action="store_true",
                    help="leave the decode append of the new position out of the step")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="do not time the scan and attention kernels inside the timed steps")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(a sharding plan is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import sparse_attention_shared_amd as csa2

    torch.cuda.set_device(0)
    csa2.device_check()
    if args.workload == "prefill":
        bench_prefill(args)
        return
    if args.workload == "replay":
        bench_replay(args)
        return
    if args.workload.startswith("config"):
        rec = extra_decode(int(args.workload[-1]), args.steps, args.warmup,
                           0 if args.no_cpu_baseline else 3.0)
        rec.update({"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "data": "synthetic"})
        print(json.dumps(rec), flush=True)
        return
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 18  # float32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("calibration copy: %d MiB x3" % args.calib_copy_mib, file=sys.stderr, flush=True)
        del src, dst
    sp = synth.config(3)
    if args.schedule == "page":
        sp = synth.Spec(**{**sp.__dict__, "schedule": synth.page_schedule_20()})
    if args.topk:
        sp = synth.Spec(**{**sp.__dict__, "k": args.topk})
    sp = synth.Spec(**{**sp.__dict__, "kv_format": args.kv})
    row = 136 if args.kv == "fp4" else 144
    print("generating inputs ...", file=sys.stderr, flush=True)
    st = DecodeSetup(sp, args.copies, not args.no_append)
    tm, attn_ms, scan_ms, tk = time_decode(st, args.steps, args.warmup,
                                           kernel_events=not args.no_kernel_events,
                                           graph=args.graph)
    rec = decode_record(st, tm, attn_ms, scan_ms, row)
    B = sp.n_seq
    kern = rec.pop("kernels")
    roofline = None
    if kern:
        # the dominant kernel: the most time per step
        name = max(kern, key=lambda n: kern[n]["ms_per_step"])
        kk = kern[name]
        roofline = {
            "kernel": {"attention": "k_attn_chunk (decode attention, one launch per layer)",
                       "scan": "k_score_dense<1> (layer-0 Full indexer scan)"}[name],
            "bound": "hbm", "achieved": kk["achieved_gbps"], "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": kk["achieved_gbps"] / PEAK_HBM_GBPS,
            "traffic": (traffic_from_profile("k_attn_chunk_b4_t131072_fp4_counters", ATTN_SRC)
                        if name == "attention" and args.kv == "fp4" and not args.topk else None),
            "launch_ms": kk["launch_ms_mean"],
            "algorithmic_bytes_per_launch": kk["algorithmic_bytes_per_launch"],
            "share_of_step": kk["ms_per_step"] / rec["ms_per_step"],
            "timing": "kernel's own start/end events (created without the system-scope "
                      "fence) on one bracketed launch per step, over %d steps right after "
                      "the timed ones (their step: %.4f ms)" % (
                          len(attn_ms), tk.ms),
        }
    result = {
        "metric": METRIC,
        "value": rec["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "ms_median": rec["ms_median"], "ms_p10": rec["ms_p10"], "ms_p90": rec["ms_p90"],
        "hbm_gbps": rec["hbm_gbps"],
        "hbm_pct_of_peak": 100.0 * rec["hbm_frac_of_peak"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("decode append + " if st.app is not None else "") +
                        "20-layer CSA2 decode stack over one shared FP4 (E2M1 + %s) global "
                        "KV cache: batch 4, context 131072, 16 q heads / 1 KV head, head_dim "
                        "128, indexer dim 64, Full pool 8192 then %s, "
                        "top-k %d, SWA 128" % ("E8M0/32" if args.kv == "fp4" else "E4M3/16",
                                               "[Reindex, Reuse x3]*" if args.schedule == "repeat"
                                               else "the pages' 1 Full / 4 Reindex / 15 Reuse",
                                               sp.k),
            "kv_scales": "E8M0/32" if args.kv == "fp4" else "E4M3/16",
            "batch": B, "context": sp.t_cap, "layers": sp.n_layers,
            "schedule": "".join("FIU"[m] for m in sp.schedule),
            "k": sp.k, "pool": sp.pool, "window": sp.window,
            "cache_copies_rotated": args.copies,
            "append": st.app is not None,
            "launch": "recorded stack replayed as a HIP graph (csa2_stack_plan_launch)"
                      if args.graph else "host launches (csa2_stack_run)",
        },
        "dtype_note": "FP4 storage (E2M1 codes + block scales), dequantised exactly to bf16 "
                      "MFMA operands, fp32 accumulation, bf16 output",
        "step_algorithmic_bytes": rec["step_algorithmic_bytes"],
        "roofline": roofline,
        "kernels": kern,
        "wall_s_timed_region": tm.wall,
    }
    x3 = st.x
    del st
    torch.cuda.empty_cache()
    if not args.no_extra:
        extra = {}
        for cid, key in ((1, "config1_single_layer_b1_t2048_bf16"),
                         (2, "config2_single_layer_b8_t32768_fp4"),
                         (4, "config4_blockwise_b1_t1048576_fp4")):
            print("extra workload %d ..." % cid, file=sys.stderr, flush=True)
            extra[key] = extra_decode(cid, args.steps, args.warmup,
                                      0 if args.no_cpu_baseline else 3.0)
        print("extra workload 5 ...", file=sys.stderr, flush=True)
        prec, px, psp = bench_prefill_run(args.steps, args.warmup)
        if not args.no_cpu_baseline:
            prec["cpu_baseline"] = cpu_baseline_prefill(px, psp, 4.0)
        prec["workload"] = psp.name
        extra["config5_prefill_q4096_t131072_fp4"] = prec
        result["extra_workloads"] = extra
    if not args.no_cpu_baseline:
        print("timing the oracle on the host ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline_stack(sp, x3, 10.0)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
