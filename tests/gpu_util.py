"""Helpers of the GPU parity tests: device copies of synthetic inputs and the
comparison rules against the oracle.

Rules (parity bar):
  * FP4 codes, scales and dequantised values: bit-exact.
  * Selections: same size; every position in the symmetric difference has an
    oracle fp32 score within 1e-3 (relative) of the oracle's boundary score
    (the k-th, or the pool's P-th); Reuse selections and causal masks exact.
  * Attention outputs: |gpu - oracle| <= 1e-2 + 2e-2 |oracle| element-wise,
    against the oracle's double-precision result on the GPU's own selection.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch

import oracle
import sparse_attention_shared_amd as csa2

ATOL, RTOL = 1e-2, 2e-2
SEL_REL = 1e-3


def dev16(a: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def dev32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class DevInputs:
    """Device copies of a synth.Inputs, with the FP4 cache packed on the GPU."""

    def __init__(self, x):
        sp = x.spec
        self.x = x
        self.kv = dev16(x.kv)
        self.k_idx = dev16(x.k_idx)
        if sp.kv_format in ("fp4", "fp4e"):
            pack = csa2.pack_fp4 if sp.kv_format == "fp4" else csa2.pack_fp4_e4m3
            self.codes, self.scales = pack(self.kv)
            self.cache = csa2.Cache(self.codes, self.k_idx, self.scales)
        else:
            self.codes = self.scales = None
            self.cache = csa2.Cache(self.kv, self.k_idx)
        self.q_pos = dev32(x.q_pos)
        self.q_seq = dev32(x.q_seq)
        self.q = [dev16(x.q[l]) for l in range(sp.n_layers)]
        self.q_idx = [dev16(x.q_idx[l]) for l in range(sp.n_layers)]
        self.local = [csa2.Local(dev16(x.local_k[l]), dev16(x.local_v[l]), sp.window, sp.lo)
                      for l in range(sp.n_layers)]


def oracle_cache(sp, kv, k_idx, m=1):
    """The oracle's view of a cache of the spec's format (m positions per entry)."""
    return oracle.Cache(kv, k_idx, fp4=sp.kv_format != "bf16",
                        scale="e4m3" if sp.kv_format == "fp4e" else "e8m0", m=m)


def boundary_check(gpu_ids, ids, scores, k, what=""):
    """Selection rule against the oracle's own ranking of (ids, scores).

    ids/scores: the candidates (positions and their oracle fp32 scores);
    returns the oracle's chosen set for reference.
    """
    gpu = [int(v) for v in gpu_ids if v >= 0]
    assert len(set(gpu)) == len(gpu), what + ": duplicate positions"
    assert gpu == sorted(gpu), what + ": not ascending"
    ref = oracle.topk(scores, k, ids.astype(np.int32))
    ref_set = set(int(v) for v in ref if v >= 0)
    assert len(gpu) == len(ref_set), "%s: %d chosen, oracle %d" % (what, len(gpu), len(ref_set))
    diff = set(gpu) ^ ref_set
    if diff:
        pos_score = {int(i): float(s) for i, s in zip(ids, scores) if i >= 0}
        sk = min(pos_score[j] for j in ref_set)  # the oracle's k-th score
        for j in diff:
            assert abs(pos_score[j] - sk) <= SEL_REL * abs(sk), \
                "%s: position %d score %r vs boundary %r" % (what, j, pos_score[j], sk)
    return ref_set


def attn_check(gpu_out: np.ndarray, ref: np.ndarray, what=""):
    g = bf16_to_f64(gpu_out)
    err = np.abs(g - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), "%s: %d bad, max abs err %.3g" % (what, int(bad.sum()), err.max())
    return float(err.max())


def par_map(fn, items):
    """fn over items on one thread per available core (the oracle's C calls
    release the GIL); results in order, the first exception re-raised."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    n = max(1, min(16, n))
    with cf.ThreadPoolExecutor(max_workers=n) as ex:
        return list(ex.map(fn, items))
