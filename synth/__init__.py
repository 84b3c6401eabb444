"""Seeded synthetic inputs for CSA2 decode and prefill workloads.

This module is shared by the CPU oracle's callers and the HIP path's callers as
*input only*: it draws random tensors and lays them out.  It holds none of the
method's arithmetic (no scoring, selection, quantisation or attention).

Recipe
------
* Every tensor is drawn from its own NumPy ``PCG64`` stream, keyed by
  ``SeedSequence(seed, spawn_key=(tensor_id, layer, seq))``.  Values are
  standard normal in float32, then rounded to bfloat16 (round to nearest even)
  and stored as ``uint16`` bit patterns.
* Global main KV: one row of 256 bf16 per token, K in channels 0..127 and V in
  channels 128..255 (one KV head, head_dim 128).  Indexer keys: 64 bf16 per
  token.  Both are shared by every decoder layer of a sequence.
* Per layer: main queries ``[nq][16][128]``, indexer queries ``[nq][64]`` and
  the local (sliding-window) K and V, held in a ring of ``cap`` slots per
  sequence where position ``p`` lives in slot ``p % cap``.
* Needles: positions drawn without replacement from their own stream; the main
  K (channels 0..127) and the indexer key at those positions are multiplied
  by 4 (exact in bf16).  Blockwise workloads plant whole 64-token blocks.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

H = 16          # query heads sharing one KV head
D = 128         # head_dim of K and V
D_IDX = 64      # indexer dimension
ROW = 2 * D     # bf16 channels per global KV row (K | V)

FULL, REINDEX, REUSE = 0, 1, 2
MODE_NAMES = {FULL: "Full", REINDEX: "Reindex", REUSE: "Reuse"}

# tensor ids of the named random streams
_T_KV, _T_KIDX, _T_Q, _T_QIDX, _T_LK, _T_LV, _T_NEEDLE = 1, 2, 3, 4, 5, 6, 7


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, tensor: int, layer: int = 0, seq: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(tensor, layer, seq))
    return np.random.Generator(np.random.PCG64(ss))


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


def schedule_from_string(s: str) -> List[int]:
    m = {"F": FULL, "I": REINDEX, "U": REUSE}
    return [m[c] for c in s]


def repeating_schedule(n_layers: int) -> List[int]:
    """Layer 0 Full, then [Reindex, Reuse, Reuse, Reuse] repeated."""
    cyc = [REINDEX, REUSE, REUSE, REUSE]
    return [FULL] + [cyc[i % 4] for i in range(n_layers - 1)]


def page_schedule_20() -> List[int]:
    """[Full + 3 Reuse] then 4 x [Reindex + 3 Reuse]: 1 Full, 4 Reindex, 15 Reuse."""
    return [FULL, REUSE, REUSE, REUSE] + [REINDEX, REUSE, REUSE, REUSE] * 4


@dataclasses.dataclass
class Spec:
    """Shape of one CSA2 workload.

    ``q_pos`` lists the query position of each query; ``q_seq`` its sequence.
    Decode has one query per sequence; a prefill chunk has many queries on one
    sequence.
    """
    name: str
    n_seq: int
    t_cap: int                 # global KV rows allocated per sequence
    q_pos: List[int]
    q_seq: List[int]
    kv_format: str             # "fp4" (E8M0 per 32), "fp4e" (E4M3 per 16) or "bf16"
    k: int                     # selected global entries per query
    window: int                # SWA window W
    pool: int = 0              # Full-layer candidate pool size in tokens (0 = none)
    block: int = 1             # 1 = tokenwise Full scoring, >1 = blockwise
    schedule: Sequence[int] = (FULL,)
    local_cap: int = 128       # ring slots of local KV per sequence
    lo: int = 0                # lowest position the window may read
    needles: int = 0           # planted needle tokens per sequence
    needle_blocks: int = 0     # planted needle blocks (of ``block`` tokens)
    seed: int = 1000

    @property
    def nq(self) -> int:
        return len(self.q_pos)

    @property
    def n_layers(self) -> int:
        return len(self.schedule)


def config(cid: int) -> Spec:
    """The five named workloads (decode configs 1-4, prefill config 5)."""
    if cid == 1:
        return Spec("single layer Full, B=1, T=2048, bf16 KV, k=256, W=128, 8 needles",
                    n_seq=1, t_cap=2048, q_pos=[2047], q_seq=[0], kv_format="bf16",
                    k=256, window=128, needles=8, seed=1001)
    if cid == 2:
        return Spec("single layer Full, B=8, T=32768, FP4 KV, k=2048, W=128",
                    n_seq=8, t_cap=32768, q_pos=[32767] * 8, q_seq=list(range(8)),
                    kv_format="fp4", k=2048, window=128, seed=1002)
    if cid == 3:
        return Spec("20-layer stack F+(I,U,U,U)*, B=4, T=131072, FP4 KV, pool 8192, k=2048, W=128",
                    n_seq=4, t_cap=131072, q_pos=[131071] * 4, q_seq=list(range(4)),
                    kv_format="fp4", k=2048, window=128, pool=8192,
                    schedule=repeating_schedule(20), seed=1003)
    if cid == 4:
        return Spec("single layer blockwise Full, B=1, T=2^20, FP4 KV, 64-token blocks, "
                    "256-block pool, k=2048, W=128, 32 needle blocks",
                    n_seq=1, t_cap=1 << 20, q_pos=[(1 << 20) - 1], q_seq=[0],
                    kv_format="fp4", k=2048, window=128, pool=256 * 64, block=64,
                    needle_blocks=32, seed=1004)
    if cid == 5:
        start, n = 126976, 4096
        return Spec("prefill chunk of 4096 queries at 126976.., T=131072, FP4 KV, k=2048, W=128",
                    n_seq=1, t_cap=131072, q_pos=list(range(start, start + n)), q_seq=[0] * n,
                    kv_format="fp4", k=2048, window=128, local_cap=4352, seed=1005)
    raise ValueError(cid)


@dataclasses.dataclass
class Inputs:
    spec: Spec
    kv: np.ndarray             # uint16 [n_seq][t_cap][256] bf16 bits (K | V)
    k_idx: np.ndarray          # uint16 [n_seq][t_cap][64]
    q: np.ndarray              # uint16 [n_layers][nq][16][128]
    q_idx: np.ndarray          # uint16 [n_layers][nq][64]
    local_k: np.ndarray        # uint16 [n_layers][n_seq][local_cap][128]
    local_v: np.ndarray        # uint16 [n_layers][n_seq][local_cap][128]
    q_pos: np.ndarray          # int32 [nq]
    q_seq: np.ndarray          # int32 [nq]
    needle_pos: List[np.ndarray]


def make_inputs(spec: Spec, layers: Optional[Sequence[int]] = None) -> Inputs:
    """Draw every tensor of ``spec`` from its named stream.

    ``layers`` restricts the per-layer tensors that are drawn (others are left
    zero); the global cache is always drawn whole.
    """
    S, T, L, nq = spec.n_seq, spec.t_cap, spec.n_layers, spec.nq
    kv = np.empty((S, T, ROW), np.uint16)
    k_idx = np.empty((S, T, D_IDX), np.uint16)
    needle_pos = []
    for s in range(S):
        kv[s] = _normal_bf16(_rng(spec.seed, _T_KV, 0, s), (T, ROW))
        k_idx[s] = _normal_bf16(_rng(spec.seed, _T_KIDX, 0, s), (T, D_IDX))
        pos = np.zeros(0, np.int64)
        nr = _rng(spec.seed, _T_NEEDLE, 0, s)
        if spec.needles:
            pos = np.sort(nr.choice(T, size=spec.needles, replace=False))
        elif spec.needle_blocks:
            nb = T // spec.block
            blocks = np.sort(nr.choice(nb, size=spec.needle_blocks, replace=False))
            pos = (blocks[:, None] * spec.block + np.arange(spec.block)[None, :]).reshape(-1)
        if pos.size:
            four = np.float32(4.0)
            kf = bf16_bits_to_f32(kv[s, pos, :D]) * four
            kv[s, pos, :D] = f32_to_bf16_bits(kf)
            kif = bf16_bits_to_f32(k_idx[s, pos]) * four
            k_idx[s, pos] = f32_to_bf16_bits(kif)
        needle_pos.append(pos)
    q = np.zeros((L, nq, H, D), np.uint16)
    q_idx = np.zeros((L, nq, D_IDX), np.uint16)
    lk = np.zeros((L, S, spec.local_cap, D), np.uint16)
    lv = np.zeros((L, S, spec.local_cap, D), np.uint16)
    want = range(L) if layers is None else layers
    for l in want:
        q[l] = _normal_bf16(_rng(spec.seed, _T_Q, l, 0), (nq, H, D))
        q_idx[l] = _normal_bf16(_rng(spec.seed, _T_QIDX, l, 0), (nq, D_IDX))
        for s in range(S):
            lk[l, s] = _normal_bf16(_rng(spec.seed, _T_LK, l, s), (spec.local_cap, D))
            lv[l, s] = _normal_bf16(_rng(spec.seed, _T_LV, l, s), (spec.local_cap, D))
    return Inputs(spec, kv, k_idx, q, q_idx, lk, lv,
                  np.asarray(spec.q_pos, np.int32), np.asarray(spec.q_seq, np.int32),
                  needle_pos)
