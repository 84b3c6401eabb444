"""ctypes wrapper of the plain C reference of CSA2 sparse attention.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the GPU
library (``sparse_attention_shared_amd``) and neither imports the other; both
take their inputs from ``synth``.

Every function here marshals numpy arrays into ``csa2_oracle.c``; all of the
arithmetic is in that file, in double precision.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FULL, REINDEX, REUSE = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.orc_fp4_pack.argtypes = [P, i64, i32, P, P]
        L.orc_fp4_unpack.argtypes = [P, P, i64, i32, P]
        L.orc_fp4e_pack.argtypes = [P, i64, i32, P, P]
        L.orc_fp4e_unpack.argtypes = [P, P, i64, i32, P]
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_value.restype = dbl
        L.orc_scores.argtypes = [P, P, i64, P]
        L.orc_scores.restype = None
        L.orc_block_scores.argtypes = [P, i64, i32, P]
        L.orc_block_scores.restype = None
        L.orc_topk.argtypes = [P, P, i64, i32, P]
        L.orc_topk.restype = i32
        L.orc_attention.argtypes = [P, P, P, i64, dbl, P]
        L.orc_attention.restype = None
        L.orc_layer.argtypes = [i32, P, P, i32, i32, i64, i32, P, P, P, P, P, P, P, P,
                                i32, i32, i32, i32, i32, i32, P, P, dbl, P]
        L.orc_attend.argtypes = [i32, P, P, i32, i64, i32, P, P, P, P, P, i32, P, P,
                                 i32, i32, i32, dbl, P]
        L.orc_stack.argtypes = [i32, P, i32, P, i32, i64, i32, P, P, P, P, P, P, P, P,
                                i32, i32, i32, i32, i32, i32, dbl, P, P, P]
        L.orc_compress.argtypes = [P, i64, i32, i32, P]
        L.orc_append.argtypes = [i32, i64, P, P, P, P, P, i32, i32, P, P, P, P]
        L.orc_replay.argtypes = [i32, P, i32, i32, i32, P, i32, i64, i32, P, P, P, P, P, P, P, P,
                                 i32, i32, i32, i32, i32, i32, P, P, dbl, P, P, P]
        L.orc_append.restype = None
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def fp4_pack(x_bf16: np.ndarray):
    """[..., dim] bf16 bits -> (codes [..., dim/2] u8, scales [..., dim/32] u8)."""
    x = _c(x_bf16, np.uint16)
    dim = x.shape[-1]
    rows = x.size // dim
    codes = np.empty(x.shape[:-1] + (dim // 2,), np.uint8)
    scales = np.empty(x.shape[:-1] + (dim // 32,), np.uint8)
    rc = lib().orc_fp4_pack(_p(x), rows, dim, _p(codes), _p(scales))
    if rc:
        raise ValueError("orc_fp4_pack rc=%d" % rc)
    return codes, scales


def fp4_unpack(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    c = _c(codes, np.uint8)
    s = _c(scales, np.uint8)
    dim = c.shape[-1] * 2
    rows = c.size // c.shape[-1]
    out = np.empty(c.shape[:-1] + (dim,), np.float64)
    rc = lib().orc_fp4_unpack(_p(c), _p(s), rows, dim, _p(out))
    if rc:
        raise ValueError("orc_fp4_unpack rc=%d" % rc)
    return out


def fp4e_pack(x_bf16: np.ndarray):
    """FP4 with one E4M3 scale per 16: [..., dim] bf16 bits -> (codes
    [..., dim/2] u8, scales [..., dim/16] u8)."""
    x = _c(x_bf16, np.uint16)
    dim = x.shape[-1]
    rows = x.size // dim
    codes = np.empty(x.shape[:-1] + (dim // 2,), np.uint8)
    scales = np.empty(x.shape[:-1] + (dim // 16,), np.uint8)
    rc = lib().orc_fp4e_pack(_p(x), rows, dim, _p(codes), _p(scales))
    if rc:
        raise ValueError("orc_fp4e_pack rc=%d" % rc)
    return codes, scales


def fp4e_unpack(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    c = _c(codes, np.uint8)
    s = _c(scales, np.uint8)
    dim = c.shape[-1] * 2
    rows = c.size // c.shape[-1]
    out = np.empty(c.shape[:-1] + (dim,), np.float64)
    rc = lib().orc_fp4e_unpack(_p(c), _p(s), rows, dim, _p(out))
    if rc:
        raise ValueError("orc_fp4e_unpack rc=%d" % rc)
    return out


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(int(code))


def scores(q_idx: np.ndarray, k_idx: np.ndarray) -> np.ndarray:
    q = _c(q_idx, np.uint16)
    k = _c(k_idx, np.uint16)
    n = k.shape[0]
    s = np.empty(n, np.float32)
    lib().orc_scores(_p(q), _p(k), n, _p(s))
    return s


def block_scores(s: np.ndarray, block: int) -> np.ndarray:
    s = _c(s, np.float32)
    out = np.empty((s.size + block - 1) // block, np.float32)
    lib().orc_block_scores(_p(s), s.size, block, _p(out))
    return out


def topk(s: np.ndarray, k: int, ids: np.ndarray | None = None) -> np.ndarray:
    s = _c(s, np.float32)
    idp = None if ids is None else _c(ids, np.int32)
    out = np.empty(k, np.int32)
    lib().orc_topk(_p(s), _p(idp), s.size, k, _p(out))
    return out


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    q = _c(q, np.uint16)
    K = _c(K, np.float64)
    V = _c(V, np.float64)
    out = np.empty((16, 128), np.float64)
    lib().orc_attention(_p(q), _p(K), _p(V), K.shape[0], scale, _p(out))
    return out


class Cache:
    """The global cache of every sequence as the oracle reads it.

    For FP4 the oracle quantises the bf16 rows with its own packer: one E8M0
    scale per 32 (``scale="e8m0"``) or one E4M3 scale per 16 (``"e4m3"``).
    """

    def __init__(self, kv_bf16: np.ndarray, k_idx: np.ndarray, fp4: bool, scale: str = "e8m0",
                 m: int = 1):
        self.t_cap = kv_bf16.shape[1]
        self.m = int(m)  # positions per entry: rows are entries of m positions
        self.fp4 = bool(fp4)
        self.fmt = 0
        self.k_idx = _c(k_idx, np.uint16)
        if self.fp4:
            self.kv = None
            if scale == "e4m3":
                self.fmt = 2
                self.codes, self.scales = fp4e_pack(kv_bf16)
            else:
                assert scale == "e8m0", scale
                self.fmt = 1
                self.codes, self.scales = fp4_pack(kv_bf16)
        else:
            self.kv = _c(kv_bf16, np.uint16)
            self.codes = self.scales = None

    def args(self):
        return (self.fmt, self.t_cap, self.m, _p(self.kv), _p(self.codes), _p(self.scales))


def layer(cache: Cache, q_pos, q_seq, mode, q, q_idx, lk, lv, window, lo, k,
          pool=0, block=1, pool_io=None, sel_io=None, scale=128 ** -0.5):
    """One layer for nq queries; returns (out [nq][16][128] f64, sel, pool)."""
    q_pos = _c(q_pos, np.int32)
    q_seq = _c(q_seq, np.int32)
    nq = q_pos.size
    q = _c(q, np.uint16)
    q_idx = _c(q_idx, np.uint16)
    lk = _c(lk, np.uint16)
    lv = _c(lv, np.uint16)
    cap = lk.shape[-2]
    pool_io = (np.full((nq, max(pool, 0)), -1, np.int32) if pool_io is None
               else _c(pool_io, np.int32).copy())
    sel_io = np.full((nq, k), -1, np.int32) if sel_io is None else _c(sel_io, np.int32).copy()
    out = np.empty((nq, 16, 128), np.float64)
    rc = lib().orc_layer(nq, _p(q_pos), _p(q_seq), mode, *cache.args(), _p(cache.k_idx),
                         _p(q), _p(q_idx), _p(lk), _p(lv), cap, window, lo, k, pool, block,
                         _p(pool_io), _p(sel_io), scale, _p(out))
    if rc:
        raise ValueError("orc_layer rc=%d" % rc)
    return out, sel_io, pool_io


def attend(cache: Cache, q_pos, q_seq, q, sel, lk, lv, window, lo, scale=128 ** -0.5):
    q_pos = _c(q_pos, np.int32)
    q_seq = _c(q_seq, np.int32)
    nq = q_pos.size
    q = _c(q, np.uint16)
    sel = _c(sel, np.int32)
    lk = _c(lk, np.uint16)
    lv = _c(lv, np.uint16)
    out = np.empty((nq, 16, 128), np.float64)
    rc = lib().orc_attend(nq, _p(q_pos), _p(q_seq), *cache.args(), _p(q), _p(sel), sel.shape[-1],
                          _p(lk), _p(lv), lk.shape[-2], window, lo, scale, _p(out))
    if rc:
        raise ValueError("orc_attend rc=%d" % rc)
    return out


def stack(cache: Cache, modes, q_pos, q, q_idx, lk, lv, window, lo, k, pool, block=1,
          scale=128 ** -0.5):
    """Decoder stack, one query per sequence; returns (out, sel [L][S][k], pool)."""
    modes = _c(modes, np.int32)
    q_pos = _c(q_pos, np.int32)
    L = modes.size
    S = q_pos.size
    q = _c(q, np.uint16)
    q_idx = _c(q_idx, np.uint16)
    lk = _c(lk, np.uint16)
    lv = _c(lv, np.uint16)
    sel = np.full((L, S, k), -1, np.int32)
    pool_out = np.full((S, max(pool, 0)), -1, np.int32)
    out = np.empty((L, S, 16, 128), np.float64)
    rc = lib().orc_stack(L, _p(modes), S, _p(q_pos), *cache.args(), _p(cache.k_idx),
                         _p(q), _p(q_idx), _p(lk), _p(lv), lk.shape[-2], window, lo, k, pool,
                         block, scale, _p(sel), _p(pool_out), _p(out))
    if rc:
        raise ValueError("orc_stack rc=%d" % rc)
    return out, sel, pool_out


def append(kv, k_idx, lk, lv, pos, kv_new, kidx_new=None, k_new=None, v_new=None):
    """Decode append on copies of the bf16 arrays: kv [S][T][256], k_idx
    [S][T][64], lk / lv [L][S][cap][128] (may be None), rows kv_new [S][256],
    kidx_new [S][64] (may be None), k_new / v_new [L][S][128].  Returns the
    updated (kv, k_idx, lk, lv)."""
    kv = _c(kv, np.uint16).copy()
    k_idx = _c(k_idx, np.uint16).copy()
    pos = _c(pos, np.int32)
    S, T = kv.shape[0], kv.shape[1]
    assert pos.size == S
    if lk is not None:
        lk = _c(lk, np.uint16).copy()
        lv = _c(lv, np.uint16).copy()
        L, cap = lk.shape[0], lk.shape[2]
        k_new = _c(k_new, np.uint16)
        v_new = _c(v_new, np.uint16)
        assert k_new.shape == (L, S, 128) and v_new.shape == (L, S, 128)
    else:
        L, cap = 0, 1
    kv_new = _c(kv_new, np.uint16)
    kidx_new = None if kidx_new is None else _c(kidx_new, np.uint16)
    lib().orc_append(S, T, _p(pos), _p(kv_new), _p(kidx_new), _p(kv), _p(k_idx), L, cap,
                     _p(k_new) if L else None, _p(v_new) if L else None,
                     _p(lk) if L else None, _p(lv) if L else None)
    return kv, k_idx, lk, lv


def replay(cache: Cache, modes, seq, pos, q, q_idx, lk, lv, window, lo, k, pool, k_new, v_new,
           block=1, scale=128 ** -0.5):
    """Bounded replay of positions pos (one sequence) through a decoder stack.
    q [L][n][16][128], q_idx [L][n][64], lk / lv [L][n_seq][cap][128] (copied,
    then updated as the replay writes the segment's rows k_new / v_new
    [L][n][128]).  Returns (out [L][n][16][128], sel [L][n][k], pool [n][pool],
    lk, lv)."""
    modes = _c(modes, np.int32)
    pos = _c(pos, np.int32)
    L, n = modes.size, pos.size
    q = _c(q, np.uint16)
    q_idx = _c(q_idx, np.uint16)
    lk = _c(lk, np.uint16).copy()
    lv = _c(lv, np.uint16).copy()
    k_new = _c(k_new, np.uint16)
    v_new = _c(v_new, np.uint16)
    assert k_new.shape == (L, n, 128) and v_new.shape == (L, n, 128)
    sel = np.full((L, n, k), -1, np.int32)
    pool_out = np.full((n, max(pool, 0)), -1, np.int32)
    out = np.empty((L, n, 16, 128), np.float64)
    rc = lib().orc_replay(L, _p(modes), lk.shape[1], seq, n, _p(pos), *cache.args(),
                          _p(cache.k_idx), _p(q), _p(q_idx), _p(lk), _p(lv), lk.shape[-2],
                          window, lo, k, pool, block, _p(k_new), _p(v_new), scale, _p(sel),
                          _p(pool_out), _p(out))
    if rc:
        raise ValueError("orc_replay rc=%d" % rc)
    return out, sel, pool_out, lk, lv


def compress(x_bf16: np.ndarray, m: int) -> np.ndarray:
    """Sequence compression: bf16 [..., groups * m, dim] -> [..., groups, dim],
    each entry the mean of its m positions rounded to bf16 (rows beyond the
    last complete group are dropped)."""
    x = _c(x_bf16, np.uint16)
    dim = x.shape[-1]
    n = x.shape[-2]
    groups = n // m
    lead = x.shape[:-2]
    x = np.ascontiguousarray(x[..., :groups * m, :])
    out = np.empty(lead + (groups, dim), np.uint16)
    total = int(np.prod(lead, dtype=np.int64)) * groups
    rc = lib().orc_compress(_p(x), total, m, dim, _p(out))
    if rc:
        raise ValueError("orc_compress rc=%d" % rc)
    return out
