"""ctypes marshalling of the libcsa2 C ABI (include/csa2.h).

Tensors are torch tensors on the current HIP device; bf16 data may be passed as
``torch.bfloat16`` or as 16-bit integer bit patterns.  Every call enqueues on
``torch.cuda.current_stream()`` and returns without synchronising.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libcsa2.so")

FULL, REINDEX, REUSE = 0, 1, 2
KV_BF16, KV_FP4, KV_FP4_E4M3 = 0, 1, 2
HEADS, HEAD_DIM, INDEX_DIM = 16, 128, 64

_P = ctypes.c_void_p
_i32, _i64, _f32, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class csa2_cache(ctypes.Structure):
    _fields_ = [("format", _i32), ("n_seq", _i32), ("t_cap", _i64), ("data", _P),
                ("scales", _P), ("k_idx", _P), ("m", _i32)]


class csa2_local(ctypes.Structure):
    _fields_ = [("k", _P), ("v", _P), ("cap", _i32), ("window", _i32), ("lo", _i32)]


class csa2_stack_desc(ctypes.Structure):
    _fields_ = [("n_layers", _i32), ("modes", ctypes.POINTER(_i32)),
                ("cache", ctypes.POINTER(csa2_cache)), ("q_pos", _P), ("k", _i32),
                ("pool", _i32), ("block", _i32), ("sm_scale", _f32),
                ("q", ctypes.POINTER(_P)), ("q_idx", ctypes.POINTER(_P)),
                ("local", ctypes.POINTER(csa2_local)), ("out", ctypes.POINTER(_P)),
                ("sel_out", ctypes.POINTER(_P)), ("pool_out", _P), ("scan_events", _P * 2),
                ("append_kv", _P), ("append_kidx", _P), ("append_k", ctypes.POINTER(_P)),
                ("append_v", ctypes.POINTER(_P)), ("attn_events", ctypes.POINTER(_P))]


class csa2_replay_desc(ctypes.Structure):
    _fields_ = [("n_layers", _i32), ("modes", ctypes.POINTER(_i32)),
                ("cache", ctypes.POINTER(csa2_cache)), ("seq", _i32), ("n", _i32),
                ("q_pos", _P), ("k", _i32), ("pool", _i32), ("block", _i32), ("sm_scale", _f32),
                ("q", ctypes.POINTER(_P)), ("q_idx", ctypes.POINTER(_P)),
                ("local", ctypes.POINTER(csa2_local)), ("local_k", ctypes.POINTER(_P)),
                ("local_v", ctypes.POINTER(_P)), ("out", ctypes.POINTER(_P)),
                ("sel_out", ctypes.POINTER(_P)), ("pool_out", _P)]


class Csa2Error(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """Load libcsa2.so (built by ``sparse_attention_shared_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise ImportError("libcsa2.so is not built (%s); run __graft_entry__.build()" % lib_path)
        L = ctypes.CDLL(lib_path)
        L.csa2_version.restype = ctypes.c_int
        L.csa2_status_str.restype = ctypes.c_char_p
        L.csa2_status_str.argtypes = [ctypes.c_int]
        L.csa2_device_check.restype = ctypes.c_int
        L.csa2_pack_fp4.argtypes = [_P, _i64, _i32, _P, _P, _P]
        L.csa2_unpack_fp4.argtypes = [_P, _P, _i64, _i32, _P, _P]
        L.csa2_pack_fp4_e4m3.argtypes = [_P, _i64, _i32, _P, _P, _P]
        L.csa2_compress.argtypes = [_P, _i64, _i32, _i32, _P, _P]
        L.csa2_unpack_fp4_e4m3.argtypes = [_P, _P, _i64, _i32, _P, _P]
        L.csa2_append.argtypes = [ctypes.POINTER(csa2_cache), _P, _P, _P, _i32,
                                  ctypes.POINTER(csa2_local), ctypes.POINTER(_P),
                                  ctypes.POINTER(_P), _P]
        L.csa2_index_score.argtypes = [ctypes.POINTER(csa2_cache), _P, _P, _P, _i32, _P, _i64,
                                       _i32, _P, _i64, _P]
        L.csa2_prefill_score.argtypes = [ctypes.POINTER(csa2_cache), _i32, _P, _P, _i32, _P, _i64,
                                         _P]
        L.csa2_prefill_topk.argtypes = [ctypes.POINTER(csa2_cache), _i32, _P, _P, _i32, _i32, _P,
                                        _P, _sz, _P]
        L.csa2_prefill_topk_workspace.argtypes = [_i32, _i64, _i32, ctypes.POINTER(_sz)]
        L.csa2_topk.argtypes = [_P, _i32, _i64, _i64, _P, _i32, _P, _i32, _P, _P, _sz, _P]
        L.csa2_topk_workspace.argtypes = [_i32, _i64, _i32, _i32, ctypes.POINTER(_sz)]
        L.csa2_expand_blocks.argtypes = [_P, _i32, _i32, _i32, _P, _P, _P]
        L.csa2_sparse_attn.argtypes = [ctypes.POINTER(csa2_cache), _P, _P, _P, _i32, _P, _i32,
                                       ctypes.POINTER(csa2_local), _f32, _P, _P, _sz, _P]
        L.csa2_sparse_attn_workspace.argtypes = [_i32, _i32, _i32, ctypes.POINTER(_sz)]
        L.csa2_sparse_attn_noalloc.argtypes = [ctypes.POINTER(csa2_cache), _P, _P, _P, _i32, _P,
                                               _i32, ctypes.POINTER(csa2_local), _f32, _P, _P]
        L.csa2_stack_workspace.argtypes = [ctypes.POINTER(csa2_stack_desc), ctypes.POINTER(_sz)]
        L.csa2_stack_run.argtypes = [ctypes.POINTER(csa2_stack_desc), _P, _sz, _P]
        L.csa2_stack_plan_create.argtypes = [ctypes.POINTER(csa2_stack_desc), _P, _sz,
                                             ctypes.POINTER(_P)]
        L.csa2_stack_plan_launch.argtypes = [_P, _P]
        L.csa2_stack_plan_destroy.argtypes = [_P]
        L.csa2_replay_workspace.argtypes = [ctypes.POINTER(csa2_replay_desc), ctypes.POINTER(_sz)]
        L.csa2_replay_run.argtypes = [ctypes.POINTER(csa2_replay_desc), _P, _sz, _P]
        for f in ("csa2_pack_fp4", "csa2_unpack_fp4", "csa2_pack_fp4_e4m3", "csa2_unpack_fp4_e4m3",
                  "csa2_append", "csa2_compress", "csa2_index_score", "csa2_prefill_score",
                  "csa2_prefill_topk", "csa2_prefill_topk_workspace", "csa2_topk",
                  "csa2_topk_workspace", "csa2_expand_blocks", "csa2_sparse_attn",
                  "csa2_sparse_attn_noalloc",
                  "csa2_sparse_attn_workspace", "csa2_stack_workspace", "csa2_stack_run",
                  "csa2_stack_plan_create", "csa2_stack_plan_launch", "csa2_stack_plan_destroy",
                  "csa2_replay_workspace", "csa2_replay_run"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(name: str, st: int) -> None:
    if st != 0:
        raise Csa2Error("%s: %s (status %d)" % (name, lib().csa2_status_str(st).decode(), st))


def version() -> int:
    return lib().csa2_version()


def device_check() -> None:
    _check("csa2_device_check", lib().csa2_device_check())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _bits16(t: torch.Tensor) -> torch.Tensor:
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return t
    raise TypeError("expected bf16 data (bfloat16 or 16-bit bit patterns), got %s" % t.dtype)


def _i32t(t: Optional[torch.Tensor]):
    if t is not None and t.dtype != torch.int32:
        raise TypeError("expected int32, got %s" % t.dtype)
    return t


class Cache:
    """The global cache shared by all decoder layers.

    BF16: ``data`` bf16 [n_seq][t_cap][256] (K | V).  FP4: ``data`` uint8 codes
    [n_seq][t_cap][128] and ``scales`` uint8 [n_seq][t_cap][8] as written by
    :func:`pack_fp4` on rows of 256 (one E8M0 scale per 32), or
    [n_seq][t_cap][16] as written by :func:`pack_fp4_e4m3` (one E4M3 scale per
    16).  ``k_idx`` bf16 [n_seq][t_cap][64].
    """

    def __init__(self, data: torch.Tensor, k_idx: torch.Tensor,
                 scales: Optional[torch.Tensor] = None, m: int = 1):
        self.fp4 = scales is not None
        self.data, self.scales, self.k_idx = data, scales, _bits16(k_idx)
        self.n_seq, self.t_cap = int(k_idx.shape[0]), int(k_idx.shape[1])
        fmt = KV_BF16
        if self.fp4:
            assert data.dtype == torch.uint8 and tuple(data.shape) == (self.n_seq, self.t_cap, 128)
            assert scales.dtype == torch.uint8 and scales.dim() == 3
            assert tuple(scales.shape[:2]) == (self.n_seq, self.t_cap) and scales.shape[2] in (8, 16)
            fmt = KV_FP4 if scales.shape[2] == 8 else KV_FP4_E4M3
        else:
            _bits16(data)
            assert tuple(data.shape) == (self.n_seq, self.t_cap, 256)
        self.format = fmt
        self.m = int(m)  # positions per entry (rows are entries)
        self.c = csa2_cache(fmt, self.n_seq, self.t_cap,
                            _ptr(data), _ptr(scales) if self.fp4 else None, _ptr(self.k_idx),
                            self.m)


class Local:
    """A layer's local KV ring: k, v bf16 [n_seq][cap][128]; position p in slot p % cap."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, window: int, lo: int = 0):
        self.k, self.v = _bits16(k), _bits16(v)
        self.cap = int(k.shape[1])
        self.c = csa2_local(_ptr(self.k), _ptr(self.v), self.cap, int(window), int(lo))


def pack_fp4(x: torch.Tensor):
    """bf16 [..., dim] -> (codes uint8 [..., dim/2], scales uint8 [..., dim/32])."""
    x = _bits16(x)
    dim = int(x.shape[-1])
    rows = x.numel() // dim if dim else 0
    codes = torch.empty(tuple(x.shape[:-1]) + (dim // 2,), dtype=torch.uint8, device=x.device)
    scales = torch.empty(tuple(x.shape[:-1]) + (dim // 32,), dtype=torch.uint8, device=x.device)
    _check("csa2_pack_fp4", lib().csa2_pack_fp4(_ptr(x), rows, dim, _ptr(codes), _ptr(scales),
                                                _stream()))
    return codes, scales


def compress(x: torch.Tensor, m: int) -> torch.Tensor:
    """Sequence compression (csa2_compress): bf16 [..., groups * m, dim] ->
    [..., groups, dim], each entry the mean of its m positions (bf16)."""
    x = _bits16(x)
    if not x.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    dim, n = int(x.shape[-1]), int(x.shape[-2])
    if n % m:
        raise ValueError("positions must fill whole groups")
    lead = tuple(x.shape[:-2])
    groups = (x.numel() // (n * dim)) * (n // m) if dim and n else 0
    out = torch.empty(lead + (n // m, dim), dtype=x.dtype, device=x.device)
    _check("csa2_compress", lib().csa2_compress(_ptr(x), groups, m, dim, _ptr(out), _stream()))
    return out


def pack_fp4_e4m3(x: torch.Tensor):
    """bf16 [..., dim] -> (codes uint8 [..., dim/2], E4M3 scales uint8 [..., dim/16])."""
    x = _bits16(x)
    dim = int(x.shape[-1])
    rows = x.numel() // dim if dim else 0
    codes = torch.empty(tuple(x.shape[:-1]) + (dim // 2,), dtype=torch.uint8, device=x.device)
    scales = torch.empty(tuple(x.shape[:-1]) + (dim // 16,), dtype=torch.uint8, device=x.device)
    _check("csa2_pack_fp4_e4m3", lib().csa2_pack_fp4_e4m3(_ptr(x), rows, dim, _ptr(codes),
                                                          _ptr(scales), _stream()))
    return codes, scales


def unpack_fp4_e4m3(codes: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    dim = int(codes.shape[-1]) * 2
    rows = codes.numel() // (dim // 2) if dim else 0
    out = torch.empty(tuple(codes.shape[:-1]) + (dim,), dtype=torch.float32, device=codes.device)
    _check("csa2_unpack_fp4_e4m3", lib().csa2_unpack_fp4_e4m3(_ptr(codes), _ptr(scales), rows, dim,
                                                              _ptr(out), _stream()))
    return out


def unpack_fp4(codes: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    dim = int(codes.shape[-1]) * 2
    rows = codes.numel() // (dim // 2) if dim else 0
    out = torch.empty(tuple(codes.shape[:-1]) + (dim,), dtype=torch.float32, device=codes.device)
    _check("csa2_unpack_fp4", lib().csa2_unpack_fp4(_ptr(codes), _ptr(scales), rows, dim,
                                                    _ptr(out), _stream()))
    return out


def append(cache: Cache, pos: torch.Tensor, kv: Optional[torch.Tensor] = None,
           kidx: Optional[torch.Tensor] = None, local: Sequence[Local] = (),
           k_new: Sequence[torch.Tensor] = (), v_new: Sequence[torch.Tensor] = ()) -> None:
    """Decode append (csa2_append): row pos[b] of the global cache takes kv[b]
    (bf16 [n_seq][256], FP4-packed for an FP4 cache) and k_idx takes kidx[b]
    (bf16 [n_seq][64]); ring slot pos[b] % cap of local[l] takes k_new[l][b] and
    v_new[l][b] (bf16 [n_seq][128]).  Sequences with pos outside [0, t_cap) are
    skipped."""
    n = len(local)
    if len(k_new) != n or len(v_new) != n:
        raise ValueError("local, k_new and v_new must have the same length")
    locs = (csa2_local * n)(*[l.c for l in local]) if n else None
    kn = (_P * n)(*[_bits16(t).data_ptr() for t in k_new]) if n else None
    vn = (_P * n)(*[_bits16(t).data_ptr() for t in v_new]) if n else None
    _check("csa2_append", lib().csa2_append(
        ctypes.byref(cache.c), _ptr(_i32t(pos)), _ptr(_bits16(kv)) if kv is not None else None,
        _ptr(_bits16(kidx)) if kidx is not None else None, n, locs, kn, vn, _stream()))


def index_score(cache: Cache, q_idx: torch.Tensor, q_pos: torch.Tensor,
                q_seq: Optional[torch.Tensor] = None, cand: Optional[torch.Tensor] = None,
                block: int = 1, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    nq = int(q_pos.shape[0])
    if cand is not None:
        n = int(cand.shape[1])
    else:
        n = (cache.t_cap + block - 1) // block
    if out is None:
        out = torch.empty((nq, n), dtype=torch.float32, device=q_pos.device)
    _check("csa2_index_score", lib().csa2_index_score(
        ctypes.byref(cache.c), _ptr(_bits16(q_idx)), _ptr(_i32t(q_pos)), _ptr(_i32t(q_seq)), nq,
        _ptr(_i32t(cand)), n if cand is not None else 0, block, _ptr(out), int(out.stride(0)),
        _stream()))
    return out


def prefill_score(cache: Cache, seq: int, q_idx: torch.Tensor, q_pos: torch.Tensor,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dense scores of a chunk of queries on one sequence (MFMA): [nq][t_cap]."""
    nq = int(q_pos.shape[0])
    if out is None:
        out = torch.empty((nq, cache.t_cap), dtype=torch.float32, device=q_pos.device)
    _check("csa2_prefill_score", lib().csa2_prefill_score(
        ctypes.byref(cache.c), int(seq), _ptr(_bits16(q_idx)), _ptr(_i32t(q_pos)), nq, _ptr(out),
        int(out.stride(0)), _stream()))
    return out


def prefill_topk_workspace(nq: int, t_cap: int, k: int) -> int:
    n = _sz()
    _check("csa2_prefill_topk_workspace",
           lib().csa2_prefill_topk_workspace(int(nq), int(t_cap), int(k), ctypes.byref(n)))
    return n.value


def prefill_topk(cache: Cache, seq: int, q_idx: torch.Tensor, q_pos: torch.Tensor, k: int,
                 out: Optional[torch.Tensor] = None,
                 ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-k positions of every query of a prefill chunk on one sequence: [nq][k]."""
    nq = int(q_pos.shape[0])
    if out is None:
        out = torch.empty((nq, k), dtype=torch.int32, device=q_pos.device)
    need = prefill_topk_workspace(nq, cache.t_cap, k)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q_pos.device)
    _check("csa2_prefill_topk", lib().csa2_prefill_topk(
        ctypes.byref(cache.c), int(seq), _ptr(_bits16(q_idx)), _ptr(_i32t(q_pos)), nq, int(k),
        _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return out


def topk_workspace(nq: int, n: int, k: int, k2: int = 0) -> int:
    ws_n = _sz()
    _check("csa2_topk_workspace", lib().csa2_topk_workspace(nq, n, k, k2, ctypes.byref(ws_n)))
    return ws_n.value


def topk(scores: torch.Tensor, k: int, ids: Optional[torch.Tensor] = None, k2: int = 0,
         ws: Optional[torch.Tensor] = None):
    """Returns (out [nq][k], out2 [nq][k2] or None); positions ascending, -1 padded.
    ``ws``: an optional workspace (zero-filled before its first use; see
    csa2_topk for when it may be reused)."""
    nq, n = int(scores.shape[0]), int(scores.shape[1])
    out = torch.empty((nq, k), dtype=torch.int32, device=scores.device)
    out2 = torch.empty((nq, k2), dtype=torch.int32, device=scores.device) if k2 else None
    need = topk_workspace(nq, n, k, k2)
    if ws is None:
        ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=scores.device)
    _check("csa2_topk", lib().csa2_topk(_ptr(scores), nq, n, int(scores.stride(0)),
                                        _ptr(_i32t(ids)), k, _ptr(out), k2, _ptr(out2), _ptr(ws),
                                        ws.numel(), _stream()))
    return out, out2


def expand_blocks(blocks: torch.Tensor, block: int, q_pos: torch.Tensor) -> torch.Tensor:
    nq, nb = int(blocks.shape[0]), int(blocks.shape[1])
    out = torch.empty((nq, nb * block), dtype=torch.int32, device=blocks.device)
    _check("csa2_expand_blocks", lib().csa2_expand_blocks(_ptr(_i32t(blocks)), nq, nb, block,
                                                          _ptr(_i32t(q_pos)), _ptr(out), _stream()))
    return out


def sparse_attn_workspace(nq: int, k: int, window: int) -> int:
    n = _sz()
    _check("csa2_sparse_attn_workspace", lib().csa2_sparse_attn_workspace(nq, k, window,
                                                                          ctypes.byref(n)))
    return n.value


def sparse_attn(cache: Cache, q: torch.Tensor, q_pos: torch.Tensor, q_seq: Optional[torch.Tensor],
                sel: torch.Tensor, local: Local, sm_scale: float = HEAD_DIM ** -0.5,
                out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    nq = int(q_pos.shape[0])
    k = int(sel.shape[1]) if sel is not None else 0
    if out is None:
        out = torch.empty((nq, HEADS, HEAD_DIM), dtype=torch.bfloat16, device=q.device)
    need = sparse_attn_workspace(nq, k, local.c.window)
    if ws is None and need > 0:
        ws = torch.zeros(need, dtype=torch.uint8, device=q.device)
    _check("csa2_sparse_attn", lib().csa2_sparse_attn(
        ctypes.byref(cache.c), _ptr(_bits16(q)), _ptr(_i32t(q_pos)), _ptr(_i32t(q_seq)), nq,
        _ptr(_i32t(sel)), k, ctypes.byref(local.c), float(sm_scale), _ptr(out), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream()))
    return out


def sparse_attn_noalloc(cache: Cache, q: torch.Tensor, q_pos: torch.Tensor,
                        q_seq: Optional[torch.Tensor], sel: torch.Tensor, local: Local,
                        sm_scale: float = HEAD_DIM ** -0.5,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """csa2_sparse_attn_noalloc: the same attention without a workspace (the
    library's fixed per-GPU scratch; calls on one GPU must not overlap)."""
    nq = int(q_pos.shape[0])
    k = int(sel.shape[1]) if sel is not None else 0
    if out is None:
        out = torch.empty((nq, HEADS, HEAD_DIM), dtype=torch.bfloat16, device=q.device)
    _check("csa2_sparse_attn_noalloc", lib().csa2_sparse_attn_noalloc(
        ctypes.byref(cache.c), _ptr(_bits16(q)), _ptr(_i32t(q_pos)), _ptr(_i32t(q_seq)), nq,
        _ptr(_i32t(sel)), k, ctypes.byref(local.c), float(sm_scale), _ptr(out), _stream()))
    return out


class _StackArgs:
    """Keeps the ctypes arrays of one stack descriptor alive."""

    def __init__(self, cache: Cache, modes: Sequence[int], q_pos: torch.Tensor,
                 q: Sequence[torch.Tensor], q_idx: Sequence[Optional[torch.Tensor]],
                 local: Sequence[Local], out: Sequence[torch.Tensor], k: int, pool: int,
                 block: int, sm_scale: float, sel_out: Optional[Sequence[torch.Tensor]],
                 pool_out: Optional[torch.Tensor], scan_events=None, append=None,
                 attn_events=None):
        L = len(modes)
        self.refs = (cache, q_pos, list(q), list(q_idx), list(local), list(out), sel_out, pool_out,
                     append)
        self.modes = (_i32 * L)(*modes)
        self.q = (_P * L)(*[t.data_ptr() for t in q])
        self.q_idx = (_P * L)(*[(t.data_ptr() if t is not None else None) for t in q_idx])
        self.local = (csa2_local * L)(*[l.c for l in local])
        self.out = (_P * L)(*[t.data_ptr() for t in out])
        self.sel = (_P * L)(*[t.data_ptr() for t in sel_out]) if sel_out is not None else None
        self.desc = csa2_stack_desc(
            L, self.modes, ctypes.pointer(cache.c), _ptr(_i32t(q_pos)), k, pool, block,
            float(sm_scale), self.q, self.q_idx, self.local, self.out,
            self.sel if self.sel is not None else None,
            _ptr(pool_out) if pool_out is not None else None,
            (_P * 2)(*(scan_events or (None, None))))
        if append is not None:
            kv, kidx, kn, vn = append
            self.desc.append_kv = _ptr(_bits16(kv)).value
            self.desc.append_kidx = _ptr(_bits16(kidx)).value if kidx is not None else None
            if kn is not None:
                if len(kn) != L or len(vn) != L:
                    raise ValueError("append rows: one (k, v) pair per layer")
                self.app_k = (_P * L)(*[(_bits16(t).data_ptr() if t is not None else None)
                                        for t in kn])
                self.app_v = (_P * L)(*[(_bits16(t).data_ptr() if t is not None else None)
                                        for t in vn])
                self.desc.append_k = self.app_k
                self.desc.append_v = self.app_v
        if attn_events is not None:
            if len(attn_events) != 2 * L:
                raise ValueError("attn_events: two events per layer")
            self.attn_ev = (_P * (2 * L))(*[(e.value if isinstance(e, ctypes.c_void_p) else e)
                                            if e is not None else None for e in attn_events])
            self.desc.attn_events = self.attn_ev


def stack_workspace(args: _StackArgs) -> int:
    n = _sz()
    _check("csa2_stack_workspace", lib().csa2_stack_workspace(ctypes.byref(args.desc),
                                                              ctypes.byref(n)))
    return n.value


def stack_run(cache: Cache, modes: Sequence[int], q_pos: torch.Tensor,
              q: Sequence[torch.Tensor], q_idx: Sequence[Optional[torch.Tensor]],
              local: Sequence[Local], k: int, pool: int = 0, block: int = 1,
              sm_scale: float = HEAD_DIM ** -0.5, want_sel: bool = True,
              ws: Optional[torch.Tensor] = None, out: Optional[Sequence[torch.Tensor]] = None,
              scan_events=None, append=None, attn_events=None, want_pool: bool = True):
    """Run a decoder stack (one decode query per sequence).

    Returns (out list of bf16 [n_seq][16][128], sel list or None, pool or None;
    the pool only with ``want_pool`` and pool > 0).
    ``scan_events``: optional pair of ``torch.cuda.Event(enable_timing=True)``
    recorded around layer 0's indexer scan; ``attn_events``: optional list of
    2 * n_layers such events (or None to skip a layer), receiving the start
    and end of each layer's attention kernel.  ``append``: optional
    ``(kv, kidx, k_new, v_new)`` written at q_pos before layer 0 (the decode
    append of csa2_append; kidx may be None, k_new / v_new None or one bf16
    [n_seq][128] tensor (or None) per layer).
    """
    S = int(q_pos.shape[0])
    dev = q_pos.device
    if out is None:
        out = [torch.empty((S, HEADS, HEAD_DIM), dtype=torch.bfloat16, device=dev) for _ in modes]
    sel = [torch.empty((S, k), dtype=torch.int32, device=dev) for _ in modes] if want_sel else None
    pool_out = torch.empty((S, pool), dtype=torch.int32, device=dev) if pool > 0 and want_pool else None
    ev = None
    if scan_events is not None:
        ev = tuple(ctypes.c_void_p(e.cuda_event) for e in scan_events)
    aev = None
    if attn_events is not None:
        aev = [ctypes.c_void_p(e.cuda_event) if e is not None else None for e in attn_events]
    args = _StackArgs(cache, modes, q_pos, q, q_idx, local, out, k, pool, block, sm_scale, sel,
                      pool_out, ev, append, aev)
    need = stack_workspace(args)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    _check("csa2_stack_run", lib().csa2_stack_run(ctypes.byref(args.desc), _ptr(ws), ws.numel(),
                                                  _stream()))
    return out, sel, pool_out


class StackPlan:
    """A decoder stack recorded once into a HIP graph (csa2_stack_plan_*).

    The output, selection, pool and workspace buffers are allocated here and
    fixed for the plan's life; :meth:`launch` replays the whole stack on the
    current stream (inputs may be updated in place between launches).
    """

    def __init__(self, cache: Cache, modes: Sequence[int], q_pos: torch.Tensor,
                 q: Sequence[torch.Tensor], q_idx: Sequence[Optional[torch.Tensor]],
                 local: Sequence[Local], k: int, pool: int = 0, block: int = 1,
                 sm_scale: float = HEAD_DIM ** -0.5, want_sel: bool = False,
                 out: Optional[Sequence[torch.Tensor]] = None, scan_events=None, append=None):
        S = int(q_pos.shape[0])
        dev = q_pos.device
        self.out = out if out is not None else [
            torch.empty((S, HEADS, HEAD_DIM), dtype=torch.bfloat16, device=dev) for _ in modes]
        self.sel = ([torch.empty((S, k), dtype=torch.int32, device=dev) for _ in modes]
                    if want_sel else None)
        self.pool = torch.empty((S, pool), dtype=torch.int32, device=dev) if pool > 0 else None
        ev = None
        if scan_events is not None:
            ev = tuple(ctypes.c_void_p(e.cuda_event) for e in scan_events)
        self.args = _StackArgs(cache, modes, q_pos, q, q_idx, local, self.out, k, pool, block,
                               sm_scale, self.sel, self.pool, ev, append)
        need = stack_workspace(self.args)
        self.ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize(dev)  # the zero fill lands before the plan is recorded
        self._plan = _P()
        _check("csa2_stack_plan_create", lib().csa2_stack_plan_create(
            ctypes.byref(self.args.desc), _ptr(self.ws), self.ws.numel(), ctypes.byref(self._plan)))

    def launch(self):
        _check("csa2_stack_plan_launch", lib().csa2_stack_plan_launch(self._plan, _stream()))
        return self.out, self.sel, self.pool

    def close(self):
        if getattr(self, "_plan", None) is not None and self._plan.value:
            lib().csa2_stack_plan_destroy(self._plan)
            self._plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class _ReplayArgs:
    """Keeps the ctypes arrays of one replay descriptor alive."""

    def __init__(self, cache: Cache, modes: Sequence[int], seq: int, q_pos: torch.Tensor,
                 q: Sequence[torch.Tensor], q_idx: Sequence[Optional[torch.Tensor]],
                 local: Sequence[Local], out: Sequence[torch.Tensor], k: int, pool: int,
                 block: int, sm_scale: float, local_k=None, local_v=None, sel_out=None,
                 pool_out: Optional[torch.Tensor] = None):
        L = len(modes)
        self.refs = (cache, q_pos, list(q), list(q_idx), list(local), list(out), sel_out,
                     pool_out, local_k, local_v)
        self.modes = (_i32 * L)(*modes)
        self.q = (_P * L)(*[_bits16(t).data_ptr() for t in q])
        self.q_idx = (_P * L)(*[(_bits16(t).data_ptr() if t is not None else None)
                                for t in q_idx])
        self.local = (csa2_local * L)(*[l.c for l in local])
        self.out = (_P * L)(*[t.data_ptr() for t in out])
        self.sel = (_P * L)(*[t.data_ptr() for t in sel_out]) if sel_out is not None else None
        rows = local_k is not None
        if rows and (len(local_k) != L or len(local_v) != L):
            raise ValueError("local rows: one (k, v) pair per layer")
        self.lk = (_P * L)(*[(_bits16(t).data_ptr() if t is not None else None)
                             for t in local_k]) if rows else None
        self.lv = (_P * L)(*[(_bits16(t).data_ptr() if t is not None else None)
                             for t in local_v]) if rows else None
        self.desc = csa2_replay_desc(
            L, self.modes, ctypes.pointer(cache.c), int(seq), int(q_pos.shape[0]),
            _ptr(_i32t(q_pos)), k, pool, block, float(sm_scale), self.q, self.q_idx, self.local,
            self.lk, self.lv, self.out, self.sel,
            _ptr(pool_out) if pool_out is not None else None)


def replay_workspace(args: _ReplayArgs) -> int:
    n = _sz()
    _check("csa2_replay_workspace", lib().csa2_replay_workspace(ctypes.byref(args.desc),
                                                                ctypes.byref(n)))
    return n.value


def replay_run(cache: Cache, modes: Sequence[int], seq: int, q_pos: torch.Tensor,
               q: Sequence[torch.Tensor], q_idx: Sequence[Optional[torch.Tensor]],
               local: Sequence[Local], k: int, pool: int = 0, block: int = 1,
               sm_scale: float = HEAD_DIM ** -0.5, local_k=None, local_v=None,
               want_sel: bool = True, ws: Optional[torch.Tensor] = None,
               out: Optional[Sequence[torch.Tensor]] = None):
    """Bounded replay (csa2_replay_run): the queries at q_pos (int32 [n], all
    on sequence ``seq``) through every layer; ``local_k`` / ``local_v``: None,
    or per layer a bf16 [n][128] tensor (or None) of the segment's local rows,
    written into the layer's ring first.  Set each Local's ``lo`` to the
    segment's first position for the window cut-off.  Returns (out list of
    bf16 [n][16][128], sel list or None, pool or None)."""
    n = int(q_pos.shape[0])
    dev = q_pos.device
    if out is None:
        out = [torch.empty((n, HEADS, HEAD_DIM), dtype=torch.bfloat16, device=dev) for _ in modes]
    sel = [torch.empty((n, k), dtype=torch.int32, device=dev) for _ in modes] if want_sel else None
    pool_out = torch.empty((n, pool), dtype=torch.int32, device=dev) if pool > 0 else None
    args = _ReplayArgs(cache, modes, seq, q_pos, q, q_idx, local, out, k, pool, block, sm_scale,
                       local_k, local_v, sel, pool_out)
    need = replay_workspace(args)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    _check("csa2_replay_run", lib().csa2_replay_run(ctypes.byref(args.desc), _ptr(ws), ws.numel(),
                                                    _stream()))
    return out, sel, pool_out
