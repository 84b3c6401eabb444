"""Python binding of libcsa2: CSA2 sparse attention over one FP4 global KV cache
shared by every decoder layer, on MI355X (gfx950).

This module only marshals arguments: tensors become device pointers, the
current torch stream becomes the HIP stream, and every step of the path runs in
the library's HIP kernels (declared in ``include/csa2.h``).  There is no
fallback: if ``libcsa2.so`` is missing or the device is not gfx950, calls raise.
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    FULL, REINDEX, REUSE, KV_BF16, KV_FP4, KV_FP4_E4M3, HEADS, HEAD_DIM, INDEX_DIM,
    Cache, Local, Csa2Error, lib, lib_path, version, device_check,
    pack_fp4, unpack_fp4, pack_fp4_e4m3, unpack_fp4_e4m3, compress, append, index_score, prefill_score, prefill_topk, prefill_topk_workspace, topk, topk_workspace, expand_blocks, sparse_attn, sparse_attn_noalloc,
    sparse_attn_workspace, stack_run, stack_workspace, StackPlan, replay_run, replay_workspace,
)
