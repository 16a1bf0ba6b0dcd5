"""MLA tree-verify attention for MI355X (gfx950).

The compute lives in ``libmla_verify.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/mla_verify.h``). This package only marshals torch
tensors into that ABI; ``synth`` draws seeded synthetic inputs.
"""
from .binding import (  # noqa: F401
    MlaError,
    compact_kv,
    head_project,
    load_library,
    plan,
    probe_gather_rows,
    probe_mfma_bf16,
    select_topk,
    topk_workspace_bytes,
    sparse_attn,
    strerror,
    verify_attn,
    verify_attn_noalloc,
    workspace_bytes,
)
