"""ctypes binding of libmla_verify.so (include/mla_verify.h).

Argument marshalling only: every step of the attention runs in the library's
HIP kernels. Tensors are torch device tensors; the call is enqueued on the
current torch stream (or the one given) and returns without synchronising.
There is no fallback: if the library is missing or fails to load, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_verify.so")

MLA_OK = 0
MLA_ERR_INVALID = -1
MLA_ERR_WORKSPACE = -2
MLA_ERR_HIP = -3
MLA_ERR_UNSUPPORTED = -4
MLA_ERR_SCRATCH = -5
NOALLOC_SCRATCH_BYTES = 64 << 20  # MLA_NOALLOC_SCRATCH_BYTES

PHASE_ALL = 0
PHASE_PARTIAL = 1
PHASE_COMBINE = 2

EXPORTED = (
    "mla_verify_plan",
    "mla_verify_workspace_bytes",
    "mla_verify_attn",
    "mla_verify_attn_noalloc",
    "mla_sparse_attn",
    "mla_verify_strerror",
    "mla_compact_kv",
    "mla_head_project",
    "mla_select_topk",
    "mla_select_topk_workspace_bytes",
    "mla_probe_mfma_bf16",
    "mla_probe_gather_rows",
)


class MlaDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32),
        ("kv_seq_stride", ctypes.c_int64),
        ("kv_rows", ctypes.c_int64),
        ("topk", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("phase", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class MlaPlanInfo(ctypes.Structure):
    _fields_ = [
        ("num_splits", ctypes.c_int32),
        ("chunk_tiles", ctypes.c_int32),
        ("row_blocks", ctypes.c_int32),
        ("num_groups", ctypes.c_int32),
        ("rows_per_group", ctypes.c_int32),
        ("split_slots", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class MlaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} ({code})")


_lib = None
_lock = threading.Lock()


def load_library(path: Optional[str] = None):
    """Load (once) and return the ctypes handle of libmla_verify.so."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                f"{p} is missing: build it with `python -m speculative_decode_verify_mla_amd.build`")
        lib = ctypes.CDLL(p)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        dims_p = ctypes.POINTER(MlaDims)
        lib.mla_verify_plan.argtypes = [dims_p, i32, ctypes.POINTER(MlaPlanInfo)]
        lib.mla_verify_plan.restype = i32
        lib.mla_verify_workspace_bytes.argtypes = [dims_p, i32]
        lib.mla_verify_workspace_bytes.restype = sz
        common = [dims_p, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, sz, vp]
        lib.mla_verify_attn.argtypes = common
        lib.mla_verify_attn.restype = i32
        lib.mla_sparse_attn.argtypes = common
        lib.mla_sparse_attn.restype = i32
        lib.mla_verify_attn_noalloc.argtypes = [dims_p, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp]
        lib.mla_verify_attn_noalloc.restype = i32
        lib.mla_compact_kv.argtypes = [dims_p, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.mla_compact_kv.restype = i32
        lib.mla_head_project.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp]
        lib.mla_head_project.restype = i32
        lib.mla_select_topk.argtypes = [i32, i32, ctypes.c_int64, i32, vp, vp, vp, vp, sz, vp]
        lib.mla_select_topk.restype = i32
        lib.mla_select_topk_workspace_bytes.argtypes = [i32, i32]
        lib.mla_select_topk_workspace_bytes.restype = sz
        lib.mla_probe_mfma_bf16.argtypes = [i32, i32, vp, vp]
        lib.mla_probe_mfma_bf16.restype = i32
        lib.mla_probe_gather_rows.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int64, vp, i32, i32,
                                              i32, vp, vp]
        lib.mla_probe_gather_rows.restype = i32
        lib.mla_verify_strerror.argtypes = [i32]
        lib.mla_verify_strerror.restype = ctypes.c_char_p
        _lib = lib
        return lib


def strerror(code: int) -> str:
    try:
        return load_library().mla_verify_strerror(int(code)).decode()
    except Exception:  # library missing: still describe the code
        return {0: "success", -1: "invalid argument", -2: "workspace missing or too small",
                -3: "HIP runtime or launch failure", -4: "device is not gfx950",
                -5: "call needs more than the fixed device scratch of the allocation-free "
                    "entry point"}.get(code, "unknown")


def make_dims(*, batch, num_q, num_heads, max_kv_len, kv_rows, kv_seq_stride=0, page_size=0,
              max_pages=0, topk=0, num_splits=0, phase=PHASE_ALL) -> MlaDims:
    return MlaDims(batch=batch, num_q=num_q, num_heads=num_heads, page_size=page_size,
                   max_pages=max_pages, max_kv_len=max_kv_len, kv_seq_stride=kv_seq_stride,
                   kv_rows=kv_rows, topk=topk, num_splits=num_splits, phase=phase, reserved=0)


def plan(dims: MlaDims, sparse: bool = False) -> MlaPlanInfo:
    info = MlaPlanInfo()
    rc = load_library().mla_verify_plan(ctypes.byref(dims), int(bool(sparse)), ctypes.byref(info))
    if rc != MLA_OK:
        raise MlaError(rc, "mla_verify_plan")
    return info


def workspace_bytes(dims: MlaDims, sparse: bool = False) -> int:
    return int(load_library().mla_verify_workspace_bytes(ctypes.byref(dims), int(bool(sparse))))


# --------------------------------------------------------------------------
# torch-tensor front end
# --------------------------------------------------------------------------
_ws_cache = {}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _workspace(device, nbytes: int, tag: str = "attn"):
    """A cached device buffer of at least nbytes per (device, tag). Calls that use
    the same cached buffer must be ordered on one stream."""
    import torch

    if nbytes == 0:
        return None
    key = (device.type, device.index, tag)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def _dims_from(q_lat, c_kv, kv_lens, *, max_kv_len, kv_seq_stride, page_table, page_size, topk,
               num_splits, phase) -> MlaDims:
    B, T, H, dl = q_lat.shape
    if dl != 512:
        raise ValueError("q_lat must be [B, T, H, 512]")
    return make_dims(batch=B, num_q=T, num_heads=H, max_kv_len=int(max_kv_len),
                     kv_rows=int(c_kv.shape[0]), kv_seq_stride=int(kv_seq_stride),
                     page_size=int(page_size) if page_table is not None else 0,
                     max_pages=int(page_table.shape[1]) if page_table is not None else 0,
                     topk=int(topk), num_splits=int(num_splits), phase=int(phase))


def _call(fn_name, dims, sparse, q_lat, q_rope, c_kv, k_rope, page_table, mask_or_idx, kv_lens,
          scale, out, lse, workspace, stream):
    import torch

    lib = load_library()
    if workspace is None:
        info = plan(dims, sparse)
        workspace = _workspace(q_lat.device, int(info.workspace_bytes))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(q_lat.device)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    rc = getattr(lib, fn_name)(ctypes.byref(dims), _ptr(q_lat), _ptr(q_rope), _ptr(c_kv),
                               _ptr(k_rope), _ptr(page_table), _ptr(mask_or_idx), _ptr(kv_lens),
                               ctypes.c_float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
                               ctypes.c_size_t(ws_bytes), sptr)
    if rc != MLA_OK:
        raise MlaError(rc, fn_name)


def _as_u16(t):
    import torch

    return t.view(torch.uint16) if t.dtype == torch.bfloat16 else t


def verify_attn(q_lat, q_rope, c_kv, k_rope, page_table, tree_mask, kv_lens, scale, out, lse, *,
                max_kv_len: int, kv_seq_stride: int = 0, page_size: int = 0, num_splits: int = 0,
                phase: int = PHASE_ALL, workspace=None, stream=None):
    """Dense tree-verify attention (mla_verify_attn). bf16 tensors may be torch.bfloat16 or uint16."""
    dims = _dims_from(q_lat, c_kv, kv_lens, max_kv_len=max_kv_len, kv_seq_stride=kv_seq_stride,
                      page_table=page_table, page_size=page_size, topk=0, num_splits=num_splits,
                      phase=phase)
    _call("mla_verify_attn", dims, False, _as_u16(q_lat), _as_u16(q_rope), _as_u16(c_kv),
          _as_u16(k_rope), page_table, tree_mask, kv_lens, scale, _as_u16(out), lse, workspace,
          stream)


def verify_attn_noalloc(q_lat, q_rope, c_kv, k_rope, page_table, tree_mask, kv_lens, scale, out,
                        lse, *, max_kv_len: int, kv_seq_stride: int = 0, page_size: int = 0,
                        num_splits: int = 0, phase: int = PHASE_ALL, stream=None):
    """Dense tree-verify attention without a workspace (mla_verify_attn_noalloc):
    the split partials use the library's fixed device scratch. Calls on one
    GPU must not overlap."""
    import torch

    dims = _dims_from(q_lat, c_kv, kv_lens, max_kv_len=max_kv_len, kv_seq_stride=kv_seq_stride,
                      page_table=page_table, page_size=page_size, topk=0, num_splits=num_splits,
                      phase=phase)
    if stream is None:
        stream = torch.cuda.current_stream(q_lat.device)
    rc = load_library().mla_verify_attn_noalloc(
        ctypes.byref(dims), _ptr(_as_u16(q_lat)), _ptr(_as_u16(q_rope)), _ptr(_as_u16(c_kv)),
        _ptr(_as_u16(k_rope)), _ptr(page_table), _ptr(tree_mask), _ptr(kv_lens),
        ctypes.c_float(scale), _ptr(_as_u16(out)), _ptr(lse), ctypes.c_void_p(stream.cuda_stream))
    if rc != MLA_OK:
        raise MlaError(rc, "mla_verify_attn_noalloc")


def sparse_attn(q_lat, q_rope, c_kv, k_rope, page_table, indices, kv_lens, scale, out, lse, *,
                max_kv_len: int, kv_seq_stride: int = 0, page_size: int = 0, num_splits: int = 0,
                phase: int = PHASE_ALL, workspace=None, stream=None):
    """Sparse top-k attention (mla_sparse_attn); indices is int32 [B, T, topk]."""
    dims = _dims_from(q_lat, c_kv, kv_lens, max_kv_len=max_kv_len, kv_seq_stride=kv_seq_stride,
                      page_table=page_table, page_size=page_size, topk=int(indices.shape[2]),
                      num_splits=num_splits, phase=phase)
    _call("mla_sparse_attn", dims, True, _as_u16(q_lat), _as_u16(q_rope), _as_u16(c_kv),
          _as_u16(k_rope), page_table, indices, kv_lens, scale, _as_u16(out), lse, workspace,
          stream)


def compact_kv(c_kv, k_rope, page_table, kv_lens, accepted, num_accepted, new_kv_lens, *,
               max_kv_len: int, kv_seq_stride: int = 0, page_size: int = 0, stream=None):
    """Post-verify KV compaction (mla_compact_kv), in place on c_kv / k_rope.

    accepted is int32 [B, T] (draft indices in path order), num_accepted int32 [B];
    new_kv_lens int32 [B] receives the compacted lengths (it may be kv_lens itself).
    """
    import torch

    B, T = accepted.shape
    dims = make_dims(batch=int(B), num_q=int(T), num_heads=1, max_kv_len=int(max_kv_len),
                     kv_rows=int(c_kv.shape[0]), kv_seq_stride=int(kv_seq_stride),
                     page_size=int(page_size) if page_table is not None else 0,
                     max_pages=int(page_table.shape[1]) if page_table is not None else 0)
    if stream is None:
        stream = torch.cuda.current_stream(c_kv.device)
    rc = load_library().mla_compact_kv(ctypes.byref(dims), _ptr(_as_u16(c_kv)), _ptr(_as_u16(k_rope)),
                                       _ptr(page_table), _ptr(kv_lens), _ptr(accepted),
                                       _ptr(num_accepted), _ptr(new_kv_lens),
                                       ctypes.c_void_p(stream.cuda_stream))
    if rc != MLA_OK:
        raise MlaError(rc, "mla_compact_kv")


def head_project(x, w, y, stream=None):
    """y[m, h, :] = x[m, h, :] . w[h] (mla_head_project): x [tokens, heads, in_dim],
    w [heads, in_dim, out_dim], y [tokens, heads, out_dim], all bf16 (or uint16)."""
    import torch

    M, H, K = x.shape
    N = w.shape[2]
    if tuple(w.shape) != (H, K, N) or tuple(y.shape) != (M, H, N):
        raise ValueError("head_project: x [M,H,K], w [H,K,N], y [M,H,N]")
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    rc = load_library().mla_head_project(int(M), int(H), int(K), int(N), _ptr(_as_u16(x)),
                                         _ptr(_as_u16(w)), _ptr(_as_u16(y)),
                                         ctypes.c_void_p(stream.cuda_stream))
    if rc != MLA_OK:
        raise MlaError(rc, "mla_head_project")


def probe_mfma_bf16(blocks: int, iters: int, sink, stream=None) -> float:
    """Enqueue the matrix-core throughput probe (mla_probe_mfma_bf16) and return
    the flops that launch performs; `sink` is a float32 device tensor of at
    least blocks x 256 elements."""
    import torch

    if sink.dtype != torch.float32 or sink.numel() < blocks * 256:
        raise ValueError("probe_mfma_bf16: sink must be float32 with blocks x 256 elements")
    if stream is None:
        stream = torch.cuda.current_stream(sink.device)
    rc = load_library().mla_probe_mfma_bf16(int(blocks), int(iters), _ptr(sink),
                                            ctypes.c_void_p(stream.cuda_stream))
    if rc != MLA_OK:
        raise MlaError(rc, "mla_probe_mfma_bf16")
    return float(blocks) * 4 * iters * 16 * 2 * 32 * 32 * 16


def probe_gather_rows(c_kv, k_rope, indices, *, kv_seq_stride: int, tokens_per_seq: int, sink,
                      stream=None, count: bool = True):
    """Enqueue the row-gather probe (mla_probe_gather_rows) over `indices` [groups,
    per_group]; with `count`, also return the bytes it gathers (1,152 per index that
    selects a row; counting synchronises with the device, so timed calls pass
    count=False). `sink` is a float32 device tensor of at least groups x
    ceil(per_group / 64) x 256 elements."""
    import torch

    idx = indices.reshape(indices.shape[0], -1) if indices.dim() != 2 else indices
    G, K = int(idx.shape[0]), int(idx.shape[1])
    if sink.dtype != torch.float32 or sink.numel() < G * ((K + 63) // 64) * 256:
        raise ValueError("probe_gather_rows: sink too small")
    if stream is None:
        stream = torch.cuda.current_stream(c_kv.device)
    rows = int(c_kv.shape[0])
    rc = load_library().mla_probe_gather_rows(_ptr(_as_u16(c_kv)), _ptr(_as_u16(k_rope)), rows,
                                              int(kv_seq_stride), _ptr(idx), G, K,
                                              int(tokens_per_seq), _ptr(sink),
                                              ctypes.c_void_p(stream.cuda_stream))
    if rc != MLA_OK:
        raise MlaError(rc, "mla_probe_gather_rows")
    if not count:
        return None
    base = (torch.arange(G, device=idx.device) // int(tokens_per_seq)) * int(kv_seq_stride)
    row = idx.to(torch.int64) + base[:, None]
    valid = (idx >= 0) & (row < rows)
    if kv_seq_stride > 0:
        valid &= idx < int(kv_seq_stride)
    return int(valid.sum().item()) * 1152


def topk_workspace_bytes(rows: int, row_len: int) -> int:
    return int(load_library().mla_select_topk_workspace_bytes(int(rows), int(row_len)))


def select_topk(scores, k: int, indices, row_lens=None, row_len: Optional[int] = None,
                workspace=None, split_rows: bool = True, stream=None):
    """Top-k positions per row of fp32 scores (mla_select_topk), ascending and -1
    padded into int32 indices [rows, k]. row_len defaults to scores.shape[1].
    split_rows=False passes no workspace (one workgroup per row); otherwise the
    given workspace, or a cached one of mla_select_topk_workspace_bytes, lets
    the library spread short batches of rows over several workgroups."""
    import torch

    rows, stride = scores.shape
    n = int(stride if row_len is None else row_len)
    if stream is None:
        stream = torch.cuda.current_stream(scores.device)
    if not split_rows:
        workspace = None
    elif workspace is None:
        workspace = _workspace(scores.device, topk_workspace_bytes(rows, n), tag="topk")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().mla_select_topk(int(rows), n, int(stride), int(k), _ptr(scores),
                                        _ptr(row_lens), _ptr(indices), _ptr(workspace),
                                        ctypes.c_size_t(ws_bytes),
                                        ctypes.c_void_p(stream.cuda_stream))
    if rc != MLA_OK:
        raise MlaError(rc, "mla_select_topk")
