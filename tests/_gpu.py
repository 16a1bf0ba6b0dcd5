"""Device-side helpers for the GPU tests: upload a synthetic workload and call the C ABI."""
from __future__ import annotations

import numpy as np
import torch

import speculative_decode_verify_mla_amd as mv
from speculative_decode_verify_mla_amd.synth import DL, DR, Workload, bf16_bits_to_f64

NAN_BF16 = 0x7FC0


def _dev_u16(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


class DeviceWorkload:
    """A workload resident on the GPU, with its output buffers."""

    def __init__(self, w: Workload, device="cuda:0"):
        self.w = w
        self.device = torch.device(device)
        d = self.device
        self.q_lat = _dev_u16(w.q_lat, d)
        self.q_rope = _dev_u16(w.q_rope, d)
        if w.row_ids is None:
            self.c_kv = _dev_u16(w.c_kv, d)
            self.k_rope = _dev_u16(w.k_rope, d)
        else:
            # only the selected rows carry values; the rest of the cache is NaN poison
            self.c_kv = torch.full((w.kv_rows, DL), NAN_BF16, dtype=torch.int16, device=d)
            self.k_rope = torch.full((w.kv_rows, DR), NAN_BF16, dtype=torch.int16, device=d)
            rows = torch.from_numpy(w.row_ids).to(d)
            self.c_kv[rows] = _dev_u16(w.c_kv, d)
            self.k_rope[rows] = _dev_u16(w.k_rope, d)
        self.kv_lens = torch.from_numpy(w.kv_lens.astype(np.int32)).to(d)
        m = w.mask_for_kernel
        self.tree_mask = None if m is None else torch.from_numpy(m.astype(np.uint8)).to(d)
        self.page_table = None if w.page_table is None else torch.from_numpy(
            w.page_table.astype(np.int32)).to(d)
        self.indices = None if w.indices is None else torch.from_numpy(
            w.indices.astype(np.int32)).to(d)
        self.out = torch.empty((w.B, w.T, w.H, DL), dtype=torch.int16, device=d)
        self.lse = torch.empty((w.B, w.T, w.H), dtype=torch.float32, device=d)

    def run(self, num_splits=0, phase=mv.binding.PHASE_ALL, out=None, lse=None, q_lat=None,
            q_rope=None, workspace=None, stream=None):
        w = self.w
        out = self.out if out is None else out
        lse = self.lse if lse is None else lse
        kw = dict(max_kv_len=w.max_kv_len, kv_seq_stride=w.kv_seq_stride, page_size=w.page_size,
                  num_splits=num_splits, phase=phase, workspace=workspace, stream=stream)
        ql = self.q_lat if q_lat is None else q_lat
        qr = self.q_rope if q_rope is None else q_rope
        if w.layout == "sparse":
            mv.sparse_attn(ql, qr, self.c_kv, self.k_rope, self.page_table, self.indices,
                           self.kv_lens, w.scale, out, lse, **kw)
        else:
            mv.verify_attn(ql, qr, self.c_kv, self.k_rope, self.page_table, self.tree_mask,
                           self.kv_lens, w.scale, out, lse, **kw)

    def workspace(self, num_splits=0):
        """A workspace of the size this workload's call needs (allocated here, not on capture)."""
        w = self.w
        dims = mv.binding._dims_from(self.q_lat, self.c_kv, self.kv_lens, max_kv_len=w.max_kv_len,
                                     kv_seq_stride=w.kv_seq_stride, page_table=self.page_table,
                                     page_size=w.page_size, topk=w.topk or 0,
                                     num_splits=num_splits, phase=0)
        n = mv.workspace_bytes(dims, sparse=w.layout == "sparse")
        return torch.empty(max(n, 16), dtype=torch.uint8, device=self.device)

    def results(self, out=None, lse=None):
        torch.cuda.synchronize(self.device)
        out = self.out if out is None else out
        lse = self.lse if lse is None else lse
        o = bf16_bits_to_f64(out.cpu().numpy().view(np.uint16))
        return o, lse.cpu().numpy().astype(np.float64)
