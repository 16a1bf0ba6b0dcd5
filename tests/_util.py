"""Test helpers: decode synthetic workloads into oracle inputs (test infrastructure)."""
from __future__ import annotations

import numpy as np

from speculative_decode_verify_mla_amd.synth import Workload, bf16_bits_to_f64
import oracle


def oracle_inputs(w: Workload):
    return dict(
        q_lat=bf16_bits_to_f64(w.q_lat),
        q_rope=bf16_bits_to_f64(w.q_rope),
        c_kv=bf16_bits_to_f64(w.c_kv),
        k_rope=bf16_bits_to_f64(w.k_rope),
    )


_DEFAULT = object()


def run_oracle(w: Workload, mask_override=_DEFAULT):
    d = oracle_inputs(w)
    mask = w.mask_for_kernel if mask_override is _DEFAULT else mask_override
    if w.layout == "sparse":
        return oracle.verify_sparse(d["q_lat"], d["q_rope"], d["c_kv"], d["k_rope"], w.kv_lens,
                                    w.indices, w.scale, kv_seq_stride=w.kv_seq_stride,
                                    page_table=w.page_table, page_size=w.page_size,
                                    row_ids=w.row_ids, kv_rows=w.kv_rows)
    return oracle.verify_dense(d["q_lat"], d["q_rope"], d["c_kv"], d["k_rope"], w.kv_lens,
                               mask, w.scale, kv_seq_stride=w.kv_seq_stride,
                               page_table=w.page_table, page_size=w.page_size,
                               row_ids=w.row_ids, kv_rows=w.kv_rows)


def bf16_round_f64(x: np.ndarray) -> np.ndarray:
    """Round-trip fp64 values through bf16 (RNE), for expressing expected bf16 outputs."""
    from speculative_decode_verify_mla_amd.synth import f32_to_bf16_bits
    return bf16_bits_to_f64(f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))
