"""The allocation-free verify entry point (mla_verify_attn_noalloc, for callers
that cannot allocate) against the workspace entry point (mla_verify_attn) it
mirrors: both run the same kernels, so the results must be identical bit for
bit, and both within the oracle bar. Two calls in a row, the second smaller,
so the second reuses the fixed device scratch the first left behind."""
import numpy as np
import pytest
import torch

import speculative_decode_verify_mla_amd as mv
from speculative_decode_verify_mla_amd import synth
from speculative_decode_verify_mla_amd.synth import Spec, generate
from tests._util import run_oracle

pytestmark = pytest.mark.gpu


def _noalloc_vs_workspace(w, tag):
    from tests._gpu import DeviceWorkload

    print(f"[case] noalloc {tag} B={w.B} T={w.T} H={w.H} layout={w.layout} "
          f"kv_lens={w.kv_lens.tolist()[:8]}", flush=True)
    d = DeviceWorkload(w)
    ws = d.workspace()
    d.run(workspace=ws)
    torch.cuda.synchronize()
    ref_out, ref_lse = d.out.clone(), d.lse.clone()
    out = torch.full_like(d.out, 0x7FC0)
    lse = torch.full_like(d.lse, float("nan"))
    mv.verify_attn_noalloc(d.q_lat, d.q_rope, d.c_kv, d.k_rope, d.page_table, d.tree_mask,
                           d.kv_lens, w.scale, out, lse, max_kv_len=w.max_kv_len,
                           kv_seq_stride=w.kv_seq_stride, page_size=w.page_size)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), f"{tag}: out differs from the workspace call"
    assert torch.equal(lse, ref_lse), f"{tag}: lse differs from the workspace call"
    o = synth.bf16_bits_to_f64(out.cpu().numpy().view(np.uint16))
    l = lse.cpu().numpy().astype(np.float64)
    r_out, r_lse = run_oracle(w)
    e_out, e_lse = float(np.abs(o - r_out).max()), float(np.abs(l - r_lse).max())
    print(f"   {tag}: max|dout|={e_out:.3e} max|dlse|={e_lse:.3e}", flush=True)
    assert e_out <= 1e-2 and e_lse <= 1e-3


def test_noalloc_equals_workspace_call_twice_second_smaller(gpu_lib):
    # 1: one long sequence, 32 splits x 8 row blocks of partials (33.9 MB of scratch)
    big = generate(Spec("na_big", B=1, T=16, H=64, layout="contig", prefix=20000), seed=41)
    dims = mv.binding._dims_from(torch.empty(1, 16, 64, 512), torch.empty(big.kv_rows, 512),
                                 None, max_kv_len=big.max_kv_len, kv_seq_stride=big.kv_seq_stride,
                                 page_table=None, page_size=0, topk=0, num_splits=0, phase=0)
    need = mv.plan(dims).workspace_bytes
    assert 0 < need <= mv.binding.NOALLOC_SCRATCH_BYTES
    _noalloc_vs_workspace(big, "first call (large)")
    # 2: a smaller, ragged paged batch over the scratch the first call left
    small = generate(Spec("na_small", B=3, T=4, H=64, layout="paged", prefix=[900, 3000, 64]),
                     seed=42)
    _noalloc_vs_workspace(small, "second call (smaller)")
