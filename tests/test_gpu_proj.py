"""GPU parity of the per-head projection (mla_head_project) against the fp64
oracle.

Tolerance from the arithmetic: products of bf16 inputs are exact in fp32, the
fp32 sum of K of them is within K * 2^-24 * sum|x||w| (K <= 1024 gives <= 2^-14),
and the bf16 result adds half an ulp, <= 2^-9 |y|. The test allows
2^-8 |y| + 2^-13 sum_k |x_k||w_kn|.
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_decode_verify_mla_amd as mv
from speculative_decode_verify_mla_amd.synth import bf16_bits_to_f64, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

SHAPES = [
    ("absorb_q", 16, 64, 128, 512),      # q_nope . W_UK, one verify step (T=16 tokens)
    ("head_out", 16, 64, 512, 128),      # out_lat . W_UV
    ("ragged_tokens", 37, 3, 48, 96),    # token tail inside a 32-token tile
    ("many_tokens", 100, 8, 128, 512),   # several token tiles
    ("minimal", 1, 1, 16, 32),
    ("wide_k", 5, 2, 1024, 64),
]


def _bf16(rng, shape, scale=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("name,M,H,K,N", SHAPES, ids=[s[0] for s in SHAPES])
def test_head_project_matches_oracle(gpu_lib, name, M, H, K, N):
    print(f"[case] head_project {name} M={M} H={H} K={K} N={N}", flush=True)
    rng = np.random.default_rng([M, H, K, N])  # stable per shape
    xb = _bf16(rng, (M, H, K))
    wb = _bf16(rng, (H, K, N), 1.0 / np.sqrt(K))
    d = torch.device("cuda:0")
    x = torch.from_numpy(xb.view(np.int16)).to(d)
    w = torch.from_numpy(wb.view(np.int16)).to(d)
    y = torch.full((M, H, N), 0x7FC0, dtype=torch.int16, device=d)
    mv.head_project(x, w, y)
    torch.cuda.synchronize()
    got = bf16_bits_to_f64(y.cpu().numpy().view(np.uint16))
    xf, wf = bf16_bits_to_f64(xb), bf16_bits_to_f64(wb)
    ref = oracle.head_project(xf, wf)
    bound = oracle.head_project(np.abs(xf), np.abs(wf))
    err = np.abs(got - ref)
    tol = 2.0 ** -8 * np.abs(ref) + 2.0 ** -13 * bound
    print(f"   max|dy|={err.max():.3e} max rel={np.max(err / np.maximum(np.abs(ref), 1e-30)):.3e}",
          flush=True)
    assert np.isfinite(got).all()
    assert np.all(err <= tol)


def test_head_project_on_both_sides_of_verify(gpu_lib):
    """q_nope -> (absorb) -> verify -> (head out) equals the oracle chain run in
    fp64 from the same bf16 tensors (each stage's output rounded to bf16 as the
    GPU path does), within the verify call's own tolerance."""
    from speculative_decode_verify_mla_amd import synth
    from tests._util import run_oracle

    w = synth.generate(synth.Spec("proj_chain", B=1, T=4, H=16, layout="contig", prefix=500), seed=51)
    print("[case] absorb -> verify -> head out", flush=True)
    rng = np.random.default_rng(52)
    M = w.B * w.T
    q_nope = _bf16(rng, (M, w.H, 128))
    w_uk = _bf16(rng, (w.H, 128, 512), 1.0 / np.sqrt(128))
    w_uv = _bf16(rng, (w.H, 512, 128), 1.0 / np.sqrt(512))
    d = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(d)
    q_lat_dev = torch.empty((M, w.H, 512), dtype=torch.int16, device=d)
    mv.head_project(t(q_nope), t(w_uk), q_lat_dev)
    torch.cuda.synchronize()
    q_lat_bits = q_lat_dev.cpu().numpy().view(np.uint16).reshape(w.B, w.T, w.H, 512)
    # the verify call on the absorbed queries
    w.q_lat[:] = q_lat_bits
    from tests._gpu import DeviceWorkload
    dw = DeviceWorkload(w)
    dw.run()
    torch.cuda.synchronize()
    o_head = torch.empty((M, w.H, 128), dtype=torch.int16, device=d)
    mv.head_project(dw.out.view(M, w.H, 512), t(w_uv), o_head)
    torch.cuda.synchronize()
    got = bf16_bits_to_f64(o_head.cpu().numpy().view(np.uint16))
    # oracle chain from the same absorbed queries
    q_lat_ref = oracle.head_project(bf16_bits_to_f64(q_nope), bf16_bits_to_f64(w_uk))
    assert np.all(np.abs(bf16_bits_to_f64(q_lat_bits).reshape(M, w.H, 512) - q_lat_ref)
                  <= 2.0 ** -8 * np.abs(q_lat_ref) + 2.0 ** -13 * oracle.head_project(
                      np.abs(bf16_bits_to_f64(q_nope)), np.abs(bf16_bits_to_f64(w_uk))))
    out_ref, _ = run_oracle(w)
    ref = oracle.head_project(out_ref.reshape(M, w.H, 512), bf16_bits_to_f64(w_uv))
    # |o| error: the verify bar (1e-2 on out) carried through |W_UV| row sums, plus rounding
    carry = 1e-2 * np.abs(bf16_bits_to_f64(w_uv)).sum(axis=1)  # [H, 128]
    err = np.abs(got - ref)
    print(f"   chain max|do|={err.max():.3e}", flush=True)
    assert np.all(err <= carry[None] + 2.0 ** -8 * np.abs(ref) + 1e-3)
