"""Serving-style use of the verify call: captured into a HIP graph and replayed,
and issued on several streams at once ("The SMEM Ceiling", section "CUDA Graph
Capture Safety"; the 4-stream benchmark of "The Shared Memory Ceiling",
section "The Message: Reasoning Before Deployment"). The eager result of every
case is checked against the fp64 oracle (max-abs 1e-2 on out, 1e-3 on lse),
and every replay and every stream's result must equal the eager call bit for
bit (the kernels are deterministic and the call keeps no state between
launches)."""
import dataclasses

import numpy as np
import pytest
import torch

from speculative_decode_verify_mla_amd import synth
from speculative_decode_verify_mla_amd.synth import DL, Spec, generate
from tests._util import run_oracle

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
LSE_TOL = 1e-3


def _check_oracle(out_t, lse_t, w, tag):
    """The device result (torch tensors) against the oracle for workload w."""
    out = synth.bf16_bits_to_f64(out_t.cpu().numpy().view(np.uint16))
    lse = lse_t.cpu().numpy().astype(np.float64)
    ref_out, ref_lse = run_oracle(w)
    e_out = float(np.abs(out - ref_out).max())
    e_lse = float(np.abs(lse - ref_lse).max())
    print(f"   {tag}: max|dout|={e_out:.3e} max|dlse|={e_lse:.3e}", flush=True)
    assert e_out <= OUT_TOL and e_lse <= LSE_TOL, (tag, e_out, e_lse)

CASES = [
    ("long_single", lambda: generate(Spec("g1", B=1, T=16, H=64, layout="contig", prefix=6000), seed=31)),
    ("ragged_paged", lambda: generate(Spec("g2", B=4, T=4, H=64, layout="paged",
                                           prefix=[5000, 40, 1200, 3000]), seed=32)),
    ("sparse", lambda: generate(Spec("g3", B=4, T=1, H=64, layout="sparse", cache_len=8000,
                                     topk=512), seed=33)),
]


def _dev(w):
    from tests._gpu import DeviceWorkload
    return DeviceWorkload(w)


def _snapshot(d):
    torch.cuda.synchronize()
    return d.out.clone(), d.lse.clone()


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_equals_eager(gpu_lib, name, make):
    w = make()
    print(f"[case] graph replay {name} B={w.B} T={w.T} layout={w.layout}", flush=True)
    d = _dev(w)
    ws = d.workspace()
    d.run(workspace=ws)
    ref_out, ref_lse = _snapshot(d)
    _check_oracle(ref_out, ref_lse, w, f"{name} eager")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        d.run(workspace=ws, stream=side)  # warm on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        d.run(workspace=ws, stream=side)
    torch.cuda.synchronize()

    # other eager work between replays: scribble over the outputs and the
    # workspace, and run an eager call with different queries
    other_q = torch.flip(d.q_lat, dims=[2]).contiguous()
    for rep in range(3):
        d.out.fill_(0x7FC0)
        d.lse.fill_(float("nan"))
        ws.fill_(0xFF)
        scratch_out = torch.empty_like(d.out)
        scratch_lse = torch.empty_like(d.lse)
        d.run(q_lat=other_q, out=scratch_out, lse=scratch_lse, workspace=ws)
        torch.cuda.synchronize()
        g.replay()
        out, lse = _snapshot(d)
        assert torch.equal(out, ref_out), f"replay {rep}: out differs"
        assert torch.equal(lse, ref_lse), f"replay {rep}: lse differs"
        if rep == 0:
            _check_oracle(out, lse, w, f"{name} replay")


def test_streams_equal_eager(gpu_lib):
    """Four calls in flight on four streams (own outputs and workspaces)."""
    w = generate(Spec("ms", B=2, T=8, H=64, layout="contig", prefix=[3000, 7000]), seed=34)
    print("[case] four streams", flush=True)
    d = _dev(w)
    n = 4
    qs = [d.q_lat] + [torch.roll(d.q_lat, shifts=k, dims=2).contiguous() for k in range(1, n)]
    outs = [torch.empty_like(d.out) for _ in range(n)]
    lses = [torch.empty_like(d.lse) for _ in range(n)]
    wss = [d.workspace() for _ in range(n)]
    refs = []
    for k in range(n):
        d.run(q_lat=qs[k], out=outs[k], lse=lses[k], workspace=wss[k])
        torch.cuda.synchronize()
        refs.append((outs[k].clone(), lses[k].clone()))
        outs[k].zero_()
        lses[k].zero_()
    # each stream's queries are the heads rolled by k: its own oracle case
    for k in range(n):
        wk = dataclasses.replace(w, q_lat=np.roll(w.q_lat, shift=k, axis=2))
        _check_oracle(*refs[k], wk, f"stream {k} eager")
    streams = [torch.cuda.Stream() for _ in range(n)]
    torch.cuda.synchronize()
    for rep in range(2):
        for k in range(n):
            streams[k].wait_stream(torch.cuda.current_stream())
            d.run(q_lat=qs[k], out=outs[k], lse=lses[k], workspace=wss[k], stream=streams[k])
        torch.cuda.synchronize()
        for k in range(n):
            assert torch.equal(outs[k], refs[k][0]) and torch.equal(lses[k], refs[k][1]), (rep, k)


def test_streams_in_a_graph_equal_oracle(gpu_lib):
    """Four calls on four streams, forked from and joined into one captured
    graph (own outputs and workspaces), replayed several times with eager work
    in between; every stream's output matches the oracle and the eager call."""
    w = generate(Spec("msg", B=1, T=8, H=64, layout="contig", prefix=5000), seed=35)
    print("[case] four streams captured in one graph", flush=True)
    d = _dev(w)
    n = 4
    qs = [d.q_lat] + [torch.roll(d.q_lat, shifts=k, dims=2).contiguous() for k in range(1, n)]
    outs = [torch.empty_like(d.out) for _ in range(n)]
    lses = [torch.empty_like(d.lse) for _ in range(n)]
    wss = [d.workspace() for _ in range(n)]
    for k in range(n):
        d.run(q_lat=qs[k], out=outs[k], lse=lses[k], workspace=wss[k])
    torch.cuda.synchronize()
    refs = [(o.clone(), l.clone()) for o, l in zip(outs, lses)]
    for k in range(n):
        wk = dataclasses.replace(w, q_lat=np.roll(w.q_lat, shift=k, axis=2))
        _check_oracle(*refs[k], wk, f"graph stream {k} eager")

    cap = torch.cuda.Stream()
    streams = [torch.cuda.Stream() for _ in range(n)]
    cap.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for k in range(n):
            streams[k].wait_stream(cap)
            d.run(q_lat=qs[k], out=outs[k], lse=lses[k], workspace=wss[k], stream=streams[k])
        for k in range(n):
            cap.wait_stream(streams[k])
    torch.cuda.synchronize()
    for rep in range(3):
        for k in range(n):
            outs[k].fill_(0x7FC0)
            lses[k].fill_(float("nan"))
            wss[k].fill_(0xFF)
        d.run(q_lat=qs[(rep + 1) % n], out=d.out, lse=d.lse, workspace=wss[0])  # eager work between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in range(n):
            assert torch.equal(outs[k], refs[k][0]) and torch.equal(lses[k], refs[k][1]), (rep, k)


def test_topk_graph_replay_equals_eager(gpu_lib):
    """Top-k over row pieces (three launches sharing a workspace) captured into a
    graph: every replay, with the workspace and output scribbled over and other
    eager selections in between, equals the eager call."""
    import speculative_decode_verify_mla_amd as mv

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(71)
    R, L, k = 6, 30000, 1500
    scores = torch.from_numpy(rng.standard_normal((R, L)).astype(np.float32)).to(dev)
    lens = torch.tensor([30000, 12000, 4097, 0, 29999, 1], dtype=torch.int32, device=dev)
    ws = torch.empty(mv.topk_workspace_bytes(R, L), dtype=torch.uint8, device=dev)
    out = torch.empty((R, k), dtype=torch.int32, device=dev)
    print(f"[case] top-k graph replay R={R} L={L} k={k} workspace={ws.numel()}", flush=True)
    mv.select_topk(scores, k, out, row_lens=lens, workspace=ws)
    torch.cuda.synchronize()
    ref = out.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    mv.select_topk(scores, k, out, row_lens=lens, workspace=ws, stream=side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        mv.select_topk(scores, k, out, row_lens=lens, workspace=ws, stream=side)
    torch.cuda.synchronize()
    other = torch.flip(scores, dims=[1]).contiguous()
    other_out = torch.empty_like(out)
    for rep in range(3):
        out.fill_(-7)
        ws.fill_(0xAB)
        mv.select_topk(other, k, other_out, row_lens=lens, workspace=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}"
