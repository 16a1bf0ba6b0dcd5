"""The matrix-core throughput probe behind bench.py's measured ceiling.

Every thread's sink value is the sum of its 16 accumulators after `iters`
rounds of one fixed bf16 product, so it is `iters` times the one-round value
(up to fp32 rounding of the running sums), and it is the same on every run.
Threads 0 and 1 of each workgroup hold the loop's shader-clock cycles and
100 MHz real-time ticks instead; over a long loop their ratio is a clock
between 0.3 and 3 GHz."""
import pytest
import torch


@pytest.mark.gpu
def test_probe_runs_scales_and_repeats(gpu_lib):
    mv = gpu_lib
    blocks = 8
    dev = torch.device("cuda:0")
    s1 = torch.full((blocks * 256,), float("nan"), device=dev)
    s4 = torch.full_like(s1, float("nan"))
    again = torch.full_like(s1, float("nan"))
    f1 = mv.probe_mfma_bf16(blocks, 1, s1)
    f4 = mv.probe_mfma_bf16(blocks, 4, s4)
    mv.probe_mfma_bf16(blocks, 1, again)
    torch.cuda.synchronize()
    assert f1 == blocks * 4 * 16 * 2 * 32 * 32 * 16 and f4 == 4 * f1
    assert torch.isfinite(s1).all() and torch.isfinite(s4).all()
    v1, v4, va = (x.view(blocks, 256)[:, 2:] for x in (s1, s4, again))
    assert v1.abs().max() > 0
    assert torch.allclose(v4, 4 * v1, rtol=1e-4, atol=1e-2)
    assert torch.equal(va, v1)
    # clock stamps: elapsed cycles and 100 MHz ticks of each workgroup's loop
    big = torch.full((256 * 256,), float("nan"), device=dev)
    mv.probe_mfma_bf16(256, 2000, big)
    torch.cuda.synchronize()
    st = big.view(256, 256)[:, :2].double()
    assert (st > 0).all()
    ghz = float(st[:, 0].sum() / st[:, 1].sum()) * 0.1
    print(f"probe clock under full matrix-core load: {ghz:.3f} GHz", flush=True)
    assert 0.3 < ghz < 3.0


@pytest.mark.gpu
def test_gather_probe_reads_the_indexed_rows(gpu_lib):
    """Each thread of the row-gather probe folds (XOR) the words it loaded: 16 B of
    each of its wave's 16 latent rows, and for lanes 0..7 words 0 and 3 of 16 B of
    the rope row. The result is checked word for word against the same fold on the
    host, with skipped indices (-1, past the sequence or the cache) contributing
    nothing."""
    import numpy as np

    mv = gpu_lib
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(5)
    seqs, stride, T, K = 2, 300, 2, 70           # groups = seqs x T, two 64-index chunks each
    rows = seqs * stride
    lat = rng.integers(0, 2**16, size=(rows, 512), dtype=np.uint16)
    rope = rng.integers(0, 2**16, size=(rows, 64), dtype=np.uint16)
    idx = rng.integers(0, stride, size=(seqs * T, K)).astype(np.int32)
    idx[0, :5] = -1
    idx[3, 7] = 10**6  # past the sequence and the cache: skipped
    idx[1, 9] = stride + 3  # past its sequence (a row of the next one): skipped
    G = seqs * T
    chunks = (K + 63) // 64
    sink = torch.zeros(G * chunks * 256, dtype=torch.float32, device=dev)
    c_kv = torch.from_numpy(lat.view(np.int16)).to(dev)
    k_rope = torch.from_numpy(rope.view(np.int16)).to(dev)
    nbytes = mv.probe_gather_rows(c_kv, k_rope, torch.from_numpy(idx).to(dev),
                                  kv_seq_stride=stride, tokens_per_seq=T, sink=sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    lat32, rope32 = lat.view(np.uint32), rope.view(np.uint32)  # [rows, 256], [rows, 32]
    want = np.zeros_like(got)
    valid = 0
    for g in range(G):
        for c in range(chunks):
            for t in range(256):
                w, l = t // 64, t % 64
                x = np.uint32(0)
                for i in range(16):
                    k = c * 64 + w * 16 + i
                    if k >= K:
                        continue
                    row = (g // T) * stride + int(idx[g, k])
                    if idx[g, k] < 0 or idx[g, k] >= stride or row >= rows:
                        continue
                    x ^= np.bitwise_xor.reduce(lat32[row, 4 * l:4 * l + 4])
                    if l < 8:
                        x ^= rope32[row, 4 * l] ^ rope32[row, 4 * l + 3]
                want[(g * chunks + c) * 256 + t] = x
    for g in range(G):
        for k in range(K):
            row = (g // T) * stride + int(idx[g, k])
            valid += idx[g, k] >= 0 and idx[g, k] < stride and row < rows
    assert nbytes == valid * 1152
    assert np.array_equal(got, want)
