"""GPU parity of top-k index selection (mla_select_topk) against the oracle:
bit-exact index lists (the tie rule makes the selection unique), and the
selection feeding the sparse attention call."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decode_verify_mla_amd as mv

pytestmark = pytest.mark.gpu


def _run(scores, k, row_lens=None, row_len=None, split_rows=True):
    d = torch.device("cuda:0")
    R, L = scores.shape
    if L % 4:  # the call reads rows 16 bytes at a time: pad the stride, keep the length
        scores = np.concatenate([scores, np.zeros((R, 4 - L % 4), np.float32)], axis=1)
        row_len = L if row_len is None else row_len
    s = torch.from_numpy(np.ascontiguousarray(scores, dtype=np.float32)).to(d)
    rl = None if row_lens is None else torch.from_numpy(np.asarray(row_lens, np.int32)).to(d)
    out = torch.full((scores.shape[0], k), 12345, dtype=torch.int32, device=d)
    mv.select_topk(s, k, out, row_lens=rl, row_len=row_len, split_rows=split_rows)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _expect(scores, k, row_lens=None, row_len=None):
    L = scores.shape[1] if row_len is None else row_len
    return oracle.select_topk(scores[:, :L], k, row_lens)


CASES = [
    ("normal", lambda r: r.standard_normal((6, 5000)), 300, None),
    ("ties", lambda r: r.integers(-4, 5, size=(5, 3000)), 257, None),
    ("all_equal", lambda r: np.full((2, 2000), 0.25), 1000, None),
    ("k1", lambda r: r.standard_normal((3, 777)), 1, None),
    ("k_over_n", lambda r: r.standard_normal((2, 300)), 512, None),
    ("ragged_rows", lambda r: r.standard_normal((5, 4096)), 700, [4096, 0, 1, 699, 2500]),
    ("one_bin", lambda r: 1.0 + r.integers(0, 3, size=(2, 5000)) * 2.0 ** -20, 1234, None),
    # rows long enough to be cut into several pieces (several workgroups per row)
    ("ties_long", lambda r: r.integers(-3, 4, size=(3, 40000)), 5000, None),
    ("all_equal_long", lambda r: np.full((2, 20000), -1.5), 7777, None),
    ("ragged_long", lambda r: r.standard_normal((4, 50000)), 3000, [50000, 8191, 4097, 0]),
    ("k_over_n_long", lambda r: r.standard_normal((2, 9000)), 12000, None),
    ("low_bits_long", lambda r: 1.0 + r.integers(0, 5, size=(2, 30000)) * 2.0 ** -22, 10001, None),
    # the selected keys packed into the first ~3 wave segments of each row:
    # ~1,000 entries per segment region, all of them staged in LDS
    ("clustered_long", lambda r: np.concatenate([10.0 + r.random((2, 3000)),
                                                 r.standard_normal((2, 62536))], axis=1), 2000, None),
]


@pytest.mark.parametrize("split_rows", [True, False], ids=["pieces", "one_wg"])
@pytest.mark.parametrize("name,make,k,row_lens", CASES, ids=[c[0] for c in CASES])
def test_topk_matches_oracle(gpu_lib, name, make, k, row_lens, split_rows):
    rng = np.random.default_rng(abs(k) + 7)
    scores = make(rng).astype(np.float32)
    print(f"[case] topk {name} rows={scores.shape[0]} L={scores.shape[1]} k={k} "
          f"split_rows={split_rows}", flush=True)
    got = _run(scores, k, row_lens, split_rows=split_rows)
    assert np.array_equal(got, _expect(scores, k, row_lens))


def test_topk_special_values_and_stride(gpu_lib):
    rng = np.random.default_rng(5)
    scores = rng.standard_normal((4, 1100)).astype(np.float32)
    scores[0, ::7] = np.nan
    scores[1, ::5] = -np.inf
    scores[1, 3] = np.inf
    scores[2, :600] = 0.0
    scores[2, 600:] = -0.0
    print("[case] topk special values, row_len 1000 of stride 1100", flush=True)
    got = _run(scores, 400, row_len=1000)
    assert np.array_equal(got, _expect(scores, 400, row_len=1000))
    # the same values over rows long enough to be cut into pieces
    big = np.tile(scores, (1, 12))
    print("[case] topk special values, row_len 12000 of stride 13200", flush=True)
    got = _run(big, 3000, row_len=12000)
    assert np.array_equal(got, _expect(big, 3000, row_len=12000))


def test_topk_long_rows(gpu_lib):
    """The sparse decode shape: 32 tokens x 131,072 candidates, k = 2048."""
    rng = np.random.default_rng(6)
    scores = rng.standard_normal((32, 131072)).astype(np.float32)
    lens = np.full(32, 131072, np.int32)
    lens[3] = 70000
    print("[case] topk 32 x 131072, k=2048", flush=True)
    exp = _expect(scores, 2048, lens)
    for split_rows in (True, False):
        got = _run(scores, 2048, lens, split_rows=split_rows)
        assert np.array_equal(got, exp), f"split_rows={split_rows}"


def test_topk_feeds_sparse_attention(gpu_lib):
    """Scores -> top-k -> sparse attention equals the oracle chain."""
    from speculative_decode_verify_mla_amd import synth
    from speculative_decode_verify_mla_amd.synth import Spec, generate
    from tests._util import run_oracle
    from tests._gpu import DeviceWorkload

    w = generate(Spec("topk_chain", B=2, T=2, H=64, layout="sparse", cache_len=6000, topk=256), seed=61)
    rng = np.random.default_rng(62)
    scores = rng.standard_normal((w.B * w.T, w.kv_seq_stride)).astype(np.float32)
    lens = np.repeat(w.kv_lens, w.T).astype(np.int32)
    idx = _run(scores, w.topk, lens, row_len=w.kv_seq_stride)
    exp = oracle.select_topk(scores, w.topk, lens)
    assert np.array_equal(idx, exp)
    print("[case] topk -> sparse attention", flush=True)
    w.indices = idx.reshape(w.B, w.T, w.topk)
    # the synthetic cache holds every row (rows_materialised = all); make it so
    full = generate(Spec("topk_chain_full", B=2, T=2, H=64, layout="contig", prefix=[5998, 5998]),
                    seed=63)
    w.c_kv, w.k_rope, w.row_ids = full.c_kv, full.k_rope, None
    d = DeviceWorkload(w)
    d.run()
    out, lse = d.results()
    ref_out, ref_lse = run_oracle(w)
    assert np.abs(out - ref_out).max() <= 1e-2 and np.abs(lse - ref_lse).max() <= 1e-3
