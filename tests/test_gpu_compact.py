"""GPU parity of post-verify KV compaction (mla_compact_kv) against the oracle:
bit-exact cache contents and lengths, contiguous and paged, with accepted
root-to-node paths of random draft trees, the degenerate cases, and new
lengths written over kv_lens itself."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decode_verify_mla_amd as mv
from speculative_decode_verify_mla_amd import synth
from speculative_decode_verify_mla_amd.synth import Spec, generate

pytestmark = pytest.mark.gpu


def _path(parents, node):
    p = []
    while node >= 0:
        p.append(node)
        node = parents[node]
    return p[::-1]


def _accepted(w, rng):
    """A root-to-node path of each sequence's draft tree (parents drawn like the workloads)."""
    acc = np.full((w.B, w.T), -1, dtype=np.int32)
    n = np.zeros(w.B, dtype=np.int32)
    for b in range(w.B):
        parents = synth.random_tree_parents(rng, w.T)
        path = _path(parents, int(rng.integers(0, w.T)))
        acc[b, :len(path)] = path
        n[b] = len(path)
    return acc, n


def _run(w, acc, nacc, alias=False):
    d = torch.device("cuda:0")
    u16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(d)
    c_kv, k_rope = u16(w.c_kv), u16(w.k_rope)
    kv_lens = torch.from_numpy(w.kv_lens.astype(np.int32)).to(d)
    pt = None if w.page_table is None else torch.from_numpy(w.page_table.astype(np.int32)).to(d)
    acc_t = torch.from_numpy(acc.astype(np.int32)).to(d)
    n_t = torch.from_numpy(nacc.astype(np.int32)).to(d)
    new_lens = kv_lens if alias else torch.empty_like(kv_lens)
    mv.compact_kv(c_kv, k_rope, pt, kv_lens, acc_t, n_t, new_lens, max_kv_len=w.max_kv_len,
                  kv_seq_stride=w.kv_seq_stride, page_size=w.page_size)
    torch.cuda.synchronize()
    return (c_kv.cpu().numpy().view(np.uint16), k_rope.cpu().numpy().view(np.uint16),
            new_lens.cpu().numpy())


def _expect(w, acc, nacc):
    return oracle.compact_kv(w.c_kv, w.k_rope, w.kv_lens, acc, nacc, w.T,
                             kv_seq_stride=w.kv_seq_stride, page_table=w.page_table,
                             page_size=w.page_size, max_kv_len=w.max_kv_len)


SPECS = [
    Spec("c_contig", B=5, T=16, H=8, layout="contig", prefix=[300, 0, 5000, 17, 64]),
    Spec("c_paged", B=6, T=8, H=8, layout="paged", prefix=[1000, 5, 64 * 3 - 8, 2000, 70, 12]),
    Spec("c_t64", B=2, T=64, H=8, layout="contig", prefix=[100, 1]),
]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
@pytest.mark.parametrize("alias", [False, True])
def test_compaction_matches_oracle(gpu_lib, spec, alias):
    w = generate(spec, seed=41)
    rng = np.random.default_rng(42)
    acc, nacc = _accepted(w, rng)
    print(f"[case] compact {spec.name} alias={alias} kv_lens={w.kv_lens.tolist()} n={nacc.tolist()}",
          flush=True)
    c, r, lens = _run(w, acc, nacc, alias=alias)
    ce, re_, le = _expect(w, acc, nacc)
    assert np.array_equal(lens, le)
    assert np.array_equal(c, ce) and np.array_equal(r, re_)


def test_compaction_degenerate_cases(gpu_lib):
    """Nothing accepted, everything accepted, bad indices, counts past T, a short sequence."""
    spec = Spec("c_deg", B=6, T=8, H=8, layout="contig", prefix=[200, 200, 200, 200, 200, 0])
    w = generate(spec, seed=43)
    w.kv_lens[5] = 3  # shorter than the draft window
    acc = np.array([[0, 1, 2, 3, 4, 5, 6, 7],
                    [0, 1, 2, 3, 4, 5, 6, 7],
                    [7, -1, 9, 2, 100, 3, 0, 0],
                    [1, 2, 3, 4, 5, 6, 7, 0],
                    [3, 5, 7, 0, 0, 0, 0, 0],
                    [5, 6, 7, 0, 0, 0, 0, 0]], dtype=np.int32)
    nacc = np.array([0, 8, 8, 50, 3, 3], dtype=np.int32)
    print("[case] compact degenerate", flush=True)
    c, r, lens = _run(w, acc, nacc)
    ce, re_, le = _expect(w, acc, nacc)
    assert np.array_equal(lens, le)
    assert np.array_equal(c, ce) and np.array_equal(r, re_)


def test_compaction_then_verify(gpu_lib):
    """Attention over the compacted sequence (its new length) sees exactly the keys
    of prefix + accepted drafts in the original cache."""
    spec = Spec("c_then_v", B=2, T=8, H=64, layout="paged", prefix=[900, 3000])
    w = generate(spec, seed=44)
    rng = np.random.default_rng(45)
    acc, nacc = _accepted(w, rng)
    print(f"[case] compact then verify n={nacc.tolist()}", flush=True)
    c, r, lens = _run(w, acc, nacc)
    f = synth.bf16_bits_to_f64
    for b in range(w.B):
        P = int(w.kv_lens[b]) - w.T
        logical = np.concatenate([np.arange(P), P + acc[b, :nacc[b]]])  # prefix + accepted
        new_logical = np.arange(int(lens[b]))
        ps = w.page_size
        phys = lambda p: w.page_table[b, p // ps] * ps + p % ps
        k_old = np.array([phys(p) for p in logical])
        k_new = np.array([phys(p) for p in new_logical])
        o1, l1 = oracle.attend(f(w.q_lat[b, 0]), f(w.q_rope[b, 0]), f(w.c_kv[k_old]), f(w.k_rope[k_old]),
                               w.scale)
        o2, l2 = oracle.attend(f(w.q_lat[b, 0]), f(w.q_rope[b, 0]), f(c[k_new]), f(r[k_new]), w.scale)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
