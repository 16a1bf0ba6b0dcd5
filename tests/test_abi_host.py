"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments with the documented codes before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

import speculative_decode_verify_mla_amd as mv
from speculative_decode_verify_mla_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libmla_verify.so is not built (run __graft_entry__.build())")
    return mv.load_library()


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(mla_\w+)\(", text, re.M)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(B.EXPORTED)


def test_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def _dims(**kw):
    base = dict(batch=1, num_q=4, num_heads=16, max_kv_len=132, kv_rows=132, kv_seq_stride=132)
    base.update(kw)
    return B.make_dims(**base)


class FakePtr:
    """Aligned non-NULL addresses that are never dereferenced (validation fails first)."""

    def __init__(self, addr):
        self.addr = addr

    def __call__(self):
        return ctypes.c_void_p(self.addr)


P = FakePtr(0x10000)
MIS = FakePtr(0x10002)


def call(lib, dims, sparse=False, ptrs=None, ws=None, ws_bytes=0, scale=0.1):
    p = dict(q_lat=P(), q_rope=P(), c_kv=P(), k_rope=P(), pt=None, mask=None, idx=P(),
             kv_lens=P(), out=P(), lse=P())
    if ptrs:
        p.update(ptrs)
    fn = lib.mla_sparse_attn if sparse else lib.mla_verify_attn
    third = p["idx"] if sparse else p["mask"]
    return fn(ctypes.byref(dims) if dims is not None else None, p["q_lat"], p["q_rope"],
              p["c_kv"], p["k_rope"], p["pt"], third, p["kv_lens"], ctypes.c_float(scale),
              p["out"], p["lse"], ws, ws_bytes, None)


@pytest.mark.parametrize("case", [
    dict(dims=None),
    dict(kw=dict(num_q=0)),
    dict(kw=dict(num_q=65)),
    dict(kw=dict(batch=0)),
    dict(kw=dict(num_heads=0)),
    dict(kw=dict(max_kv_len=3)),            # max_kv_len < T
    dict(kw=dict(kv_seq_stride=100)),       # stride < max_kv_len
    dict(kw=dict(batch=2)),                 # second sequence past kv_rows
    dict(kw=dict(num_splits=-1)),
    dict(kw=dict(batch=40000, max_kv_len=1 << 22, kv_seq_stride=1 << 22,
                 kv_rows=40000 << 22)),  # batch x tiles past 2^31
    dict(kw=dict(phase=3)),
    dict(ptrs=dict(q_lat=None)),
    dict(ptrs=dict(out=None)),
    dict(ptrs=dict(kv_lens=None)),
    dict(ptrs=dict(c_kv=MIS())),            # misaligned
    dict(ptrs=dict(pt=P())),                # page table without page size
    dict(kw=dict(page_size=64, max_pages=3)),  # page size without page table
    dict(kw=dict(page_size=32, max_pages=5), ptrs=dict(pt=P())),  # not a multiple of 64
    dict(kw=dict(page_size=64, max_pages=2), ptrs=dict(pt=P())),  # 2*64 < max_kv_len
    dict(scale=float("nan")),
    dict(scale=0.0),                        # the softmax scale must be positive
    dict(scale=-0.1),
    dict(scale=float("inf")),
])
def test_invalid_arguments(lib, case):
    dims = None if "dims" in case else _dims(**case.get("kw", {}))
    rc = call(lib, dims, ptrs=case.get("ptrs"), scale=case.get("scale", 0.1))
    assert rc == B.MLA_ERR_INVALID


def test_reserved_must_be_zero(lib):
    d = _dims()
    d.reserved = 1
    assert call(lib, d) == B.MLA_ERR_INVALID


def test_sparse_invalid(lib):
    d = _dims(topk=0, num_q=1)
    assert call(lib, d, sparse=True) == B.MLA_ERR_INVALID
    d = _dims(topk=16, num_q=1)
    assert call(lib, d, sparse=True, ptrs=dict(idx=None)) == B.MLA_ERR_INVALID
    big = (1 << 21) + 64
    d = _dims(topk=16, num_q=1, max_kv_len=big, kv_rows=big, kv_seq_stride=big)
    assert call(lib, d, sparse=True) == B.MLA_ERR_INVALID


def test_workspace_too_small(lib):
    d = _dims(num_q=16, num_heads=64, max_kv_len=65552, kv_rows=65552, kv_seq_stride=65552)
    need = mv.workspace_bytes(d)
    assert need > 0
    assert call(lib, d) == B.MLA_ERR_WORKSPACE
    assert call(lib, d, ws=ctypes.c_void_p(0x100000), ws_bytes=need - 1) == B.MLA_ERR_WORKSPACE
    assert call(lib, d, ws=ctypes.c_void_p(0x100008), ws_bytes=need) == B.MLA_ERR_WORKSPACE


def test_plan_shapes():
    # long-prefix verify: 8 row blocks x 32 splits = one workgroup per CU on 256 CUs
    d = _dims(num_q=16, num_heads=64, max_kv_len=65552, kv_rows=65552, kv_seq_stride=65552)
    p = mv.plan(d)
    assert (p.row_blocks, p.num_groups, p.rows_per_group) == (8, 1, 1024)
    assert p.num_splits * p.chunk_tiles >= 1025 > (p.num_splits - 1) * p.chunk_tiles
    assert p.split_slots == p.num_splits == 32
    assert p.workspace_bytes == p.split_slots * 8 * 4 * (32 * 512 * 2 + 3 * 32 * 4)
    # tiny chain: one split, no workspace
    p1 = mv.plan(_dims())
    assert p1.num_splits == 1 and p1.workspace_bytes == 0
    # sparse decode: groups are tokens, rows are heads
    d5 = _dims(batch=32, num_q=1, num_heads=64, topk=2048, max_kv_len=131072,
               kv_rows=32 * 131072, kv_seq_stride=131072)
    p5 = mv.plan(d5, sparse=True)
    assert (p5.num_groups, p5.rows_per_group, p5.row_blocks) == (32, 64, 1)
    # a single sequence takes exactly the requested splits (capped at its tiles),
    # its tiles spread evenly: 10 tiles over 7 splits are 3 x 2 + 4 x 1
    p5b = mv.plan(_dims(num_splits=7, max_kv_len=640, kv_rows=640, kv_seq_stride=640))
    assert (p5b.num_splits, p5b.chunk_tiles) == (7, 2)
    p7 = mv.plan(_dims(num_splits=7, max_kv_len=896, kv_rows=896, kv_seq_stride=896))
    assert p7.num_splits == 7 and p7.chunk_tiles == 2
    p8 = mv.plan(_dims(num_splits=50))
    assert p8.num_splits == 3  # 132 keys = 3 tiles


def test_plan_single_sequence_fewest_splits_of_the_shortest_chunk():
    # Kimi-like verify (65 tiles, 8 row blocks, at most 32 slots): no split can
    # hold fewer than 3 tiles at most, and 22 splits of at most 3 reach that
    # (32 splits of 2-3 would only add partials to write and combine)
    d = _dims(num_q=16, num_heads=64, max_kv_len=4112, kv_rows=4112, kv_seq_stride=4112)
    p = mv.plan(d)
    assert (p.row_blocks, p.split_slots, p.num_splits, p.chunk_tiles) == (8, 22, 22, 3)
    assert p.workspace_bytes == 22 * 8 * 4 * (32 * 512 * 2 + 3 * 32 * 4)
    # a requested count is taken as it is (capped at the tiles)
    p2 = mv.plan(_dims(num_q=16, num_heads=64, max_kv_len=4112, kv_rows=4112,
                       kv_seq_stride=4112, num_splits=32))
    assert (p2.num_splits, p2.chunk_tiles) == (32, 3)


def _plan_tuple(d, sparse=False):
    p = mv.plan(d, sparse=sparse)
    return (p.num_splits, p.chunk_tiles, p.row_blocks, p.num_groups, p.rows_per_group,
            p.split_slots, p.workspace_bytes)


PLAN_DIMS = [
    (dict(num_q=16, num_heads=64, max_kv_len=65552, kv_rows=65552, kv_seq_stride=65552), False),
    (dict(batch=8, num_q=8, num_heads=64, max_kv_len=30186, kv_rows=8 * 30186,
          kv_seq_stride=30186), False),
    (dict(batch=32, num_q=1, num_heads=64, topk=2048, max_kv_len=131072,
          kv_rows=32 * 131072, kv_seq_stride=131072), True),
]


def test_plan_is_a_function_of_dims_only():
    """The plan (and so the workspace size) makes no HIP call: a process whose
    HIP runtime sees no device at all plans exactly as this one does."""
    import json
    import subprocess
    import sys

    here = [_plan_tuple(_dims(**kw), sparse=sp) for kw, sp in PLAN_DIMS]
    code = (
        "import json, sys; sys.path.insert(0, %r)\n"
        "from tests.test_abi_host import PLAN_DIMS, _plan_tuple, _dims\n"
        "print(json.dumps([_plan_tuple(_dims(**kw), sparse=sp) for kw, sp in PLAN_DIMS]))\n"
    ) % (os.path.dirname(os.path.dirname(os.path.abspath(__file__))),)
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                         timeout=120)
    assert res.returncode == 0, res.stderr
    assert json.loads(res.stdout.strip().splitlines()[-1]) == [list(t) for t in here]
    # and every figure follows from the dims alone (256 compute units)
    assert here[0][:6] == (32, 33, 8, 1, 1024, 32)
    assert here[1][5] == 64 and here[2][:6] == (8, 4, 1, 32, 64, 256)


def test_plan_ragged_batch_slots():
    # A ragged batch gets slots for one workgroup per CU; the kernels share them
    # out by the actual lengths, so the plan no longer multiplies by the batch.
    d = _dims(batch=8, num_q=8, num_heads=64, max_kv_len=30186, kv_rows=8 * 30186,
              kv_seq_stride=30186)
    p = mv.plan(d)
    assert (p.row_blocks, p.num_groups) == (4, 8)
    assert p.split_slots == 64  # 256 CUs / 4 row blocks
    # records, then one (first slot, splits) pair per sequence for the combine
    assert p.workspace_bytes == 64 * 4 * 4 * (32 * 512 * 2 + 3 * 32 * 4) + 8 * 8
    # a requested split count is per sequence
    p2 = mv.plan(_dims(batch=8, num_q=8, num_heads=64, max_kv_len=30186, kv_rows=8 * 30186,
                       kv_seq_stride=30186, num_splits=3))
    assert (p2.num_splits, p2.split_slots) == (3, 24)
    # never fewer slots than sequences
    p3 = mv.plan(_dims(batch=300, num_q=4, num_heads=64, max_kv_len=5000,
                       kv_rows=300 * 5000, kv_seq_stride=5000))
    assert p3.split_slots >= 300


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, 99):
        assert isinstance(lib.mla_verify_strerror(code), bytes)
    assert mv.strerror(B.MLA_ERR_WORKSPACE) == "workspace missing or too small"


def test_compact_invalid_arguments(lib):
    d = _dims(batch=2, num_q=4, max_kv_len=132, kv_rows=264, kv_seq_stride=132)
    ok = dict(c=P(), r=P(), pt=None, kv=P(), acc=P(), n=P(), new=P())

    def call_c(dims, **kw):
        p = dict(ok, **kw)
        return lib.mla_compact_kv(ctypes.byref(dims) if dims is not None else None, p["c"], p["r"],
                                  p["pt"], p["kv"], p["acc"], p["n"], p["new"], None)

    assert call_c(None) == B.MLA_ERR_INVALID
    for k in ("c", "r", "kv", "acc", "n", "new"):
        assert call_c(d, **{k: None}) == B.MLA_ERR_INVALID, k
    assert call_c(d, c=MIS()) == B.MLA_ERR_INVALID
    assert call_c(d, pt=P()) == B.MLA_ERR_INVALID  # page table without a page size
    assert call_c(_dims(batch=2, num_q=65, max_kv_len=132, kv_rows=264, kv_seq_stride=132)) == \
        B.MLA_ERR_INVALID


def test_topk_and_projection_invalid_arguments(lib):
    f = lib.mla_select_topk
    assert f(0, 100, 100, 8, P(), None, P(), None, 0, None) == B.MLA_ERR_INVALID   # no rows
    assert f(2, 100, 99, 8, P(), None, P(), None, 0, None) == B.MLA_ERR_INVALID    # stride < length
    assert f(2, 98, 98, 8, P(), None, P(), None, 0, None) == B.MLA_ERR_INVALID     # stride % 4
    assert f(2, 100, 100, 0, P(), None, P(), None, 0, None) == B.MLA_ERR_INVALID   # k = 0
    assert f(2, 100, 100, 8, None, None, P(), None, 0, None) == B.MLA_ERR_INVALID
    assert f(2, 100, 100, 8, FakePtr(0x10004)(), None, P(), None, 0, None) == B.MLA_ERR_INVALID
    assert f(2, 100000, 100000, 8, P(), None, P(), MIS(), 1 << 30, None) == B.MLA_ERR_INVALID
    # rows long enough to be split over workgroups need the whole workspace
    assert f(2, 100000, 100000, 8, P(), None, P(), P(), 16, None) == B.MLA_ERR_WORKSPACE
    g = lib.mla_head_project
    assert g(4, 2, 24, 64, P(), P(), P(), None) == B.MLA_ERR_INVALID          # in_dim % 16
    assert g(4, 2, 32, 48, P(), P(), P(), None) == B.MLA_ERR_INVALID          # out_dim % 32
    assert g(4, 2, 2048, 64, P(), P(), P(), None) == B.MLA_ERR_INVALID        # in_dim > 1024
    assert g(0, 2, 32, 64, P(), P(), P(), None) == B.MLA_ERR_INVALID
    assert g(4, 2, 32, 64, MIS(), P(), P(), None) == B.MLA_ERR_INVALID


def test_topk_workspace_bytes(lib):
    w = lib.mla_select_topk_workspace_bytes
    # at most 32 pieces: per piece 256 bins + 4 counts (4 B each) and a 16-byte
    # digit-0 record, and entry room for every score plus one 1024-score step
    # per piece (8 B each)
    assert w(32, 131072) == 32 * 32 * 1056 + 32 * (131072 + 32 * 1024) * 8
    assert w(1, 4096) == 0          # one piece: no workspace
    assert w(3, 9000) == 3 * 3 * 1056 + 3 * (9000 + 3 * 1024) * 8
    assert w(0, 100) == 0 and w(2, 0) == 0


def test_probe_invalid_arguments(lib):
    sink = ctypes.c_void_p(0x10000)
    for blocks, iters, s in ((0, 1, sink), (65537, 1, sink), (1, 0, sink), (1, 1000001, sink),
                             (1, 1, None), (1, 1, ctypes.c_void_p(0x10002))):
        assert lib.mla_probe_mfma_bf16(blocks, iters, s, None) == B.MLA_ERR_INVALID


def test_gather_probe_invalid_arguments(lib):
    P16 = ctypes.c_void_p(0x10000)
    ok = dict(c=P16, r=P16, rows=100, stride=10, idx=P16, g=2, k=64, t=1, s=P16)
    for bad in (dict(c=None), dict(r=ctypes.c_void_p(0x10008)), dict(idx=ctypes.c_void_p(0x10002)),
                dict(s=None), dict(rows=0), dict(stride=-1), dict(g=0), dict(k=0), dict(t=0)):
        a = {**ok, **bad}
        rc = lib.mla_probe_gather_rows(a["c"], a["r"], a["rows"], a["stride"], a["idx"], a["g"], a["k"],
                                       a["t"], a["s"], None)
        assert rc == B.MLA_ERR_INVALID, bad


def test_noalloc_rejects_calls_beyond_its_scratch(lib):
    """A call whose partials exceed the fixed 64 MiB device scratch is refused
    with MLA_ERR_SCRATCH before any HIP call (300 sequences x 2 row blocks x
    4 records of 33,152 bytes = 79.6 MB); its workspace twin would accept it
    with a large enough workspace."""
    d = _dims(batch=300, num_q=4, num_heads=64, max_kv_len=5000, kv_rows=300 * 5000,
              kv_seq_stride=5000)
    need = mv.workspace_bytes(d)
    assert need > B.NOALLOC_SCRATCH_BYTES
    p = P()
    rc = lib.mla_verify_attn_noalloc(ctypes.byref(d), p, p, p, p, None, None, p,
                                     ctypes.c_float(0.1), p, p, None)
    assert rc == B.MLA_ERR_SCRATCH
    assert "scratch" in mv.strerror(B.MLA_ERR_SCRATCH)
    # invalid arguments are still MLA_ERR_INVALID first
    rc = lib.mla_verify_attn_noalloc(ctypes.byref(d), None, p, p, p, None, None, p,
                                     ctypes.c_float(0.1), p, p, None)
    assert rc == B.MLA_ERR_INVALID
