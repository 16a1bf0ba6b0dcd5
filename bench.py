#!/usr/bin/env python3
"""Benchmark of the MLA tree-verify attention call on one MI355X.

Default workload: long-prefix verify, B=1, H=64 heads, prefix 65,536, T=16
random draft tree (Dl=512 latent + Dr=64 rope, bf16 N(0,1) synthetic inputs).
One "step" is one whole verify call (split-KV kernel + log-sum-exp combine)
with every input already resident in HBM.

Prints ONE JSON line: µs/call (value), achieved HBM GB/s, the split kernel's
roofline position (its average duration from HIP events on the launch
stream), and the fp64 CPU oracle timed on the host as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verify-attn µs/call + achieved HBM GB/s (% of peak), H=64, 64k prefix"
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
LATENT_ROW_BYTES = 512 * 2
ROPE_ROW_BYTES = 64 * 2
KERNEL_SOURCES = ("speculative_decode_verify_mla_amd/csrc/mla_kernels.hip",
                  "speculative_decode_verify_mla_amd/csrc/mla_device.h",
                  "speculative_decode_verify_mla_amd/csrc/mla_api.hip",
                  "speculative_decode_verify_mla_amd/csrc/mla_internal.h")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# The naive kernel the pages measure against ("The Shared Memory Ceiling",
# section "The Guard: Turning a Limitation into a Demonstration"): it holds the
# fp32 query row (Dl + Dr) and the fp32 score row (kv_len) in on-chip memory,
# and its launch is skipped ("n/a") when that exceeds the memory a block gets.
# ---------------------------------------------------------------------------
def naive_score_row_bytes(kv_len: int, dl: int = 512, dr: int = 64) -> int:
    return (dl + dr + int(kv_len)) * 4


def naive_row_fits(kv_len: int, limit_bytes: int) -> bool:
    return naive_score_row_bytes(kv_len) <= limit_bytes


# ---------------------------------------------------------------------------
# Algorithmic work of one call (each visible KV row counted once per sequence)
# ---------------------------------------------------------------------------
def work_model(w):
    import numpy as np

    B, T, H = w.B, w.T, w.H
    rows = B * T * H
    q_bytes = rows * (LATENT_ROW_BYTES + ROPE_ROW_BYTES)
    out_bytes = rows * LATENT_ROW_BYTES + rows * 4
    if w.layout == "sparse":
        kv_rows = sum(len(np.unique(w.indices[b])) for b in range(B))
        visible = int(np.sum((w.indices >= 0) & (w.indices < w.kv_lens[:, None, None]))) * H
        meta = w.indices.nbytes + w.kv_lens.nbytes
        if w.page_table is not None:
            meta += w.page_table.nbytes
    else:
        kv_rows = int(w.kv_lens.sum())
        prefix = w.kv_lens - T
        visible = int(sum(H * (prefix[b] * T + int(w.tree_mask[b].sum())) for b in range(B)))
        meta = w.kv_lens.nbytes + (0 if w.mask_for_kernel is None else w.tree_mask.nbytes)
        if w.page_table is not None:
            meta += w.page_table.nbytes
    kv_bytes = kv_rows * (LATENT_ROW_BYTES + ROPE_ROW_BYTES)
    flops = 2.0 * visible * (512 + 64 + 512)
    return dict(kv_bytes=kv_bytes, q_bytes=q_bytes, out_bytes=out_bytes, meta_bytes=meta,
                total_bytes=kv_bytes + q_bytes + out_bytes + meta, flops=flops,
                visible_pairs=visible)


# ---------------------------------------------------------------------------
def _oracle_sample(w, budget_s: float):
    """(groups done, wall seconds) of the fp64 oracle cycling over the call's
    (sequence, draft-token) groups for about budget_s seconds."""
    import oracle
    from speculative_decode_verify_mla_amd.synth import bf16_bits_to_f64

    q_lat, q_rope = bf16_bits_to_f64(w.q_lat), bf16_bits_to_f64(w.q_rope)
    c_kv, k_rope = bf16_bits_to_f64(w.c_kv), bf16_bits_to_f64(w.k_rope)
    tokens = [(b, t) for b in range(w.B) for t in range(w.T)]
    done = 0
    t0 = time.perf_counter()
    while True:
        b, t = tokens[done % len(tokens)]
        if w.layout == "sparse":
            sl = (slice(b, b + 1), slice(t, t + 1))
            oracle.verify_sparse(q_lat[sl], q_rope[sl], c_kv, k_rope, w.kv_lens[b:b + 1],
                                 w.indices[b:b + 1, t:t + 1], w.scale,
                                 kv_seq_stride=w.kv_seq_stride,
                                 page_table=None if w.page_table is None else w.page_table[b:b + 1],
                                 page_size=w.page_size, row_ids=_rows_of(w, b))
        else:
            _token_oracle(oracle, q_lat, q_rope, c_kv, k_rope, w, b, t)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    return done, time.perf_counter() - t0


def cpu_baseline(w, budget_s: float, single_thread: bool = False):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same call,
    with the BLAS threads it finds; with single_thread, also with one thread."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    ntok = w.B * w.T
    done, el = _oracle_sample(w, budget_s)
    res = dict(value=el / done * ntok * 1e6, unit="us/call", cores=int(threads), kind="oracle",
               sample=f"{done} (sequence, draft-token) groups of {w.H} heads each, cycling "
                      f"through the call's {ntok}, fp64 numpy oracle, {el:.1f} s wall; "
                      f"scaled to one whole call",
               cpu_model=_cpu_model(), host_cpus=os.cpu_count())
    if single_thread:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                d1, e1 = _oracle_sample(w, min(budget_s, 5.0))
            res["single_thread_us_per_call"] = e1 / d1 * ntok * 1e6
            res["single_thread_sample"] = f"{d1} groups, {e1:.1f} s wall, BLAS limited to 1 thread"
        except Exception as e:  # threadpoolctl missing: say so
            res["single_thread_us_per_call"] = None
            res["single_thread_sample"] = f"not measured ({e.__class__.__name__})"
    return res


def _cpu_model():
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess

    try:
        if _profiled():
            raise RuntimeError("no child programs under the profiler")
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                name = line.split(":", 1)[1].strip()
                if name:
                    return name
    except Exception:
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _rows_of(w, b):
    """Materialised-row ids as seen from a one-sequence slice (sequence b becomes 0)."""
    if w.row_ids is None:
        return None
    if w.page_table is not None:
        return w.row_ids
    return w.row_ids - b * w.kv_seq_stride


def _token_oracle(oracle, q_lat, q_rope, c_kv, k_rope, w, b, t):
    """The oracle's own per-token step: visible positions, gather, attend."""
    import numpy as np

    mrow = None if w.mask_for_kernel is None else w.tree_mask[b, t]
    pos = oracle.dense_visible_positions(int(w.kv_lens[b]), w.T, t, mrow)
    if w.page_table is None:
        phys = b * w.kv_seq_stride + pos
    else:
        phys = w.page_table[b][pos // w.page_size].astype(np.int64) * w.page_size + pos % w.page_size
    return oracle.attend(q_lat[b, t], q_rope[b, t], c_kv[phys], k_rope[phys], w.scale)


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3,
                    help="workload of synth.CONFIGS: 1 tiny chain, 2 Kimi-K2-like (4k prefix), "
                         "3 long prefix (64k, the headline), 4 batched paged, 5 sparse top-k, "
                         "6 single-token decode over the 64k prefix")
    ap.add_argument("--copies", type=int, default=0,
                    help="input copies cycled through so repeats miss the 256 MB Infinity Cache "
                         "(0 = enough for twice its size, at least 4)")
    ap.add_argument("--splits", type=int, default=0, help="0 = library's automatic plan")
    ap.add_argument("--spike", type=float, default=0.0,
                    help="long-prefix workload only: plant, in the last tile of every split, a key scoring "
                         "this many nats above the rest for every query row (0 = off)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle CPU work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--op", choices=("verify", "compact", "proj", "topk", "sweep"), default="verify",
                    help="verify: the attention call (default); compact: post-verify KV "
                         "compaction; proj: the per-head projections around it; topk: "
                         "top-k index selection for the sparse path; sweep: the verify call "
                         "over prefixes 1k..64k at T=16 and T=1")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device-to-device copy (hardware counter scale)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the verify call is a "
              f"single-GPU kernel and this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import speculative_decode_verify_mla_amd as mv
    from speculative_decode_verify_mla_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        # A copy kernel of known size: 256 MiB read + 256 MiB written per launch.
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 5 launches of a 268435456-byte device copy")
        return
    mv.load_library()
    log(f"device {torch.cuda.get_device_name(0)}; workload config {args.config}")
    if args.op == "compact":
        bench_compact(args, dev)
        return
    if args.op == "proj":
        bench_proj(args, dev)
        return
    if args.op == "topk":
        bench_topk(args, dev)
        return
    if args.op == "sweep":
        bench_sweep(args, dev)
        return

    w = synth.config(args.config)
    spiked = None
    if args.spike > 0:
        if args.config != 3:
            raise SystemExit("--spike applies to the long-prefix workload (--config 3) only")
        w, spiked = plant_spikes(w, args, args.spike)
    wm = work_model(w)
    log(f"workload {w.spec.name}{' (spiked)' if spiked else ''}: B={w.B} T={w.T} H={w.H} "
        f"kv_lens={w.kv_lens.tolist()[:8]} algorithmic bytes {wm['total_bytes']/1e6:.2f} MB "
        f"flops {wm['flops']:.4e}")
    ncopies = args.copies if args.copies > 0 else auto_copies(wm["total_bytes"], 4)
    vc = VerifyCall(w, dev, ncopies, args.splits)
    log(f"plan: split_slots={vc.info.split_slots} (splits={vc.info.num_splits} chunk_tiles="
        f"{vc.info.chunk_tiles} at max_kv_len) row_blocks={vc.info.row_blocks} groups="
        f"{vc.info.num_groups} workgroups={vc.workgroups} workspace={vc.info.workspace_bytes/1e6:.1f} MB; "
        f"inputs x{ncopies} copies ({ncopies * wm['total_bytes'] / 1e6:.0f} MB of algorithmic bytes)")
    stream = vc.stream
    call = vc.call
    copies = vc.copies
    smi_before = smi_snapshot()

    # ---- ceilings first: the matrix-core probe runs for at least SETTLE_S seconds,
    # which also takes the GPU out of its idle clock state, so the timed calls run
    # at the clock a busy GPU holds (from idle, the first few ms of calls run at
    # ~1.5 GHz instead of ~1.85: 20 calls after 5 warm-up calls measured 161.5
    # instead of 151.3 us on the long-prefix workload) --------------------------
    gather = vc.gather_probe() if w.layout == "sparse" else None
    ceil = measured_ceilings(dev, gather, settle_s=SETTLE_S)
    # host-side gaps of a few ms (allocations, syncs, Python) let the clock fall
    # again, so every timed loop below is enqueued right behind ~15 ms of probe
    # work with no host wait in between
    busy = KeepBusy(dev, stream)

    # ---- warmup -----------------------------------------------------------------------
    busy()
    for i in range(args.warmup):
        call(copies[i % len(copies)])
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} calls)")

    # ---- timed region: K whole calls, inputs cycled across copies -------------------------
    K = args.steps
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        call(copies[i % len(copies)])
    t_end.record(stream)
    # the shader clock right after the timed calls, from a short matrix-core load
    # enqueued behind them (no host gap in between)
    clk = ClockProbe(dev, stream)
    clk.launch()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / K
    clock_after = clk.read()
    log(f"timed {K} calls: {ms_per_step*1e3:.2f} us/call (cold-rotated); shader clock right after: "
        f"{clock_after} GHz")

    # ---- per-call spread (events around each call, outside the timed region) -----------
    evc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    busy()
    for i in range(K):
        evc[i][0].record(stream)
        call(copies[i % len(copies)])
        evc[i][1].record(stream)
    torch.cuda.synchronize()
    per_call = np.sort(np.array([a.elapsed_time(b) * 1e3 for a, b in evc]))
    pct = {f"p{q}": round(float(np.percentile(per_call, q)), 3) for q in (10, 50, 90)}
    log(f"per-call us: {pct}")

    # ---- warm (one copy, Infinity-Cache resident) for context ----------------------------
    busy()
    t_start.record(stream)
    for i in range(K):
        call(copies[0])
    t_end.record(stream)
    torch.cuda.synchronize()
    warm_us = t_start.elapsed_time(t_end) / K * 1e3

    # ---- the same rotated calls replayed from one captured HIP graph -----------------------
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    call(copies[0], st=side)  # warm on the capture stream
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for c in copies:
            call(c, st=side)
    torch.cuda.synchronize()
    reps = max(1, K // len(copies))
    busy()
    t_start.record(stream)
    for _ in range(reps):
        graph.replay()
    t_end.record(stream)
    torch.cuda.synchronize()
    graph_us = t_start.elapsed_time(t_end) / (reps * len(copies)) * 1e3
    log(f"graph replay: {graph_us:.2f} us/call ({reps} replays of {len(copies)} calls)")
    del graph

    # ---- four calls in flight on four streams (own outputs and workspaces) -----------------
    streams4_us = vc.streams_throughput(4, K, busy)
    log(f"4 streams: {streams4_us:.2f} us per call ({K} calls dealt over 4 streams)")

    # ---- per-kernel durations: back-to-back launches of each phase between two events -------
    # on the launch stream (the rotated copies as in the timed region); each average
    # is one launch's duration plus the gap to the next launch on the same queue
    busy()
    t_start.record(stream)
    for i in range(K):
        call(copies[i % len(copies)], mv.binding.PHASE_PARTIAL)
    t_end.record(stream)
    torch.cuda.synchronize()
    split_ms = t_start.elapsed_time(t_end) / K
    combine_ms = 0.0
    if vc.info.workspace_bytes > 0:
        busy()
        t_start.record(stream)
        for i in range(K):
            call(copies[i % len(copies)], mv.binding.PHASE_COMBINE)
        t_end.record(stream)
        torch.cuda.synchronize()
        combine_ms = t_start.elapsed_time(t_end) / K
    log(f"split kernel {split_ms*1e3:.2f} us, combine {combine_ms*1e3:.2f} us "
        f"(back-to-back launches, event-timed)")

    # ---- roofline of the dominant (split) kernel ------------------------------------------
    t_hbm = wm["total_bytes"] / (PEAK_HBM_GBPS * 1e9)
    t_mfma = wm["flops"] / (PEAK_BF16_TFLOPS * 1e12)
    split_s = split_ms * 1e-3
    if t_mfma >= t_hbm:
        achieved = wm["flops"] / split_s / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_BF16_TFLOPS,
                    unit="TFLOP/s", frac=round(achieved / PEAK_BF16_TFLOPS, 4))
    else:
        split_bytes = wm["kv_bytes"] + wm["q_bytes"] + wm["meta_bytes"]
        achieved = split_bytes / split_s / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBPS,
                    unit="GB/s", frac=round(achieved / PEAK_HBM_GBPS, 4))
    roof["traffic"] = None if spiked else load_traffic(w.spec.name)
    roof["kernel"] = "mla_split_kernel"
    # The same kernel against what this GPU measurably sustains (measured before
    # the timed calls): a full-load bf16 MFMA loop (matrix-core bound), or for
    # HBM-bound calls the same rows gathered with no compute (sparse) or else a
    # 256 MiB device copy.
    if roof["bound"] == "mfma":
        measured = ceil["mfma_bf16_TFLOPs"]
    else:
        measured = ceil.get("gather_GBps", ceil["copy_GBps"])
    roof["measured_peak"] = measured
    roof["frac_of_measured"] = round(roof["achieved"] / measured, 4)
    smi_after = smi_snapshot()

    value_us = ms_per_step * 1e3
    gbps = wm["total_bytes"] / (value_us * 1e-6) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the fp64 oracle on the host for ~{args.cpu_budget:.0f} s")
        cpu = cpu_baseline(w, args.cpu_budget, single_thread=args.config in (1, 2))

    name = w.spec.name + (f"_spiked{args.spike:g}" if spiked else "")
    line = {
        "metric": METRIC,
        "value": round(value_us, 3),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, random draft tree)",
        "config": {"workload": name, "batch": w.B, "draft_tokens": w.T, "heads": w.H,
                   "prefix": (w.kv_lens - w.T).tolist() if w.layout != "sparse" else None,
                   "kv_lens": w.kv_lens.tolist()[:8] if w.B <= 8 else f"{w.B} x {int(w.kv_lens[0])}",
                   "latent_dim": 512, "rope_dim": 64, "layout": w.layout,
                   "topk": w.topk or None, "split_slots": int(vc.info.split_slots),
                   "workgroups": vc.workgroups, "input_copies": ncopies,
                   "spikes": None if not spiked else {"nats": args.spike, "keys": spiked}},
        "achieved_hbm_GBps": round(gbps, 1),
        "hbm_frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
        "per_call_us": pct,
        "warm_us_per_call": round(warm_us, 3),
        "graph_us_per_call": round(graph_us, 3),
        "streams4_us_per_call": round(streams4_us, 3),
        "split_kernel_us": round(split_ms * 1e3, 3),
        "combine_kernel_us": round(combine_ms * 1e3, 3),
        "algorithmic_bytes": int(wm["total_bytes"]),
        "algorithmic_flops": wm["flops"],
        "roofline": roof,
        "measured_ceilings": ceil,
        "clocks": {"settle_s": SETTLE_S, "shader_GHz_after_timed_calls": clock_after,
                   "shader_GHz_full_mfma_load": ceil.get("probe_clock_GHz"),
                   "smi_before": smi_before, "smi_after": smi_after},
        "cpu_baseline": cpu,
        "kernel_source": kernel_source_hash(),
        "device": device_info(dev),
    }
    print(json.dumps(line), flush=True)


MALL_BYTES = 256 * 2**20  # MI355X Infinity Cache
SETTLE_S = 0.25  # seconds of matrix-core probe before any timed call
MAX_COPIES = 128


def auto_copies(call_bytes, least):
    """Input copies whose algorithmic bytes add up to twice the Infinity Cache,
    so that cycling through them reads from HBM (at least `least`; at most
    MAX_COPIES, which leaves calls of under 4 MB cache-resident)."""
    return int(min(MAX_COPIES, max(least, -(-2 * MALL_BYTES // int(call_bytes)))))


def plant_spikes(w, args, nats):
    """Workload 3 with, in the last tile of every split the plan makes, one key
    scoring `nats` above the rest for every query row (the streaming softmax's
    worst case: its exponent reference must rise in every split)."""
    import speculative_decode_verify_mla_amd as mv
    from speculative_decode_verify_mla_amd import synth

    tiles = -(-int(w.kv_lens[0]) // 64)
    dims = mv.binding.make_dims(batch=1, num_q=w.T, num_heads=w.H, max_kv_len=w.max_kv_len,
                                kv_rows=w.kv_rows, kv_seq_stride=w.kv_seq_stride,
                                num_splits=args.splits)
    n = int(mv.plan(dims).num_splits)
    bounds = [s * tiles // n for s in range(n + 1)]  # the even spread of one sequence's tiles
    return synth.plant_late_spikes(w, bounds, nats)


class VerifyCall:
    """One workload resident on the device in several input copies, with its
    outputs, workspace and a closure that enqueues one whole call."""

    def __init__(self, w, dev, ncopies, splits):
        import numpy as np
        import torch

        import speculative_decode_verify_mla_amd as mv
        from speculative_decode_verify_mla_amd.synth import DL, DR

        self.w, self.dev, self.mv = w, dev, mv

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

        base = {"q_lat": up(w.q_lat), "q_rope": up(w.q_rope)}
        if w.row_ids is None:
            base["c_kv"], base["k_rope"] = up(w.c_kv), up(w.k_rope)
        else:
            base["c_kv"] = torch.full((w.kv_rows, DL), 0x7FC0, dtype=torch.int16, device=dev)
            base["k_rope"] = torch.full((w.kv_rows, DR), 0x7FC0, dtype=torch.int16, device=dev)
            rows = torch.from_numpy(w.row_ids).to(dev)
            base["c_kv"][rows] = up(w.c_kv)
            base["k_rope"][rows] = up(w.k_rope)
        self.copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(ncopies - 1)]
        self.kv_lens = torch.from_numpy(w.kv_lens).to(dev)
        self.mask = None if w.mask_for_kernel is None else torch.from_numpy(w.tree_mask).to(dev)
        self.pt = None if w.page_table is None else torch.from_numpy(w.page_table).to(dev)
        self.idx = None if w.indices is None else torch.from_numpy(w.indices).to(dev)
        self.out = torch.empty((w.B, w.T, w.H, DL), dtype=torch.int16, device=dev)
        self.lse = torch.empty((w.B, w.T, w.H), dtype=torch.float32, device=dev)
        self.kw = dict(max_kv_len=w.max_kv_len, kv_seq_stride=w.kv_seq_stride,
                       page_size=w.page_size, num_splits=splits)
        dims = mv.binding._dims_from(base["q_lat"], base["c_kv"], self.kv_lens, page_table=self.pt,
                                     topk=0 if self.idx is None else self.idx.shape[2], phase=0,
                                     **self.kw)
        self.info = mv.plan(dims, sparse=w.layout == "sparse")
        self.ws = self.new_workspace()
        # split-kernel grid: row blocks x (group, split) slots; dense slots are
        # shared out on the device by the actual kv_lens
        self.workgroups = int(self.info.split_slots) * int(self.info.row_blocks)
        self.stream = torch.cuda.current_stream(dev)

    def new_workspace(self):
        import torch
        return torch.empty(max(int(self.info.workspace_bytes), 16), dtype=torch.uint8, device=self.dev)

    def call(self, c, phase=0, st=None, out=None, lse=None, ws=None):
        mv, w = self.mv, self.w
        st = self.stream if st is None else st
        out = self.out if out is None else out
        lse = self.lse if lse is None else lse
        ws = self.ws if ws is None else ws
        if w.layout == "sparse":
            mv.sparse_attn(c["q_lat"], c["q_rope"], c["c_kv"], c["k_rope"], self.pt, self.idx,
                           self.kv_lens, w.scale, out, lse, workspace=ws, stream=st, phase=phase,
                           **self.kw)
        else:
            mv.verify_attn(c["q_lat"], c["q_rope"], c["c_kv"], c["k_rope"], self.pt, self.mask,
                           self.kv_lens, w.scale, out, lse, workspace=ws, stream=st, phase=phase,
                           **self.kw)

    def streams_throughput(self, n, calls, busy=None):
        """µs per call with `calls` whole calls dealt round-robin over n streams
        (each stream its own outputs and workspace, inputs cycling over the
        copies), from one event on the launch stream before the first and one
        after all streams joined it again."""
        import torch

        streams = [torch.cuda.Stream(self.dev) for _ in range(n)]
        outs = [torch.empty_like(self.out) for _ in range(n)]
        lses = [torch.empty_like(self.lse) for _ in range(n)]
        wss = [self.new_workspace() for _ in range(n)]
        for k in range(n):  # warm each stream once
            self.call(self.copies[k % len(self.copies)], st=streams[k], out=outs[k], lse=lses[k],
                      ws=wss[k])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if busy is not None:
            busy()
        e0.record(self.stream)
        for s in streams:
            s.wait_stream(self.stream)
        for i in range(calls):
            k = i % n
            self.call(self.copies[i % len(self.copies)], st=streams[k], out=outs[k], lse=lses[k],
                      ws=wss[k])
        for s in streams:
            self.stream.wait_stream(s)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / calls * 1e3

    def gather_probe(self):
        """A callable enqueuing the row-gather probe over the call's own rows,
        cycling over the same input copies as the timed calls (so that, like
        them, it reads from HBM); with count=True it also returns the bytes."""
        import torch

        w, mv = self.w, self.mv
        gsink = torch.empty(w.B * w.T * ((w.topk + 63) // 64) * 256, dtype=torch.float32, device=self.dev)
        turn = [0]

        def gather(count=False):
            c = self.copies[turn[0] % len(self.copies)]
            turn[0] += 1
            return mv.probe_gather_rows(c["c_kv"], c["k_rope"], self.idx.reshape(w.B * w.T, -1),
                                        kv_seq_stride=w.kv_seq_stride, tokens_per_seq=w.T,
                                        sink=gsink, stream=self.stream, count=count)
        return gather


class KeepBusy:
    """Enqueues `launches` matrix-core probe launches (~0.6 ms each on one
    workgroup per CU) with no host wait, so work enqueued next starts on a GPU
    that has not idled."""

    def __init__(self, dev, stream, launches=24, iters=2000):
        import torch

        self.blocks = torch.cuda.get_device_properties(dev).multi_processor_count
        self.sink = torch.empty(self.blocks * 256, dtype=torch.float32, device=dev)
        self.stream, self.launches, self.iters = stream, launches, iters

    def __call__(self):
        import speculative_decode_verify_mla_amd as mv
        for _ in range(self.launches):
            mv.probe_mfma_bf16(self.blocks, self.iters, self.sink, stream=self.stream)


class ClockProbe:
    """A short launch of the matrix-core probe (one workgroup per CU) whose
    in-kernel stamps give the shader clock: s_memtime cycles over 100 MHz
    s_memrealtime ticks."""

    def __init__(self, dev, stream, iters=200):
        import torch

        self.blocks = torch.cuda.get_device_properties(dev).multi_processor_count
        self.sink = torch.empty(self.blocks * 256, dtype=torch.float32, device=dev)
        self.stream, self.iters = stream, iters

    def launch(self):
        import speculative_decode_verify_mla_amd as mv
        mv.probe_mfma_bf16(self.blocks, self.iters, self.sink, stream=self.stream)

    def read(self):
        s = self.sink.view(self.blocks, 256)[:, :2].double().sum(dim=0).tolist()
        return round(s[0] / s[1] * 0.1, 3) if s[1] > 0 else None


def _profiled():
    """True under rocprofv3: its preloaded library initialises the GPU in every
    child process too, so no child program may be started then."""
    pre = os.environ.get("LD_PRELOAD", "")
    return "rocprof" in pre or any(k.startswith("ROCPROF") for k in os.environ)


def smi_snapshot():
    """Clocks, power and driver as rocm-smi reports them (JSON), or None
    (also when profiled: see _profiled)."""
    import subprocess

    if _profiled():
        return None
    try:
        res = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--showdriverversion",
                              "--showproductname", "--json"],
                             capture_output=True, text=True, timeout=30)
        d = json.loads(res.stdout)
    except Exception:
        return None
    keep = {}
    for card, vals in d.items():
        if not isinstance(vals, dict):
            continue
        keep[card] = {k: v for k, v in vals.items()
                      if any(x in k.lower() for x in ("clock", "power", "driver", "card series",
                                                        "card model", "gfx", "sku"))}
    return keep or None


def bench_sweep(args, dev):
    """The verify call over prefixes 1k .. 64k, at T=16 (random tree) and T=1,
    H=64, contiguous cache. Beside each figure: the fp32 score row a kernel
    holding the whole row in LDS would need, (512 + 64 + kv_len) x 4 bytes, and
    whether it fits one workgroup's 160 KiB of LDS on this GPU ("n/a" past it)."""
    import numpy as np
    import torch

    from speculative_decode_verify_mla_amd import synth

    lds = 160 * 1024
    measured_ceilings(dev, None, settle_s=SETTLE_S)  # out of the idle clock state first
    busy = KeepBusy(dev, torch.cuda.current_stream(dev))
    rows = []
    for T in (16, 1):
        for L in (1024, 2048, 4096, 8192, 16384, 32768, 65536):
            spec = synth.Spec(f"sweep_t{T}_l{L}", B=1, T=T, H=64, layout="contig", prefix=L)
            w = synth.generate(spec, seed=100 + T)
            wm = work_model(w)
            ncopies = auto_copies(wm["total_bytes"], 2)
            vc = VerifyCall(w, dev, ncopies, 0)
            busy()
            for i in range(args.warmup):
                vc.call(vc.copies[i % ncopies])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(vc.stream)
            for i in range(args.steps):
                vc.call(vc.copies[i % ncopies])
            e1.record(vc.stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / args.steps * 1e3
            naive = naive_score_row_bytes(int(w.kv_lens[0]))
            r = {"T": T, "prefix": L, "us_per_call": round(us, 3),
                 "hbm_GBps": round(wm["total_bytes"] / (us * 1e-6) / 1e9, 1),
                 "TFLOPs": round(wm["flops"] / (us * 1e-6) / 1e12, 1),
                 "splits": int(vc.info.num_splits), "workgroups": vc.workgroups,
                 "naive_score_row_bytes": naive,
                 "naive_row_in_lds": "fits" if naive_row_fits(int(w.kv_lens[0]), lds) else "n/a"}
            log(f"sweep T={T:2d} prefix={L:6d}: {us:9.2f} us  {r['hbm_GBps']:7.1f} GB/s  "
                f"{r['TFLOPs']:7.1f} TFLOP/s  splits={r['splits']}  naive row {naive} B: "
                f"{r['naive_row_in_lds']}")
            rows.append(r)
            del vc
            torch.cuda.empty_cache()
    line = {"metric": "verify-attn µs/call over prefix length (H=64; T=16 tree and T=1)",
            "value": None, "unit": "us/call", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "higher_is_better": False, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) bf16)", "config": {"workload": "prefix_sweep"},
            "sweep": rows, "kernel_source": kernel_source_hash()}
    print(json.dumps(line), flush=True)


def device_info(dev):
    import torch

    p = torch.cuda.get_device_properties(dev)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count,
            "hbm_GiB": round(p.total_memory / 2**30, 1), "hip": torch.version.hip}


def measured_ceilings(dev, gather=None, settle_s=0.0):
    """Best-of-5 rates of (a) the library's matrix-core probe, 16 independent
    bf16 32x32x16 MFMA chains per wave on every CU (with the shader clock its
    in-kernel stamps read), (b) a 256 MiB device-to-device copy (read + write
    bytes) and, when `gather` is given (a call that enqueues the library's
    row-gather probe, and returns its bytes when called with count=True), (c)
    that gather. All are event-timed on the current stream, the copy over 4 and
    the gather over 14 back-to-back launches (cycling over the input copies).
    With settle_s, the matrix-core probe first runs back to back for that many
    seconds."""
    import torch

    import speculative_decode_verify_mla_amd as mv

    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn, reps=5, warm=2, after=None, batch=1):
        """Best of `reps` timings of `batch` back-to-back calls, per call: a
        short kernel timed alone between two events would include the launch
        (several microseconds)."""
        for _ in range(warm):
            fn()
        t = float("inf")
        for _ in range(reps):
            e0.record(stream)
            for _ in range(batch):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            t = min(t, e0.elapsed_time(e1) * 1e-3 / batch)
            if after is not None:
                after()
        return t

    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    iters = 2000
    flops = float(blocks) * 4 * iters * 16 * 2 * 32 * 32 * 16
    clocks = []

    def read_clock():
        s = sink.view(blocks, 256)[:, :2].double().sum(dim=0).tolist()
        if s[1] > 0:
            clocks.append(s[0] / s[1] * 0.1)

    if settle_s > 0:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < settle_s:
            for _ in range(8):
                mv.probe_mfma_bf16(blocks, iters, sink, stream=stream)
            torch.cuda.synchronize()
    t_mfma = best(lambda: mv.probe_mfma_bf16(blocks, iters, sink, stream=stream), after=read_clock)
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    t_copy = best(lambda: dst.copy_(src), batch=4)
    out = {"mfma_bf16_TFLOPs": round(flops / t_mfma / 1e12, 1),
           "probe_clock_GHz": round(max(clocks), 3) if clocks else None,
           "copy_GBps": round(2 * src.numel() / t_copy / 1e9, 1)}
    del src, dst, sink
    if gather is not None:
        nbytes = gather(count=True)
        out["gather_GBps"] = round(nbytes / best(gather, batch=14) / 1e9, 1)
    log(f"measured ceilings: {out}")
    return out


def _time_small_op(fn, steps, warmup, dev):
    """(eager us/call, graph us/call) of a small launch-bound op: eager is
    limited by host enqueue (Python + ctypes), the graph replays `steps`
    captured calls with no host work in between (the kernels' own rate)."""
    import torch

    stream = torch.cuda.current_stream(dev)
    for i in range(warmup):
        fn(i, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        fn(i, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    eager = e0.elapsed_time(e1) / steps * 1e3
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    fn(0, side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for i in range(steps):
            fn(i, side)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    graph = e0.elapsed_time(e1) / steps * 1e3
    del g
    return eager, graph


def bench_compact(args, dev):
    """Post-verify KV compaction on a dense workload: every sequence accepts a
    root-to-node path of a random draft tree (parents drawn like the workload's)."""
    import numpy as np
    import torch

    import speculative_decode_verify_mla_amd as mv
    from speculative_decode_verify_mla_amd import synth

    w = synth.config(args.config)
    if w.layout == "sparse":
        raise SystemExit("--op compact needs a dense (verify) workload")
    rng = np.random.default_rng(1000 + args.config)
    acc = np.full((w.B, w.T), -1, dtype=np.int32)
    nacc = np.zeros(w.B, dtype=np.int32)
    for b in range(w.B):
        parents = synth.random_tree_parents(rng, w.T)
        node, path = int(rng.integers(0, w.T)), []
        while node >= 0:
            path.append(node)
            node = int(parents[node])
        path = path[::-1]
        acc[b, :len(path)] = path
        nacc[b] = len(path)
    u16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    c_kv, k_rope = u16(w.c_kv), u16(w.k_rope)
    kv_lens = torch.from_numpy(w.kv_lens.astype(np.int32)).to(dev)
    pt = None if w.page_table is None else torch.from_numpy(w.page_table.astype(np.int32)).to(dev)
    acc_t, n_t = torch.from_numpy(acc).to(dev), torch.from_numpy(nacc).to(dev)
    new_lens = torch.empty_like(kv_lens)
    stream = torch.cuda.current_stream(dev)

    def call(i, st):
        mv.compact_kv(c_kv, k_rope, pt, kv_lens, acc_t, n_t, new_lens, max_kv_len=w.max_kv_len,
                      kv_seq_stride=w.kv_seq_stride, page_size=w.page_size, stream=st)

    K = args.steps
    eager_us, us = _time_small_op(call, K, args.warmup, dev)
    log(f"compaction: {us:.2f} us/call from a captured graph, {eager_us:.2f} us/call eager")
    moved = int(sum(max(0, min(int(n), w.T)) for n in nacc)) * (LATENT_ROW_BYTES + ROPE_ROW_BYTES)
    alg_bytes = 2 * moved + 4 * w.B * (w.T + 3)  # rows read + written, indices and lengths
    gbps = alg_bytes / (us * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_budget, 5.0):
            oracle.compact_kv(w.c_kv, w.k_rope, w.kv_lens, acc, nacc, w.T, kv_seq_stride=w.kv_seq_stride,
                              page_table=w.page_table, page_size=w.page_size, max_kv_len=w.max_kv_len)
            reps += 1
        el = time.perf_counter() - t0
        cpu = dict(value=el / reps * 1e6, unit="us/call", cores=1, kind="oracle",
                   sample=f"{reps} whole calls of the numpy oracle (it copies the cache once per call)")
    line = {
        "metric": "kv-compaction µs/call (post-verify, accepted path to the front of the draft region)",
        "value": round(us, 3), "unit": "us/call", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "u16", "data": "synthetic (seeded), root-to-node accepted paths",
        "config": {"workload": w.spec.name, "batch": w.B, "draft_tokens": w.T,
                   "accepted": nacc.tolist()},
        "algorithmic_bytes": alg_bytes, "achieved_hbm_GBps": round(gbps, 2),
        "eager_us_per_call": round(eager_us, 3), "timing": "graph replay of the timed calls",
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 5), "traffic": None,
                     "kernel": "mla_compact_kernel"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_proj(args, dev):
    """Query absorption (q_nope . W_UK, 128 -> 512) and per-head output
    (out_lat . W_UV, 512 -> 128) for one verify step of the workload's tokens."""
    import numpy as np
    import torch

    import speculative_decode_verify_mla_amd as mv
    from speculative_decode_verify_mla_amd import synth

    w = synth.config(args.config)
    M, H = w.B * w.T, w.H
    rng = np.random.default_rng(2000 + args.config)
    bf = lambda shape, sc=1.0: torch.from_numpy(synth.f32_to_bf16_bits(
        (rng.standard_normal(shape) * sc).astype(np.float32)).view(np.int16)).to(dev)
    res = {}
    for name, K, N in (("absorb_q", 128, 512), ("head_out", 512, 128)):
        copies = [(bf((M, H, K)), bf((H, K, N), 1 / np.sqrt(K))) for _ in range(max(args.copies, 1))]
        y = torch.empty((M, H, N), dtype=torch.int16, device=dev)

        def call(i, st, copies=copies, y=y):
            mv.head_project(*copies[i % len(copies)], y, stream=st)

        eager_us, us = _time_small_op(call, args.steps, args.warmup, dev)
        nbytes = 2 * (M * H * K + H * K * N + M * H * N)
        res[name] = dict(us=round(us, 3), eager_us=round(eager_us, 3), bytes=nbytes,
                         GBps=round(nbytes / (us * 1e-6) / 1e9, 1), flops=2 * M * H * K * N)
        log(f"{name}: M={M} H={H} {K}->{N}: {us:.2f} us (graph), {eager_us:.2f} us eager, "
            f"{res[name]['GBps']} GB/s")
    tot_us = res["absorb_q"]["us"] + res["head_out"]["us"]
    tot_b = res["absorb_q"]["bytes"] + res["head_out"]["bytes"]
    gbps = tot_b / (tot_us * 1e-6) / 1e9
    line = {
        "metric": "absorbed-MLA projections µs per verify step (q_nope.W_UK + out_lat.W_UV)",
        "value": round(tot_us, 3), "unit": "us/step", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(tot_us / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1))",
        "config": {"workload": w.spec.name, "tokens": M, "heads": H, "copies": len(copies)},
        "timing": "graph replay of the timed calls (weights rotate over the copies)",
        "kernels": res,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None,
                     "kernel": "mla_proj_kernel"},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_topk(args, dev):
    """Top-k selection over one score per cached position, for every query token
    of the sparse workload (by default the sparse top-k one: 32 tokens x 131,072,
    k = 2048)."""
    import numpy as np
    import torch

    import speculative_decode_verify_mla_amd as mv
    from speculative_decode_verify_mla_amd import synth

    cfg = args.config if args.config in (5,) else 5
    w = synth.config(cfg)
    R, L, k = w.B * w.T, int(w.kv_seq_stride), int(w.topk)
    rng = np.random.default_rng(3000 + cfg)
    copies = [torch.from_numpy(rng.standard_normal((R, L)).astype(np.float32)).to(dev)
              for _ in range(max(args.copies, 1))]
    lens = torch.from_numpy(np.repeat(w.kv_lens, w.T).astype(np.int32)).to(dev)
    out = torch.empty((R, k), dtype=torch.int32, device=dev)

    def call(i, st):
        mv.select_topk(copies[i % len(copies)], k, out, row_lens=lens, stream=st)

    def call_one_wg(i, st):
        mv.select_topk(copies[i % len(copies)], k, out, row_lens=lens, split_rows=False, stream=st)

    pieces_ws = mv.topk_workspace_bytes(R, L)
    eager_us, us = _time_small_op(call, args.steps, args.warmup, dev)
    _, one_wg_us = _time_small_op(call_one_wg, args.steps, args.warmup, dev)
    nbytes = R * L * 4 + R * k * 4 + R * 4
    gbps = nbytes / (us * 1e-6) / 1e9
    log(f"top-k: {R} rows x {L}, k={k}: {us:.2f} us (graph), {eager_us:.2f} us eager, {gbps:.0f} GB/s; "
        f"one workgroup per row: {one_wg_us:.2f} us (graph)")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        host = copies[0].cpu().numpy()
        t0 = time.perf_counter()
        oracle.select_topk(host[:4], k, np.repeat(w.kv_lens, w.T)[:4])
        el = time.perf_counter() - t0
        cpu = dict(value=el / 4 * R * 1e6, unit="us/call", cores=1, kind="oracle",
                   sample=f"4 of the {R} rows (numpy lexsort), scaled to the whole call")
    line = {
        "metric": "top-k index selection µs/call (sparse decode indices)", "value": round(us, 3),
        "unit": "us/call", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded N(0,1) scores)",
        "config": {"workload": w.spec.name, "rows": R, "candidates": L, "k": k},
        "eager_us_per_call": round(eager_us, 3), "timing": "graph replay of the timed calls",
        "one_workgroup_per_row_us": round(one_wg_us, 3), "workspace_bytes": int(pieces_ws),
        "algorithmic_bytes": nbytes, "achieved_hbm_GBps": round(gbps, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None,
                     "kernel": "mla_topk_hist_kernel + mla_topk_compact_kernel + mla_topk_place_kernel (whole call)"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def load_traffic(workload: str):
    """HBM traffic per split-kernel launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    try:
        with open(p) as f:
            d = json.load(f)
        if d.get("kernel_source") != kernel_source_hash():
            return None
        return d.get("traffic_bytes")
    except Exception:
        return None


if __name__ == "__main__":
    main()
