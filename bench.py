"""Benchmark of the block-sparse attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

A step is one pass of the whole path over one batch: build the BlockMask
(classification + schedule kernels) and run the fused forward, on the causal
S=8192 workload (B=1, H=8, E=64, bf16, i.i.d. N(0,1) inputs). W untimed
steps, then K steps timed between two device synchronisations. The forward
kernel is also timed alone with events on the stream it runs on (batches of
back-to-back launches), for the roofline figure. The second headline workload (sliding window 256
over S=32768) is measured the same way and reported in the same line, and so
are the mask and head-sharing variants (bottom-right causal, grouped-query
heads, bidirectional documents, key padding, split-KV / packed-row decode,
and a user-supplied dense mask) under "workloads".

The backward (dq, dk, dv after one forward) of the causal workload is timed
the same way and reported under "backward" (10 E flops per live pair).

Prints one JSON line. ``value`` is live-pair TFLOPS of the whole step
(4 * E flops per unmasked (query, key) pair); ``forward_only`` has the
forward kernel alone, which is what the FlexAttention-on-MPS table times.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_sparse_attention_35_amd as bsa  # noqa: E402
import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "ms/forward and live-pair TFLOPS (% bf16 MFMA peak), S=8192 causal & S=32768 W=256"
HEADLINE = "causal_8192_bf16"
SECOND = "sliding_32768_w256_bf16"
# Mask and head-sharing variants of the same kernel, reported in "workloads".
VARIANTS = ("causal_lower_right_2048x8192_bf16", "gqa_causal_8192_h32_kv8_bf16",
            "document_bidirectional_8192_f16_softcap", "causal_8192_keypad_b2_bf16",
            "decode_gqa_b8_h32_kv8_s8192_bf16", "custom_blocks_8192_bf16")
# The other configurations of the method's workloads (the fp32 accuracy case,
# the window sweep at S=8192, documents with the soft-cap), timed the same way.
CONFIGS = ("causal_256_f32", "sliding_8192_w64_bf16", "sliding_8192_w256_bf16", "sliding_8192_w1024_bf16",
           "sliding_8192_w4096_bf16", "document_8192_f16_softcap")


def padded_causal_pairs(L: int, start: int, end: int) -> int:
    """Causal pairs (j <= i) of L queries whose keys are limited to
    [start, end): query i has max(0, min(i, end - 1) - start + 1) keys."""
    i = np.arange(L, dtype=np.int64)
    return int(np.maximum(0, np.minimum(i, end - 1) - start + 1).sum())


def live_pairs(w: wl.Workload) -> int:
    """Live (query, key) pairs of one head (averaged over the batch when
    the key padding differs per entry) from the closed forms of the rules."""
    L, S = w.L, w.S
    if w.key_ranges:
        if w.kind != wl.MASK_CAUSAL or L != S:
            raise ValueError("no closed form for this padded workload")
        return sum(padded_causal_pairs(L, a, b) for a, b in w.key_ranges) // w.B
    if w.kind == wl.MASK_CAUSAL and L == S:
        return S * (S + 1) // 2
    if w.kind == wl.MASK_SLIDING_WINDOW and L == S and w.window <= S:
        W = w.window
        return W * S - W * (W - 1) // 2
    if w.kind == wl.MASK_DOCUMENT and L == S:
        edges = [0, *w.doc_bounds, S]
        return sum((b - a) * (b - a + 1) // 2 for a, b in zip(edges[:-1], edges[1:]))
    if w.kind == wl.MASK_NONE:
        return L * S
    if w.kind == wl.MASK_CAUSAL_LOWER_RIGHT:
        # query i sees keys 0 .. i + S - L
        return L * (S - L + 1) + L * (L - 1) // 2 if L <= S else S * (S + 1) // 2
    if w.kind == wl.MASK_SLIDING_WINDOW_LOWER_RIGHT:
        return sum(min(w.window, i + S - L + 1) for i in range(L) if i + S - L >= 0)
    if w.kind == wl.MASK_DOCUMENT_BIDIRECTIONAL and L == S:
        edges = [0, *w.doc_bounds, S]
        return sum((b - a) ** 2 for a, b in zip(edges[:-1], edges[1:]))
    if w.kind == wl.MASK_CUSTOM:
        return int(wl.make_mask(w).sum())  # the pairs the user mask keeps
    raise ValueError("no closed form for this workload")


def algorithmic_bytes(w: wl.Workload) -> int:
    """Read Q, K, V once, write O once and the fp32 logsumexp (K and V have
    kv_heads heads)."""
    esize = {"f32": 4, "bf16": 2, "f16": 2}[w.dtype]
    n, nkv = w.B * w.H, w.B * w.kv_heads
    return (n * w.L * w.E * 2 + nkv * w.S * w.E * 2) * esize + n * w.L * 4


def run_workload(w: wl.Workload, steps: int, warmup: int, dev, use_graph: bool = False):
    q, k, v = (x.to(dev) for x in wl.make_qkv(w, 0))
    doc = wl.make_doc(w)
    doc_t = torch.from_numpy(doc).to(dev) if doc is not None else None
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.L, dtype=torch.float32, device=dev)
    if w.kind == wl.MASK_CUSTOM:
        # the user mask is packed once; a step rebuilds the BlockMask from its bits
        bm = bsa.create_block_mask_from_dense(torch.from_numpy(wl.make_mask(w)).to(dev))
    else:
        bm = bsa.create_block_mask(w.kind, w.L, w.S, window=w.window or None, document_id=doc_t,
                                   device=dev)
    score_mod = "softcap" if w.softcap else None
    ks = ke = None
    if w.key_ranges:
        ks = torch.tensor([a for a, _ in w.key_ranges], dtype=torch.int32, device=dev)
        ke = torch.tensor([b for _, b in w.key_ranges], dtype=torch.int32, device=dev)

    # an explicit zero-filled workspace, so nothing is allocated inside a graph
    nws = bsa.workspace_size(q, bm)
    ws = torch.zeros(nws, dtype=torch.uint8, device=dev) if nws > 0 else None

    def step():
        bm.rebuild()
        bsa.attention(q, k, v, bm, score_mod=score_mod, softcap=w.softcap or 30.0,
                      scale=w.scale, out=o, lse=lse, key_start=ks, key_end=ke, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # The step's two launches (mask build, forward) captured once in a HIP
    # graph and replayed; a replay must give the eager step's bits.
    replay, timing = step, "eager"
    if use_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        o_graph, lse_graph = o.clone(), lse.clone()
        step()
        torch.cuda.synchronize()
        if not (torch.equal(o, o_graph) and torch.equal(lse, lse_graph)):
            raise RuntimeError(f"{w.name}: graph replay differs from the eager step")
        replay, timing = g.replay, "graph"
        for _ in range(warmup // 4):
            replay()
        torch.cuda.synchronize()

    # Timed region: exactly `steps` whole steps between two synchronisations.
    t0 = time.perf_counter()
    for _ in range(steps):
        replay()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps

    # Per-launch durations with events on the stream the kernels run on: the
    # mask build alone, and the forward alone as back-to-back batches of
    # launches (so host launch gaps between steps are not counted).
    stream = torch.cuda.current_stream(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        bm.rebuild()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    mask_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    def fwd():
        bsa.attention(q, k, v, bm, score_mod=score_mod, softcap=w.softcap or 30.0,
                      scale=w.scale, out=o, lse=lse, key_start=ks, key_end=ke, workspace=ws)

    # Each timed batch is queued behind two untimed launches, so the host
    # stays ahead of the GPU and no host-side pause lands between the events;
    # the garbage collector is off while the batches are queued.
    batch = 10
    events = []
    gc.disable()
    try:
        for _ in range(max(1, steps // batch)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            fwd()
            fwd()
            e0.record(stream)
            for _ in range(batch):
                fwd()
            e1.record(stream)
            events.append((e0, e1))
        torch.cuda.synchronize()
    finally:
        gc.enable()
    fwd_ms = np.array([a.elapsed_time(b) / batch for a, b in events])
    return dict(wall_ms=wall_ms, mask_ms=mask_ms, fwd_ms=fwd_ms, timing=timing)


_KIND_LABEL = {wl.MASK_NONE: "none", wl.MASK_CAUSAL: "causal", wl.MASK_SLIDING_WINDOW: "sliding_window",
               wl.MASK_DOCUMENT: "document", wl.MASK_CAUSAL_LOWER_RIGHT: "causal_lower_right",
               wl.MASK_SLIDING_WINDOW_LOWER_RIGHT: "sliding_window_lower_right",
               wl.MASK_DOCUMENT_BIDIRECTIONAL: "document_bidirectional", wl.MASK_CUSTOM: "custom"}


def forward_kernel_label(w: wl.Workload) -> str:
    """The forward kernel a workload's launch runs, as a kernel trace names it:
    fp32 has its own kernel; at most 32 query rows per K/V head (L times the
    heads sharing it) run packed; sliding windows of at most 15 blocks with at
    least 1024 work items (B*H*query blocks) run the chained form."""
    kind = _KIND_LABEL[w.kind]
    if w.dtype == "f32":
        return f"fwd32_kernel<{kind}>"
    if w.L >= 1 and w.L * (w.H // (w.H_kv or w.H)) <= 32:
        return f"packed_kernel<{w.dtype}, {kind}>"
    chained = (w.kind in (wl.MASK_SLIDING_WINDOW, wl.MASK_SLIDING_WINDOW_LOWER_RIGHT)
               and w.window <= 15 * 128 and w.B * w.H * -(-w.L // 128) >= 1024)
    return f"{'fwd16_chain_kernel' if chained else 'fwd16_kernel'}<{w.dtype}, {kind}>"


def roofline(w: wl.Workload, r, traffic):
    """Roofline of the workload's forward kernel: matrix-bound (against the
    MFMA peak of its dtype) when its live flops per algorithmic byte reach the
    peak's flops per byte of HBM bandwidth, else bandwidth-bound."""
    peak_flops = PEAK_FP32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
    out = {"kernel": forward_kernel_label(w), "launch_ms": r["forward_ms"]["mean"]}
    if r["live_gflop"] * 1e9 / r["algorithmic_bytes"] >= peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9):
        out.update(bound="mfma", achieved=r["forward_tflops"], peak=peak_flops, unit="TFLOP/s",
                   frac=r["forward_tflops"] / peak_flops, per_launch_flop=r["live_gflop"] * 1e9)
    else:
        out.update(bound="hbm", achieved=r["forward_gbs"], peak=PEAK_HBM_GBS, unit="GB/s",
                   frac=r["forward_gbs"] / PEAK_HBM_GBS, per_launch_bytes=r["algorithmic_bytes"])
    out["traffic"] = traffic
    return {k: out[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel",
                                "per_launch_flop", "per_launch_bytes", "launch_ms") if k in out}


def run_backward(w: wl.Workload, steps: int, warmup: int, dev):
    """Per-call time of the backward (attn_backward: D and the transposed mask,
    then the dK/dV and dQ kernels) after one forward, in batches of back-to-back
    launches timed with events on the stream they run on."""
    q, k, v = (x.to(dev) for x in wl.make_qkv(w, 0))
    dout = torch.from_numpy(np.random.default_rng(99).standard_normal(
        (w.B, w.H, w.L, w.E), dtype=np.float32)).to(w.torch_dtype).to(dev)
    doc = wl.make_doc(w)
    bm = bsa.create_block_mask(w.kind, w.L, w.S, window=w.window or None,
                               document_id=None if doc is None else torch.from_numpy(doc).to(dev),
                               device=dev)
    sm = "softcap" if w.softcap else None
    o, lse = bsa.attention(q, k, v, bm, score_mod=sm, softcap=w.softcap or 30.0, scale=w.scale,
                           return_lse=True)

    def bwd():
        bsa.attention_backward(q, k, v, o, lse, dout, bm, score_mod=sm, softcap=w.softcap or 30.0,
                               scale=w.scale)

    for _ in range(max(1, warmup // 4)):
        bwd()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    batch, times = 5, []
    gc.disable()
    try:
        events = []
        for _ in range(max(1, steps // (2 * batch))):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            bwd()
            e0.record(stream)
            for _ in range(batch):
                bwd()
            e1.record(stream)
            events.append((e0, e1))
        torch.cuda.synchronize()
        times = [a.elapsed_time(b) / batch for a, b in events]
    finally:
        gc.enable()
    ms = float(np.mean(times))
    # 5 products of 2 E flops per live pair (S, dP, dV, dK, dQ; the second
    # score product of the dQ kernel is recomputation, not counted)
    flops = 10.0 * w.E * live_pairs(w) * w.B * w.H
    return {"workload": w.name, "ms": ms, "min_ms": float(np.min(times)),
            "tflops": flops / (ms * 1e-3) / 1e12,
            "frac_bf16_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def summarize(w: wl.Workload, r):
    flops = 4.0 * w.E * live_pairs(w) * w.B * w.H
    fwd_avg = float(r["fwd_ms"].mean())
    nbytes = algorithmic_bytes(w)
    return {
        "workload": w.name,
        "ms_per_step": r["wall_ms"],
        "step_timing": r["timing"],
        "step_tflops": flops / (r["wall_ms"] * 1e-3) / 1e12,
        "forward_ms": {"mean": fwd_avg, "median": float(np.median(r["fwd_ms"])),
                       "min": float(r["fwd_ms"].min()), "max": float(r["fwd_ms"].max())},
        "forward_tflops": flops / (fwd_avg * 1e-3) / 1e12,
        "forward_frac_bf16_peak": flops / (fwd_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        # fp32 runs on the fp32 MFMA, whose peak is its own
        **({"forward_frac_fp32_peak": flops / (fwd_avg * 1e-3) / 1e12 / PEAK_FP32_TFLOPS}
           if w.dtype == "f32" else {}),
        "forward_gbs": nbytes / (fwd_avg * 1e-3) / 1e9,
        "forward_frac_hbm_peak": nbytes / (fwd_avg * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "dominant_kernel_traffic": measured_traffic(w.name),
        "mask_build_ms": {"mean": float(r["mask_ms"].mean()), "median": float(np.median(r["mask_ms"]))},
        "live_gflop": flops / 1e9,
        "algorithmic_bytes": nbytes,
    }


TRAFFIC_PROFILES = [os.path.join(ROOT, "profiles", f) for f in (
    "fwd16_hbm_traffic_causal_sliding_documents.md",
    "packed_decode_gqa_b8_h32_kv8_s8192_hbm_traffic.md")]
FWD_SOURCE = os.path.join(ROOT, "block_sparse_attention_35_amd", "csrc", "fwd_kernels.h")


def measured_traffic(workload: str):
    """HBM bytes per launch of the workload's dominant kernel from the
    committed rocprofv3 counter summaries, or None when the forward source has
    changed since they were taken."""
    try:
        src_hash = hashlib.sha256(open(FWD_SOURCE, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    for path in TRAFFIC_PROFILES:
        try:
            text = open(path).read()
        except OSError:
            continue
        for line in text.splitlines():
            if line.startswith("traffic-bytes "):
                fields = dict(f.split("=", 1) for f in line.split()[1:])
                if fields.get("source") == src_hash and workload in fields:
                    return int(fields[workload])
    return None


# The method's configurations (the oracle is timed on each of them).
ORACLE_CONFIGS = ("causal_256_f32", HEADLINE, "sliding_8192_w64_bf16", "sliding_8192_w256_bf16",
                  "sliding_8192_w1024_bf16", "sliding_8192_w4096_bf16", SECOND, "document_8192_f16_softcap")


def live_in_rows(w: wl.Workload, rows: np.ndarray) -> int:
    """Live (query, key) pairs of the given flat rows (b*H + h)*L + i, for
    the rule kinds of the method's configurations (L == S)."""
    i = (rows % w.L).astype(np.int64)
    if w.kind == wl.MASK_CAUSAL:
        return int((i + 1).sum())
    if w.kind == wl.MASK_SLIDING_WINDOW:
        return int(np.minimum(i + 1, w.window).sum())
    if w.kind == wl.MASK_DOCUMENT:
        starts = np.array([0, *w.doc_bounds], dtype=np.int64)
        first = starts[np.searchsorted(starts, i, side="right") - 1]
        return int((i - first + 1).sum())
    raise ValueError("no per-row live count for this workload")


def oracle_timing(w: wl.Workload, budget_s: float):
    """The fp64 oracle on a bounded, seeded sample of the workload's rows.
    It evaluates every key of a row (the plain definition: scores of masked
    pairs are computed, then replaced by -inf), so it is credited both with
    the live pairs of the rows (the GPU metric's unit) and with all L*S
    pairs it computes (dense rate)."""
    import oracle

    q, k, v = wl.make_qkv(w, 0)
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    doc = wl.make_doc(w)
    rng = np.random.default_rng(7)
    n_rows = w.B * w.H * w.L
    probe = rng.choice(n_rows, size=min(64, n_rows), replace=False)
    t0 = time.perf_counter()
    oracle.attention(qd, kd, vd, w.kind, w.scale, w.window, doc, w.softcap, rows=probe)
    per_row = (time.perf_counter() - t0) / probe.size
    count = int(min(n_rows, max(64, budget_s / max(per_row, 1e-9))))
    rows = np.arange(n_rows) if count >= n_rows else np.sort(rng.choice(n_rows, size=count, replace=False))
    t0 = time.perf_counter()
    oracle.attention(qd, kd, vd, w.kind, w.scale, w.window, doc, w.softcap, rows=rows)
    secs = time.perf_counter() - t0
    live_flops = 4.0 * w.E * live_in_rows(w, rows)
    dense_flops = 4.0 * w.E * w.S * rows.size
    return {"workload": w.name, "rows": int(rows.size), "of_rows": n_rows, "seconds": secs,
            "projected_full_seconds": secs * n_rows / rows.size,
            "live_tflops": live_flops / secs / 1e12, "dense_tflops": dense_flops / secs / 1e12}


def cpu_baseline(budget_s: float):
    """The oracle timed on every configuration of the method (a bounded
    sample of rows each); the headline entry is the causal workload's, in the
    metric's unit (live-pair TFLOPS)."""
    import oracle

    per = {}
    for n in ORACLE_CONFIGS:
        print(f"bench: oracle {n} ...", file=sys.stderr, flush=True)
        per[n] = oracle_timing(wl.WORKLOADS[n], budget_s / len(ORACLE_CONFIGS))
    h = per[HEADLINE]
    return {"value": h["live_tflops"], "unit": "TFLOPS (live pairs)", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{h['rows']} of {h['of_rows']} query rows of {HEADLINE} drawn uniformly "
                      f"(seed 7), fp64, {h['seconds']:.1f} s wall; every other configuration "
                      f"timed the same way under per_config (about {budget_s / len(ORACLE_CONFIGS):.1f} s each)",
            "dense_tflops": h["dense_tflops"], "seconds": h["seconds"], "per_config": per}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as a replayed HIP graph (slower here than separate launches)")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of oracle time over all configurations")
    ap.add_argument("--workloads", default=",".join((HEADLINE, SECOND) + VARIANTS + CONFIGS))
    ap.add_argument("--backward", default=HEADLINE,
                    help="workloads whose backward is timed too (comma list; empty for none)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size "
                         "kernel that scales HBM traffic counters in profiler runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path runs on a single MI355X; heads are independent, so several GPUs "
              "would each take a share of the heads with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    names = args.workloads.split(",")
    results = {}
    for n in names:
        w = wl.WORKLOADS[n]
        print(f"bench: {n} ...", file=sys.stderr, flush=True)
        results[n] = summarize(w, run_workload(w, args.steps, args.warmup, dev, use_graph=args.graph))
        print(f"bench: {n} forward {results[n]['forward_ms']['mean']:.4f} ms "
              f"{results[n]['forward_tflops']:.1f} TFLOPS", file=sys.stderr, flush=True)

    backward = {}
    for n in [x for x in args.backward.split(",") if x]:
        print(f"bench: {n} backward ...", file=sys.stderr, flush=True)
        backward[n] = run_backward(wl.WORKLOADS[n], args.steps, args.warmup, dev)
        print(f"bench: {n} backward {backward[n]['ms']:.4f} ms {backward[n]['tflops']:.1f} TFLOPS",
              file=sys.stderr, flush=True)

    head = results[names[0]]
    w = wl.WORKLOADS[names[0]]
    line = {
        "metric": METRIC,
        "value": head["step_tflops"],
        "unit": "TFLOPS (live pairs, whole step: mask build + forward)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded i.i.d. N(0,1) q/k/v rounded to the workload dtype",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "S": w.S, "E": w.E,
                   "mask": _KIND_LABEL[w.kind], "block": 128, "scale": w.scale},
        "frac_bf16_peak": head["step_tflops"] / PEAK_BF16_TFLOPS,
        "forward_only": {"ms": head["forward_ms"], "tflops": head["forward_tflops"],
                         "frac_bf16_peak": head["forward_frac_bf16_peak"]},
        "mask_build_ms": head["mask_build_ms"],
        "roofline": roofline(w, head, measured_traffic(names[0])),
        "workloads": results,
        "backward": backward,
    }
    if SECOND in results:
        s = results[SECOND]
        line["sliding_32768_w256"] = {
            "forward_ms": s["forward_ms"], "tflops": s["forward_tflops"],
            "frac_bf16_peak": s["forward_frac_bf16_peak"], "gbs": s["forward_gbs"],
            "frac_hbm_peak": s["forward_gbs"] / PEAK_HBM_GBS, "step_ms": s["ms_per_step"],
            "traffic": measured_traffic(SECOND),
            "roofline": roofline(wl.WORKLOADS[SECOND], s, measured_traffic(SECOND))}
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
