#!/usr/bin/env python3
"""KDA prefill benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]

One step is one full KDA layer over the workload: for the segment-path
workloads (default: 131,072 tokens, H=32, d=128, bf16, 16 leveled segments,
Blelloch scan, checkpoints every 4096 tokens) package -> scan -> fix-up
writing the checkpoint rungs; for the chunked workloads one kda_prefill call.  Inputs are
seeded synthetic tensors already resident in HBM when timing starts.

Prints one JSON line with tokens/s per layer, the dominant kernel's roofline
(algorithmic bytes over its HIP-event-timed duration against 8 TB/s HBM), the
chunked form's algorithmic MFMA fraction, the fp64 oracle timed on a bounded
sample on the host cores, and (under "decode") the one-token decode kernel on
a 64-sequence batch against its own HBM roofline.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def chunk_flops_per_token_head(C: int, dk: int, dv: int) -> float:
    """Algorithmic flops of the chunkwise form per token and head (triangles
    exploited): Gram A and P, UT inverse, W and U~, and the three state
    products U = U~ - W S, O = Qbar S + P U, S <- gamma S + Kbar^T U."""
    gram = dk * (C - 1) + dk * (C + 1)
    wy = (C + 1) * dk + (C + 1) * dv
    inv = C * C / 3.0
    state = 2 * dk * dv * 3 + (C + 1) * dv
    return gram + wy + inv + state


def bytes_per_token_head(dk: int, dv: int, io_bytes: int) -> int:
    """q, k, v, o in the I/O dtype, g and beta in fp32."""
    return io_bytes * (2 * dk + 2 * dv) + 4 * dk + 4


def recorded_traffic(workload: str, kernel_mode: str, entry: str | None = None):
    """HBM bytes per launch of a kernel from profiles/hbm_traffic.json (two
    rocprofv3 --pmc runs, FETCH_SIZE and WRITE_SIZE, each scaled by what the
    same counter reads for a plain copy of known size), or None when that
    record is for another workload or the kernel's sources changed since.
    `entry` selects a nested record (e.g. "decode")."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if entry is not None:
        rec = rec.get(entry, {})
    if rec.get("workload") != workload or kernel_mode not in rec.get("kernel", ""):
        return None
    h = hashlib.sha256()
    for p in rec["sources"]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return rec["traffic_bytes"] if h.hexdigest() == rec["source_sha256"] else None


def recorded_mfma(workload: str, kernel_mode: str, launch_ms: float):
    """Matrix-core figures of the dominant kernel from the same record's
    rocprofv3 --pmc run (SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16):
    the busy fraction of the MFMA pipes, and the hardware MFMA flops per launch
    over this run's launch time against the dense bf16 peak.  None when the
    record is for another workload or the kernel's sources changed since."""
    if recorded_traffic(workload, kernel_mode) is None:
        return None
    rec = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json"))).get("mfma")
    if not rec:
        return None
    tf = rec["mfma_flops_per_launch"] / (launch_ms * 1e-3) / 1e12
    return {"busy_frac": rec["mfma_busy_frac"], "flops_per_launch": rec["mfma_flops_per_launch"],
            "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "source": "profiles/hbm_traffic.json"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the device reaches its steady clock after a few tens of milliseconds of
    # this load (measured: 2.18 ms per step after 3 warm-up steps, 2.02-2.07
    # after 20 or more); untimed steps are cheap (about 2 ms each)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", type=int, default=3, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    ap.add_argument("--no-resume", action="store_true", help="skip the resume measurement")
    ap.add_argument("--no-conv", action="store_true", help="skip the short-conv measurement")
    ap.add_argument("--no-long-memory", action="store_true",
                    help="skip the long-memory segment-path measurement")
    ap.add_argument("--no-chunked", action="store_true",
                    help="skip the 8,192-token single-sequence measurement (both paths)")
    ap.add_argument("--decode-launches", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--roofline-launches", type=int, default=5,
                    help="extra launches of the dominant kernel timed alone for the roofline")
    ap.add_argument("--no-reference", action="store_true",
                    help="skip the device reference points (1 GiB copy, bf16 GEMM)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes three times (a known-size "
                         "reference for the HBM traffic counters) and exit")
    return ap.parse_args()


def copy_probe(nbytes: int):
    import torch
    n = nbytes // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "launches": 3}), flush=True)


def reference_rates(reps: int = 10) -> dict:
    """Reference points measured on this device, for context beside the
    spec peaks (neither is part of the library): a 1 GiB device-to-device
    copy (torch copy_, bytes read + written per second) and a bf16 matrix
    product of 8192 x 8192 x 8192 (torch matmul, a library GEMM, contiguous
    operands).  Median over reps, HIP events around each."""
    import torch
    stream = torch.cuda.current_stream()

    def median_ms(fn):
        fn()
        pairs = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in pairs]))
    n = (1 << 30) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    copy_ms = median_ms(lambda: y.copy_(x))
    del x, y
    m = 8192
    a = torch.randn((m, m), device="cuda").to(torch.bfloat16)
    b = torch.randn((m, m), device="cuda").to(torch.bfloat16)
    gemm_ms = median_ms(lambda: torch.matmul(a, b))
    del a, b
    torch.cuda.empty_cache()
    return {"copy_1gib_gbs": round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9, 1),
            "bf16_gemm_8192_tflops": round(2 * m ** 3 / (gemm_ms * 1e-3) / 1e12, 1)}


def cpu_baseline(w, target_s: float) -> dict:
    """The fp64 oracle as it stands, on the first tokens of sequence 0, all heads."""
    import oracle
    oracle.build(force=False)
    threads = oracle.threads()
    L0 = int(w.lengths[0])

    def run(ntok):
        a = int(w.cu_seqlens[0])
        sl = slice(a, a + ntok)
        q, k, v, g, b = (np.ascontiguousarray(getattr(w, n)[sl]) for n in ("q", "k", "v", "g", "beta"))
        from workloads import to_f64
        args = [to_f64(q, w.dtype), to_f64(k, w.dtype), to_f64(v, w.dtype),
                g.astype(np.float64), b.astype(np.float64)]
        S0 = None if w.S0 is None else w.S0[0:1]
        t = time.perf_counter()
        oracle.prefill(*args, [0, ntok], S0=S0, nthreads=threads)
        return time.perf_counter() - t

    probe = min(L0, 512)
    dt = run(probe)
    ntok = int(min(L0, max(probe, probe * target_s / max(dt, 1e-6))))
    ntok = max(64, (ntok // 64) * 64) if L0 >= 64 else L0
    dt = run(ntok)
    return {"value": round(ntok / dt, 2), "unit": "tokens/s", "cores": int(min(threads, w.H)),
            "kind": "oracle",
            "sample": f"first {ntok} tokens of sequence 0, all {w.H} heads, fp64 token loop, "
                      f"{threads} threads over heads ({dt:.1f} s)"}


def resume_measure(K, w, t, launches: int) -> dict:
    """kda_prefill_resume over the segment workload's tokens read as one
    sequence per segment, each continuing in place from a pool slot at its
    absolute start position, rungs every `ckpt_interval` tokens on the
    absolute grid.  HIP events around each call; algorithmic bytes as for
    prefill (1540 B per token-head) plus the states read, written and rung."""
    import torch
    from workloads import ckpt_offsets
    nseg = len(w.seg_start) - 1
    lengths = np.diff(w.seg_start)
    pos0 = torch.from_numpy(w.seg_start[:-1].astype(np.int64)).cuda()
    iv = w.ckpt_interval or 4096
    off_np = ckpt_offsets(lengths, iv, pos0=w.seg_start[:-1])
    off = torch.from_numpy(off_np).cuda()
    gen = torch.Generator(device="cuda").manual_seed(46003)
    pool = 0.1 * torch.randn((nseg, w.H, w.dk, w.dv), generator=gen, device="cuda")
    idx = torch.arange(nseg, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    ck = torch.empty((int(off_np[-1]), w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    o = torch.empty_like(t["v"])

    def call():   # outputs preallocated: no allocation or host synchronisation inside the call
        K.kda_prefill_resume(t["q"], t["k"], t["v"], t["g"], t["beta"], t["seg_start"], pool, idx,
                             idx, pos0=pos0, ckpt_interval=iv, ckpt_offsets=off, ckpt_out=ck, out=o)
    # untimed calls first: the first calls of this launch run slower
    # (measured: 2.35 ms falling to 1.75 ms over about seven calls)
    for _ in range(8):
        call()
    torch.cuda.synchronize()
    pairs = []
    for _ in range(launches):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in pairs]))
    io_bytes = 2 if w.dtype == "bf16" else 4
    alg = (w.T * w.H * bytes_per_token_head(w.dk, w.dv, io_bytes)
           + 4 * w.H * w.dk * w.dv * (2 * nseg + int(off_np[-1])))
    gbs = alg / (ms * 1e-3) / 1e9
    return {"workload": f"{w.name} as {nseg} sequences resumed in place at their absolute starts",
            "kernel": "chunk_engine<prefill> from a state pool", "tokens_per_s": round(w.T / (ms * 1e-3), 1),
            "launch_ms": round(ms, 4), "launches_timed": launches, "rungs": int(off_np[-1]),
            "alg_bytes_per_launch": int(alg),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def conv_measure(K, w, t, launches: int) -> dict:
    """kda_short_conv (width 4, SiLU, one sequence) over each of q, k, v of
    the workload, three launches per repetition, HIP events around each
    repetition.  Algorithmic bytes: every input element read once and every
    output element written once, in the I/O dtype."""
    import torch
    C = w.H * w.dk
    gen = torch.Generator(device="cuda").manual_seed(46006)
    weights = [torch.randn((C, 4), generator=gen, device="cuda") * 0.5 for _ in range(3)]
    bias = [0.1 * torch.randn(C, generator=gen, device="cuda") for _ in range(3)]
    xs = [t[n].reshape(w.T, C) for n in ("q", "k", "v")]
    ys = [torch.empty_like(x) for x in xs]
    cu = t["cu_seqlens"]
    stream = torch.cuda.current_stream()

    def call():
        for x, y, wt, b in zip(xs, ys, weights, bias):
            K.kda_short_conv(x, cu, wt, b, activation=K.KDA_ACT_SILU, out=y)
    call()
    pairs = []
    for _ in range(launches):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in pairs]))
    io_bytes = 2 if w.dtype == "bf16" else 4
    alg = 3 * 2 * w.T * C * io_bytes
    gbs = alg / (ms * 1e-3) / 1e9
    return {"workload": f"q, k, v of {w.name} ({w.T} x {C} each), width 4, SiLU",
            "kernel": "conv_kernel<bf16,4>", "tokens_per_s": round(w.T / (ms * 1e-3), 1),
            "ms_qkv": round(ms, 4), "launches_timed": 3 * launches, "alg_bytes": int(alg),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def _time_calls(call, launches: int, warm: int = 3) -> float:
    """Mean milliseconds per call, HIP events on the current stream around each."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        call()
    torch.cuda.synchronize()
    pairs = []
    for _ in range(launches):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in pairs]))


def long_memory_measure(K, w, t, launches: int) -> dict:
    """The segment step on the same q, k, v and segmentation with long-memory
    gates: log alpha = -softplus(N(0,1) - 9) (about -1.2e-4 per token) and
    beta = sigmoid(N(0,1) - 6), drawn on the device from a seeded generator.
    Every M stays far from zero, so the M blocks run their whole segment,
    the scan forms every product and every rung carries the propagated
    incoming state.  When the package does not split its segments (enough
    (segment, head) units), the step keeps a fix-up operator over whole
    segments: the M blocks write X for every row, the fix-up is one product,
    o += S_in^T X, and the rungs come from kda_checkpoint_write with sub_M.
    Otherwise (split segments) it runs the headline's step, whose fix-up then
    walks the recurrence.  Algorithmic bytes: the package pass (1540 B per
    token-head at d = 128 bf16) plus the M blocks' reads of q, k, g, beta and
    writes of X and the fix-up's read of X and of o and write of o (operator),
    or the M blocks' reads of k, g, beta and the fix-up's reads of q, k, g,
    beta and of o and write of o (recurrence); states, packages and rungs as
    the step moves them."""
    import ctypes
    import torch
    import torch.nn.functional as F
    gen = torch.Generator(device="cuda").manual_seed(46007)
    T, H, dk, dv = w.T, w.H, w.dk, w.dv
    g = -F.softplus(torch.randn((T, H, dk), generator=gen, device="cuda") - 9.0)
    beta = torch.sigmoid(torch.randn((T, H), generator=gen, device="cuda") - 6.0)
    S0 = None if t["S0"] is None else t["S0"][0].contiguous()
    interval = w.ckpt_interval
    nseg = len(w.seg_start) - 1
    seg_len = np.diff(np.asarray(w.seg_start, dtype=np.int64))
    cfg = K.make_config(H, dk, dv, t["q"].dtype)
    whole = K.LIB.kda_segment_package_workspace(ctypes.byref(cfg), T, nseg) == 0
    rows = T // interval if interval else 0
    ev = {}
    stream = torch.cuda.current_stream()

    def mark(name):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        ev.setdefault(name, []).append(e)

    if whole:
        fx = K.FixOp(nseg, H, dk, t["q"].dtype, "cuda", chunks=int(-(-seg_len.max() // 64)))
        ck_out = torch.empty((rows, H, dk, dv), dtype=torch.float32, device="cuda") if rows else None
    else:
        fx = K.FixOp(nseg, H, dk, t["q"].dtype, "cuda", interval=interval)

    def step(timed):
        if timed:
            mark("a")
        o, M, D, sM, sD = K.kda_segment_package_fx(t["q"], t["k"], t["v"], g, beta,
                                                   t["seg_start"], fx, ckpt_interval=interval,
                                                   want_sub_M=whole)
        if timed:
            mark("b")
        S_in, _ = K.kda_segment_scan(M, D, S0, algo=w.scan_algo)
        if timed:
            mark("c")
        if whole:
            K.kda_output_fixup_fx(t["q"], t["k"], g, beta, t["seg_start"], S_in, o, fx)
            if rows:
                K.kda_checkpoint_write(t["seg_start"], S_in, sM, sD, T=T, interval=interval,
                                       out=ck_out)
        else:
            K.kda_output_fixup_fx(t["q"], t["k"], g, beta, t["seg_start"], S_in, o, fx, sub_D=sD,
                                  interval=interval, out=sD)
        if timed:
            mark("d")
        return M

    M = step(False)
    torch.cuda.synchronize()
    m_norm_min = float(torch.linalg.matrix_norm(M).min())
    route = fx.route.cpu().numpy()
    for _ in range(3):
        step(False)
    torch.cuda.synchronize()
    for _ in range(launches):
        step(True)
    torch.cuda.synchronize()

    def avg(a, b):
        return float(np.mean([x.elapsed_time(y) for x, y in zip(ev[a], ev[b])]))
    ms = avg("a", "d")
    io = 2 if w.dtype == "bf16" else 4
    if whole:   # M blocks: q, k, g, beta read, X written; fix-up: X and o read, o written
        per_tok = (bytes_per_token_head(dk, dv, io) + (2 * io * dk + 4 * dk + 4 + io * dk)
                   + (io * dk + 2 * io * dv))
        rung_bytes = 4 * H * (3 * dk * dv + 2 * dk * dk) * rows   # sub_D, sub_M, rung
    else:       # M blocks: k, g, beta read; fix-up: q, k, g, beta and o read, o written
        per_tok = (bytes_per_token_head(dk, dv, io) + (io * dk + 4 * dk + 4)
                   + (2 * io * dk + 4 * dk + 4 + 2 * io * dv))
        rung_bytes = 2 * 4 * H * dk * dv * rows
    alg = T * H * per_tok + 4 * H * (dk * dv + dk * dk) * nseg + rung_bytes
    gbs = alg / (ms * 1e-3) / 1e9
    return {"workload": f"{w.name} with long-memory gates (log alpha ~ -1.2e-4 per token)",
            "fixup": ("operator over whole segments, rungs by kda_checkpoint_write" if whole
                      else "recurrence (split segments: the operator covers no segment)"),
            "units_on_recurrence": int(route.sum()),
            "min_frobenius_norm_M": round(m_norm_min, 4),
            "tokens_per_s": round(T / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
            "steps_timed": launches,
            "breakdown_ms": {"package": round(avg("a", "b"), 4), "scan": round(avg("b", "c"), 4),
                             "fixup_and_rungs": round(avg("c", "d"), 4)},
            "alg_bytes_per_step": int(alg),
            "hbm": {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def single_sequence_measure(K, launches: int) -> dict:
    """kda_prefill on the 8,192-token single sequence (H = 32, d = 128,
    bf16, S0 ~ N(0, 0.1^2)) by both of its paths: the chunked engine in one
    pass (a 256-byte workspace: one workgroup per head and value-column
    block) and the queried workspace, with which kda_prefill runs the
    sequence as segments (packages, sequential scan, fix-up).  HIP events
    around each call; algorithmic bytes as for prefill."""
    import torch
    from workloads import standard_workload
    from workloads.device import to_torch
    w = standard_workload(1)
    t = to_torch(w)
    o = torch.empty_like(t["v"])
    Sf = torch.empty((1, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    tiny = torch.empty(256, dtype=torch.uint8, device="cuda")
    out = {"workload": w.name}
    io = 2 if w.dtype == "bf16" else 4
    alg = w.T * w.H * bytes_per_token_head(w.dk, w.dv, io) + 4 * w.H * w.dk * w.dv * 2
    for name, ws in (("one_pass", tiny), ("segmented", None)):
        def call():
            K.kda_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"], t["S0"],
                          out=o, workspace=ws)
        ms = _time_calls(call, max(launches, 10))
        gbs = alg / (ms * 1e-3) / 1e9
        out[name] = {"tokens_per_s": round(w.T / (ms * 1e-3), 1), "ms_per_call": round(ms, 4),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def decode_measure(K, launches: int) -> dict:
    """kda_decode on 64 sequences x 32 heads (d=128, bf16, gate logits,
    128-slot pool with in-place rows, forks, fresh and discarded states).
    The states touched by one call (~230 MiB) would fit in the 256 MiB
    last-level cache, so a 1 GiB buffer is read through before every timed
    call (a read leaves clean lines, whose eviction costs the timed call
    nothing, and pushes the previous call's dirty states back to HBM) and
    each call is bracketed by its own HIP events: the figure is a cold-HBM
    one.  Algorithmic bytes: each state read and written once
    (fp32), q, k, v, o in bf16, g and beta in fp32."""
    import torch
    from workloads import standard_decode_batch
    from workloads.device import decode_to_torch
    b = standard_decode_batch()
    t = decode_to_torch(b)
    n_slots = b.pool.shape[0]
    state = 4 * b.H * b.dk * b.dv
    nread = int(np.sum((b.read_idx >= 0) & (b.read_idx < n_slots)))
    nwrite = int(np.sum((b.write_idx >= 0) & (b.write_idx < n_slots)))
    alg = state * (nread + nwrite) + b.N * b.H * (2 * (2 * b.dk + 2 * b.dv) + 4 * b.dk + 4)
    stream = torch.cuda.current_stream()

    def call():
        K.kda_decode(t["q"], t["k"], t["v"], t["g"], t["beta"], t["pool"], t["read_idx"],
                     t["write_idx"], gate_logits=True)
    for _ in range(5):
        call()
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=t["q"].device)
    pairs = []
    for _ in range(launches):
        flush.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in pairs]))
    gbs = alg / (ms * 1e-3) / 1e9
    return {"workload": b.name, "kernel": "decode_kernel<128,128,bf16>",
            "tokens_per_s": round(b.N / (ms * 1e-3), 1), "launch_us": round(ms * 1e3, 2),
            "launches_timed": launches, "cache": "1 GiB read before each timed call",
            "alg_bytes_per_launch": int(alg),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": recorded_traffic(b.name, "decode_kernel", "decode")}}


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1 "
                                   "(the library has no cross-GPU package exchange)"}))
        sys.exit(2)
    import torch
    from workloads import standard_workload, ckpt_offsets
    from workloads.device import to_torch
    import gated_delta_rule_46_amd.kda as K

    w = standard_workload(args.config)
    t = to_torch(w)
    dev = t["q"].device
    T, H, dk, dv = w.T, w.H, w.dk, w.dv
    segmented = w.seg_start is not None
    io_bytes = 2 if w.dtype == "bf16" else 4
    stream = torch.cuda.current_stream()

    ev = {}

    def mark(name):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        ev.setdefault(name, []).append(e)

    if segmented:
        S0 = None if t["S0"] is None else t["S0"][0].contiguous()
        interval = w.ckpt_interval
        nseg = len(w.seg_start) - 1
        # the fix-up operator: the M blocks keep the identity's outputs of the
        # first chunks of each segment, and the fix-up is a product with them
        fx = K.FixOp(nseg, H, dk, t["q"].dtype, dev, interval=interval)

        def step(timed):
            if timed:
                mark("pkg0")
            o, M, D, _, sD = K.kda_segment_package_fx(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                                      t["seg_start"], fx, ckpt_interval=interval,
                                                      want_sub_M=False)
            if timed:
                mark("pkg1")
            S_in, S_fin = K.kda_segment_scan(M, D, S0, algo=w.scan_algo)
            if timed:
                mark("scan1")
            # the fix-up forms the checkpoint rungs in the same launch, in place in
            # sub_D (rows past the propagated state's end are final already)
            K.kda_output_fixup_fx(t["q"], t["k"], t["g"], t["beta"], t["seg_start"], S_in, o, fx,
                                  sub_D=sD, interval=interval, out=sD)
            if timed:
                mark("fix1")
            return o
        main_kernel = "package_engine (value blocks, then M blocks with the fix-up operator)"
        rows = T // interval if interval else 0
        # D and rung sub_D, and M, written by the launch; the rows of X it writes
        # are counted once the warm-up has filled the operator (len)
        extra_bytes = 4 * H * dk * dv * (nseg + rows) + 4 * H * dk * dk * nseg

        def dominant():
            # the launch the step runs first: kda_segment_package_fx
            K.kda_segment_package_fx(t["q"], t["k"], t["v"], t["g"], t["beta"], t["seg_start"],
                                     fx, ckpt_interval=interval, want_sub_M=False)

        def value_blocks():
            # the value blocks alone (kda_segment_package without M)
            K.kda_segment_package(t["q"], t["k"], t["v"], t["g"], t["beta"], t["seg_start"],
                                  ckpt_interval=interval, want_M=False)
    else:
        off = ck_out = None
        if w.ckpt_interval:
            off_np = ckpt_offsets(w.lengths, w.ckpt_interval)
            off = torch.from_numpy(off_np).to(dev)
            if w.N > 1:   # rung states preallocated: no host synchronisation inside a step
                ck_out = torch.empty((int(off_np[-1]), H, dk, dv), dtype=torch.float32, device=dev)

        def step(timed):
            if timed:
                mark("pkg0")
            o, Sf, ck = K.kda_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                                      t["S0"], ckpt_interval=w.ckpt_interval, ckpt_offsets=off,
                                      ckpt_out=ck_out)
            if timed:
                mark("pkg1")
            return o
        # one long sequence on few heads runs segmented inside kda_prefill
        # (several launches); otherwise the call is one engine launch
        main_kernel = ("kda_prefill (segmented: packages, scan, fix-up)"
                       if w.N == 1 and K.LIB.kda_prefill_workspace(
                           ctypes.byref(K.make_config(H, dk, dv, t["q"].dtype)), T, 1) > 256
                       else "chunk_engine<prefill>")
        rows = int(ckpt_offsets(w.lengths, w.ckpt_interval)[-1]) if w.ckpt_interval else 0
        extra_bytes = 4 * H * dk * dv * (2 * w.N + rows)             # S0, S_final, checkpoints

        def dominant():
            step(False)
        value_blocks = None

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1000.0 * elapsed / args.steps
    if segmented:   # rows of X the package launch writes (per 64-column block), read after the steps
        step(False)
        torch.cuda.synchronize()
        lens = np.clip(fx.len.cpu().numpy().astype(np.int64), 0, fx.chunks)
        seg_len = np.diff(np.asarray(w.seg_start, dtype=np.int64))
        x_rows = sum(int(np.minimum(lens[j] * 64, seg_len[j]).sum()) for j in range(nseg))
        extra_bytes += x_rows * 64 * io_bytes

    def avg_ms(a, b):
        return float(np.mean([x.elapsed_time(y) for x, y in zip(ev[a], ev[b])]))

    # the dominant kernel timed alone with HIP events on the launch stream
    for _ in range(args.roofline_launches):
        mark("dom0")
        dominant()
        mark("dom1")
    if value_blocks is not None:
        for _ in range(args.roofline_launches):
            mark("vb0")
            value_blocks()
            mark("vb1")
    torch.cuda.synchronize()
    kernel_ms = avg_ms("dom0", "dom1")
    breakdown = {"package" if segmented else "prefill": round(avg_ms("pkg0", "pkg1"), 4)}
    # spread of the timed steps (each step's first and last event; the value
    # above is total time over steps, host gaps included)
    last = "fix1" if segmented else "pkg1"
    per_step = np.array([x.elapsed_time(y) for x, y in zip(ev["pkg0"], ev[last])])
    step_spread = {"p10": round(float(np.percentile(per_step, 10)), 4),
                   "p50": round(float(np.percentile(per_step, 50)), 4),
                   "p90": round(float(np.percentile(per_step, 90)), 4)}
    if segmented:
        breakdown.update(scan=round(avg_ms("pkg1", "scan1"), 4),
                         fixup_and_rungs=round(avg_ms("scan1", "fix1"), 4))
    alg_bytes = T * H * bytes_per_token_head(dk, dv, io_bytes) + extra_bytes
    achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9
    flops = T * H * chunk_flops_per_token_head(64, dk, dv)
    tok_s = T / (ms_per_step * 1e-3)
    result = {
        "metric": "KDA prefill tokens/s per layer (H=32, d=128) + % MI355X bf16 MFMA peak",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": T, "H": H, "dk": dk, "dv": dv, "chunk": 64,
                   "path": "segment" if segmented else "chunked",
                   "segments": (len(w.seg_start) - 1) if segmented else None,
                   "scan": ("blelloch" if w.scan_algo == 1 else "sequential") if segmented else None,
                   "sequences": w.N, "ckpt_interval": w.ckpt_interval},
        "mfma_frac": round(flops / (ms_per_step * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
        "mfma_tflops_alg": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "roofline": {"bound": "hbm", "kernel": main_kernel, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(w.name, "package_engine" if segmented else "prefill"),
                     "alg_bytes_per_launch": int(alg_bytes),
                     "launch_ms": round(kernel_ms, 4), "launches_timed": args.roofline_launches},
        "breakdown_ms": breakdown,
        "step_ms_spread": step_spread,
    }
    if value_blocks is not None:
        vb_ms = avg_ms("vb0", "vb1")
        vb_bytes = T * H * bytes_per_token_head(dk, dv, io_bytes) + 4 * H * dk * dv * (nseg + rows)
        vb_gbs = vb_bytes / (vb_ms * 1e-3) / 1e9
        result["roofline_value_blocks"] = {
            "kernel": "chunk_engine<package> value blocks alone (kda_segment_package without M)",
            "achieved": round(vb_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(vb_gbs / HBM_PEAK_GBS, 4), "alg_bytes_per_launch": int(vb_bytes),
            "launch_ms": round(vb_ms, 4), "launches_timed": args.roofline_launches}
    mf = recorded_mfma(w.name, "package_engine" if segmented else "prefill", kernel_ms)
    if mf is not None:
        result["roofline"]["mfma_rocprof"] = mf
    if segmented and not args.no_long_memory:
        result["long_memory"] = long_memory_measure(K, w, t, args.roofline_launches)
    if segmented and not args.no_resume:
        result["resume"] = resume_measure(K, w, t, args.roofline_launches)
    if not args.no_conv:
        result["short_conv"] = conv_measure(K, w, t, args.roofline_launches)
    t = None   # the workload's device tensors are not needed past this point
    torch.cuda.empty_cache()
    if args.config == 3 and not args.no_chunked:
        result["single_sequence_8192"] = single_sequence_measure(K, args.roofline_launches)
    if not args.no_decode:
        result["decode"] = decode_measure(K, args.decode_launches)
    if not args.no_reference:
        ref = reference_rates()
        result["reference"] = ref
        result["roofline"]["frac_of_measured_copy"] = round(achieved / ref["copy_1gib_gbs"], 4)
        result["mfma_frac_of_measured_gemm"] = round(
            flops / (ms_per_step * 1e-3) / 1e12 / ref["bf16_gemm_8192_tflops"], 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
