"""kda_prefill_noalloc: the prefill entry point that allocates nothing (its
scratch is a fixed array inside the library) against kda_prefill with a
workspace from the caller, through the C ABI.

Two calls in a row on the same device, the second smaller, so the second
runs on scratch the first left behind: a single 8,192-token sequence (H = 32,
d = 128, bf16: run as segments inside the scratch), then a single 2,048-token
sequence (H = 4: segments again, fewer and shorter), then a varlen batch (the
longest-first schedule in the scratch, checkpoints).  Each result is compared
with kda_prefill on the same inputs (rel-L2 at the bf16 bars, and reported
when bit-identical) and with the oracle.
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import ckpt_offsets, make_workload, standard_workload
from workloads.device import to_numpy_f64, to_torch

pytestmark = pytest.mark.gpu

OUT_TOL, STATE_TOL = 2e-2, 1e-2


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_delta_rule_46_amd.kda as kda
    return kda


def _run(K, w, interval):
    import torch
    t = to_torch(w)
    off = None
    if interval:
        off = torch.from_numpy(ckpt_offsets(w.lengths, interval)).cuda()
    o1, S1, c1 = K.kda_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"], t["S0"],
                               ckpt_interval=interval, ckpt_offsets=off)
    # every output preallocated: the no-allocation call then allocates nothing
    o2 = torch.empty_like(o1)
    S2 = torch.empty_like(S1)
    c2 = None if c1 is None else torch.full_like(c1, float("nan"))
    torch.cuda.synchronize()
    stats0 = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    free0 = torch.cuda.mem_get_info()[0]
    K.kda_prefill_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"], t["S0"],
                          ckpt_interval=interval, ckpt_offsets=off, out=o2, final_out=S2,
                          ckpt_out=c2)
    torch.cuda.synchronize()
    stats1 = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    free1 = torch.cuda.mem_get_info()[0]
    assert stats1 == stats0, "the no-allocation call went through torch's allocator"
    say(f"  device free memory before / after the call: {free0} / {free1}")
    return (o1, S1, c1), (o2, S2, c2)


def _compare(name, a, b, ref, tol):
    import torch
    same = bool(torch.equal(a, b))
    x, y = to_numpy_f64(b), to_numpy_f64(a)
    e = oracle.rel_l2(x, y)
    e_ref = oracle.rel_l2(x, ref)
    say(f"  {name}: vs kda_prefill rel-L2 {e:.3e} (bit-identical: {same}), vs oracle {e_ref:.3e}")
    assert np.all(np.isfinite(x))
    assert e <= tol and e_ref <= tol


def _case(K, w, interval=0):
    ref = oracle.prefill(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("g"), w.f64("beta"),
                         w.cu_seqlens, S0=w.S0, ckpt_interval=interval,
                         ckpt_offsets=ckpt_offsets(w.lengths, interval) if interval else None)
    (o1, S1, c1), (o2, S2, c2) = _run(K, w, interval)
    _compare("o", o1, o2, ref[0], OUT_TOL)
    _compare("S_final", S1, S2, ref[1], STATE_TOL)
    if interval:
        _compare("rungs", c1, c2, ref[2], STATE_TOL)


def test_noalloc_two_calls_second_smaller(K):
    say("no-allocation prefill, call 1: T=8192 H=32 d=128 bf16 (segmented in the scratch)")
    _case(K, standard_workload(1))
    say("no-allocation prefill, call 2: T=2048 H=4 d=128 bf16 (segmented, smaller)")
    _case(K, make_workload("noalloc-2", [2048], 4, 128, 128, "bf16", 4970, s0_std=0.1))
    say("no-allocation prefill, call 3: varlen [300, 77, 129, 1] H=2 d=64 bf16, rungs every 64")
    _case(K, make_workload("noalloc-3", [300, 77, 129, 1], 2, 64, 64, "bf16", 4971, s0_std=0.2),
          interval=64)


def test_noalloc_rejects_oversized_schedule(K):
    """More sequences than the fixed scratch can schedule: a clear error
    before anything runs."""
    import ctypes
    import torch
    n = K.NOALLOC_SCRATCH_BYTES // 4 + 1
    c = K.make_config(1, 64, 64, torch.float32)
    buf = torch.empty(64, dtype=torch.float32, device="cuda")
    p = buf.data_ptr()
    st = K.LIB.kda_prefill_noalloc(ctypes.byref(c), p, p, p, p, p, p, n, 64, None, None, p,
                                   None, None)
    assert st == K.KDA_ERR_WORKSPACE
    assert "scratch" in K.LIB.kda_last_error().decode()
