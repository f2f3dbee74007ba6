"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances are rel-L2 over the compared tensor: 1e-4 for fp32 I/O; for bf16
I/O 2e-2 on outputs and 1e-2 on states.  The full-size workloads are in
test_gpu_fullsize.py.
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import make_workload, standard_workload, ckpt_offsets
from workloads.device import to_torch, to_numpy_f64

pytestmark = pytest.mark.gpu

OUT_TOL = {"f32": 1e-4, "bf16": 2e-2}
STATE_TOL = {"f32": 1e-4, "bf16": 1e-2}


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_delta_rule_46_amd.kda as kda
    return kda


def sync():
    import torch
    torch.cuda.synchronize()


def oracle_full(w, interval=0):
    off = ckpt_offsets(w.lengths, interval) if interval else None
    return oracle.prefill(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("g"), w.f64("beta"),
                          w.cu_seqlens, S0=w.S0, scale=w.scale, qk_l2norm=w.qk_l2norm,
                          ckpt_interval=interval, ckpt_offsets=off)


def oracle_unit(w, n, h, interval=0):
    u = w.unit(n, h)
    L = int(w.lengths[n])
    off = ckpt_offsets([L], interval) if interval else None
    return oracle.prefill(u["q"], u["k"], u["v"], u["g"], u["beta"], [0, L], S0=u["S0"],
                          scale=w.scale, qk_l2norm=w.qk_l2norm, ckpt_interval=interval,
                          ckpt_offsets=off)


def run_prefill_t(K, w, interval=0):
    """Runs kda_prefill; returns device tensors (o, S_final, ckpt)."""
    import torch
    t = to_torch(w)
    off = None
    if interval:
        off = torch.from_numpy(ckpt_offsets(w.lengths, interval)).cuda()
    o, Sf, ck = K.kda_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"], t["S0"],
                              ckpt_interval=interval, ckpt_offsets=off, scale=w.scale,
                              qk_l2norm=bool(w.qk_l2norm))
    sync()
    del t
    return o, Sf, ck


def run_prefill(K, w, interval=0):
    o, Sf, ck = run_prefill_t(K, w, interval)
    return to_numpy_f64(o), to_numpy_f64(Sf), (None if ck is None else to_numpy_f64(ck))


def assert_close(name, got, ref, tol):
    err = oracle.rel_l2(got, ref)
    say(f"{name}: rel-L2 {err:.3e} (tol {tol:g})")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert err <= tol, f"{name}: rel-L2 {err:.3e} > {tol:g}"


# ---------------------------------------------------------------------------
# chunked prefill, small sizes compared in full
# ---------------------------------------------------------------------------
def test_prefill_config0_fp32(K):
    say("prefill config0 fp32 T=256 H=1 d=64")
    w = standard_workload(0)
    o, Sf, _ = run_prefill(K, w)
    ro, rS, _ = oracle_full(w)
    assert_close("o", o, ro, OUT_TOL["f32"])
    assert_close("S_final", Sf, rS, STATE_TOL["f32"])


@pytest.mark.parametrize("d,T,H", [(128, 300, 2), (64, 200, 3), (128, 64, 1), (128, 17, 2)])
def test_prefill_bf16_ragged(K, d, T, H):
    say(f"prefill bf16 d={d} T={T} H={H}")
    w = make_workload("t", [T], H, d, d, "bf16", 101 + d + T, s0_std=0.1)
    o, Sf, _ = run_prefill(K, w)
    ro, rS, _ = oracle_full(w)
    assert_close("o", o, ro, OUT_TOL["bf16"])
    assert_close("S_final", Sf, rS, STATE_TOL["bf16"])


def test_prefill_fp32_long_memory(K):
    say("prefill fp32 d=64 long-memory gates T=700 H=2")
    w = make_workload("t", [700], 2, 64, 64, "f32", 7, s0_std=0.5, gate_shift=-9.0, beta_shift=-6.0)
    o, Sf, _ = run_prefill(K, w)
    ro, rS, _ = oracle_full(w)
    assert_close("o", o, ro, OUT_TOL["f32"])
    assert_close("S_final", Sf, rS, STATE_TOL["f32"])


@pytest.mark.parametrize("dtype,d,H,T,iv", [("bf16", 128, 4, 8192, 1024), ("f32", 64, 2, 3000, 0),
                                             ("bf16", 64, 8, 4160, 256)])
def test_prefill_single_sequence_split_and_single_pass(K, dtype, d, H, T, iv):
    """One sequence on few heads: kda_prefill splits it into segments when
    the workspace holds them (the queried size), and runs one pass with a
    minimal workspace; both against the oracle, with rungs at the sequence's
    own positions."""
    import torch
    w = make_workload("split", [T], H, d, d, dtype, 4631, s0_std=0.1)
    t = to_torch(w)
    ref = oracle_full(w, iv)
    for name, ws in (("split", None), ("one pass", torch.empty(256, dtype=torch.uint8, device="cuda"))):
        say(f"prefill {name}: T={T} H={H} d={d} {dtype} interval={iv}")
        o, Sf, ck = K.kda_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                                  t["S0"], ckpt_interval=iv, workspace=ws)
        sync()
        assert_close(f"{name} o", to_numpy_f64(o), ref[0], OUT_TOL[dtype])
        assert_close(f"{name} S_final", to_numpy_f64(Sf), ref[1], STATE_TOL[dtype])
        if iv:
            assert ck.shape[0] == T // iv
            assert_close(f"{name} rungs", to_numpy_f64(ck), ref[2], STATE_TOL[dtype])


def test_prefill_varlen_checkpoints(K):
    lens = [70, 1, 128, 200, 0, 64, 129, 256]
    say(f"prefill varlen fp32 d=64 lens={lens} ckpt=64")
    w = make_workload("t", lens, 2, 64, 64, "f32", 8, s0_std=0.3)
    o, Sf, ck = run_prefill(K, w, interval=64)
    ro, rS, rck = oracle_full(w, interval=64)
    assert_close("o", o, ro, OUT_TOL["f32"])
    assert_close("S_final", Sf, rS, STATE_TOL["f32"])
    assert ck.shape == rck.shape
    assert_close("ckpt", ck, rck, STATE_TOL["f32"])


def test_prefill_ckpt_out_preallocated(K):
    """Rung states in a caller-supplied tensor (no host synchronisation in
    the binding) are the same bits as in the binding's own allocation, for
    prefill and for resume from a pool."""
    import torch
    lens = [300, 64, 513, 1]
    say(f"prefill / resume with preallocated rung states, bf16 d=128 lens={lens} ckpt=128")
    w = make_workload("t", lens, 2, 128, 128, "bf16", 9, s0_std=0.2)
    t = to_torch(w)
    off_np = ckpt_offsets(w.lengths, 128)
    off = torch.from_numpy(off_np).cuda()
    o1, S1, c1 = K.kda_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"], t["S0"],
                               ckpt_interval=128, ckpt_offsets=off)
    buf = torch.full((int(off_np[-1]), 2, 128, 128), float("nan"), device="cuda")
    o2, S2, c2 = K.kda_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"], t["S0"],
                               ckpt_interval=128, ckpt_offsets=off, ckpt_out=buf)
    sync()
    assert c2.data_ptr() == buf.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(c1, c2)
    pool = t["S0"].clone()
    idx = torch.arange(len(lens), dtype=torch.int32, device="cuda")
    pos0 = torch.zeros(len(lens), dtype=torch.int64, device="cuda")
    r1, d1 = K.kda_prefill_resume(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                                  pool.clone(), idx, idx, pos0=pos0, ckpt_interval=128,
                                  ckpt_offsets=off)
    buf2 = torch.full_like(buf, float("nan"))
    r2, d2 = K.kda_prefill_resume(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                                  pool.clone(), idx, idx, pos0=pos0, ckpt_interval=128,
                                  ckpt_offsets=off, ckpt_out=buf2)
    sync()
    assert torch.equal(r1, r2) and torch.equal(d1, d2) and torch.equal(d2, c1)


@pytest.mark.parametrize("dtype,d,l2,scale", [("bf16", 128, 0, 1.0), ("bf16", 128, 1, 0.08838834764831845),
                                          ("f32", 64, 0, 0.5), ("bf16", 64, 1, 0.125)])
def test_prefill_scale_and_no_l2norm(K, dtype, d, l2, scale):
    """Chunked prefill with a query scale and with the in-kernel L2 norm off
    (q, k scaled by 2^-4 so that the recurrence contracts)."""
    from workloads import scale_qk_pow2
    lens = [200, 77, 129]
    say(f"prefill {dtype} d={d} l2norm={l2} scale={scale:g} lens={lens}")
    w = make_workload("t", lens, 2, d, d, dtype, 31 + d + l2, s0_std=0.2, scale=scale, qk_l2norm=l2)
    if not l2:
        scale_qk_pow2(w, -4)
    o, Sf, ck = run_prefill(K, w, interval=64)
    ro, rS, rck = oracle_full(w, interval=64)
    assert_close("o", o, ro, OUT_TOL[dtype])
    assert_close("S_final", Sf, rS, STATE_TOL[dtype])
    assert_close("ckpt", ck, rck, STATE_TOL[dtype])


@pytest.mark.parametrize("algo", [0, 1])
def test_segment_path_scale_and_no_l2norm(K, algo):
    """The segment path (packages, scan, fix-up, rungs) with a query scale and
    the L2 norm off, long-memory gates so every stage carries a nonzero M."""
    from workloads import scale_qk_pow2
    say(f"segment path bf16 d=128 l2norm=0 scale=0.5 algo={algo} long-memory")
    seg = [0, 192, 640, 704, 1090]
    w = make_workload("t", [1090], 2, 128, 128, "bf16", 40 + algo, s0_std=0.5, gate_shift=-9.0,
                      beta_shift=-6.0, seg_start=seg, scale=0.5, qk_l2norm=0)
    scale_qk_pow2(w, -4)
    r = _segment_case(K, w, algo, interval=128)
    assert np.count_nonzero(r["M"]) > 0
    ro, rS, rck = oracle_full(w, interval=128)
    assert_close("o", r["o"], ro, OUT_TOL["bf16"])
    assert_close("S_final", r["S_final"], rS[0], STATE_TOL["bf16"])
    assert_close("ckpt", r["ckpt"], rck, STATE_TOL["bf16"])


def test_prefill_varlen_bf16(K):
    lens = [513, 64, 1000, 31, 2048]
    say(f"prefill varlen bf16 d=128 lens={lens} ckpt=512")
    w = make_workload("t", lens, 2, 128, 128, "bf16", 9, s0_std=0.1)
    o, Sf, ck = run_prefill(K, w, interval=512)
    ro, rS, rck = oracle_full(w, interval=512)
    assert_close("o", o, ro, OUT_TOL["bf16"])
    assert_close("S_final", Sf, rS, STATE_TOL["bf16"])
    assert_close("ckpt", ck, rck, STATE_TOL["bf16"])


def test_prefill_empty_and_zero_length(K):
    import torch
    say("prefill N=0 and all-zero-length sequences")
    w = make_workload("t", [0, 0], 1, 64, 64, "f32", 10, s0_std=1.0)
    o, Sf, _ = run_prefill(K, w)
    assert o.shape == (0, 1, 64)
    np.testing.assert_array_equal(Sf, w.S0.astype(np.float64))
    t = to_torch(make_workload("t", [5], 1, 64, 64, "f32", 11, s0_std=None))
    o2, Sf2, _ = K.kda_prefill(t["q"][:0], t["k"][:0], t["v"][:0], t["g"][:0], t["beta"][:0],
                               torch.zeros(1, dtype=torch.int64, device="cuda"), None)
    sync()
    assert o2.shape[0] == 0 and Sf2.shape[0] == 0


# ---------------------------------------------------------------------------
# closed forms on the GPU
# ---------------------------------------------------------------------------
def test_gpu_beta_zero_pure_decay(K):
    import torch
    say("closed form: beta = 0, fp32 d=64")
    # gentle gates so the decayed state stays inside fp32 range after 200 tokens
    w = make_workload("t", [200], 2, 64, 64, "f32", 12, s0_std=1.0, gate_shift=-4.0)
    w.beta[:] = 0.0
    o, Sf, _ = run_prefill(K, w)
    q = w.f64("q")
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6)
    G = np.cumsum(w.f64("g"), axis=0)
    ref_o = np.einsum("hij,thi->thj", w.S0[0].astype(np.float64), np.exp(G) * qn)
    assert_close("o (beta=0)", o, ref_o, OUT_TOL["f32"])
    assert_close("S_final (beta=0)", Sf[0], np.exp(G[-1])[:, :, None] * w.S0[0], STATE_TOL["f32"])


def test_gpu_orthonormal_recall(K):
    import torch
    say("closed form: alpha=1, beta=1, orthonormal keys, fp32 d=64")
    dk = 64
    n = 48
    rng = np.random.default_rng(13)
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:n].astype(np.float32)
    w = make_workload("t", [n], 1, dk, dk, "f32", 14, s0_std=1.0)
    w.k[:, 0] = keys
    w.q[:, 0] = keys
    w.g[:] = 0.0
    w.beta[:] = 1.0
    o, Sf, _ = run_prefill(K, w)
    # querying the key just written returns its value (up to the 1e-6 norm eps)
    assert_close("recall o_t = v_t", o[:, 0], w.f64("v")[:, 0] / np.sqrt(1 + 1e-6) ** 2, 1e-4)
    recall = Sf[0, 0].T @ keys.T.astype(np.float64)
    assert_close("S^T k_i = v_i", recall, w.f64("v")[:, 0].T / np.sqrt(1 + 1e-6) ** 2, 1e-4)


# ---------------------------------------------------------------------------
# segment path
# ---------------------------------------------------------------------------
def _segment_case(K, w, algo, interval, heads=None):
    import torch
    t = to_torch(w)
    T = w.T
    nseg = len(w.seg_start) - 1
    S0 = None if t["S0"] is None else t["S0"][0].contiguous()
    ol, M, D, sM, sD = K.kda_segment_package(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                             t["seg_start"], ckpt_interval=interval,
                                             scale=w.scale, qk_l2norm=bool(w.qk_l2norm))
    S_in, S_fin = K.kda_segment_scan(M, D, S0, algo=algo)
    o = ol.clone()
    K.kda_output_fixup(t["q"], t["k"], t["g"], t["beta"], t["seg_start"], S_in, o,
                       scale=w.scale, qk_l2norm=bool(w.qk_l2norm))
    ck = None
    if interval:
        ck = K.kda_checkpoint_write(t["seg_start"], S_in, sM, sD, T=T, interval=interval,
                                    dtype=t["q"].dtype)
    sync()
    del t
    if heads is not None:   # full-size cases: bring back only the sampled heads
        hs = list(heads)
        return dict(o=to_numpy_f64(o[:, hs]), S_final=to_numpy_f64(S_fin[hs]),
                    M=to_numpy_f64(M[:, hs]), S_in=to_numpy_f64(S_in[:, hs]),
                    ckpt=None if ck is None else to_numpy_f64(ck[:, hs]))
    return dict(o_local=to_numpy_f64(ol), M=to_numpy_f64(M), D=to_numpy_f64(D), S_in=to_numpy_f64(S_in),
                S_final=to_numpy_f64(S_fin), o=to_numpy_f64(o),
                ckpt=None if ck is None else to_numpy_f64(ck))


@pytest.mark.parametrize("algo", [0, 1])
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("bf16", 64)])
def test_segment_path_long_memory(K, algo, dtype, d):
    """Long-memory gates keep M, the scan and the fix-up all nonzero."""
    say(f"segment path {dtype} d={d} algo={algo} long-memory, 5 segments, ragged tail")
    T = 1300
    seg = [0, 256, 320, 768, 1024, 1300]
    w = make_workload("t", [T], 2, d, d, dtype, 15 + d + algo, s0_std=0.5, gate_shift=-9.0,
                      beta_shift=-6.0, seg_start=seg)
    r = _segment_case(K, w, algo, interval=128)
    q, k, v, g, b = (w.f64(x) for x in ("q", "k", "v", "g", "beta"))
    tol_o, tol_s = OUT_TOL[dtype], STATE_TOL[dtype]
    Ms, Ds = [], []
    for j in range(len(seg) - 1):
        Mr, Dr, olr = oracle.package(q, k, v, g, b, seg[j], seg[j + 1])
        Ms.append(Mr)
        Ds.append(Dr)
        assert_close(f"M[{j}]", r["M"][j], Mr, tol_s)
        assert_close(f"D[{j}]", r["D"][j], Dr, tol_s)
        assert_close(f"o_local[{j}]", r["o_local"][seg[j]:seg[j + 1]], olr[seg[j]:seg[j + 1]], tol_o)
    S_in_ref, S_fin_ref = oracle.scan_sequential(Ms, Ds, w.S0[0].astype(np.float64))
    assert_close("S_in", r["S_in"], S_in_ref, tol_s)
    ro, rS, rck = oracle_full(w, interval=128)
    assert_close("S_final", r["S_final"], rS[0], tol_s)
    assert_close("o", r["o"], ro, tol_o)
    assert_close("ckpt", r["ckpt"], rck, tol_s)


@pytest.mark.parametrize("algo", [0, 1])
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_segment_path_memory_off_every_fourth_channel(K, algo, dtype, d):
    """beta = 0 makes every M diagonal.  Channels 0 mod 4 get the configs'
    fast gates and forget within a few chunks; the others get long-memory
    gates.  So M, and the fix-up's propagated state, keep nonzero rows only
    in the channels that are not 0 mod 4.  These are the elements a zero test
    misses if it reads one float in four.  Each stage is compared with the
    oracle."""
    say(f"segment path {dtype} d={d} algo={algo}: beta=0, fast gates on channels 0 mod 4")
    T = 1300
    seg = [0, 448, 896, 1300]
    w = make_workload("t", [T], 2, d, d, dtype, 4100 + d + algo, s0_std=0.5, seg_start=seg)
    slow = make_workload("t", [T], 2, d, d, dtype, 4100 + d + algo, gate_shift=-9.0)
    keep = np.arange(d) % 4 != 0
    w.g[:, :, keep] = slow.g[:, :, keep]
    w.beta[...] = 0.0
    r = _segment_case(K, w, algo, interval=128)
    q, k, v, g, b = (w.f64(x) for x in ("q", "k", "v", "g", "beta"))
    tol_o, tol_s = OUT_TOL[dtype], STATE_TOL[dtype]
    Ms, Ds = [], []
    for j in range(len(seg) - 1):
        Mr, Dr, olr = oracle.package(q, k, v, g, b, seg[j], seg[j + 1])
        # the premise: M diagonal, below fp32's smallest value on the fast
        # channels and near 1 on the others
        diag = np.abs(np.diagonal(Mr, axis1=1, axis2=2))
        assert np.count_nonzero(Mr - np.stack([np.diag(x) for x in np.diagonal(Mr, axis1=1, axis2=2)])) == 0
        assert diag[:, ~keep].max() < 1e-46 and diag[:, keep].min() > 0.5
        Ms.append(Mr)
        Ds.append(Dr)
        assert_close(f"M[{j}]", r["M"][j], Mr, tol_s)
        assert_close(f"D[{j}]", r["D"][j], Dr, tol_s)
    S_in_ref, _ = oracle.scan_sequential(Ms, Ds, w.S0[0].astype(np.float64))
    assert_close("S_in", r["S_in"], S_in_ref, tol_s)
    ro, rS, rck = oracle_full(w, interval=128)
    assert_close("S_final", r["S_final"], rS[0], tol_s)
    assert_close("o", r["o"], ro, tol_o)
    assert_close("ckpt", r["ckpt"], rck, tol_s)


@pytest.mark.parametrize("nseg", [4096, 2500])
def test_scan_blelloch_largest_tree(K, nseg):
    """The Blelloch scan at its largest padded size (4096 packages): a tree
    level lists up to 2048 products.  A few M are zero."""
    import torch
    from workloads import make_packages
    H, d = 2, 64
    zero = tuple(range(5, nseg, 97))
    say(f"Blelloch scan nseg={nseg} (padded 4096), H={H}, d={d}, {len(zero)} zero M")
    M, D, S0 = make_packages(nseg, H, d, d, 7300 + nseg, zero=zero)
    tM, tD, tS0 = (torch.from_numpy(x).cuda() for x in (M, D, S0))
    S_in, S_fin = K.kda_segment_scan(tM, tD, tS0, algo=1)
    sync()
    S_in_ref, S_fin_ref = oracle.scan_sequential([m.astype(np.float64) for m in M],
                                                 [x.astype(np.float64) for x in D],
                                                 S0.astype(np.float64))
    assert_close("S_in", to_numpy_f64(S_in), S_in_ref, OUT_TOL["f32"])
    assert_close("S_final", to_numpy_f64(S_fin), S_fin_ref, STATE_TOL["f32"])


@pytest.mark.parametrize("algo", [0, 1])
def test_scan_M_nonzero_off_every_fourth_column(K, algo):
    """Packages whose M is nonzero only in columns that are not 0 mod 4 are
    not zero packages: the scans form their products."""
    import torch
    from workloads import make_packages
    nseg, H, d = 6, 3, 128
    M, D, S0 = make_packages(nseg, H, d, d, 4170 + algo)
    M[:, :, :, 0::4] = 0.0
    M[2, 1] = 0.0
    M[2, 1, 7, 5] = 0.5           # one nonzero element
    say(f"scan algo={algo}: M zero in every column 0 mod 4")
    tM, tD, tS0 = (torch.from_numpy(x).cuda() for x in (M, D, S0))
    S_in, S_fin = K.kda_segment_scan(tM, tD, tS0, algo=algo)
    sync()
    S_in_ref, S_fin_ref = oracle.scan_sequential([m.astype(np.float64) for m in M],
                                                 [x.astype(np.float64) for x in D],
                                                 S0.astype(np.float64))
    assert_close("S_in", to_numpy_f64(S_in), S_in_ref, OUT_TOL["f32"])
    assert_close("S_final", to_numpy_f64(S_fin), S_fin_ref, STATE_TOL["f32"])


@pytest.mark.parametrize("algo", [0, 1])
@pytest.mark.parametrize("nseg,zero", [(13, (1, 4, 5, 9, 12)), (16, (0, 2, 3, 7, 8, 11, 15)),
                                       (16, tuple(range(1, 16))), (5, ()), (1, ()), (1, (0,)),
                                       (2, (0,)), (3, (1,)), (33, (0, 5, 6, 7, 20, 31, 32))])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("with_s0", [True, False])
def test_scan_mixed_zero_packages(K, algo, nseg, zero, d, with_s0):
    """Scans over packages where some M are exactly zero and others are not:
    the zero flags decide which products and moves the scan skips."""
    import torch
    from workloads import make_packages
    say(f"scan algo={algo} nseg={nseg} zero M at {list(zero)} d={d} S0={with_s0}")
    M, D, S0 = make_packages(nseg, 3, d, d, 60 + nseg + d + len(zero), zero=zero)
    tM, tD = torch.from_numpy(M).cuda(), torch.from_numpy(D).cuda()
    tS0 = torch.from_numpy(S0).cuda() if with_s0 else None
    S_in, S_fin = K.kda_segment_scan(tM, tD, tS0, algo=algo)
    sync()
    ref_S0 = S0.astype(np.float64) if with_s0 else np.zeros((3, d, d))
    S_in_ref, S_fin_ref = oracle.scan_sequential([m.astype(np.float64) for m in M],
                                                 [x.astype(np.float64) for x in D], ref_S0)
    assert_close("S_in", to_numpy_f64(S_in), S_in_ref, OUT_TOL["f32"])
    assert_close("S_final", to_numpy_f64(S_fin), S_fin_ref, STATE_TOL["f32"])
    # the inputs are left as they were
    assert np.array_equal(tM.cpu().numpy(), M) and np.array_equal(tD.cpu().numpy(), D)


@pytest.mark.parametrize("H,dk,dv,nseg,zero", [(10, 128, 64, 9, (0, 3, 4, 8)),
                                               (17, 64, 128, 17, (2, 5, 6, 9, 16)),
                                               (8, 128, 128, 8, tuple(range(8)))])
def test_scan_sequential_heads_and_shapes(K, H, dk, dv, nseg, zero):
    """Sequential scan with head counts that are not (or are) a multiple of 8,
    dk != dv, and package counts across the batches of the walk."""
    import torch
    from workloads import make_packages
    say(f"sequential scan H={H} dk={dk} dv={dv} nseg={nseg} zero M at {list(zero)}")
    M, D, S0 = make_packages(nseg, H, dk, dv, 7100 + H + nseg, zero=zero)
    tM, tD, tS0 = (torch.from_numpy(x).cuda() for x in (M, D, S0))
    S_in, S_fin = K.kda_segment_scan(tM, tD, tS0, algo=0)
    sync()
    S_in_ref, S_fin_ref = oracle.scan_sequential([m.astype(np.float64) for m in M],
                                                 [x.astype(np.float64) for x in D],
                                                 S0.astype(np.float64))
    assert_close("S_in", to_numpy_f64(S_in), S_in_ref, OUT_TOL["f32"])
    assert_close("S_final", to_numpy_f64(S_fin), S_fin_ref, STATE_TOL["f32"])
    if len(zero) == nseg:   # every step a copy: exact
        assert np.array_equal(to_numpy_f64(S_fin), D[-1].astype(np.float64))


@pytest.mark.parametrize("H,dk,dv,nseg,zero", [(10, 128, 64, 9, (0, 3, 4, 8)),
                                               (8, 128, 128, 8, tuple(range(8)))])
def test_scan_sequential_without_workspace(K, H, dk, dv, nseg, zero):
    """The sequential scan's workspace is optional: without it every
    workgroup tests M itself, with it one launch tests each M once.  Both give
    the same bits."""
    import ctypes
    import torch
    from workloads import make_packages
    say(f"sequential scan with and without its workspace H={H} nseg={nseg}")
    M, D, S0 = make_packages(nseg, H, dk, dv, 7300 + H + nseg, zero=zero)
    tM, tD, tS0 = (torch.from_numpy(x).cuda() for x in (M, D, S0))
    S_in, S_fin = K.kda_segment_scan(tM, tD, tS0, algo=0)
    cfg = K.kda_config(H, dk, dv, K.CHUNK, K.KDA_DTYPE_BF16, 1.0, 1)
    assert K.LIB.kda_segment_scan_workspace(ctypes.byref(cfg), nseg, 0) > 0
    S_in2, S_fin2 = torch.empty_like(S_in), torch.empty_like(S_fin)
    st = K.LIB.kda_segment_scan(ctypes.byref(cfg), nseg, K._p(tM), K._p(tD), K._p(tS0),
                                K._p(S_in2), K._p(S_fin2), 0, None, 0, K._stream(None))
    sync()
    assert st == 0
    assert torch.equal(S_in, S_in2) and torch.equal(S_fin, S_fin2)


def test_segment_path_config_gates_bf16(K):
    """The configs' gates: M underflows to exactly zero after a few chunks."""
    say("segment path bf16 d=128 config gates, 4 segments of 512")
    w = make_workload("t", [2048], 2, 128, 128, "bf16", 16, s0_std=0.1,
                      seg_start=[0, 512, 1024, 1536, 2048])
    r = _segment_case(K, w, 1, interval=256)
    assert np.count_nonzero(r["M"]) == 0
    ro, rS, rck = oracle_full(w, interval=256)
    assert_close("o", r["o"], ro, OUT_TOL["bf16"])
    assert_close("S_final", r["S_final"], rS[0], STATE_TOL["bf16"])
    assert_close("ckpt", r["ckpt"], rck, STATE_TOL["bf16"])


def test_segment_single_segment_equals_prefill(K):
    say("segment path with one segment vs chunked prefill (fp32 d=64)")
    w = make_workload("t", [333], 1, 64, 64, "f32", 17, s0_std=0.2, seg_start=[0, 333])
    r = _segment_case(K, w, 0, interval=0)
    o, Sf, _ = run_prefill(K, w)
    assert_close("o vs prefill", r["o"], o, 1e-5)
    assert_close("S_final vs prefill", r["S_final"], Sf[0], 1e-5)


def test_segment_package_without_M(K):
    say("package without M: o_local, D, sub_D identical to the full call (bf16 d=128)")
    import torch
    w = make_workload("t", [1024], 2, 128, 128, "bf16", 23, s0_std=None,
                      seg_start=[0, 320, 640, 1024])
    t = to_torch(w)
    full = K.kda_segment_package(t["q"], t["k"], t["v"], t["g"], t["beta"], t["seg_start"],
                                 ckpt_interval=128)
    part = K.kda_segment_package(t["q"], t["k"], t["v"], t["g"], t["beta"], t["seg_start"],
                                 ckpt_interval=128, want_M=False)
    sync()
    assert part[1] is None and part[3] is None
    assert torch.equal(full[0], part[0])
    assert torch.equal(full[2], part[2])
    assert torch.equal(full[4], part[4])


@pytest.mark.parametrize("gates", ["config", "long"])
def test_package_split_without_M(K, gates):
    """Split packages without M (2 segments of 4096 tokens on 2 heads, 8
    sub-segments each): the merge composes D alone, the last sub-segments'
    M staying in the workspace.  o_local, D and sub_D are bit-identical to
    the split call with M, which the split tests compare with the oracle."""
    import torch
    shift = {} if gates == "config" else dict(gate_shift=-9.0, beta_shift=-6.0)
    w = make_workload("split-noM", [8192], 2, 128, 128, "bf16", 5530, s0_std=None,
                      seg_start=[0, 4096, 8192], **shift)
    say(f"split package without M, gates={gates}")
    t = to_torch(w)
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"], t["seg_start"])
    full = K.kda_segment_package(*args, ckpt_interval=512)
    part = K.kda_segment_package(*args, ckpt_interval=512, want_M=False)
    sync()
    assert part[1] is None and part[3] is None
    if gates == "long":
        assert float(full[1].abs().max()) > 1e-3, "long-memory gates should leave M nonzero"
    for name, i in (("o_local", 0), ("D", 2), ("sub_D", 4)):
        assert torch.equal(full[i], part[i]), name


def test_validate_inputs_counts_planted_faults(K):
    """The debug input check is silent on the workloads' inputs and counts
    exactly the faults planted on a copy of them (integer counts)."""
    import torch
    w = make_workload("validate", [300, 0, 517, 64], 2, 128, 128, "bf16", 5700, s0_std=None)
    t = to_torch(w)
    T, H, dk = w.T, 2, 128
    say("input validation on clean and faulty inputs")
    clean = K.kda_validate_inputs(T=T, H=H, dk=dk, g=t["g"], beta=t["beta"], bounds=t["cu_seqlens"])
    assert clean == dict.fromkeys(K.CHECK_NAMES, 0), clean
    seg = torch.tensor([0, 128, 448, T], dtype=torch.int64, device="cuda")
    assert K.kda_validate_inputs(T=T, H=H, dk=dk, g=t["g"], bounds=seg, chunk_aligned=True) \
        == dict.fromkeys(K.CHECK_NAMES, 0)
    # planted: three g > 0, one NaN, one block of 16 summing below -80 in one
    # channel, two non-finite betas, bounds out of order / off the chunk grid
    g, beta = t["g"].clone(), t["beta"].clone()
    g[5, 0, 3] = 0.5
    g[400, 1, 100] = 1e-3
    g[880, 1, 0] = 2.0
    g[77, 0, 64] = float("nan")
    start = 300 + 32                                  # a block start of sequence 2 (starts at 300)
    g[start:start + 16, 1, 17] = -6.0                 # 16 x -6 = -96 < -80
    beta[10, 1] = float("inf")
    beta[600, 0] = float("nan")
    r = K.kda_validate_inputs(T=T, H=H, dk=dk, g=g, beta=beta, bounds=t["cu_seqlens"])
    assert r == {"bounds": 0, "g_positive": 3, "g_nonfinite": 1, "g_block_floor": 1,
                 "beta_nonfinite": 2}, r
    bad_cu = t["cu_seqlens"].clone()
    bad_cu[2] = bad_cu[1] - 1                          # a decrease
    assert K.kda_validate_inputs(T=T, H=H, dk=dk, bounds=bad_cu, g=t["g"])["bounds"] == 1
    bad_seg = torch.tensor([0, 100, 448, T + 1], dtype=torch.int64, device="cuda")
    # 100 off the chunk grid, the last entry not T (the block sums stop at T)
    assert K.kda_validate_inputs(T=T, H=H, dk=dk, g=t["g"], bounds=bad_seg,
                                 chunk_aligned=True)["bounds"] == 2


# ---------------------------------------------------------------------------
# Prefill resumed from a state pool
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_prefill_resume_parity(K, dtype, d):
    """Four sequences continue from pool slots (in place, fork, zero state,
    state discarded) at absolute positions 0, 128, 192, 4096 with rungs
    every 128 tokens on the absolute grid; outputs, written slots and rungs
    against the oracle, untouched slots bit-identical."""
    import torch
    lengths = [300, 64, 257, 100]
    pos0 = [0, 128, 192, 4096]
    w = make_workload("resume", lengths, 3, d, d, dtype, 4611, s0_std=None)
    t = to_torch(w)
    n_slots = 6
    rng = np.random.default_rng(4612)
    pool_np = (0.1 * rng.standard_normal((n_slots, 3, d, d))).astype(np.float32)
    read = np.array([2, 4, -1, 1], dtype=np.int32)
    write = np.array([2, 5, 0, -1], dtype=np.int32)
    iv = 128
    off = ckpt_offsets(lengths, iv, pos0=pos0)
    say(f"prefill resume {dtype} d={d}: lengths {lengths} pos0 {pos0} rungs {int(off[-1])}")
    pool = torch.from_numpy(pool_np).cuda()
    before = pool.clone()
    o, ck = K.kda_prefill_resume(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                                 pool, torch.from_numpy(read).cuda(), torch.from_numpy(write).cuda(),
                                 pos0=torch.tensor(pos0, dtype=torch.int64, device="cuda"),
                                 ckpt_interval=iv, ckpt_offsets=torch.from_numpy(off).cuda())
    sync()
    o_ref, pool_ref, ck_ref = oracle.prefill_resume(w.f64("q"), w.f64("k"), w.f64("v"),
                                                    w.f64("g"), w.f64("beta"), w.cu_seqlens,
                                                    pool_np, read, write, pos0=pos0,
                                                    ckpt_interval=iv)
    assert ck.shape[0] == ck_ref.shape[0] == int(off[-1])
    assert_close("resume o", to_numpy_f64(o), o_ref, OUT_TOL[dtype])
    assert_close("resume written slots", to_numpy_f64(pool[[0, 2, 5]]), pool_ref[[0, 2, 5]],
                 STATE_TOL[dtype])
    assert_close("resume rungs", to_numpy_f64(ck), ck_ref, STATE_TOL[dtype])
    assert torch.equal(pool[[1, 3, 4]], before[[1, 3, 4]])


def test_prefill_resume_from_own_rung_is_exact(K):
    """Resuming from a rung the GPU wrote reproduces the GPU's continuous
    run bit for bit: same chunk grid, same fp32 state, same arithmetic."""
    import torch
    lengths = [1000, 777]
    w = make_workload("resume-own", lengths, 4, 128, 128, "bf16", 4613, s0_std=0.1)
    iv = 256
    o, Sf, ck = run_prefill_t(K, w, interval=iv)
    # sequence 0 resumes at 512 (its rung 2), sequence 1 at 256 (its rung 1)
    starts = [512, 256]
    off = ckpt_offsets(lengths, iv)
    t = to_torch(w)
    sel = torch.cat([torch.arange(512, 1000), torch.arange(1000 + 256, 1777)]).cuda()
    pool = torch.stack([ck[int(off[0]) + 1], ck[int(off[1]) + 0]]).contiguous()
    cu = torch.tensor([0, 488, 488 + 521], dtype=torch.int64, device="cuda")
    off2 = ckpt_offsets([488, 521], iv, pos0=starts)
    idx = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    say("prefill resume from the GPU's own rungs, bf16 d=128")
    o2, ck2 = K.kda_prefill_resume(t["q"][sel].contiguous(), t["k"][sel].contiguous(),
                                   t["v"][sel].contiguous(), t["g"][sel].contiguous(),
                                   t["beta"][sel].contiguous(), cu, pool, idx, idx,
                                   pos0=torch.tensor(starts, dtype=torch.int64, device="cuda"),
                                   ckpt_interval=iv, ckpt_offsets=torch.from_numpy(off2).cuda())
    sync()
    assert torch.equal(o2, o[sel])
    assert torch.equal(pool, Sf)
    # later rungs: sequence 0 at 768 (row 2 of 3), sequence 1 at 512 and 768 (rows 1, 2 of 3)
    assert torch.equal(ck2, ck[[2, int(off[1]) + 1, int(off[1]) + 2]])


# ---------------------------------------------------------------------------
# Decode against a state pool
# ---------------------------------------------------------------------------
def _decode_case(K, b, name):
    import torch
    from workloads.device import decode_to_torch
    say(f"decode {name}: N={b.N} H={b.H} dk={b.dk} dv={b.dv} {b.dtype} logits={b.gate_logits}")
    t = decode_to_torch(b)
    pool_in = t["pool"].clone()
    o = K.kda_decode(t["q"], t["k"], t["v"], t["g"], t["beta"], t["pool"], t["read_idx"],
                     t["write_idx"], gate_logits=b.gate_logits, scale=b.scale,
                     qk_l2norm=bool(b.qk_l2norm))
    sync()
    o_ref, pool_ref = oracle.decode(b.f64("q"), b.f64("k"), b.f64("v"), b.f64("g"),
                                    b.f64("beta"), b.pool, b.read_idx, b.write_idx,
                                    gate_logits=b.gate_logits, scale=b.scale,
                                    qk_l2norm=b.qk_l2norm)
    assert_close(f"decode {name} o", to_numpy_f64(o), o_ref, OUT_TOL[b.dtype])
    n_slots = b.pool.shape[0]
    written = sorted({int(w) for w in b.write_idx if 0 <= w < n_slots})
    if written:
        assert_close(f"decode {name} written states", to_numpy_f64(t["pool"][written]),
                     pool_ref[written], STATE_TOL[b.dtype])
    kept = [i for i in range(n_slots) if i not in written]
    assert torch.equal(t["pool"][kept], pool_in[kept]), "a slot that is not written changed"


@pytest.mark.parametrize("dtype,dk,dv,logits", [("bf16", 128, 128, True), ("bf16", 64, 64, False),
                                                ("f32", 64, 64, True), ("f32", 128, 64, False),
                                                ("bf16", 64, 128, True)])
def test_decode_parity(K, dtype, dk, dv, logits):
    from workloads import make_decode_batch
    b = make_decode_batch("decode-small", 20, 3, dk, dv, dtype, 4601, gate_logits=logits)
    _decode_case(K, b, f"{dtype} {dk}x{dv}")


@pytest.mark.parametrize("dtype,d,l2,scale", [("bf16", 128, 0, 1.0), ("f32", 64, 1, 0.125)])
def test_decode_scale_and_no_l2norm(K, dtype, d, l2, scale):
    """Decode with a query scale and with the in-kernel L2 norm off (q, k
    scaled by 2^-4 so that the update contracts)."""
    from workloads import make_decode_batch, scale_qk_pow2
    b = make_decode_batch("decode-opts", 24, 3, d, d, dtype, 4602, gate_logits=True)
    b.scale, b.qk_l2norm = scale, l2
    if not l2:
        scale_qk_pow2(b, -4)
    _decode_case(K, b, f"{dtype} d={d} l2norm={l2} scale={scale}")


def test_decode_standard_batch(K):
    """64 sequences, H=32, d=128, bf16, 128-slot pool, gate logits: the
    decode workload the benchmark times, compared in full."""
    from workloads import standard_decode_batch
    _decode_case(K, standard_decode_batch(), "n64")


def test_decode_out_of_range_slots(K):
    """Indices outside [0, n_slots) read a zero state and write nothing."""
    from workloads import make_decode_batch
    b = make_decode_batch("decode-oob", 6, 2, 64, 64, "f32", 4602, n_slots=12,
                          read_idx=[0, 12, -3, 1, 99, 2], write_idx=[6, 7, 8, 12, 9, -1])
    _decode_case(K, b, "out of range")


def test_decode_chain_equals_prefill(K):
    """Sixteen decode steps in place on one slot against the oracle's
    prefill of the same sixteen tokens from that slot's state."""
    import torch
    w = make_workload("decode-chain", [16], 2, 128, 128, "bf16", 4603, s0_std=0.1)
    t = to_torch(w)
    pool = torch.zeros((3, 2, 128, 128), dtype=torch.float32, device="cuda")
    pool[2] = t["S0"][0]
    idx = torch.tensor([2], dtype=torch.int32, device="cuda")
    say("decode chain: 16 steps, H=2, d=128, bf16")
    outs = []
    for s_ in range(16):
        outs.append(K.kda_decode(t["q"][s_:s_ + 1], t["k"][s_:s_ + 1], t["v"][s_:s_ + 1],
                                 t["g"][s_:s_ + 1], t["beta"][s_:s_ + 1], pool, idx, idx))
    sync()
    o_ref, Sf_ref, _ = oracle_full(w)
    assert_close("decode chain o", to_numpy_f64(torch.cat(outs)), o_ref, OUT_TOL["bf16"])
    assert_close("decode chain state", to_numpy_f64(pool[2]), Sf_ref[0], STATE_TOL["bf16"])
    assert float(pool[:2].abs().max()) == 0.0


def test_decode_empty_batch(K):
    import torch
    pool = torch.randn((2, 1, 64, 64), device="cuda")
    before = pool.clone()
    e = torch.empty((0, 1, 64), dtype=torch.bfloat16, device="cuda")
    o = K.kda_decode(e, e, e, torch.empty((0, 1, 64), device="cuda"),
                     torch.empty((0, 1), device="cuda"), pool,
                     torch.empty(0, dtype=torch.int32, device="cuda"),
                     torch.empty(0, dtype=torch.int32, device="cuda"))
    sync()
    assert o.shape == (0, 1, 64) and torch.equal(pool, before)


# ---------------------------------------------------------------------------
# Short causal convolution
# ---------------------------------------------------------------------------
def _conv_case(K, c, act, name):
    import torch
    from workloads.device import conv_to_torch
    W = c.weight.shape[1]
    say(f"short conv {name}: T={c.x.shape[0]} C={c.x.shape[1]} W={W} {c.dtype} act={act}")
    t = conv_to_torch(c)
    before = t["windows"].clone()
    y = K.kda_short_conv(t["x"], t["cu_seqlens"], t["weight"], t["bias"], windows=t["windows"],
                         read_idx=t["read_idx"], write_idx=t["write_idx"], activation=act)
    sync()
    y_ref, win_ref = oracle.short_conv(c.f64("x"), c.cu_seqlens, c.weight, c.bias,
                                       windows=c.f64("windows"), read_idx=c.read_idx,
                                       write_idx=c.write_idx, activation=act)
    assert_close(f"short conv {name} y", to_numpy_f64(y), y_ref, OUT_TOL[c.dtype])
    # windows hold inputs: bit-exact
    np.testing.assert_array_equal(to_numpy_f64(t["windows"]), win_ref)
    n_slots = c.windows.shape[0]
    written = {int(w) for w in c.write_idx if 0 <= w < n_slots}
    kept = [i for i in range(n_slots) if i not in written]
    assert torch.equal(t["windows"][kept], before[kept])


@pytest.mark.parametrize("dtype,W,act", [("bf16", 4, 1), ("bf16", 2, 0), ("f32", 8, 1), ("f32", 3, 0)])
def test_short_conv_parity(K, dtype, W, act):
    """Ragged sequences (1 to 300 rows, one empty) across 64-row tiles, with
    in-place, forked, fresh and discarded windows."""
    from workloads import make_conv_case
    c = make_conv_case("conv-small", [300, 1, 0, 65, 2, 130, 7, 64], 264, W, dtype, 4621)
    _conv_case(K, c, act, f"{dtype} W={W}")


def test_short_conv_decode_batch(K):
    """One token per sequence (64 sequences) over q, k, v side by side:
    the decode form of the convolution, windows shifted in their slots."""
    from workloads import make_conv_case
    c = make_conv_case("conv-decode", [1] * 64, 3 * 32 * 128, 4, "bf16", 4622)
    _conv_case(K, c, 1, "decode n64")


def test_short_conv_halo_equals_whole_sequence(K):
    """Per-segment convolution fed by kda_conv_halo equals the whole
    sequence's convolution bit for bit (same fp32 sums per output)."""
    import torch
    from workloads import make_conv_case
    c = make_conv_case("conv-halo", [4096], 512, 4, "bf16", 4623, n_slots=1,
                       read_idx=[-1], write_idx=[-1])
    from workloads.device import conv_to_torch
    t = conv_to_torch(c)
    say("conv halo: 4096 rows, 512 channels, W=4, 5 segments")
    y_all = K.kda_short_conv(t["x"], t["cu_seqlens"], t["weight"], t["bias"], activation=1)
    bounds = torch.tensor([0, 640, 1280, 2048, 3072, 4096], dtype=torch.int64, device="cuda")
    halos = torch.zeros((6, 3, 512), dtype=torch.bfloat16, device="cuda")
    K.kda_conv_halo(t["x"], bounds, 4, halos, torch.arange(1, 6, dtype=torch.int32, device="cuda"))
    y_seg = K.kda_short_conv(t["x"], bounds, t["weight"], t["bias"], windows=halos,
                             read_idx=torch.arange(0, 5, dtype=torch.int32, device="cuda"),
                             activation=1)
    sync()
    assert torch.equal(y_seg, y_all)
    assert torch.equal(halos[1], t["x"][637:640])
    assert float(halos[0].float().abs().max()) == 0.0


def test_short_conv_full_size_sampled(K):
    """q of the 131,072-token workload (4096 channels, bf16, W = 4, SiLU) in
    the launch bench.py times; 512 sampled rows recomputed by the oracle from
    their own W rows."""
    import torch
    w = standard_workload(3)
    T, H, dk = w.q.shape
    C = H * dk
    rng = np.random.default_rng(4624)
    weight = (rng.standard_normal((C, 4)) / 2.0).astype(np.float32)
    bias = (0.1 * rng.standard_normal(C)).astype(np.float32)
    t = to_torch(w)
    x = t["q"].reshape(T, C)
    say("short conv full size: T=131072, C=4096, bf16")
    y = K.kda_short_conv(x, torch.tensor([0, T], dtype=torch.int64, device="cuda"),
                         torch.from_numpy(weight).cuda(), torch.from_numpy(bias).cuda(), activation=1)
    sync()
    rows = np.sort(rng.choice(T, 512, replace=False))
    rows[0] = 0
    got = to_numpy_f64(y[torch.from_numpy(rows).cuda()])
    from workloads import to_f64
    xq = w.q.reshape(T, C)
    ref = np.stack([oracle.short_conv(to_f64(xq[max(0, r - 3):r + 1], "bf16"), [0, min(r, 3) + 1],
                                      weight, bias, activation=1)[0][-1] for r in rows])
    assert_close("short conv full-size sampled rows", got, ref, OUT_TOL["bf16"])


# ---------------------------------------------------------------------------
# Non-finite inputs propagate; exact-zero shortcuts do not mask them
# ---------------------------------------------------------------------------
BF16_NAN = 0x7FC0


def test_nan_propagation_prefill(K):
    """A NaN in one key channel of one token reaches every later output of
    that (sequence, head) and its final state and later rungs (the oracle's
    answer: the normalised key, then the state, is NaN from that token on).
    Chunks before it and every other sequence and head match the oracle."""
    lens = [300, 500, 200]
    w = make_workload("nan", lens, 2, 128, 128, "bf16", 4900, s0_std=0.1)
    n, h, rel = 1, 1, 150
    tok = lens[0] + rel
    w.k[tok, h, 5] = BF16_NAN
    say(f"NaN in k at token {tok} (sequence {n}, head {h}), prefill bf16 d=128, rungs every 128")
    o, Sf, ck = run_prefill(K, w, interval=128)
    ro, rS, rck = oracle_full(w, interval=128)
    off = ckpt_offsets(w.lengths, 128)
    # the oracle itself: NaN from the token on, finite before
    assert np.isnan(ro[tok:tok + lens[1] - rel, h]).all() and np.isfinite(ro[:tok, h]).all()
    chunk0 = lens[0] + (rel // 64) * 64          # first row of the chunk holding the NaN
    end = lens[0] + lens[1]
    assert np.isnan(o[tok:end, h]).all(), "rows from the NaN token on must all be NaN"
    assert np.isnan(Sf[n, h]).all()
    assert_close("o before the NaN's chunk", o[lens[0]:chunk0, h], ro[lens[0]:chunk0, h], OUT_TOL["bf16"])
    for m in range(3):
        for hh in range(2):
            if (m, hh) == (n, h):
                continue
            a, b = w.cu_seqlens[m], w.cu_seqlens[m + 1]
            assert_close(f"o[seq {m}, head {hh}]", o[a:b, hh], ro[a:b, hh], OUT_TOL["bf16"])
            assert_close(f"S_final[seq {m}, head {hh}]", Sf[m, hh], rS[m, hh], STATE_TOL["bf16"])
    rows = range(int(off[n]), int(off[n + 1]))   # rungs at 128, 256, 384 of sequence 1
    assert_close("rung before the NaN", ck[rows[0], h], rck[rows[0], h], STATE_TOL["bf16"])
    for r in rows[1:]:
        assert np.isnan(ck[r, h]).all()
    assert np.isfinite(ck[:, 0]).all()


@pytest.mark.parametrize("algo", [0, 1])
@pytest.mark.parametrize("gates", ["config", "long"])
def test_nan_propagation_segment_path(K, algo, gates):
    """A NaN in a key of segment 1 (head 1) reaches every later output of
    that head, its final state and later rungs through the packages, the
    scan, the fix-up and the checkpoint writer.  With the configs' gates the
    next segment's M is exactly zero: the scans must still form 0 * NaN
    rather than pass D on.  Head 0 and segment 0 match the oracle."""
    shift = {} if gates == "config" else dict(gate_shift=-9.0, beta_shift=-6.0)
    seg = [0, 512, 1024, 1536, 2048]
    w = make_workload("nan-seg", [2048], 2, 128, 128, "bf16", 4901 + algo, s0_std=0.3,
                      seg_start=seg, **shift)
    h, tok = 1, 600
    w.k[tok, h, 77] = BF16_NAN
    say(f"NaN in k at token {tok} head {h}, segment path algo={algo} gates={gates}")
    r = _segment_case(K, w, algo, interval=128)
    ro, rS, rck = oracle_full(w, interval=128)
    if gates == "config":
        assert np.count_nonzero(r["M"][2, h]) == 0     # the shortcut is really taken
    else:
        assert np.count_nonzero(r["M"][2, h]) > 0
    assert np.isnan(r["M"][1, h]).all() and np.isnan(r["D"][1, h]).all()
    assert np.isnan(r["S_in"][2:, h]).all()
    assert np.isnan(r["o"][tok:, h]).all(), "rows from the NaN token on must all be NaN"
    assert np.isnan(r["S_final"][h]).all()
    assert_close("o, segment 0, head 1", r["o"][:512, h], ro[:512, h], OUT_TOL["bf16"])
    assert_close("o, head 0", r["o"][:, 0], ro[:, 0], OUT_TOL["bf16"])
    assert_close("S_final, head 0", r["S_final"][0], rS[0, 0], STATE_TOL["bf16"])
    assert_close("rungs 128 .. 512, head 1", r["ckpt"][:4, h], rck[:4, h], STATE_TOL["bf16"])
    assert np.isnan(r["ckpt"][4:, h]).all()
    assert_close("rungs, head 0", r["ckpt"][:, 0], rck[:, 0], STATE_TOL["bf16"])


@pytest.mark.parametrize("algo", [0, 1])
def test_scan_zero_M_against_nonfinite(K, algo):
    """Scans over random packages where a zero M meets an infinite or NaN
    operand: the zero shortcut is taken only against finite values, so the
    result has NaN exactly in the columns the product 0 * x makes NaN, and
    every other column equals the oracle's scan."""
    import torch
    from workloads import make_packages
    nseg, H, d = 6, 2, 64
    M, D, S0 = make_packages(nseg, H, d, d, 4950 + algo, zero=(1, 2, 4))
    D[0, 1, 3, 7] = np.inf         # head 1: column 7 of D_0, then of S_in[1]
    S0[0, 5, 9] = np.nan           # head 0: column 9 of S0
    say(f"scan algo={algo} with inf / NaN operands against zero M")
    tM, tD, tS0 = (torch.from_numpy(x).cuda() for x in (M, D, S0))
    S_in, S_fin = K.kda_segment_scan(tM, tD, tS0, algo=algo)
    sync()
    S_in, S_fin = to_numpy_f64(S_in), to_numpy_f64(S_fin)
    # the oracle's scan of the same algorithm: with infinities the order of
    # the products decides between inf and NaN (A (B x) and (A B) x differ),
    # so the Blelloch tree is compared with the oracle's Blelloch tree
    scan = oracle.scan_blelloch if algo == 1 else oracle.scan_sequential
    with np.errstate(invalid="ignore"):
        ref_in, ref_fin = scan([m.astype(np.float64) for m in M],
                               [x.astype(np.float64) for x in D], S0.astype(np.float64))
    # numpy's matmul is IEEE: the oracle marks the same entries
    for name, got, ref in (("S_in", S_in, ref_in), ("S_final", S_fin, ref_fin)):
        assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{name}: NaN pattern differs"
        assert np.array_equal(np.isinf(got), np.isinf(ref)), f"{name}: inf pattern differs"
        fin = np.isfinite(ref)
        assert_close(f"{name} (finite entries)", got[fin], ref[fin], 1e-4)
    # the NaN columns really appear after a zero M
    assert np.isnan(ref_in[2, 1, :, 7]).all() and np.isnan(ref_in[1, 0, :, 9]).all()


# ---------------------------------------------------------------------------
# Stream ordering of checkpoint stores
# ---------------------------------------------------------------------------
def test_checkpoint_stream_ordering(K):
    """Rung states read on a second stream after an event recorded on the
    compute stream right after the producing call are the fresh ones: every
    kernel of kda_prefill and of the segment path runs on the stream it is
    given.  Each rung buffer is filled with NaN first, behind a long queue of
    work on the compute stream.  The copy made without waiting on the event
    is reported (how much of it was fresh), not asserted."""
    import torch
    w = make_workload("order", [8192], 4, 128, 128, "bf16", 4960, s0_std=0.1,
                      seg_start=[0, 2048, 4096, 6144, 8192])
    t = to_torch(w)
    compute, store = torch.cuda.Stream(), torch.cuda.Stream()
    ref = None
    fresh_unfenced = []
    for rep in range(3):
        for path in ("prefill", "segment"):
            ck = torch.full((8192 // 1024, 4, 128, 128), float("nan"), dtype=torch.float32,
                            device="cuda")
            torch.cuda.synchronize()    # the NaN sentinel is in place before anything runs
            with torch.cuda.stream(compute):
                for _ in range(4):      # queue ahead of the producer
                    K.kda_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"], t["S0"],
                                  workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
                if path == "prefill":
                    K.kda_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"], t["S0"],
                                  ckpt_interval=1024, ckpt_out=ck,
                                  ckpt_offsets=torch.tensor([0, 8], device="cuda"),
                                  workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
                else:
                    o, M, D, sM, sD = K.kda_segment_package(t["q"], t["k"], t["v"], t["g"],
                                                            t["beta"], t["seg_start"],
                                                            ckpt_interval=1024)
                    S_in, _ = K.kda_segment_scan(M, D, t["S0"][0].contiguous(), algo=1)
                    K.kda_checkpoint_write(t["seg_start"], S_in, sM, sD, T=8192, interval=1024,
                                           out=ck)
                ev = torch.cuda.Event()
                ev.record(compute)
            with torch.cuda.stream(store):
                early = ck.clone()      # no wait: may read the buffer before the rungs land
                store.wait_event(ev)
                late = ck.clone()
            ck.record_stream(store)
            torch.cuda.synchronize()
            fresh_unfenced.append(float(torch.isfinite(early).float().mean()))
            assert bool(torch.isfinite(late).all()), f"{path}: a fenced read saw a stale rung"
            got = to_numpy_f64(late)
            if ref is None:
                ref = oracle_full(w, interval=1024)[2]
            assert_close(f"{path} rungs read on the store stream (rep {rep})", got, ref,
                         STATE_TOL["bf16"])
    say(f"fresh fraction of the copies made without the fence: {fresh_unfenced}")


# ---------------------------------------------------------------------------
# Head dims dk != dv
# ---------------------------------------------------------------------------
SHAPES = [("bf16", 64, 128), ("bf16", 128, 64), ("f32", 64, 128), ("f32", 128, 128),
          ("f32", 128, 64)]


@pytest.mark.parametrize("dtype,dk,dv", SHAPES)
@pytest.mark.parametrize("H", [2, 32])
def test_prefill_dk_ne_dv(K, dtype, dk, dv, H):
    """Chunked prefill of varlen sequences with dk != dv, rungs every 64
    tokens; with 32 heads x 8 sequences the value columns run as 128-wide
    blocks where dv = 128 (bf16), with 2 heads as 64-wide blocks."""
    lens = [300, 77, 129, 64, 1, 200, 33, 130] if H == 32 else [300, 77, 129, 1]
    say(f"prefill {dtype} dk={dk} dv={dv} H={H} lens={lens}")
    w = make_workload("shape", lens, H, dk, dv, dtype, 5000 + dk + 3 * dv + H, s0_std=0.2)
    o, Sf, ck = run_prefill(K, w, interval=64)
    ro, rS, rck = oracle_full(w, interval=64)
    assert_close("o", o, ro, OUT_TOL[dtype])
    assert_close("S_final", Sf, rS, STATE_TOL[dtype])
    assert_close("ckpt", ck, rck, STATE_TOL[dtype])


@pytest.mark.parametrize("dtype,dk,dv", SHAPES)
@pytest.mark.parametrize("algo", [0, 1])
@pytest.mark.parametrize("H", [2, 32])
def test_segment_path_dk_ne_dv(K, dtype, dk, dv, algo, H):
    """The segment path with dk != dv and long-memory gates (nonzero M in
    every segment): M, D, o_local per segment, S_in, outputs, final state and
    rungs.  With 32 heads x 8 segments the value blocks are 128 wide where
    dv = 128 (bf16) while the M blocks stay dk wide."""
    seg = [0, 256, 320, 768, 1024, 1300] if H == 2 else [0, 128, 256, 384, 512, 640, 768, 832, 960]
    T = seg[-1]
    say(f"segment path {dtype} dk={dk} dv={dv} H={H} algo={algo}, {len(seg) - 1} segments, long memory")
    w = make_workload("shape-seg", [T], H, dk, dv, dtype, 5100 + dk + 3 * dv + algo + H,
                      s0_std=0.5, gate_shift=-9.0, beta_shift=-6.0, seg_start=seg)
    r = _segment_case(K, w, algo, interval=128)
    q, k, v, g, b = (w.f64(x) for x in ("q", "k", "v", "g", "beta"))
    tol_o, tol_s = OUT_TOL[dtype], STATE_TOL[dtype]
    Ms, Ds = [], []
    for j in range(len(seg) - 1):
        Mr, Dr, olr = oracle.package(q, k, v, g, b, seg[j], seg[j + 1])
        Ms.append(Mr)
        Ds.append(Dr)
        assert_close(f"M[{j}]", r["M"][j], Mr, tol_s)
        assert_close(f"D[{j}]", r["D"][j], Dr, tol_s)
        assert_close(f"o_local[{j}]", r["o_local"][seg[j]:seg[j + 1]], olr[seg[j]:seg[j + 1]], tol_o)
    S_in_ref, _ = oracle.scan_sequential(Ms, Ds, w.S0[0].astype(np.float64))
    assert_close("S_in", r["S_in"], S_in_ref, tol_s)
    ro, rS, rck = oracle_full(w, interval=128)
    assert_close("S_final", r["S_final"], rS[0], tol_s)
    assert_close("o", r["o"], ro, tol_o)
    assert_close("ckpt", r["ckpt"], rck, tol_s)


@pytest.mark.parametrize("dtype,dk,dv", SHAPES)
def test_single_sequence_split_dk_ne_dv(K, dtype, dk, dv):
    """One 4,096-token sequence on 4 heads: kda_prefill runs it as segments
    (queried workspace) and in one pass (minimal workspace); both against the
    oracle, with rungs every 512 tokens."""
    import torch
    w = make_workload("split-shape", [4096], 4, dk, dv, dtype, 5200 + dk + dv, s0_std=0.1)
    t = to_torch(w)
    ref = oracle_full(w, 512)
    for name, ws in (("split", None), ("one pass", torch.empty(256, dtype=torch.uint8, device="cuda"))):
        say(f"prefill {name}: T=4096 H=4 {dtype} dk={dk} dv={dv}")
        o, Sf, ck = K.kda_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                                  t["S0"], ckpt_interval=512, workspace=ws)
        sync()
        assert_close(f"{name} o", to_numpy_f64(o), ref[0], OUT_TOL[dtype])
        assert_close(f"{name} S_final", to_numpy_f64(Sf), ref[1], STATE_TOL[dtype])
        assert_close(f"{name} rungs", to_numpy_f64(ck), ref[2], STATE_TOL[dtype])


# ---------------------------------------------------------------------------
# Fix-up writing the checkpoint rungs (one launch)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("gates", ["config", "long"])
@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 64, 64), ("bf16", 64, 128),
                                         ("f32", 128, 128)])
def test_fixup_ckpt_equals_checkpoint_write(K, gates, dtype, dk, dv):
    """kda_output_fixup_ckpt leaves the same outputs as kda_output_fixup (bit
    for bit) and writes the rungs that kda_checkpoint_write forms from the
    sub-packages (same map, other rounding), both against the oracle, and
    the same rungs bit for bit when they are formed in place in sub_D; rungs
    at segment ends, inside segments, right after a segment start, and after
    the propagated state has reached zero."""
    import torch
    shift = {} if gates == "config" else dict(gate_shift=-9.0, beta_shift=-6.0)
    seg = [0, 448, 512, 1216, 1536, 2112]
    w = make_workload("fixup-rungs", [2112], 2, dk, dv, dtype, 5300 + dk + dv, s0_std=0.5,
                      seg_start=seg, **shift)
    say(f"fix-up with rungs {dtype} dk={dk} dv={dv} gates={gates}")
    t = to_torch(w)
    iv = 64 if gates == "config" else 128
    ol, M, D, sM, sD = K.kda_segment_package(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                             t["seg_start"], ckpt_interval=iv)
    S_in, _ = K.kda_segment_scan(M, D, t["S0"][0].contiguous(), algo=1)
    o1, o2 = ol.clone(), ol.clone()
    K.kda_output_fixup(t["q"], t["k"], t["g"], t["beta"], t["seg_start"], S_in, o1)
    ck_fused = K.kda_output_fixup_ckpt(t["q"], t["k"], t["g"], t["beta"], t["seg_start"], S_in, o2,
                                       sD, interval=iv)
    ck_two = K.kda_checkpoint_write(t["seg_start"], S_in, sM, sD, T=w.T, interval=iv,
                                    dtype=t["q"].dtype)
    # the rungs formed in place in sub_D: the same values, bit for bit
    o3, sD3 = ol.clone(), sD.clone()
    ck_inplace = K.kda_output_fixup_ckpt(t["q"], t["k"], t["g"], t["beta"], t["seg_start"], S_in,
                                         o3, sD3, interval=iv, out=sD3)
    sync()
    assert torch.equal(o1, o2) and torch.equal(o2, o3)
    assert ck_inplace.data_ptr() == sD3.data_ptr() and torch.equal(ck_inplace, ck_fused)
    ro, rS, rck = oracle_full(w, interval=iv)
    tol = STATE_TOL[dtype]
    assert_close("rungs, fused", to_numpy_f64(ck_fused), rck, tol)
    assert_close("rungs, checkpoint write", to_numpy_f64(ck_two), rck, tol)
    assert_close("fused vs two-call rungs", to_numpy_f64(ck_fused), to_numpy_f64(ck_two), tol)
    assert_close("o", to_numpy_f64(o2), ro, OUT_TOL[dtype])


# ---------------------------------------------------------------------------
# Fix-up operator: X from the M blocks, the fix-up as a product with X
# ---------------------------------------------------------------------------
FIXOP_SEG = [0, 448, 512, 1216, 1536, 2112]
# segment [960, 1216) has the rung at 1024 among its first rows
FIXOP_SEG_RUNG = [0, 448, 960, 1216, 1536, 2112]


def _fixop_case(K, w, iv, chunks=6):
    """package_fx -> Blelloch scan -> fix-up from the operator with the rungs
    formed in place, beside the plain package and the recurrence's fix-up."""
    import torch
    t = to_torch(w)
    nseg = len(w.seg_start) - 1
    fx = K.FixOp(nseg, w.H, w.dk, t["q"].dtype, "cuda", chunks=chunks, interval=iv)
    S0 = t["S0"][0].contiguous()
    ol, M, D, _, sD = K.kda_segment_package_fx(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                               t["seg_start"], fx, ckpt_interval=iv,
                                               want_sub_M=False)
    S_in, S_fin = K.kda_segment_scan(M, D, S0, algo=1)
    o = ol.clone()
    ck = K.kda_output_fixup_fx(t["q"], t["k"], t["g"], t["beta"], t["seg_start"], S_in, o, fx,
                               sub_D=sD, interval=iv, out=sD)
    ol2, M2, D2, _, sD2 = K.kda_segment_package(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                                t["seg_start"], ckpt_interval=iv,
                                                want_sub_M=False, split=False)
    o2 = ol2.clone()
    ck2 = K.kda_output_fixup_ckpt(t["q"], t["k"], t["g"], t["beta"], t["seg_start"], S_in, o2,
                                  sD2, interval=iv)
    sync()
    return dict(t=t, fx=fx, o_local=(ol, ol2), M=(M, M2), D=(D, D2), o=(o, o2), ck=(ck, ck2),
                S_in=S_in)


@pytest.mark.parametrize("gates,iv,seg", [("config", 1024, FIXOP_SEG), ("config", 64, FIXOP_SEG),
                                          ("long", 1024, FIXOP_SEG), ("config", 1024, FIXOP_SEG_RUNG),
                                          ("config", 128, FIXOP_SEG_RUNG)],
                         ids=["rungs-past", "rungs-64", "long", "rung-in-rows", "rungs-128"])
@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 64, 64), ("bf16", 64, 128),
                                         ("bf16", 128, 64)])
def test_fixop_segment_path(K, gates, iv, seg, dtype, dk, dv):
    """The fix-up operator path against the oracle and against the
    recurrence's fix-up.  The packages are the plain call's, bit for bit.
    With the configs' gates the identity vanishes within a few chunks
    (len >= 0).  With rungs every 1024 tokens every segment is corrected from
    X; a single rung among a segment's corrected rows (the segment starting at
    960) is formed from Pi.  Two rungs among those rows (rungs every 64 tokens)
    send the segment to the recurrence, bit for bit as the plain fix-up.  With
    long-memory gates the segments longer than the
    operator's 6 chunks never vanish (len = -1) and walk the recurrence; the
    shorter ones are covered whole by X."""
    import torch
    shift = {} if gates == "config" else dict(gate_shift=-9.0, beta_shift=-6.0)
    w = make_workload("fixop", [2112], 2, dk, dv, dtype, 5400 + dk + dv + iv, s0_std=0.5,
                      seg_start=seg, **shift)
    say(f"fix-up operator {dtype} dk={dk} dv={dv} gates={gates} rungs every {iv} segments {seg}")
    r = _fixop_case(K, w, iv)
    lens = r["fx"].len.cpu().numpy()
    say(f"  len per (segment, head, 64-column block): {lens.reshape(len(seg) - 1, -1).tolist()}")
    route = r["fx"].route.cpu().numpy()
    say(f"  route per (segment, head): {route.tolist()}")
    nch = np.diff(seg) // 64 + (np.diff(seg) % 64 > 0)
    if gates == "config":
        assert (lens >= 1).all() and (lens <= 6).all()
    else:   # a segment of at most 6 chunks is covered whole; the longer ones never vanish
        for j, n in enumerate(nch):
            assert (lens[j] == (n if n <= 6 else -1)).all(), (j, lens[j].tolist())
    for name in ("o_local", "M", "D"):
        assert torch.equal(*r[name]), f"{name} differs from the plain package call"
    ro, rS, rck = oracle_full(w, interval=iv)
    o, o2 = (to_numpy_f64(x) for x in r["o"])
    ck, ck2 = (to_numpy_f64(x) for x in r["ck"])
    assert_close("o (operator)", o, ro, OUT_TOL[dtype])
    assert_close("rungs (operator, in place)", ck, rck, STATE_TOL[dtype])
    assert_close("o: operator vs recurrence", o, o2, OUT_TOL[dtype])
    assert_close("rungs: operator vs recurrence", ck, ck2, STATE_TOL[dtype])
    # a segment routed to the recurrence is the plain fix-up's, bit for bit
    for j in range(len(seg) - 1):
        for hh in range(w.H):
            if route[j, hh]:
                assert np.array_equal(o[seg[j]:seg[j + 1], hh], o2[seg[j]:seg[j + 1], hh]), (j, hh)
    if gates == "config" and iv == 64:   # two rungs among the first rows of segment 0
        assert route[0].all()
    if gates == "config" and seg is FIXOP_SEG_RUNG:   # one rung among them: Pi
        assert not route[2].any()


def test_fixop_whole_segments_long_memory(K):
    """Long-memory gates: no propagated identity vanishes.  An operator that
    keeps every row of each segment (chunks = the longest segment) still
    covers them all (len = each segment's chunk count, route 0), so the
    fix-up is one product; the rungs come from kda_checkpoint_write with
    sub_M.  Outputs and rungs against the oracle, outputs against the
    recurrence's fix-up."""
    import torch
    seg = [0, 1024, 2560, 4096]
    w = make_workload("fixop-whole", [4096], 2, 128, 128, "bf16", 5620, s0_std=0.5,
                      seg_start=seg, gate_shift=-9.0, beta_shift=-6.0)
    say("fix-up operator over whole segments, long-memory gates")
    t = to_torch(w)
    iv = 512
    chunks = max(b - a for a, b in zip(seg[:-1], seg[1:])) // 64
    fx = K.FixOp(3, 2, 128, t["q"].dtype, "cuda", chunks=chunks)
    # unsplit: a split segment's operator comes from its first sub-segment only
    ol, M, D, sM, sD = K.kda_segment_package_fx(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                                t["seg_start"], fx, ckpt_interval=iv,
                                                want_sub_M=True, split=False)
    S_in, _ = K.kda_segment_scan(M, D, t["S0"][0].contiguous(), algo=1)
    o, o2 = ol.clone(), ol.clone()
    K.kda_output_fixup_fx(t["q"], t["k"], t["g"], t["beta"], t["seg_start"], S_in, o, fx)
    ck = K.kda_checkpoint_write(t["seg_start"], S_in, sM, sD, T=4096, interval=iv)
    K.kda_output_fixup(t["q"], t["k"], t["g"], t["beta"], t["seg_start"], S_in, o2)
    sync()
    lens, route = fx.len.cpu().numpy(), fx.route.cpu().numpy()
    want = np.array([(b - a) // 64 for a, b in zip(seg[:-1], seg[1:])])
    say(f"  len {lens.reshape(3, -1).tolist()} route {route.tolist()}")
    assert (lens == want[:, None, None]).all() and (route == 0).all()
    assert float(M.abs().max()) > 1e-3, "long-memory gates should leave M nonzero"
    ro, _, rck = oracle_full(w, interval=iv)
    assert_close("o (operator)", to_numpy_f64(o), ro, OUT_TOL["bf16"])
    assert_close("o: operator vs recurrence", to_numpy_f64(o), to_numpy_f64(o2), OUT_TOL["bf16"])
    assert_close("rungs", to_numpy_f64(ck), rck, STATE_TOL["bf16"])


@pytest.mark.parametrize("nseg", [4, 8, 16])
def test_fixop_workgroups_per_unit(K, nseg):
    """The operator's launch takes one to several workgroups per (segment,
    head) unit, by the unit count: with 32 heads, 4, 8 and 16 segments give
    128, 256 and 512 units, so each unit's chunks and rung quarters are
    spread over 4, 2 and 1 workgroups.  Rungs every 128 tokens put one among
    each segment's corrected rows (formed from Pi).  Outputs and rungs against
    the recurrence's fix-up on every head, and against the oracle on two."""
    import torch
    T, iv = 1024 * nseg, 128
    seg = list(range(0, T + 1, 1024))
    w = make_workload("fixop-spread", [T], 32, 128, 128, "bf16", 5600 + nseg, s0_std=0.5,
                      seg_start=seg)
    say(f"fix-up operator over {nseg} x 32 units, rungs every {iv}")
    t = to_torch(w)
    fx = K.FixOp(nseg, 32, 128, t["q"].dtype, "cuda", interval=iv)
    ol, M, D, _, sD = K.kda_segment_package_fx(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                               t["seg_start"], fx, ckpt_interval=iv,
                                               want_sub_M=False)
    S_in, _ = K.kda_segment_scan(M, D, t["S0"][0].contiguous(), algo=0)
    o, o2 = ol.clone(), ol.clone()
    ck2 = K.kda_output_fixup_ckpt(t["q"], t["k"], t["g"], t["beta"], t["seg_start"], S_in, o2,
                                  sD.clone(), interval=iv)
    ck = K.kda_output_fixup_fx(t["q"], t["k"], t["g"], t["beta"], t["seg_start"], S_in, o, fx,
                               sub_D=sD, interval=iv, out=sD)
    sync()
    lens, route = fx.len.cpu().numpy(), fx.route.cpu().numpy()
    assert (route == 0).all() and (lens >= 2).all(), "the operator should cover every unit"
    assert_close("o: operator vs recurrence", to_numpy_f64(o), to_numpy_f64(o2), OUT_TOL["bf16"])
    assert_close("rungs: operator vs recurrence", to_numpy_f64(ck), to_numpy_f64(ck2),
                 STATE_TOL["bf16"])
    for h in (0, 31):
        ro, _, rck = oracle_unit(w, 0, h, interval=iv)
        assert_close(f"o head {h}", to_numpy_f64(o[:, h]), ro[:, 0], OUT_TOL["bf16"])
        assert_close(f"rungs head {h}", to_numpy_f64(ck[:, h]), rck[:, 0], STATE_TOL["bf16"])


@pytest.mark.parametrize("gates", ["config", "long"])
def test_fixop_split_segments(K, gates):
    """The operator when kda_segment_package splits segments into
    sub-segments (4 segments of 4096 tokens on 2 heads).  The first
    sub-segment of each segment writes its operator.  With the configs' gates
    the identity vanishes inside it; with long-memory gates it does not
    (len = -1, the recurrence).  Outputs and rungs against the oracle, and
    against the recurrence's fix-up."""
    import torch
    shift = {} if gates == "config" else dict(gate_shift=-9.0, beta_shift=-6.0)
    seg = [0, 4096, 8192, 12288, 16384]
    w = make_workload("fixop-split", [16384], 2, 128, 128, "bf16", 5495, s0_std=0.5,
                      seg_start=seg, **shift)
    say(f"fix-up operator on split segments (4 x 4096, H=2, bf16 d=128), gates={gates}")
    t = to_torch(w)
    iv = 1024
    fx = K.FixOp(4, 2, 128, t["q"].dtype, "cuda", interval=iv)
    ol, M, D, _, sD = K.kda_segment_package_fx(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                               t["seg_start"], fx, ckpt_interval=iv,
                                               want_sub_M=False)
    S_in, _ = K.kda_segment_scan(M, D, t["S0"][0].contiguous(), algo=0)
    o = ol.clone()
    ck = K.kda_output_fixup_fx(t["q"], t["k"], t["g"], t["beta"], t["seg_start"], S_in, o, fx,
                               sub_D=sD, interval=iv, out=sD)
    o2 = ol.clone()
    ck2 = K.kda_output_fixup_ckpt(t["q"], t["k"], t["g"], t["beta"], t["seg_start"], S_in, o2,
                                  sD.clone(), interval=iv)
    sync()
    lens, route = fx.len.cpu().numpy(), fx.route.cpu().numpy()
    say(f"  len {lens.reshape(4, -1).tolist()} route {route.tolist()}")
    if gates == "config":
        assert (lens >= 1).all() and (route == 0).all()
    else:
        assert (lens == -1).all() and (route == 1).all()
    ro, rS, rck = oracle_full(w, interval=iv)
    assert_close("o (operator)", to_numpy_f64(o), ro, OUT_TOL["bf16"])
    assert_close("rungs (operator)", to_numpy_f64(ck), rck, STATE_TOL["bf16"])
    assert_close("o: operator vs recurrence", to_numpy_f64(o), to_numpy_f64(o2), OUT_TOL["bf16"])


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 64, 64)])
def test_fixop_rows_are_the_identity_outputs(K, dtype, dk, dv):
    """Rows of X against the oracle's definition: the outputs of segment j
    run from the identity as its incoming state (dk value columns), with
    zero values.  Compared over the chunks its len covers."""
    w = make_workload("fixop-x", [2112], 2, dk, dv, dtype, 5480 + dk, s0_std=0.5,
                      seg_start=FIXOP_SEG)
    say(f"fix-up operator rows vs the identity's outputs, {dtype} dk={dk}")
    r = _fixop_case(K, w, 1024)
    X = to_numpy_f64(r["fx"].X)
    lens = r["fx"].len.cpu().numpy()
    q, k, g, b = (w.f64(x) for x in ("q", "k", "g", "beta"))
    H = w.H
    for j in range(len(FIXOP_SEG) - 1):
        a, e = FIXOP_SEG[j], FIXOP_SEG[j + 1]
        n = e - a
        S0 = np.broadcast_to(np.eye(dk), (1, H, dk, dk)).copy()
        xo, _, _ = oracle.prefill(q[a:e], k[a:e], np.zeros((n, H, dk)), g[a:e], b[a:e], [0, n],
                                  S0=S0, scale=w.scale, qk_l2norm=w.qk_l2norm)
        for h in range(H):
            for blk in range(dk // 64):
                rows = min(n, int(lens[j, h, blk]) * 64)
                cols = slice(64 * blk, 64 * blk + 64)
                assert_close(f"X[{j}] head {h} columns {cols.start}..{cols.stop - 1}, {rows} rows",
                             X[j, :rows, h, cols], xo[:rows, h, cols], OUT_TOL[dtype])
                # past the vanishing point the identity's outputs are exactly zero
                assert np.abs(xo[rows:, h, cols]).max(initial=0.0) < 1e-30


def test_fixop_nonfinite_incoming_state(K):
    """An incoming state with a NaN walks the recurrence: the outputs carry
    NaN exactly where the plain fix-up puts it (the NaN reaches every S_in of
    head 1 through the scan), and head 0's segments are corrected from X."""
    import torch
    w = make_workload("fixop-nan", [2112], 2, 128, 128, "bf16", 5490, s0_std=0.5,
                      seg_start=FIXOP_SEG)
    w.S0[0, 1, 3, 7] = np.nan
    say("fix-up operator with a NaN in S0 (segment 0, head 1)")
    r = _fixop_case(K, w, 1024)
    o, o2 = (to_numpy_f64(x) for x in r["o"])
    assert np.isnan(o).any()
    assert np.array_equal(np.isnan(o), np.isnan(o2))
    fin = ~np.isnan(o2)
    assert_close("o (finite entries): operator vs recurrence", o[fin], o2[fin], OUT_TOL["bf16"])


# ---------------------------------------------------------------------------
# Packages of segments split into sub-segments (CUs otherwise idle)
# ---------------------------------------------------------------------------
SPLIT_CASES = [
    # dtype, dk, dv, H, T, seg_start, gates, rung interval
    ("bf16", 128, 128, 2, 4096, [0, 640, 1984, 2048, 4096], "config", 128),
    ("bf16", 128, 128, 2, 4096, [0, 640, 1984, 2048, 4096], "long", 128),
    ("f32", 64, 64, 4, 16384, [0, 8192, 16384], "long", 1024),
    ("bf16", 64, 128, 2, 8192, [0, 4096, 8192], "config", 512),
    ("f32", 128, 128, 2, 4096, [0, 1536, 4096], "long", 512),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-H{c[3]}-T{c[4]}-{c[6]}")
def test_package_split_into_subsegments(K, case):
    """With its workspace, kda_segment_package splits segments whose
    (segment, head) units would leave compute units idle (2 to 8
    sub-segments here, one segment of a single chunk), merges the
    sub-packages, and gives the unsplit call's o_local, M, D and rung
    sub-packages; each against the oracle too."""
    import ctypes
    import torch
    dtype, dk, dv, H, T, seg, gates, iv = case
    shift = {} if gates == "config" else dict(gate_shift=-9.0, beta_shift=-6.0)
    w = make_workload("split-pkg", [T], H, dk, dv, dtype, 5400 + dk + dv + H, s0_std=0.3,
                      seg_start=seg, **shift)
    t = to_torch(w)
    cfg = K.make_config(H, dk, dv, t["q"].dtype)
    wsb = K.LIB.kda_segment_package_workspace(ctypes.byref(cfg), T, len(seg) - 1)
    say(f"package split {case}: workspace {wsb} bytes")
    assert wsb > 0, "the call should split these segments"
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"], t["seg_start"])
    sp = K.kda_segment_package(*args, ckpt_interval=iv)
    un = K.kda_segment_package(*args, ckpt_interval=iv, split=False)
    sync()
    tol_o, tol_s = OUT_TOL[dtype], STATE_TOL[dtype]
    for name, i, tol in (("o_local", 0, tol_o), ("M", 1, tol_s), ("D", 2, tol_s),
                         ("sub_M", 3, tol_s), ("sub_D", 4, tol_s)):
        assert_close(f"split vs unsplit {name}", to_numpy_f64(sp[i]), to_numpy_f64(un[i]), tol)
    q, k, v, g, b = (w.f64(x) for x in ("q", "k", "v", "g", "beta"))
    rows = T // iv
    ref_sM = np.zeros((rows, H, dk, dk))
    ref_sD = np.zeros((rows, H, dk, dv))
    for j in range(len(seg) - 1):
        Mr, Dr, olr = oracle.package(q, k, v, g, b, seg[j], seg[j + 1])
        assert_close(f"M[{j}]", to_numpy_f64(sp[1][j]), Mr, tol_s)
        assert_close(f"D[{j}]", to_numpy_f64(sp[2][j]), Dr, tol_s)
        assert_close(f"o_local[{j}]", to_numpy_f64(sp[0][seg[j]:seg[j + 1]]),
                     olr[seg[j]:seg[j + 1]], tol_o)
        for p in range((seg[j] // iv + 1) * iv, seg[j + 1] + 1, iv):
            Mp, Dp, _ = oracle.package(q, k, v, g, b, seg[j], p)
            ref_sM[p // iv - 1], ref_sD[p // iv - 1] = Mp, Dp
    # with the configs' gates a rung 512 tokens into a segment has a map below
    # fp32 range (|Pi_p| ~ 1e-150 in fp64, exactly 0 in fp32): such rungs are
    # compared in absolute terms against the O(1) states they act on
    got_sM = to_numpy_f64(sp[3])
    for r in range(rows):
        if np.linalg.norm(ref_sM[r]) < 1e-20:
            assert np.abs(got_sM[r] - ref_sM[r]).max() < 1e-20, f"sub_M row {r}"
        else:
            assert_close(f"sub_M row {r}", got_sM[r], ref_sM[r], tol_s)
    assert_close("sub_D", to_numpy_f64(sp[4]), ref_sD, tol_s)
    # the whole path through the split packages
    o, Sf, ck = K.kda_segment_prefill(*args, t["S0"][0].contiguous(), algo=1, ckpt_interval=iv)
    sync()
    ro, rS, rck = oracle_full(w, interval=iv)
    assert_close("o", to_numpy_f64(o), ro, tol_o)
    assert_close("S_final", to_numpy_f64(Sf), rS[0], tol_s)
    assert_close("rungs", to_numpy_f64(ck), rck, tol_s)
