"""CPU checks of the comparison machinery the GPU parity tests rest on.

``oracle.rel_l2`` is pinned to hand-computed values, and the full-size
segment checks (tests/checks.py) are shown to fail on the mistakes they exist
to catch: a missing or partial output fix-up, a wrong sign in it, and wrong
rungs.  The "mistakes" are planted in oracle results on the CPU.
"""
import numpy as np
import pytest

import oracle
from checks import OUT_TOL, STATE_TOL, SegmentChecks, UnitErrors, seg_walk, slice_inputs
from workloads import make_workload


# ---------------------------------------------------------------------------
# rel_l2
# ---------------------------------------------------------------------------
def test_rel_l2_hand_values():
    # ||(1,2,3) - (1,2,2)|| / ||(1,2,2)|| = 1 / 3
    assert oracle.rel_l2([1.0, 2.0, 3.0], [1.0, 2.0, 2.0]) == pytest.approx(1.0 / 3.0, rel=1e-15)
    # ||(0,0) - (3,4)|| / 5 = 1
    assert oracle.rel_l2([0.0, 0.0], [3.0, 4.0]) == 1.0
    # reference all zero: the absolute norm, sqrt(9 + 16) = 5
    assert oracle.rel_l2([3.0, 4.0], [0.0, 0.0]) == 5.0
    # identical tensors: exactly zero
    x = np.random.default_rng(1).standard_normal((7, 3, 5))
    assert oracle.rel_l2(x, x.copy()) == 0.0
    # a uniform relative perturbation e gives e
    assert oracle.rel_l2(x * (1 + 3e-3), x) == pytest.approx(3e-3, rel=1e-9)
    # the 2-D case is the Frobenius norm over the whole tensor: 1 / sqrt(2),
    # not the mean of the per-row figures (0 and 1)
    a = np.array([[1.0, 0.0], [0.0, 0.0]])
    b = np.array([[1.0, 0.0], [0.0, 1.0]])
    assert oracle.rel_l2(a, b) == pytest.approx(2 ** -0.5, rel=1e-15)


def test_rel_l2_rejects_shape_mismatch_and_fails_on_nan():
    with pytest.raises(ValueError):
        oracle.rel_l2(np.zeros((4, 1)), np.zeros(4))
    with pytest.raises(ValueError):
        oracle.rel_l2(np.zeros((2, 3)), np.zeros((3, 2)))
    x = np.ones(10)
    y = x.copy()
    y[3] = np.nan
    e = oracle.rel_l2(y, x)
    assert not (e <= 1.0)
    y[3] = np.inf
    assert not (oracle.rel_l2(y, x) <= 1.0)


def test_rel_l2_negative_control_at_the_tolerances():
    """Noise of relative norm 3e-2 on outputs and 1.5e-2 on states fails the
    bf16 bars; 5e-3 and 2e-5 pass them and the fp32 bar respectively."""
    rng = np.random.default_rng(2)
    ref = rng.standard_normal((64, 4, 128))
    noise = rng.standard_normal(ref.shape)
    noise *= np.linalg.norm(ref) / np.linalg.norm(noise)
    assert not oracle.rel_l2(ref + 3e-2 * noise, ref) <= OUT_TOL["bf16"]
    assert not oracle.rel_l2(ref + 1.5e-2 * noise, ref) <= STATE_TOL["bf16"]
    assert oracle.rel_l2(ref + 5e-3 * noise, ref) <= OUT_TOL["bf16"]
    assert oracle.rel_l2(ref + 2e-5 * noise, ref) <= OUT_TOL["f32"]
    assert not oracle.rel_l2(ref + 2e-4 * noise, ref) <= OUT_TOL["f32"]


def test_unit_errors_accumulate_exactly():
    """A unit's error summed over pieces equals rel_l2 over the joined tensor."""
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((100, 8))
    got = ref + 0.01 * rng.standard_normal(ref.shape)
    e = UnitErrors("t")
    e.add("u", got[:30], ref[:30])
    e.add("u", got[30:], ref[30:])
    assert e.rel()["u"] == pytest.approx(oracle.rel_l2(got, ref), rel=1e-12)
    with pytest.raises(ValueError):
        e.add("u", got[:3], ref[:4])


# ---------------------------------------------------------------------------
# The full-size segment checks catch a missing or wrong fix-up
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def seg_case():
    """The 16,384-token workload's shape shrunk to 4 segments of 1024 tokens,
    2 heads: config gates (incoming states forgotten within a few chunks),
    S0 ~ N(0, 0.1^2), rungs every 512 tokens."""
    w = make_workload("checks", [4096], 2, 128, 128, "bf16", 4700, s0_std=0.1,
                      seg_start=[0, 1024, 2048, 3072, 4096])
    segs = list(seg_walk(w, [0, 1], interval=512, corrections=True))
    q, k, v, g, b = (w.f64(x) for x in ("q", "k", "v", "g", "beta"))
    o_local = np.zeros((w.T, 2, 128))
    for s in segs:
        _, _, ol = oracle.package(q, k, v, g, b, s["a"], s["b"])
        o_local[s["a"]:s["b"]] = ol[s["a"]:s["b"]]
    return w, segs, o_local


def _checks(segs, o_of, corr_of=None, rungs_of=None):
    c = SegmentChecks([0, 1])
    for s in segs:
        c.add(s, o=o_of(s), S_in=s["S_in"], corr=None if corr_of is None else corr_of(s),
              rungs=None if rungs_of is None else rungs_of(s))
    return c


def test_seg_walk_matches_the_whole_sequence(seg_case):
    """Walking segment by segment carries the state exactly: outputs, final
    state and rungs equal one oracle run over the whole sequence, and the
    correction equals the outputs minus the zero-state outputs."""
    w, segs, o_local = seg_case
    from workloads import ckpt_offsets
    ro, rS, rck = oracle.prefill(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("g"), w.f64("beta"),
                                 w.cu_seqlens, S0=w.S0, ckpt_interval=512,
                                 ckpt_offsets=ckpt_offsets(w.lengths, 512))
    o = np.concatenate([s["o"] for s in segs])
    assert oracle.rel_l2(o, ro) < 1e-13
    assert oracle.rel_l2(segs[-1]["S_out"], rS[0]) < 1e-13
    rows = dict(r for s in segs for r in s["rungs"])
    assert sorted(rows) == list(range(8))
    assert oracle.rel_l2(np.stack([rows[i] for i in range(8)]), rck) < 1e-13
    for s in segs:
        assert oracle.rel_l2(s["corr"], s["o"] - o_local[s["a"]:s["b"]]) < 1e-10


def test_checks_pass_the_oracle_and_fail_without_fixup(seg_case):
    w, segs, o_local = seg_case
    good = _checks(segs, lambda s: s["o"], lambda s: s["corr"])
    good.check(OUT_TOL["bf16"], STATE_TOL["bf16"])
    # no fix-up at all: outputs are o_local, the correction is zero
    bad = _checks(segs, lambda s: o_local[s["a"]:s["b"]], lambda s: np.zeros_like(s["corr"]))
    u, e_win = bad.o_win.worst()
    print(f"missing fix-up: worst window rel-L2 {e_win:.3e} at {u}; "
          f"per-head rel-L2 {bad.o_head.worst()[1]:.3e}")
    with pytest.raises(AssertionError):
        bad.o_win.check(OUT_TOL["bf16"])
    with pytest.raises(AssertionError):
        bad.corr.check(OUT_TOL["bf16"])
    assert bad.corr.worst()[1] == 1.0


def test_checks_fail_on_a_partial_or_wrong_fixup(seg_case):
    w, segs, o_local = seg_case
    # segment 0's S0 correction dropped, every other segment right
    part = _checks(segs, lambda s: o_local[s["a"]:s["b"]] if s["j"] == 0 else s["o"],
                   lambda s: np.zeros_like(s["corr"]) if s["j"] == 0 else s["corr"])
    with pytest.raises(AssertionError):
        part.o_win.check(OUT_TOL["bf16"])
    assert part.o_win.worst()[0][0] == 0
    # correction subtracted instead of added
    sign = _checks(segs, lambda s: o_local[s["a"]:s["b"]] - s["corr"], lambda s: -s["corr"])
    with pytest.raises(AssertionError):
        sign.o_win.check(OUT_TOL["bf16"])
    with pytest.raises(AssertionError):
        sign.corr.check(OUT_TOL["bf16"])
    # the correction of the previous segment's incoming state (wrong S_in)
    prev = {s["j"]: s for s in segs}

    def shifted(s):
        if s["j"] == 0:
            return s["corr"]
        q, k, v, g, b = slice_inputs(w, s["a"], s["b"], [0, 1])
        c, _, _ = oracle.prefill(q, k, np.zeros_like(v), g, b, [0, s["b"] - s["a"]],
                                 S0=prev[s["j"] - 1]["S_in"][None])
        return c
    wrong = _checks(segs, lambda s: s["o"], shifted)
    with pytest.raises(AssertionError):
        wrong.corr.check(OUT_TOL["bf16"])


def test_checks_fail_on_wrong_rungs(seg_case):
    w, segs, _ = seg_case

    def rungs_scaled(s):
        return {row: r * (1.02 if row == 3 else 1.0) for row, r in s["rungs"]}

    bad = _checks(segs, lambda s: s["o"], rungs_of=rungs_scaled)
    with pytest.raises(AssertionError):
        bad.rungs.check(STATE_TOL["bf16"])

    def rungs_swapped(s):   # rung rows off by one inside a segment
        rr = dict(s["rungs"])
        keys = sorted(rr)
        return {k: rr[keys[(i + 1) % len(keys)]] for i, k in enumerate(keys)} if len(keys) > 1 else rr
    bad2 = _checks(segs, lambda s: s["o"], rungs_of=rungs_swapped)
    with pytest.raises(AssertionError):
        bad2.rungs.check(STATE_TOL["bf16"])
