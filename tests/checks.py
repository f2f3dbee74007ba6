"""Full-size parity checks shared by the GPU tests and their CPU negative
controls.

The oracle is run segment by segment over one sequence, carrying the state, so
every segment's incoming state S_in^j, its outputs, its rungs and the output
contribution of S_in^j alone (the fix-up's correction: the same segment run
from S_in^j with all values set to zero, since the outputs are affine in the
incoming state and the values) are known per (segment, head) without holding
the whole 131,072-token sequence in fp64.

Comparisons are reported per unit (head, or (segment, head)) as rel-L2, and the
worst unit decides.  ``UnitErrors`` accumulates squared error sums so a head's
error over all segments is exact, not an average of per-segment figures.
"""
from __future__ import annotations

import numpy as np

import oracle
from workloads import to_f64

OUT_TOL = {"f32": 1e-4, "bf16": 2e-2}
STATE_TOL = {"f32": 1e-4, "bf16": 1e-2}
FIXUP_ROWS = 64      # rows at the start of each segment checked on their own


def slice_inputs(w, a, b, heads):
    """fp64 q, k, v, g, beta of rows [a, b) for the listed heads."""
    hs = list(heads)
    q = to_f64(w.q[a:b][:, hs], w.dtype)
    k = to_f64(w.k[a:b][:, hs], w.dtype)
    v = to_f64(w.v[a:b][:, hs], w.dtype)
    g = np.asarray(w.g[a:b][:, hs], dtype=np.float64)
    beta = np.asarray(w.beta[a:b][:, hs], dtype=np.float64)
    return q, k, v, g, beta


def seg_walk(w, heads, interval=0, corrections=False):
    """Oracle over the segments of one-sequence workload w for the given
    heads.  Yields one dict per segment j:
        j, a, b        the segment's rows
        S_in           [nh, dk, dv] state entering the segment
        o              [b-a, nh, dv] outputs
        corr           [b-a, nh, dv] outputs of the segment run from S_in with
                       zero values (only with corrections=True)
        rungs          [(row, [nh, dk, dv]), ...] states at absolute positions
                       p = m*interval inside (a, b]
        S_out          [nh, dk, dv] state leaving the segment
    """
    hs = list(heads)
    S = (np.zeros((len(hs), w.dk, w.dv)) if w.S0 is None
         else np.asarray(w.S0[0][hs], dtype=np.float64))
    seg = w.seg_start
    for j in range(len(seg) - 1):
        a, b = int(seg[j]), int(seg[j + 1])
        q, k, v, g, beta = slice_inputs(w, a, b, hs)
        pool = S[None]
        o, out, rk = oracle.prefill_resume(q, k, v, g, beta, [0, b - a], pool, [0], [0],
                                           pos0=[a], ckpt_interval=interval,
                                           scale=w.scale, qk_l2norm=w.qk_l2norm)
        rungs = []
        if interval:
            first = a // interval + 1
            for i in range(rk.shape[0]):
                rungs.append((first + i - 1, rk[i]))
        corr = None
        if corrections:
            corr, _, _ = oracle.prefill(q, k, np.zeros_like(v), g, beta, [0, b - a], S0=pool,
                                        scale=w.scale, qk_l2norm=w.qk_l2norm)
        yield dict(j=j, a=a, b=b, S_in=S, o=o, corr=corr, rungs=rungs, S_out=out[0])
        S = out[0]


class UnitErrors:
    """Squared-error and squared-reference sums per unit label."""

    def __init__(self, what: str):
        self.what = what
        self.num = {}
        self.den = {}

    def add(self, unit, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        if got.shape != ref.shape:
            raise ValueError(f"{self.what}: shapes differ: {got.shape} vs {ref.shape}")
        d = got - ref
        self.num[unit] = self.num.get(unit, 0.0) + float(np.sum(d * d))
        self.den[unit] = self.den.get(unit, 0.0) + float(np.sum(ref * ref))

    def rel(self) -> dict:
        out = {}
        for u, n in self.num.items():
            den = self.den[u]
            out[u] = float(np.sqrt(n / den)) if den > 0 else float(np.sqrt(n))
        return out

    def worst(self):
        r = self.rel()
        if not r:
            raise ValueError(f"{self.what}: nothing compared")
        u = max(r, key=lambda x: (np.nan_to_num(r[x], nan=np.inf)))
        return u, r[u]

    def check(self, tol: float, say=print):
        """Fails when any unit's rel-L2 exceeds tol (NaN fails too)."""
        r = self.rel()
        u, e = self.worst()
        vals = np.array(list(r.values()))
        say(f"{self.what}: {len(r)} units, rel-L2 max {e:.3e} at {u}, "
            f"median {np.median(vals):.3e} (tol {tol:g})")
        bad = {k: v for k, v in r.items() if not (v <= tol)}
        assert not bad, f"{self.what}: {len(bad)} units above {tol:g}, worst {u}: {e:.3e}"
        return e


def per_head(errs: UnitErrors, seg_label, heads, got, ref):
    """Adds got/ref [rows, nh, d] head by head (unit = head label)."""
    for i, h in enumerate(heads):
        errs.add(h if seg_label is None else (seg_label, h), got[:, i], ref[:, i])


class SegmentChecks:
    """The unit errors the full-size segment tests assert on, filled one
    segment at a time (from seg_walk):
      o per head over the whole sequence;
      o over the first FIXUP_ROWS rows of every (segment, head), where the
        fix-up's correction is concentrated;
      the fix-up's correction alone per (segment, head), when given;
      S_in per (segment, head) and rungs per (row, head), when given."""

    def __init__(self, heads):
        self.heads = list(heads)
        self.o_head = UnitErrors("o per head")
        self.o_win = UnitErrors(f"o, first {FIXUP_ROWS} rows of each (segment, head)")
        self.corr = UnitErrors("fix-up correction per (segment, head)")
        self.s_in = UnitErrors("S_in per (segment, head)")
        self.rungs = UnitErrors("rungs per (row, head)")

    def add(self, s, o=None, S_in=None, corr=None, rungs=None):
        """o, corr: [b-a, nh, dv]; S_in: [nh, dk, dv]; rungs: {row: [nh, dk, dv]}."""
        hs = self.heads
        if o is not None:
            per_head(self.o_head, None, hs, o, s["o"])
            n = min(FIXUP_ROWS, s["b"] - s["a"])
            per_head(self.o_win, s["j"], hs, o[:n], s["o"][:n])
        if corr is not None:
            per_head(self.corr, s["j"], hs, corr, s["corr"])
        if S_in is not None:
            for i, h in enumerate(hs):
                self.s_in.add((s["j"], h), S_in[i], s["S_in"][i])
        if rungs is not None:
            for row, ref in s["rungs"]:
                for i, h in enumerate(hs):
                    self.rungs.add((row, h), rungs[row][i], ref[i])

    def check(self, out_tol, state_tol, say=print):
        worst = {}
        for e, tol in ((self.o_head, out_tol), (self.o_win, out_tol), (self.corr, out_tol),
                       (self.s_in, state_tol), (self.rungs, state_tol)):
            if e.num:
                worst[e.what] = e.check(tol, say)
        return worst
