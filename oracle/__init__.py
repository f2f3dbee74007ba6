"""fp64 CPU oracle for KDA prefill -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the GPU library (gated_delta_rule_46_amd)
and never imports it.

* ``prefill``  -- token-by-token recurrence (kda_oracle.c), outputs, final
  states and checkpoints.
* ``package``  -- the affine map S_out = M S_in + D of a token range and the
  range's outputs from a zero state (kda_oracle.c).
* ``compose`` / ``scan_sequential`` / ``scan_blelloch`` -- package algebra
  written from its definition with numpy matmuls (pegainfer PR #970,
  whale-lane commit text: (M,D) packages combined all-prefix, with a Blelloch
  prefix-scan fallback).
* ``decode`` -- one new token per sequence against a pool of states read and
  written through slot indices (ROCm/ATOM PR #2709, review notes: the fused
  sigmoid-gated delta-rule update takes a read-side state index beside the
  write table).  It is the token recurrence above on sequences of length 1;
  gate logits are activated first with ``softplus`` / ``sigmoid`` written
  from their definitions.
* ``prefill_resume`` -- prefill that continues sequences from pool slots, with
  rungs at absolute positions of the original sequence (ROCm/ATOM PR #2709,
  Changes: prefix caching of KDA state, checkpoints on the chunk grid): the
  token recurrence run piece by piece between rung positions, each piece's
  final state being the rung.
* ``short_conv`` / ``conv_halo`` -- the causal depthwise convolution over
  tokens that KDA applies to q, k, v, with per-sequence windows (kern PR #44:
  short-conv gather and window update per sequence; ROCm/ATOM PR #2709: the
  conv state follows a fork through a read index) and the halo tail a
  segment publishes for the next (pegainfer PR #970), from the definition.
* ``mirror`` -- the fp64 chunkwise form (used only to pin chunk-size
  independence and the chunk algebra; never as the oracle).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

__all__ = ["build", "prefill", "package", "compose", "identity_package", "scan_sequential",
           "scan_blelloch", "rel_l2", "threads", "softplus", "sigmoid", "decode",
           "prefill_resume", "silu", "short_conv", "conv_halo"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        d, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.kda_oracle_prefill.argtypes = [i64, i32, i32, i32, d, d, d, d, d, d, i32, d,
                                           ctypes.c_double, i32, i32, d, d, d, d, i32]
        lib.kda_oracle_prefill.restype = ctypes.c_int
        lib.kda_oracle_package.argtypes = [i64, i32, i32, i32, d, d, d, d, d, i64, i64,
                                           ctypes.c_double, i32, d, d, d, i32]
        lib.kda_oracle_package.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    return max(1, os.cpu_count() or 1)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def prefill(q, k, v, g, beta, cu_seqlens, S0=None, scale=1.0, qk_l2norm=1,
            ckpt_interval=0, ckpt_offsets=None, nthreads=None):
    """Token-by-token KDA prefill in fp64.

    q, k, g: [T,H,dk]; v: [T,H,dv]; beta: [T,H]; cu_seqlens: [N+1]; S0: [N,H,dk,dv].
    Returns (o [T,H,dv], S_final [N,H,dk,dv], ckpt [rows,H,dk,dv] or None).
    """
    q, k, v, g, beta = (_c64(x) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    S0 = _c64(S0)
    o = np.zeros((T, H, dv))
    Sf = np.zeros((N, H, dk, dv))
    ck = None
    off = None
    if ckpt_interval:
        off = np.ascontiguousarray(ckpt_offsets, dtype=np.int64)
        ck = np.zeros((int(off[-1]), H, dk, dv))
    rc = _load().kda_oracle_prefill(T, H, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta),
                                    _p(cu), N, _p(S0), float(scale), int(qk_l2norm),
                                    int(ckpt_interval), _p(off), _p(ck), _p(o), _p(Sf),
                                    int(nthreads or threads()))
    if rc != 0:
        raise ValueError("kda_oracle_prefill rejected its arguments")
    return o, Sf, ck


def package(q, k, v, g, beta, a, b, scale=1.0, qk_l2norm=1, nthreads=None):
    """Package (M [H,dk,dk], D [H,dk,dv]) of rows [a, b) plus o_local [T,H,dv]
    (rows a..b-1 filled: outputs of the range started from a zero state)."""
    q, k, v, g, beta = (_c64(x) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    M = np.zeros((H, dk, dk))
    D = np.zeros((H, dk, dv))
    o = np.zeros((T, H, dv))
    rc = _load().kda_oracle_package(T, H, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta),
                                    int(a), int(b), float(scale), int(qk_l2norm),
                                    _p(M), _p(D), _p(o), int(nthreads or threads()))
    if rc != 0:
        raise ValueError("kda_oracle_package rejected its arguments")
    return M, D, o


# ---------------------------------------------------------------------------
# Decode against a state pool
# ---------------------------------------------------------------------------
def softplus(x):
    """log(1 + e^x) in fp64, as log(e^0 + e^x) without overflow."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def sigmoid(x):
    """1 / (1 + e^-x) in fp64."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def decode(q, k, v, g, beta, pool, read_idx, write_idx, gate_logits=False, scale=1.0,
           qk_l2norm=1):
    """One decode step: sequence n takes row n of q, k, v [N,H,d], g [N,H,dk],
    beta [N,H].  With gate_logits, log alpha = -softplus(g) and
    beta = sigmoid(beta).  Sequence n starts from pool[read_idx[n]] (zeros
    when the index is outside [0, n_slots)) and its new state goes to
    pool[write_idx[n]] (nowhere when outside).  All reads happen before any
    write.  Returns (o [N,H,dv], new pool), both fp64."""
    q, k, v, g, beta = (_c64(x) for x in (q, k, v, g, beta))
    N, H, dk = q.shape
    dv = v.shape[2]
    pool = np.asarray(pool, dtype=np.float64)
    n_slots = pool.shape[0]
    if gate_logits:
        g = -softplus(g)
        beta = sigmoid(beta)
    S0 = np.zeros((N, H, dk, dv))
    for n in range(N):
        r = int(read_idx[n])
        if 0 <= r < n_slots:
            S0[n] = pool[r]
    o, Sf, _ = prefill(q, k, v, g, beta, np.arange(N + 1), S0=S0, scale=scale,
                       qk_l2norm=qk_l2norm)
    out = pool.copy()
    for n in range(N):
        w = int(write_idx[n])
        if 0 <= w < n_slots:
            out[w] = Sf[n]
    return o, out


def prefill_resume(q, k, v, g, beta, cu_seqlens, pool, read_idx, write_idx, pos0=None,
                   ckpt_interval=0, scale=1.0, qk_l2norm=1):
    """Sequence n (rows cu[n]..cu[n+1]) starts from pool[read_idx[n]] (zeros
    outside [0, n_slots)) at absolute position pos0[n]; its final state goes
    to pool[write_idx[n]].  Rungs at absolute P = m*interval with
    pos0 < P <= pos0 + len, in sequence order then position order.
    Returns (o [T,H,dv], new pool, rungs [rows,H,dk,dv] or None), fp64."""
    q, k, v, g, beta = (_c64(x) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    pool = np.asarray(pool, dtype=np.float64)
    n_slots = pool.shape[0]
    p0 = np.zeros(N, dtype=np.int64) if pos0 is None else np.asarray(pos0, dtype=np.int64)
    o = np.zeros((T, H, dv))
    out = pool.copy()
    finals = {}
    rungs = []
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        r = int(read_idx[n])
        S = pool[r].copy() if 0 <= r < n_slots else np.zeros((H, dk, dv))
        cuts = [a]
        if ckpt_interval:
            P = (int(p0[n]) // ckpt_interval + 1) * ckpt_interval
            while P <= int(p0[n]) + (b - a):
                cuts.append(a + P - int(p0[n]))
                P += ckpt_interval
        if cuts[-1] != b:
            cuts.append(b)
        for i in range(len(cuts) - 1):
            x, y = cuts[i], cuts[i + 1]
            on, Sn, _ = prefill(q[x:y], k[x:y], v[x:y], g[x:y], beta[x:y], [0, y - x], S0=S[None],
                                scale=scale, qk_l2norm=qk_l2norm)
            o[x:y] = on
            S = Sn[0]
            if ckpt_interval and (int(p0[n]) + y - a) % ckpt_interval == 0:
                rungs.append(S.copy())
        finals[n] = S
    for n in range(N):
        w = int(write_idx[n])
        if 0 <= w < n_slots:
            out[w] = finals[n]
    ck = np.stack(rungs) if rungs else (np.zeros((0, H, dk, dv)) if ckpt_interval else None)
    return o, out, ck


# ---------------------------------------------------------------------------
# Short causal convolution over tokens
# ---------------------------------------------------------------------------
def silu(z):
    """z * sigmoid(z) in fp64."""
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


def short_conv(x, cu_seqlens, weight, bias=None, windows=None, read_idx=None, write_idx=None,
               activation=0):
    """y_t[c] = act(bias[c] + sum_j weight[c, j] * xx[t + j, c]) for each
    sequence, where xx is the sequence's window (W-1 rows, zeros when absent)
    followed by its rows of x [T, C]; the last tap multiplies the current
    token.  Returns (y [T, C], new windows [n_slots, W-1, C] or None); the new
    window of sequence n (last W-1 rows of xx) goes to slot write_idx[n]
    after every window has been read.  All fp64."""
    x = np.asarray(x, dtype=np.float64)
    weight = np.asarray(weight, dtype=np.float64)
    T, C = x.shape
    W = weight.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    old = None if windows is None else np.asarray(windows, dtype=np.float64)
    new = None if old is None else old.copy()
    n_slots = 0 if old is None else old.shape[0]
    y = np.zeros((T, C))
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        r = -1 if read_idx is None else int(read_idx[n])
        win = old[r] if 0 <= r < n_slots else np.zeros((W - 1, C))
        xx = np.concatenate([win, x[a:b]], axis=0)
        L = b - a
        acc = np.zeros((L, C)) if bias is None else np.broadcast_to(
            np.asarray(bias, dtype=np.float64), (L, C)).copy()
        for j in range(W):
            acc += weight[:, j] * xx[j:j + L]
        y[a:b] = silu(acc) if activation == 1 else acc
        w = -1 if write_idx is None else int(write_idx[n])
        if 0 <= w < n_slots:
            new[w] = xx[-(W - 1):]
    return y, new


def conv_halo(x, bounds, width, windows, write_idx):
    """Slot write_idx[j] <- the width-1 rows of x before bounds[j+1] (zeros
    before row 0).  Returns the new windows (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.asarray(windows, dtype=np.float64).copy()
    for j in range(len(bounds) - 1):
        w = int(write_idx[j])
        if not 0 <= w < out.shape[0]:
            continue
        e = int(bounds[j + 1])
        for kk in range(width - 1):
            row = e - (width - 1) + kk
            out[w, kk] = x[row] if row >= 0 else 0.0
    return out


# ---------------------------------------------------------------------------
# Package algebra, from its definition: S -> M S + D, composition "later after
# earlier": (Mb, Db) o (Ma, Da) = (Mb Ma, Mb Da + Db), identity (I, 0).
# ---------------------------------------------------------------------------
def compose(later, earlier):
    Mb, Db = later
    Ma, Da = earlier
    return Mb @ Ma, Mb @ Da + Db


def identity_package(H, dk, dv):
    return np.broadcast_to(np.eye(dk), (H, dk, dk)).copy(), np.zeros((H, dk, dv))


def scan_sequential(Ms, Ds, S0):
    """S_in[0] = S0; S_in[j+1] = M_j S_in[j] + D_j.  Returns (S_in [nseg,...], S_final)."""
    S = np.array(S0, dtype=np.float64)
    S_in = []
    for M, D in zip(Ms, Ds):
        S_in.append(S)
        S = M @ S + D
    return np.stack(S_in), S


def scan_blelloch(Ms, Ds, S0):
    """Exclusive prefix of the packages by a Blelloch up-sweep / down-sweep
    (padded with identity packages to a power of two), then S_in[j] = Pre_j(S0)."""
    n = len(Ms)
    H, dk, _ = Ms[0].shape
    dv = Ds[0].shape[2]
    size = 1
    while size < n:
        size *= 2
    P = [(np.array(Ms[j]), np.array(Ds[j])) for j in range(n)]
    P += [identity_package(H, dk, dv) for _ in range(size - n)]
    step = 1
    while step < size:                       # up-sweep
        for i in range(2 * step - 1, size, 2 * step):
            P[i] = compose(P[i], P[i - step])
        step *= 2
    total = P[size - 1]
    P[size - 1] = identity_package(H, dk, dv)
    step = size // 2
    while step >= 1:                         # down-sweep
        for i in range(2 * step - 1, size, 2 * step):
            left = P[i - step]
            P[i - step] = P[i]
            P[i] = compose(left, P[i])
        step //= 2
    S0 = np.asarray(S0, dtype=np.float64)
    S_in = np.stack([P[j][0] @ S0 + P[j][1] for j in range(n)])
    S_final = total[0] @ S0 + total[1]
    return S_in, S_final


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over the whole tensor, in fp64.

    The two arrays must have the same shape (no broadcasting).  A NaN or an
    infinity anywhere in either makes the result NaN or infinite, which fails
    every ``<= tol`` comparison.  With ref all zeros the absolute norm of x is
    returned."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError(f"rel_l2: shapes differ: {x.shape} vs {ref.shape}")
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    if den == 0.0:
        return float(num)
    return float(num / den)
