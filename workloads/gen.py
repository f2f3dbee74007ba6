"""Seeded synthetic KDA prefill workloads.

Every array is drawn from numpy's PCG64 with a fixed seed, in float32, and then
rounded once (round-to-nearest-even) to the workload's I/O dtype.  Both the
fp64 oracle and the GPU path consume exactly these rounded values.

Draw recipe (one independent substream per tensor and head, so heads can be
generated in parallel and a single (sequence, head) unit can be re-derived):

    rng([seed, TENSOR_ID, head])           q, k, v : N(0, 1)      shape [T, d]
                                           beta    : sigmoid(N(0,1) + beta_shift)   [T]
                                           g       : -softplus(N(0,1) + gate_shift) [T, dk]
    rng([seed, TENSOR_ID, head, seq])      S0      : N(0, s0_std^2)   [dk, dv]

with seed = 46000 + workload index for the five standard workloads.  The
"long-memory" variants shift the logits (gate_shift=-9, beta_shift=-6) so the
per-token decay is about 1.2e-4 and a state survives thousands of tokens.

The module draws and lays out random numbers only; it contains none of the
method's arithmetic (normalisation, decay, recurrence).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload", "make_workload", "standard_workload", "STANDARD",
    "bf16_round_bits", "bf16_bits_to_f32", "to_f64", "leveled_segments",
    "varlen_lengths", "ckpt_offsets", "GATE_COST_Q", "SEGMENT_FLOOR",
    "DecodeBatch", "make_decode_batch", "decode_slots", "standard_decode_batch",
    "ConvCase", "make_conv_case", "make_packages", "scale_qk_pow2",
]

T_Q, T_K, T_V, T_BETA, T_G, T_S0, T_POOL, T_CONV = 0, 1, 2, 3, 4, 5, 6, 7

# Segment cost model coefficient and the per-segment token floor quoted by the
# pegainfer "cross-process CP whale gang" PR (commit "whale rendezvous":
# t ~ len + Q*depth*len with Q = 2.7e-6, FlashKDA saturation floor 2048).
GATE_COST_Q = 2.7e-6
SEGMENT_FLOOR = 2048


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------------------
# bf16 rounding (round to nearest even), bit-exact and NaN-preserving
# ----------------------------------------------------------------------------
def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    r = ((u + bias) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored input (bf16 bits or float32) -> float64 values."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# Workload description
# ----------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    T: int
    H: int
    dk: int
    dv: int
    dtype: str                      # "f32" or "bf16": I/O dtype of q, k, v, o
    chunk: int
    cu_seqlens: np.ndarray          # int64 [N+1]
    q: np.ndarray                   # [T,H,dk] uint16 bf16 bits or float32
    k: np.ndarray
    v: np.ndarray                   # [T,H,dv]
    g: np.ndarray                   # [T,H,dk] float32, log-decay (<= 0)
    beta: np.ndarray                # [T,H] float32
    S0: np.ndarray | None           # [N,H,dk,dv] float32 or None (= zeros)
    seg_start: np.ndarray | None = None   # int64 [nseg+1] for the segment path
    scan_algo: int = 0              # 0 sequential, 1 Blelloch
    ckpt_interval: int = 0          # tokens between checkpoints, 0 = none
    scale: float = 1.0
    qk_l2norm: int = 1
    meta: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return int(len(self.cu_seqlens) - 1)

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens)

    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if name in ("q", "k", "v"):
            return to_f64(a, self.dtype)
        return np.asarray(a, dtype=np.float64)

    def unit(self, n: int, h: int) -> dict:
        """float64 inputs of one (sequence, head) unit, shaped [L,1,d]."""
        a, b = int(self.cu_seqlens[n]), int(self.cu_seqlens[n + 1])
        out = {}
        for name in ("q", "k", "v", "g"):
            x = getattr(self, name)[a:b, h:h + 1]
            out[name] = to_f64(x, self.dtype) if name in ("q", "k", "v") else x.astype(np.float64)
        out["beta"] = self.beta[a:b, h:h + 1].astype(np.float64)
        out["S0"] = None if self.S0 is None else self.S0[n:n + 1, h:h + 1].astype(np.float64)
        return out


def _gen_head(seed, tid, h, shape, kind, shift=0.0):
    rng = np.random.default_rng([seed, tid, h])
    x = rng.standard_normal(shape, dtype=np.float32)
    if kind == "normal":
        return x
    if shift:
        x = x + np.float32(shift)
    if kind == "sigmoid":
        return (np.float32(1.0) / (np.float32(1.0) + np.exp(-x))).astype(np.float32)
    if kind == "neg_softplus":
        return (-np.logaddexp(np.float32(0.0), x)).astype(np.float32)
    raise ValueError(kind)


def _fill(out, seed, tid, kind, shift, dtype_round, T, H, d):
    """Fill out[T,H,d] (or [T,H] when d == 0) head by head in parallel."""
    def work(h):
        shape = (T, d) if d else (T,)
        x = _gen_head(seed, tid, h, shape, kind, shift)
        if dtype_round == "bf16":
            out[:, h] = bf16_round_bits(x)
        else:
            out[:, h] = x
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(work, range(H)))


def make_workload(name: str, lengths, H: int, dk: int, dv: int, dtype: str, seed: int,
                  chunk: int = 64, s0_std: float | None = 0.1, gate_shift: float = 0.0,
                  beta_shift: float = 0.0, seg_start=None, scan_algo: int = 0,
                  ckpt_interval: int = 0, scale: float = 1.0, qk_l2norm: int = 1) -> Workload:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    io = np.uint16 if dtype == "bf16" else np.float32
    q = np.empty((T, H, dk), dtype=io)
    k = np.empty((T, H, dk), dtype=io)
    v = np.empty((T, H, dv), dtype=io)
    g = np.empty((T, H, dk), dtype=np.float32)
    beta = np.empty((T, H), dtype=np.float32)
    _fill(q, seed, T_Q, "normal", 0.0, dtype, T, H, dk)
    _fill(k, seed, T_K, "normal", 0.0, dtype, T, H, dk)
    _fill(v, seed, T_V, "normal", 0.0, dtype, T, H, dv)
    _fill(beta, seed, T_BETA, "sigmoid", beta_shift, "f32", T, H, 0)
    _fill(g, seed, T_G, "neg_softplus", gate_shift, "f32", T, H, dk)
    S0 = None
    N = len(lengths)
    if s0_std:
        S0 = np.empty((N, H, dk, dv), dtype=np.float32)
        for n in range(N):
            for h in range(H):
                rng = np.random.default_rng([seed, T_S0, h, n])
                S0[n, h] = rng.standard_normal((dk, dv), dtype=np.float32) * np.float32(s0_std)
    ss = None if seg_start is None else np.asarray(seg_start, dtype=np.int64)
    return Workload(name=name, T=T, H=H, dk=dk, dv=dv, dtype=dtype, chunk=chunk,
                    cu_seqlens=cu, q=q, k=k, v=v, g=g, beta=beta, S0=S0, seg_start=ss,
                    scan_algo=scan_algo, ckpt_interval=ckpt_interval, scale=scale,
                    qk_l2norm=qk_l2norm,
                    meta=dict(seed=seed, s0_std=s0_std, gate_shift=gate_shift,
                              beta_shift=beta_shift))


# ----------------------------------------------------------------------------
# Segment leveling and varlen lengths
# ----------------------------------------------------------------------------
def leveled_segments(T: int, nseg: int, Q: float = GATE_COST_Q, align: int = 64,
                     floor: int = SEGMENT_FLOOR) -> np.ndarray:
    """Segment starts [nseg+1] for the quadratic cost model t ~ len*(1 + Q*depth).

    depth of segment j = its start offset p_j.  Solve L_j (1 + Q p_j) = c for all
    j with sum L_j = T (bisection on c), then round the cumulative boundaries to
    multiples of `align`.  Deeper segments get fewer tokens.
    """
    def lens_for(c):
        p, out = 0.0, []
        for _ in range(nseg):
            L = c / (1.0 + Q * p)
            out.append(L)
            p += L
        return out, p

    lo, hi = 0.0, float(T)
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        _, tot = lens_for(mid)
        if tot < T:
            lo = mid
        else:
            hi = mid
    Ls, _ = lens_for(0.5 * (lo + hi))
    cum = np.cumsum(Ls)[:-1]
    b = [0] + [int(round(x / align)) * align for x in cum] + [T]
    b = np.asarray(b, dtype=np.int64)
    if np.any(np.diff(b) < floor):
        raise ValueError("segment below the floor")
    return b


def varlen_lengths(seed: int, n: int, lo: int = 512, hi: int = 32768) -> np.ndarray:
    """Log-uniform lengths in [lo, hi] (first draws of rng(seed))."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(np.log(lo), np.log(hi), n)
    return np.clip(np.floor(np.exp(u)).astype(np.int64), lo, hi)


def ckpt_offsets(lengths, interval: int, pos0=None) -> np.ndarray:
    """First checkpoint row of each sequence: rungs at p = m*interval <= len, m >= 1.

    With pos0 (absolute start positions), rungs sit at absolute multiples P of
    the interval with pos0 < P <= pos0 + len."""
    lengths = np.asarray(lengths, dtype=np.int64)
    if interval > 0 and pos0 is not None:
        p0 = np.asarray(pos0, dtype=np.int64)
        per = (p0 + lengths) // interval - p0 // interval
    else:
        per = lengths // interval if interval > 0 else np.zeros_like(lengths)
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    off[1:] = np.cumsum(per)
    return off


# ----------------------------------------------------------------------------
# The five standard workloads
# ----------------------------------------------------------------------------
STANDARD = {
    0: "single sequence, H=1, T=256, d=64, fp32, S0=0",
    1: "single sequence, H=32, T=8192, d=128, bf16, S0~N(0,0.1), chunked path",
    2: "segment path, H=32, T=16384, d=128, bf16, 4x4096 segments, sequential scan",
    3: "segment path, H=32, T=131072, d=128, bf16, 16 leveled segments, Blelloch scan",
    4: "varlen batch, 64 sequences log-uniform 512-32768, H=32, d=128, bf16, ckpt 4096",
}


def standard_workload(idx: int, s0_std: float | None = None, **over) -> Workload:
    seed = 46000 + idx
    if idx == 0:
        return make_workload("kda-t256-h1-d64-f32", [256], 1, 64, 64, "f32", seed,
                             s0_std=s0_std, **over)
    if idx == 1:
        return make_workload("kda-t8192-h32-d128-bf16", [8192], 32, 128, 128, "bf16", seed,
                             s0_std=0.1 if s0_std is None else s0_std, **over)
    if idx == 2:
        return make_workload("kda-seg4x4096-t16384-h32-d128-bf16", [16384], 32, 128, 128,
                             "bf16", seed, s0_std=0.1 if s0_std is None else s0_std,
                             seg_start=np.arange(0, 16385, 4096), scan_algo=0, **over)
    if idx == 3:
        return make_workload("kda-seg16-leveled-t131072-h32-d128-bf16", [131072], 32, 128, 128,
                             "bf16", seed, s0_std=0.1 if s0_std is None else s0_std,
                             seg_start=leveled_segments(131072, 16), scan_algo=1,
                             ckpt_interval=4096, **over)
    if idx == 4:
        L = varlen_lengths(seed, 64)
        return make_workload("kda-varlen64-h32-d128-bf16", L, 32, 128, 128, "bf16", seed,
                             s0_std=0.1 if s0_std is None else s0_std, ckpt_interval=4096,
                             **over)
    raise ValueError(idx)


# ----------------------------------------------------------------------------
# Decode batches: one new token per sequence, states in a slot pool
# ----------------------------------------------------------------------------
@dataclass
class DecodeBatch:
    name: str
    N: int
    H: int
    dk: int
    dv: int
    dtype: str
    q: np.ndarray                   # [N,H,dk] uint16 bf16 bits or float32
    k: np.ndarray
    v: np.ndarray                   # [N,H,dv]
    g: np.ndarray                   # [N,H,dk] float32: logits when gate_logits, else log-decay
    beta: np.ndarray                # [N,H] float32: logits when gate_logits, else beta
    gate_logits: bool
    pool: np.ndarray                # [n_slots,H,dk,dv] float32
    read_idx: np.ndarray            # int32 [N]
    write_idx: np.ndarray           # int32 [N]
    scale: float = 1.0
    qk_l2norm: int = 1

    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if name in ("q", "k", "v"):
            return to_f64(a, self.dtype)
        return np.asarray(a, dtype=np.float64)


def decode_slots(N: int, n_slots: int):
    """Slot pattern of a decode batch with N <= n_slots // 2.

    Sequence n reads slot perm[n] (a fixed permutation of 0..N-1).  Even n
    update in place; odd n fork into slot N + n, which nothing reads.  Every
    8th sequence (n % 8 == 3) starts from a zero state (read index -1) and
    every 16th (n % 16 == 5) keeps no state (write index -1).  Write slots are
    then distinct and never another sequence's read slot.
    """
    if 2 * N > n_slots:
        raise ValueError("the pattern needs n_slots >= 2N")
    perm = np.random.default_rng([N, n_slots]).permutation(N).astype(np.int32)
    read = perm.copy()
    write = np.where(np.arange(N) % 2 == 0, perm, N + np.arange(N)).astype(np.int32)
    read[np.arange(N) % 8 == 3] = -1
    write[np.arange(N) % 16 == 5] = -1
    return read, write


def make_decode_batch(name: str, N: int, H: int, dk: int, dv: int, dtype: str, seed: int,
                      n_slots: int | None = None, gate_logits: bool = True,
                      s_std: float = 0.1, read_idx=None, write_idx=None) -> DecodeBatch:
    n_slots = 2 * N if n_slots is None else n_slots
    io = np.uint16 if dtype == "bf16" else np.float32
    q = np.empty((N, H, dk), dtype=io)
    k = np.empty((N, H, dk), dtype=io)
    v = np.empty((N, H, dv), dtype=io)
    g = np.empty((N, H, dk), dtype=np.float32)
    beta = np.empty((N, H), dtype=np.float32)
    _fill(q, seed, T_Q, "normal", 0.0, dtype, N, H, dk)
    _fill(k, seed, T_K, "normal", 0.0, dtype, N, H, dk)
    _fill(v, seed, T_V, "normal", 0.0, dtype, N, H, dv)
    _fill(beta, seed, T_BETA, "normal" if gate_logits else "sigmoid", 0.0, "f32", N, H, 0)
    _fill(g, seed, T_G, "normal" if gate_logits else "neg_softplus", 0.0, "f32", N, H, dk)
    pool = np.empty((n_slots, H, dk, dv), dtype=np.float32)

    def slot(i):
        rng = np.random.default_rng([seed, T_POOL, i])
        pool[i] = rng.standard_normal((H, dk, dv), dtype=np.float32) * np.float32(s_std)
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(slot, range(n_slots)))
    if read_idx is None or write_idx is None:
        r, w = decode_slots(N, n_slots)
        read_idx = r if read_idx is None else read_idx
        write_idx = w if write_idx is None else write_idx
    return DecodeBatch(name=name, N=N, H=H, dk=dk, dv=dv, dtype=dtype, q=q, k=k, v=v, g=g,
                       beta=beta, gate_logits=gate_logits, pool=pool,
                       read_idx=np.asarray(read_idx, dtype=np.int32),
                       write_idx=np.asarray(write_idx, dtype=np.int32))


def standard_decode_batch(**over) -> DecodeBatch:
    """64 sequences (the varlen batch's count), H=32, d=128, bf16, 128-slot pool."""
    return make_decode_batch("kda-decode-n64-h32-d128-bf16", 64, 32, 128, 128, "bf16",
                             46005, **over)


# ----------------------------------------------------------------------------
# Short convolution cases
# ----------------------------------------------------------------------------
@dataclass
class ConvCase:
    name: str
    dtype: str
    x: np.ndarray                   # [T, C] uint16 bf16 bits or float32
    cu_seqlens: np.ndarray          # int64 [N+1]
    weight: np.ndarray              # [C, W] float32
    bias: np.ndarray                # [C] float32
    windows: np.ndarray             # [n_slots, W-1, C] in x's storage
    read_idx: np.ndarray            # int32 [N]
    write_idx: np.ndarray           # int32 [N]

    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if name in ("x", "windows"):
            return to_f64(a, self.dtype)
        return np.asarray(a, dtype=np.float64)


def make_conv_case(name: str, lengths, C: int, W: int, dtype: str, seed: int,
                   n_slots: int | None = None, read_idx=None, write_idx=None) -> ConvCase:
    """x ~ N(0,1) [T, C]; taps ~ N(0, 1/W); bias ~ N(0, 0.1^2); windows ~
    N(0,1); slots by decode_slots unless given."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    T, N = int(cu[-1]), len(lengths)
    n_slots = 2 * N if n_slots is None else n_slots
    rng = np.random.default_rng([seed, T_CONV])
    x = rng.standard_normal((T, C), dtype=np.float32)
    win = rng.standard_normal((n_slots, W - 1, C), dtype=np.float32)
    weight = (rng.standard_normal((C, W), dtype=np.float32) / np.float32(np.sqrt(W))).astype(np.float32)
    bias = (rng.standard_normal(C, dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    if dtype == "bf16":
        x, win = bf16_round_bits(x), bf16_round_bits(win)
    if read_idx is None or write_idx is None:
        r, w = decode_slots(N, n_slots)
        read_idx = r if read_idx is None else read_idx
        write_idx = w if write_idx is None else write_idx
    return ConvCase(name=name, dtype=dtype, x=x, cu_seqlens=cu, weight=weight, bias=bias,
                    windows=win, read_idx=np.asarray(read_idx, dtype=np.int32),
                    write_idx=np.asarray(write_idx, dtype=np.int32))


def make_packages(nseg: int, H: int, dk: int, dv: int, seed: int, zero=(), m_std: float | None = None):
    """Random fp32 segment packages for scan tests: M ~ N(0, m_std^2) (default
    0.5/sqrt(dk), spectral norm about 1), D ~ N(0, 1), S0 ~ N(0, 0.1^2); the M
    of every segment listed in `zero` is exactly zero.  Returns (M [nseg,H,dk,dk],
    D [nseg,H,dk,dv], S0 [H,dk,dv]), all float32."""
    rng = np.random.default_rng([seed, 8])
    sd = 0.5 / np.sqrt(dk) if m_std is None else m_std
    M = (rng.standard_normal((nseg, H, dk, dk)) * sd).astype(np.float32)
    D = rng.standard_normal((nseg, H, dk, dv)).astype(np.float32)
    S0 = (rng.standard_normal((H, dk, dv)) * 0.1).astype(np.float32)
    for j in zero:
        M[j] = 0.0
    return M, D, S0


def scale_qk_pow2(w, e: int):
    """Multiplies the stored q and k of a workload or decode batch by 2**e in
    place (exact in fp32 and bf16 for these magnitudes): inputs for runs
    without the in-kernel L2 norm, whose keys must stay short enough for the
    delta rule to contract (|k|^2 = dk * 4**e on average)."""
    for name in ("q", "k"):
        a = getattr(w, name)
        if w.dtype == "bf16":
            a[...] = bf16_round_bits(bf16_bits_to_f32(a) * np.float32(2.0 ** e))
        else:
            a *= np.float32(2.0 ** e)
