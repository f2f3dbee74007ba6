"""Thin Python binding of libkda.so (include/kda.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream, every step of the computation runs in the library's HIP kernels.  The
functions carry the C ABI's names.  If libkda.so has not been built, importing
this module raises ImportError; nothing falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_OK, KDA_ERR_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_ALIGN, KDA_ERR_WORKSPACE, KDA_ERR_DEVICE = range(6)
KDA_DTYPE_F32, KDA_DTYPE_BF16 = 0, 1
KDA_SCAN_SEQUENTIAL, KDA_SCAN_BLELLOCH = 0, 1
CHUNK = 64

EXPORTS = ("kda_prefill_workspace", "kda_prefill", "kda_prefill_noalloc", "kda_prefill_resume",
           "kda_segment_package", "kda_segment_package_workspace",
           "kda_segment_scan_workspace", "kda_segment_scan", "kda_output_fixup",
           "kda_output_fixup_ckpt", "kda_segment_package_fx", "kda_output_fixup_fx",
           "kda_checkpoint_write", "kda_decode", "kda_short_conv", "kda_conv_halo",
           "kda_validate_inputs", "kda_status_string", "kda_last_error", "kda_version")
# fields of kda_validate_inputs' report
KDA_CHECK_FIELDS = 8
CHECK_NAMES = ("bounds", "g_positive", "g_nonfinite", "g_block_floor", "beta_nonfinite")
KDA_ACT_NONE, KDA_ACT_SILU = 0, 1


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class kda_config(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("qk_l2norm", ctypes.c_int32)]


class kda_ckpt(ctypes.Structure):
    _fields_ = [("interval", ctypes.c_int32), ("offsets", ctypes.c_void_p),
                ("states", ctypes.c_void_p)]


class kda_fixop(ctypes.Structure):
    _fields_ = [("chunks", ctypes.c_int32), ("interval", ctypes.c_int32), ("X", ctypes.c_void_p),
                ("len", ctypes.c_void_p), ("route", ctypes.c_void_p), ("Pi", ctypes.c_void_p)]


class kda_state_pool(ctypes.Structure):
    _fields_ = [("states", ctypes.c_void_p), ("n_slots", ctypes.c_int64),
                ("read_idx", ctypes.c_void_p), ("write_idx", ctypes.c_void_p)]


class kda_conv_state(ctypes.Structure):
    _fields_ = [("states", ctypes.c_void_p), ("n_slots", ctypes.c_int64),
                ("read_idx", ctypes.c_void_p), ("write_idx", ctypes.c_void_p)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m gated_delta_rule_46_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    P, S, I32, I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    cfgp, ckp = ctypes.POINTER(kda_config), ctypes.POINTER(kda_ckpt)
    poolp = ctypes.POINTER(kda_state_pool)
    fxp = ctypes.POINTER(kda_fixop)
    convp = ctypes.POINTER(kda_conv_state)
    sig = {
        "kda_prefill_workspace": (S, [cfgp, I64, I32]),
        "kda_prefill": (ctypes.c_int, [cfgp, P, P, P, P, P, P, I32, I64, P, P, P, ckp, P, S, P]),
        "kda_prefill_noalloc": (ctypes.c_int, [cfgp, P, P, P, P, P, P, I32, I64, P, P, P, ckp, P]),
        "kda_prefill_resume": (ctypes.c_int, [cfgp, P, P, P, P, P, P, I32, I64, P, poolp, P, ckp,
                                              P, S, P]),
        "kda_segment_package": (ctypes.c_int, [cfgp, P, P, P, P, P, I64, P, I32, P, P, P, ckp,
                                               P, P, P, S, P]),
        "kda_segment_scan_workspace": (S, [cfgp, I32, I32]),
        "kda_segment_package_workspace": (S, [cfgp, I64, I32]),
        "kda_segment_scan": (ctypes.c_int, [cfgp, I32, P, P, P, P, P, I32, P, S, P]),
        "kda_output_fixup": (ctypes.c_int, [cfgp, P, P, P, P, I64, P, I32, P, P, P, S, P]),
        "kda_output_fixup_ckpt": (ctypes.c_int, [cfgp, P, P, P, P, I64, P, I32, P, P, ckp, P, P,
                                                 S, P]),
        "kda_segment_package_fx": (ctypes.c_int, [cfgp, P, P, P, P, P, I64, P, I32, P, P, P,
                                                  ckp, P, P, fxp, P, S, P]),
        "kda_output_fixup_fx": (ctypes.c_int, [cfgp, P, P, P, P, I64, P, I32, P, P, ckp, P, fxp,
                                               P]),
        "kda_checkpoint_write": (ctypes.c_int, [cfgp, ckp, I64, P, I32, P, P, P, P]),
        "kda_decode": (ctypes.c_int, [cfgp, I32, P, P, P, P, P, I32, poolp, P, P]),
        "kda_short_conv": (ctypes.c_int, [I32, I32, I32, I32, P, I64, P, I32, P, P, convp, P, P]),
        "kda_conv_halo": (ctypes.c_int, [I32, I32, I32, P, I64, P, I32, convp, P]),
        "kda_validate_inputs": (ctypes.c_int, [cfgp, I64, P, I32, I32, P, P, P, P]),
        "kda_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "kda_last_error": (ctypes.c_char_p, []),
        "kda_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()
LIB_PATH = _LIB_PATH


def version() -> str:
    return LIB.kda_version().decode()


def _check(status: int, where: str):
    if status != KDA_OK:
        raise KdaError(status, where, LIB.kda_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ckpt_rows(ckpt_offsets, ckpt_out):
    """Rung rows: from a caller-supplied output tensor (no host sync), else
    read from the last offset on the host (a device-to-host copy)."""
    if ckpt_out is not None:
        return int(ckpt_out.shape[0])
    return int(ckpt_offsets[-1].item())


def _ckpt_tensor(ckpt_out, rows, H, dk, dv, dev):
    if ckpt_out is not None:
        _need(ckpt_out, "ckpt_out", (rows, H, dk, dv), torch.float32, dev)
        return ckpt_out
    return torch.empty((max(rows, 0), H, dk, dv), dtype=torch.float32, device=dev)


def make_config(H: int, dk: int, dv: int, dtype: torch.dtype, scale: float = 1.0,
                qk_l2norm: bool = True) -> kda_config:
    if dtype == torch.bfloat16:
        io = KDA_DTYPE_BF16
    elif dtype == torch.float32:
        io = KDA_DTYPE_F32
    else:
        raise TypeError(f"q/k/v must be bfloat16 or float32, got {dtype}")
    return kda_config(H, dk, dv, CHUNK, io, float(scale), int(bool(qk_l2norm)))


def _need(t, name, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _inputs(q, k, v, g, beta):
    T, H, dk = q.shape
    dv = v.shape[2]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be device tensors")
    _need(q, "q", (T, H, dk), q.dtype, dev)
    _need(k, "k", (T, H, dk), q.dtype, dev)
    _need(v, "v", (T, H, dv), q.dtype, dev)
    _need(g, "g", (T, H, dk), torch.float32, dev)
    _need(beta, "beta", (T, H), torch.float32, dev)
    return T, H, dk, dv, dev


def _round256(b):
    return (b + 255) // 256 * 256


def kda_prefill(q, k, v, g, beta, cu_seqlens, S0=None, *, want_final=True, ckpt_interval=0,
                ckpt_offsets=None, ckpt_out=None, scale=1.0, qk_l2norm=True, out=None,
                workspace=None, stream=None):
    """Chunked prefill.  Returns (o, S_final or None, checkpoint states or None).

    cu_seqlens: int64 [N+1] device tensor.  ckpt_offsets: int64 [N+1] device
    tensor of first rung rows (required with ckpt_interval for N > 1); the
    total rung count is read from its last element on the host, unless
    ckpt_out (fp32 [rows,H,dk,dv], rows = ckpt_offsets[-1], the caller's
    guarantee, as the kernels write the rows the offsets name) is given: then
    the call makes no host synchronisation.  workspace:
    a uint8 device tensor to use instead of one of the queried size (a single
    sequence takes the segmented path only when it is large enough).
    """
    T, H, dk, dv, dev = _inputs(q, k, v, g, beta)
    N = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int64, dev)
    cfg = make_config(H, dk, dv, q.dtype, scale, qk_l2norm)
    if S0 is not None:
        _need(S0, "S0", (N, H, dk, dv), torch.float32, dev)
    o = out if out is not None else torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    _need(o, "out", (T, H, dv), q.dtype, dev)
    Sf = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if want_final else None
    ck = None
    ckp = None
    if ckpt_interval:
        if ckpt_offsets is None:
            if N != 1:
                raise ValueError("ckpt_offsets is required for more than one sequence")
            rows = T // ckpt_interval
        else:
            _need(ckpt_offsets, "ckpt_offsets", (N + 1,), torch.int64, dev)
            rows = _ckpt_rows(ckpt_offsets, ckpt_out)
        ck = _ckpt_tensor(ckpt_out, rows, H, dk, dv, dev)
        ckp = ctypes.pointer(kda_ckpt(int(ckpt_interval), _p(ckpt_offsets), _p(ck) if rows else
                                      ctypes.c_void_p(torch.empty(1, device=dev).data_ptr())))
    if workspace is not None:
        ws, wsb = workspace, workspace.numel()
    else:
        wsb = LIB.kda_prefill_workspace(ctypes.byref(cfg), T, N)
        if ckpt_interval and N == 1 and ckpt_offsets is None and wsb > 256:
            # room for the rung sub-packages of the segmented path
            rows = T // ckpt_interval
            wsb += _round256(rows * H * dk * dv * 4)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    st = LIB.kda_prefill(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(g), _p(beta), _p(cu_seqlens),
                         N, T, _p(S0), _p(Sf), _p(o), ckp, _p(ws), wsb, _stream(stream))
    _check(st, "kda_prefill")
    return o, Sf, ck


NOALLOC_SCRATCH_BYTES = 64 << 20   # KDA_NOALLOC_SCRATCH_BYTES


def kda_prefill_noalloc(q, k, v, g, beta, cu_seqlens, S0=None, *, ckpt_interval=0,
                        ckpt_offsets=None, ckpt_out=None, scale=1.0, qk_l2norm=True, out=None,
                        final_out=None, want_final=True, stream=None):
    """kda_prefill through the entry point that allocates nothing: the
    library's fixed per-device scratch replaces the workspace.  Outputs are
    allocated here unless passed (out, final_out, ckpt_out), so a caller that
    passes all of them makes no allocation at all.  Returns (o, S_final or
    None, checkpoint states or None)."""
    T, H, dk, dv, dev = _inputs(q, k, v, g, beta)
    N = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int64, dev)
    cfg = make_config(H, dk, dv, q.dtype, scale, qk_l2norm)
    if S0 is not None:
        _need(S0, "S0", (N, H, dk, dv), torch.float32, dev)
    o = out if out is not None else torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    _need(o, "out", (T, H, dv), q.dtype, dev)
    Sf = final_out
    if Sf is None and want_final:
        Sf = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    if Sf is not None:
        _need(Sf, "final_out", (N, H, dk, dv), torch.float32, dev)
    ck = None
    ckp = None
    if ckpt_interval:
        if ckpt_offsets is None:
            if N != 1:
                raise ValueError("ckpt_offsets is required for more than one sequence")
            rows = T // ckpt_interval
        else:
            _need(ckpt_offsets, "ckpt_offsets", (N + 1,), torch.int64, dev)
            rows = _ckpt_rows(ckpt_offsets, ckpt_out)
        ck = _ckpt_tensor(ckpt_out, rows, H, dk, dv, dev)
        ckp = ctypes.pointer(kda_ckpt(int(ckpt_interval), _p(ckpt_offsets),
                                      _p(ck) if rows else ctypes.c_void_p(o.data_ptr())))
    st = LIB.kda_prefill_noalloc(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(g), _p(beta),
                                 _p(cu_seqlens), N, T, _p(S0), _p(Sf), _p(o), ckp, _stream(stream))
    _check(st, "kda_prefill_noalloc")
    return o, Sf, ck


def kda_prefill_resume(q, k, v, g, beta, cu_seqlens, pool, read_idx, write_idx, *, pos0=None,
                       ckpt_interval=0, ckpt_offsets=None, ckpt_out=None, scale=1.0,
                       qk_l2norm=True, out=None, stream=None):
    """Chunked prefill continuing each sequence from pool[read_idx[n]]; the
    final state goes to pool[write_idx[n]] (pool updated in place).  pos0:
    int64 [N] absolute start positions (multiples of 64) that place the
    checkpoint rungs; ckpt_offsets: int64 [N+1] first rung rows (required
    with ckpt_interval for N > 1); ckpt_out: optional preallocated rung
    states, as in kda_prefill (no host synchronisation then).  Returns (o,
    checkpoint states or None)."""
    T, H, dk, dv, dev = _inputs(q, k, v, g, beta)
    N = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int64, dev)
    n_slots = pool.shape[0]
    _need(pool, "pool", (n_slots, H, dk, dv), torch.float32, dev)
    _need(read_idx, "read_idx", (N,), torch.int32, dev)
    _need(write_idx, "write_idx", (N,), torch.int32, dev)
    if pos0 is not None:
        _need(pos0, "pos0", (N,), torch.int64, dev)
    cfg = make_config(H, dk, dv, q.dtype, scale, qk_l2norm)
    o = out if out is not None else torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    _need(o, "out", (T, H, dv), q.dtype, dev)
    ck = None
    ckp = None
    if ckpt_interval:
        if ckpt_offsets is None:
            raise ValueError("ckpt_offsets is required with ckpt_interval")
        _need(ckpt_offsets, "ckpt_offsets", (N + 1,), torch.int64, dev)
        rows = _ckpt_rows(ckpt_offsets, ckpt_out)
        ck = _ckpt_tensor(ckpt_out, rows, H, dk, dv, dev)
        ckp = ctypes.pointer(kda_ckpt(int(ckpt_interval), _p(ckpt_offsets), _p(ck) if rows else
                                      ctypes.c_void_p(torch.empty(1, device=dev).data_ptr())))
    pl = kda_state_pool(ctypes.c_void_p(pool.data_ptr()), n_slots,
                        ctypes.c_void_p(read_idx.data_ptr()), ctypes.c_void_p(write_idx.data_ptr()))
    wsb = LIB.kda_prefill_workspace(ctypes.byref(cfg), T, N)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    st = LIB.kda_prefill_resume(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(g), _p(beta),
                                _p(cu_seqlens), N, T, _p(pos0), ctypes.byref(pl), _p(o), ckp,
                                _p(ws), wsb, _stream(stream))
    _check(st, "kda_prefill_resume")
    return o, ck


def kda_segment_package(q, k, v, g, beta, seg_start, *, ckpt_interval=0, scale=1.0,
                        qk_l2norm=True, want_M=True, want_sub_M=True, split=True, stream=None):
    """Per-segment packages.  Returns (o_local, M, D, sub_M, sub_D); M and
    sub_M are None when want_M is False (the M launch is then skipped), sub_M
    also when want_sub_M is False (rungs then from kda_output_fixup_ckpt).
    split: hand the library the workspace that lets it split segments into
    sub-segments when they would leave compute units idle."""
    T, H, dk, dv, dev = _inputs(q, k, v, g, beta)
    nseg = seg_start.numel() - 1
    _need(seg_start, "seg_start", (nseg + 1,), torch.int64, dev)
    cfg = make_config(H, dk, dv, q.dtype, scale, qk_l2norm)
    o_local = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    M = torch.empty((nseg, H, dk, dk), dtype=torch.float32, device=dev) if want_M else None
    D = torch.empty((nseg, H, dk, dv), dtype=torch.float32, device=dev)
    sub_M = sub_D = None
    ckp = None
    if ckpt_interval:
        rows = T // ckpt_interval
        if want_M and want_sub_M:
            sub_M = torch.empty((rows, H, dk, dk), dtype=torch.float32, device=dev)
        sub_D = torch.empty((rows, H, dk, dv), dtype=torch.float32, device=dev)
        if rows:
            ckp = ctypes.pointer(kda_ckpt(int(ckpt_interval), None, None))
    wsb = LIB.kda_segment_package_workspace(ctypes.byref(cfg), T, nseg) if split else 0
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
    st = LIB.kda_segment_package(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(g), _p(beta), T,
                                 _p(seg_start), nseg, _p(o_local), _p(M), _p(D), ckp,
                                 _p(sub_M) if (ckp and sub_M is not None) else None,
                                 _p(sub_D) if ckp else None,
                                 _p(ws), wsb, _stream(stream))
    _check(st, "kda_segment_package")
    return o_local, M, D, sub_M, sub_D


class FixOp:
    """Fix-up operator buffers (kda_fixop): X [nseg, chunks * 64, H, dk] in
    the I/O dtype, len [nseg, H, dk // 64] and route [nseg, H] int32, and with
    a checkpoint interval Pi [nseg, H, dk, dk] fp32."""

    def __init__(self, nseg, H, dk, dtype, device, chunks=6, interval=0):
        self.chunks = int(chunks)
        self.interval = int(interval)
        self.Pi = (torch.empty((nseg, H, dk, dk), dtype=torch.float32, device=device)
                   if self.interval else None)
        self.X = torch.empty((nseg, self.chunks * CHUNK, H, dk), dtype=dtype, device=device)
        self.len = torch.empty((nseg, H, dk // 64), dtype=torch.int32, device=device)
        self.route = torch.empty((nseg, H), dtype=torch.int32, device=device)

    def c(self):
        return kda_fixop(self.chunks, self.interval, ctypes.c_void_p(self.X.data_ptr()),
                         ctypes.c_void_p(self.len.data_ptr()),
                         ctypes.c_void_p(self.route.data_ptr()),
                         ctypes.c_void_p(self.Pi.data_ptr()) if self.Pi is not None else None)


def kda_segment_package_fx(q, k, v, g, beta, seg_start, fx, *, ckpt_interval=0, scale=1.0,
                           qk_l2norm=True, want_sub_M=True, split=True, stream=None):
    """kda_segment_package that also fills the fix-up operator fx (a FixOp).
    Returns (o_local, M, D, sub_M, sub_D).  split: as kda_segment_package."""
    T, H, dk, dv, dev = _inputs(q, k, v, g, beta)
    nseg = seg_start.numel() - 1
    _need(seg_start, "seg_start", (nseg + 1,), torch.int64, dev)
    _need(fx.X, "fx.X", (nseg, fx.chunks * CHUNK, H, dk), q.dtype, dev)
    _need(fx.len, "fx.len", (nseg, H, dk // 64), torch.int32, dev)
    cfg = make_config(H, dk, dv, q.dtype, scale, qk_l2norm)
    o_local = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    M = torch.empty((nseg, H, dk, dk), dtype=torch.float32, device=dev)
    D = torch.empty((nseg, H, dk, dv), dtype=torch.float32, device=dev)
    sub_M = sub_D = None
    ckp = None
    if ckpt_interval:
        rows = T // ckpt_interval
        if want_sub_M:
            sub_M = torch.empty((rows, H, dk, dk), dtype=torch.float32, device=dev)
        sub_D = torch.empty((rows, H, dk, dv), dtype=torch.float32, device=dev)
        if rows:
            ckp = ctypes.pointer(kda_ckpt(int(ckpt_interval), None, None))
    fxc = fx.c()
    wsb = LIB.kda_segment_package_workspace(ctypes.byref(cfg), T, nseg) if split else 0
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
    st = LIB.kda_segment_package_fx(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(g), _p(beta), T,
                                    _p(seg_start), nseg, _p(o_local), _p(M), _p(D), ckp,
                                    _p(sub_M) if (ckp and sub_M is not None) else None,
                                    _p(sub_D) if ckp else None, ctypes.byref(fxc), _p(ws), wsb,
                                    _stream(stream))
    _check(st, "kda_segment_package_fx")
    return o_local, M, D, sub_M, sub_D


def kda_segment_scan(M, D, S0=None, *, algo=KDA_SCAN_SEQUENTIAL, stream=None):
    """Prefix scan of the packages.  Returns (S_in [nseg,H,dk,dv], S_final [H,dk,dv])."""
    nseg, H, dk, _ = M.shape
    dv = D.shape[3]
    dev = M.device
    _need(M, "M", (nseg, H, dk, dk), torch.float32, dev)
    _need(D, "D", (nseg, H, dk, dv), torch.float32, dev)
    if S0 is not None:
        _need(S0, "S0", (H, dk, dv), torch.float32, dev)
    cfg = kda_config(H, dk, dv, CHUNK, KDA_DTYPE_BF16, 1.0, 1)
    S_in = torch.empty((nseg, H, dk, dv), dtype=torch.float32, device=dev)
    S_final = torch.empty((H, dk, dv), dtype=torch.float32, device=dev)
    wsb = LIB.kda_segment_scan_workspace(ctypes.byref(cfg), nseg, algo)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    st = LIB.kda_segment_scan(ctypes.byref(cfg), nseg, _p(M), _p(D), _p(S0), _p(S_in),
                              _p(S_final), algo, _p(ws), wsb, _stream(stream))
    _check(st, "kda_segment_scan")
    return S_in, S_final


def kda_output_fixup(q, k, g, beta, seg_start, S_in, o, *, scale=1.0, qk_l2norm=True,
                     stream=None):
    """o (holding o_local) is corrected in place from S_in; returns o."""
    T, H, dk = q.shape
    dev = q.device
    dv = o.shape[2]
    nseg = seg_start.numel() - 1
    _need(k, "k", (T, H, dk), q.dtype, dev)
    _need(g, "g", (T, H, dk), torch.float32, dev)
    _need(beta, "beta", (T, H), torch.float32, dev)
    _need(o, "o", (T, H, dv), q.dtype, dev)
    _need(seg_start, "seg_start", (nseg + 1,), torch.int64, dev)
    _need(S_in, "S_in", (nseg, H, dk, dv), torch.float32, dev)
    cfg = make_config(H, dk, dv, q.dtype, scale, qk_l2norm)
    st = LIB.kda_output_fixup(ctypes.byref(cfg), _p(q), _p(k), _p(g), _p(beta), T,
                              _p(seg_start), nseg, _p(S_in), _p(o), None, 0, _stream(stream))
    _check(st, "kda_output_fixup")
    return o


def kda_output_fixup_ckpt(q, k, g, beta, seg_start, S_in, o, sub_D, *, interval, out=None,
                          scale=1.0, qk_l2norm=True, stream=None):
    """The fix-up of o (in place) and the checkpoint rungs [T // interval, H,
    dk, dv] in one launch; returns the rung states (into `out` when given)."""
    T, H, dk = q.shape
    dev = q.device
    dv = o.shape[2]
    nseg = seg_start.numel() - 1
    rows = T // interval
    _need(k, "k", (T, H, dk), q.dtype, dev)
    _need(g, "g", (T, H, dk), torch.float32, dev)
    _need(beta, "beta", (T, H), torch.float32, dev)
    _need(o, "o", (T, H, dv), q.dtype, dev)
    _need(seg_start, "seg_start", (nseg + 1,), torch.int64, dev)
    _need(S_in, "S_in", (nseg, H, dk, dv), torch.float32, dev)
    _need(sub_D, "sub_D", (rows, H, dk, dv), torch.float32, dev)
    states = out if out is not None else torch.empty((rows, H, dk, dv), dtype=torch.float32,
                                                     device=dev)
    _need(states, "out", (rows, H, dk, dv), torch.float32, dev)
    cfg = make_config(H, dk, dv, q.dtype, scale, qk_l2norm)
    ck = kda_ckpt(int(interval), None, ctypes.c_void_p(states.data_ptr()))
    st = LIB.kda_output_fixup_ckpt(ctypes.byref(cfg), _p(q), _p(k), _p(g), _p(beta), T,
                                   _p(seg_start), nseg, _p(S_in), _p(o),
                                   ctypes.byref(ck) if rows else None, _p(sub_D) if rows else None,
                                   None, 0, _stream(stream))
    _check(st, "kda_output_fixup_ckpt")
    return states


def kda_output_fixup_fx(q, k, g, beta, seg_start, S_in, o, fx, *, sub_D=None, interval=0,
                        out=None, scale=1.0, qk_l2norm=True, stream=None):
    """The fix-up of o (in place) with the operator fx (a FixOp, or None), and
    with sub_D and interval also the checkpoint rungs (into `out` when given,
    which may be sub_D itself); returns the rung states or None."""
    T, H, dk = q.shape
    dev = q.device
    dv = o.shape[2]
    nseg = seg_start.numel() - 1
    _need(k, "k", (T, H, dk), q.dtype, dev)
    _need(g, "g", (T, H, dk), torch.float32, dev)
    _need(beta, "beta", (T, H), torch.float32, dev)
    _need(o, "o", (T, H, dv), q.dtype, dev)
    _need(seg_start, "seg_start", (nseg + 1,), torch.int64, dev)
    _need(S_in, "S_in", (nseg, H, dk, dv), torch.float32, dev)
    states = None
    ck = None
    rows = T // interval if interval else 0
    if rows:
        _need(sub_D, "sub_D", (rows, H, dk, dv), torch.float32, dev)
        states = out if out is not None else torch.empty((rows, H, dk, dv), dtype=torch.float32,
                                                         device=dev)
        _need(states, "out", (rows, H, dk, dv), torch.float32, dev)
        ck = kda_ckpt(int(interval), None, ctypes.c_void_p(states.data_ptr()))
    if fx is not None:
        _need(fx.X, "fx.X", (nseg, fx.chunks * CHUNK, H, dk), q.dtype, dev)
        _need(fx.len, "fx.len", (nseg, H, dk // 64), torch.int32, dev)
    fxc = fx.c() if fx is not None else None
    cfg = make_config(H, dk, dv, q.dtype, scale, qk_l2norm)
    st = LIB.kda_output_fixup_fx(ctypes.byref(cfg), _p(q), _p(k), _p(g), _p(beta), T,
                                 _p(seg_start), nseg, _p(S_in), _p(o),
                                 ctypes.byref(ck) if ck is not None else None,
                                 _p(sub_D) if rows else None,
                                 ctypes.byref(fxc) if fxc is not None else None, _stream(stream))
    _check(st, "kda_output_fixup_fx")
    return states


def kda_validate_inputs(*, T, H, dk, g=None, beta=None, bounds=None, chunk_aligned=False,
                        stream=None):
    """Debug check of device-side inputs (kda_validate_inputs): bounds are
    cu_seqlens, or segment starts with chunk_aligned=True.  Waits for the
    stream and returns the report as a dict of counts (all zero: inside what
    the kernels assume)."""
    dev = next(x.device for x in (g, beta, bounds) if x is not None)
    if g is not None:
        _need(g, "g", (T, H, dk), torch.float32, dev)
    if beta is not None:
        _need(beta, "beta", (T, H), torch.float32, dev)
    n = 0
    if bounds is not None:
        n = bounds.numel() - 1
        _need(bounds, "bounds", (n + 1,), torch.int64, dev)
    report = torch.empty(KDA_CHECK_FIELDS, dtype=torch.int32, device=dev)
    cfg = make_config(H, dk, dk, torch.bfloat16)
    st = LIB.kda_validate_inputs(ctypes.byref(cfg), int(T), _p(bounds), n, int(bool(chunk_aligned)),
                                 _p(g), _p(beta), _p(report), _stream(stream))
    _check(st, "kda_validate_inputs")
    r = report.cpu().tolist()
    return dict(zip(CHECK_NAMES, r))


def kda_checkpoint_write(seg_start, S_in, sub_M, sub_D, *, T, interval, dtype=torch.bfloat16,
                         out=None, stream=None):
    """Segment-path checkpoint states [T // interval, H, dk, dv] (into `out`
    when given)."""
    rows, H, dk, dv = sub_D.shape
    dev = S_in.device
    nseg = seg_start.numel() - 1
    _need(seg_start, "seg_start", (nseg + 1,), torch.int64, dev)
    _need(S_in, "S_in", (nseg, H, dk, dv), torch.float32, dev)
    _need(sub_M, "sub_M", (rows, H, dk, dk), torch.float32, dev)
    cfg = make_config(H, dk, dv, dtype)
    states = out if out is not None else torch.empty((rows, H, dk, dv), dtype=torch.float32,
                                                     device=dev)
    _need(states, "out", (rows, H, dk, dv), torch.float32, dev)
    if rows == 0:
        return states
    ck = kda_ckpt(int(interval), None, ctypes.c_void_p(states.data_ptr()))
    st = LIB.kda_checkpoint_write(ctypes.byref(cfg), ctypes.byref(ck), int(T), _p(seg_start),
                                  nseg, _p(S_in), _p(sub_M), _p(sub_D), _stream(stream))
    _check(st, "kda_checkpoint_write")
    return states


def kda_segment_prefill(q, k, v, g, beta, seg_start, S0=None, *, algo=KDA_SCAN_BLELLOCH,
                        ckpt_interval=0, scale=1.0, qk_l2norm=True, stream=None):
    """The whole segment path on one stream: package -> scan -> fix-up with
    the checkpoint rungs.  Returns (o, S_final, checkpoint states or None)."""
    o, M, D, _, sub_D = kda_segment_package(q, k, v, g, beta, seg_start,
                                            ckpt_interval=ckpt_interval, scale=scale,
                                            qk_l2norm=qk_l2norm, want_sub_M=False, stream=stream)
    S_in, S_final = kda_segment_scan(M, D, S0, algo=algo, stream=stream)
    if ckpt_interval:
        ck = kda_output_fixup_ckpt(q, k, g, beta, seg_start, S_in, o, sub_D,
                                   interval=ckpt_interval, scale=scale, qk_l2norm=qk_l2norm,
                                   stream=stream)
        return o, S_final, ck
    kda_output_fixup(q, k, g, beta, seg_start, S_in, o, scale=scale, qk_l2norm=qk_l2norm,
                     stream=stream)
    return o, S_final, None


def kda_decode(q, k, v, g, beta, pool, read_idx, write_idx, *, gate_logits=False, scale=1.0,
               qk_l2norm=True, out=None, stream=None):
    """One decode step for N sequences (row n of q, k, v, g, beta).

    pool: fp32 [n_slots,H,dk,dv] states, updated in place at write_idx;
    read_idx / write_idx: int32 [N] device tensors (negative = zero state /
    not written).  gate_logits: g and beta are logits activated in the kernel.
    Returns o [N,H,dv].
    """
    N, H, dk, dv, dev = _inputs(q, k, v, g, beta)
    n_slots = pool.shape[0]
    _need(pool, "pool", (n_slots, H, dk, dv), torch.float32, dev)
    _need(read_idx, "read_idx", (N,), torch.int32, dev)
    _need(write_idx, "write_idx", (N,), torch.int32, dev)
    cfg = make_config(H, dk, dv, q.dtype, scale, qk_l2norm)
    o = out if out is not None else torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _need(o, "out", (N, H, dv), q.dtype, dev)
    pl = kda_state_pool(ctypes.c_void_p(pool.data_ptr()), n_slots, ctypes.c_void_p(read_idx.data_ptr()),
                        ctypes.c_void_p(write_idx.data_ptr()))
    st = LIB.kda_decode(ctypes.byref(cfg), N, _p(q), _p(k), _p(v), _p(g), _p(beta),
                        int(bool(gate_logits)), ctypes.byref(pl), _p(o), _stream(stream))
    _check(st, "kda_decode")
    return o


def _io_dtype(dtype):
    if dtype == torch.bfloat16:
        return KDA_DTYPE_BF16
    if dtype == torch.float32:
        return KDA_DTYPE_F32
    raise TypeError(f"x must be bfloat16 or float32, got {dtype}")


def _conv_state(windows, read_idx, write_idx, N, C, W, dtype, dev):
    if windows is None:
        if read_idx is not None or write_idx is not None:
            raise ValueError("read_idx / write_idx need windows")
        return None
    n_slots = windows.shape[0]
    _need(windows, "windows", (n_slots, W - 1, C), dtype, dev)
    if read_idx is not None:
        _need(read_idx, "read_idx", (N,), torch.int32, dev)
    if write_idx is not None:
        _need(write_idx, "write_idx", (N,), torch.int32, dev)
    return kda_conv_state(ctypes.c_void_p(windows.data_ptr()), n_slots, _p(read_idx), _p(write_idx))


def kda_short_conv(x, cu_seqlens, weight, bias=None, *, windows=None, read_idx=None,
                   write_idx=None, activation=KDA_ACT_NONE, out=None, stream=None):
    """Causal depthwise convolution over tokens of x [T, C] (bf16 or fp32),
    weight [C, W] fp32, bias [C] fp32 or None, sequences by cu_seqlens
    (int64 [N+1]).  windows [n_slots, W-1, C] (x's dtype) with read_idx /
    write_idx (int32 [N]) carry each sequence's window in and out; the new
    windows are written in place.  Returns y [T, C]."""
    T, C = x.shape
    W = weight.shape[1]
    dev = x.device
    N = cu_seqlens.numel() - 1
    _need(x, "x", (T, C), x.dtype, dev)
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int64, dev)
    _need(weight, "weight", (C, W), torch.float32, dev)
    if bias is not None:
        _need(bias, "bias", (C,), torch.float32, dev)
    y = out if out is not None else torch.empty((T, C), dtype=x.dtype, device=dev)
    _need(y, "out", (T, C), x.dtype, dev)
    st = _conv_state(windows, read_idx, write_idx, N, C, W, x.dtype, dev)
    rc = LIB.kda_short_conv(_io_dtype(x.dtype), C, W, int(activation), _p(x), T, _p(cu_seqlens), N,
                            _p(weight), _p(bias), ctypes.byref(st) if st is not None else None,
                            _p(y), _stream(stream))
    _check(rc, "kda_short_conv")
    return y


def kda_conv_halo(x, bounds, width, windows, write_idx, *, stream=None):
    """Copies the width-1 rows before each bounds[j+1] of x [T, C] into
    windows[write_idx[j]] (zeros before row 0); returns windows."""
    T, C = x.shape
    dev = x.device
    nseg = bounds.numel() - 1
    _need(bounds, "bounds", (nseg + 1,), torch.int64, dev)
    st = _conv_state(windows, None, write_idx, nseg, C, width, x.dtype, dev)
    if st is None:
        raise ValueError("windows is required")
    rc = LIB.kda_conv_halo(_io_dtype(x.dtype), C, int(width), _p(x), T, _p(bounds), nseg,
                           ctypes.byref(st), _stream(stream))
    _check(rc, "kda_conv_halo")
    return windows
