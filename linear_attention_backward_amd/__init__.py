"""KDA (gated delta rule) chunkwise backward for MI355X -- Python binding.

Thin ctypes front end of libkda.so (include/kda.h).  Torch tensors supply
device memory and the current HIP stream; every step of the computation runs in
the library's HIP kernels.  If libkda.so is missing or cannot be loaded every
call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_OK = 0
KDA_ERR_INVALID_ARGUMENT = -1
KDA_ERR_UNSUPPORTED = -2
KDA_ERR_WORKSPACE_TOO_SMALL = -3
KDA_ERR_HIP = -4
KDA_ERR_SCRATCH_TOO_SMALL = -5
KDA_NOALLOC_SCRATCH_BYTES = 64 << 20
KDA_DTYPE_F32 = 0
KDA_DTYPE_BF16 = 1
KDA_WS_BWD = 0
KDA_WS_FWD = 1
KDA_WS_FWD_REF = 2
KDA_GATE_LN = 0
KDA_GATE_LOG2 = 1
CHUNK = 64

STAGES = ("chunk_table", "prep", "scan", "grad", "dalog", "recompute", "l2norm")

_P = ctypes.c_void_p


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int), ("K", ctypes.c_int),
                ("V", ctypes.c_int), ("chunk", ctypes.c_int), ("act_dtype", ctypes.c_int),
                ("num_seqs", ctypes.c_int), ("cu_seqlens_host", _P), ("cu_seqlens_dev", _P),
                ("gate_units", ctypes.c_int), ("qk_l2norm", ctypes.c_int)]


class BwdIO(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("q", "k", "v", "g_raw", "beta", "A_log", "h0", "dO", "dht",
                                  "h_saved", "dq", "dk", "dv", "dg_raw", "dbeta", "dA_log", "dh0",
                                  "dstates", "dt_bias", "ddt_bias")]


class FwdIO(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("q", "k", "v", "g_raw", "beta", "A_log", "h0", "o", "ht",
                                  "h_saved", "dt_bias")]


class KdaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("kda status %d: %s" % (status, msg))
        self.status = status


_lib = None


def load_library():
    """Load libkda.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libkda.so not built: run `python -m linear_attention_backward_amd.build`"
                              " (or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        PP = ctypes.POINTER(Problem)
        lib.kda_abi_version.restype = ctypes.c_int
        lib.kda_status_string.argtypes = [ctypes.c_int]
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_workspace_size.argtypes = [PP, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
        lib.kda_num_chunks.argtypes = [PP, ctypes.POINTER(ctypes.c_int64)]
        lib.kda_bwd.argtypes = [PP, ctypes.POINTER(BwdIO), _P, ctypes.c_size_t, _P]
        lib.kda_fwd_ref.argtypes = [PP, ctypes.POINTER(FwdIO), _P, ctypes.c_size_t, _P]
        lib.kda_fwd.argtypes = [PP, ctypes.POINTER(FwdIO), _P, ctypes.c_size_t, _P]
        lib.kda_bwd_noalloc.argtypes = [PP, ctypes.POINTER(BwdIO), _P]
        lib.kda_timing_enable.argtypes = [ctypes.c_int]
        lib.kda_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int), ctypes.c_int]
        for f in ("kda_workspace_size", "kda_num_chunks", "kda_bwd", "kda_fwd_ref", "kda_fwd",
                  "kda_bwd_noalloc", "kda_timing_enable", "kda_timing_read"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(st: int):
    if st != KDA_OK:
        raise KdaError(st, load_library().kda_status_string(st).decode())


def status_string(st: int) -> str:
    return load_library().kda_status_string(st).decode()


def abi_version() -> int:
    return load_library().kda_abi_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class _Prob:
    """A kda_problem plus the host copy of cu_seqlens it points at."""

    def __init__(self, B, T, H, K, V, dtype_code, cu_host=None, cu_dev=None, gate_units=0,
                 qk_l2norm=0):
        self.cu_host = None
        if cu_host is not None:
            self.cu_host = (ctypes.c_int32 * len(cu_host))(*[int(x) for x in cu_host])
        self.p = Problem(B, T, H, K, V, CHUNK, dtype_code,
                         (len(cu_host) - 1) if cu_host is not None else 0,
                         ctypes.cast(self.cu_host, _P) if self.cu_host is not None else None,
                         _ptr(cu_dev) if cu_dev is not None else None, gate_units, qk_l2norm)

    def ref(self):
        return ctypes.byref(self.p)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return KDA_DTYPE_BF16
    if t.dtype == torch.float32:
        return KDA_DTYPE_F32
    raise TypeError("activations must be bfloat16 or float32, got %s" % t.dtype)


def _shape(q, v, cu_seqlens):
    """(B, T, H, K, V) for [B,T,H,K] or packed [T,H,K] activations."""
    if q.dim() == 4:
        B, T, H, K = q.shape
    elif q.dim() == 3:
        B = 1
        T, H, K = q.shape
    else:
        raise ValueError("q must be [B,T,H,K] or [T,H,K]")
    V = v.shape[-1]
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed sequences need B == 1")
    return B, T, H, K, V


def _make_prob(q, v, cu_seqlens, gate_log2=False, qk_l2norm=False):
    import torch
    B, T, H, K, V = _shape(q, v, cu_seqlens)
    cu_host = cu_dev = None
    if cu_seqlens is not None:
        cu_host = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist")
                                    else cu_seqlens)]
        cu_dev = torch.tensor(cu_host, dtype=torch.int32, device=q.device)
    prob = _Prob(B, T, H, K, V, _dtype_code(q), cu_host, cu_dev,
                 KDA_GATE_LOG2 if gate_log2 else KDA_GATE_LN, 1 if qk_l2norm else 0)
    prob.cu_dev_tensor = cu_dev  # keep alive
    return prob, (B, T, H, K, V)


def num_chunks(prob: _Prob) -> int:
    n = ctypes.c_int64(0)
    _check(load_library().kda_num_chunks(prob.ref(), ctypes.byref(n)))
    return int(n.value)


def workspace_size(prob: _Prob, which: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().kda_workspace_size(prob.ref(), which, ctypes.byref(n)))
    return int(n.value)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _n_chunks_host(B, T, cu_seqlens):
    """Chunk count for shape checks (the library's kda_num_chunks gives the same)."""
    if cu_seqlens is None:
        return B * ((T + CHUNK - 1) // CHUNK)
    cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
    return sum((cu[i + 1] - cu[i] + CHUNK - 1) // CHUNK for i in range(len(cu) - 1))


def _validate(q, v, cu_seqlens, named, act_named=(), h_saved=None):
    """Check every tensor against the shapes, dtypes and layout the kernels assume,
    before anything reaches the library: the kernels read dense row-major memory of
    exactly these sizes, so a wrong dtype would make them read past a buffer and a
    strided view would be read as if it were dense.

    named: (name, tensor, shape, dtype) with None tensors skipped; act_named: (name,
    tensor) that must match q's shape-with-last-dim and dtype.  Returns (B, T, H, K, V, N).
    """
    import torch
    B, T, H, K, V = _shape(q, v, cu_seqlens)
    N = (len(cu_seqlens) - 1) if cu_seqlens is not None else B
    lead = tuple(q.shape[:-1])
    checks = [("q", q, lead + (K,), q.dtype)]
    for name, t in act_named:
        d = V if name in ("v", "dO") else K
        checks.append((name, t, lead + (d,), q.dtype))
    for name, t, shp, dt in named:
        checks.append((name, t, shp(lead, B, T, H, K, V, N), dt))
    if h_saved is not None:
        checks.append(("h_saved", h_saved, (_n_chunks_host(B, T, cu_seqlens), H, K, V), q.dtype))
    _dtype_code(q)
    for name, t, shp, dt in checks:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
        if t.dtype != dt:
            raise ValueError("%s must be %s, got %s" % (name, dt, t.dtype))
        if tuple(t.shape) != tuple(shp):
            raise ValueError("%s must have shape %s, got %s" % (name, tuple(shp), tuple(t.shape)))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous (dense row-major)" % name)
    devs = {t.device for _, t, _, _ in checks if t is not None}
    if len(devs) > 1:
        raise ValueError("all tensors must be on one device, got %s" % sorted(map(str, devs)))
    _require_cuda(*[t for _, t, _, _ in checks])
    return B, T, H, K, V, N


def _gate_specs(g_raw, beta, A_log, h0, dt_bias):
    import torch
    f32 = torch.float32
    return [("g_raw", g_raw, lambda L, B, T, H, K, V, N: L + (K,), f32),
            ("beta", beta, lambda L, B, T, H, K, V, N: L, f32),
            ("A_log", A_log, lambda L, B, T, H, K, V, N: (H,), f32),
            ("h0", h0, lambda L, B, T, H, K, V, N: (N, H, K, V), f32),
            ("dt_bias", dt_bias, lambda L, B, T, H, K, V, N: (H, K), f32)]


def kda_fwd_ref(q, k, v, g_raw, beta, A_log, h0=None, cu_seqlens=None, want_o=True,
                want_ht=True, want_states=True, stream=None, workspace=None, dt_bias=None,
                gate_log2=False, qk_l2norm=False, _entry="kda_fwd_ref"):
    """Reference forward: returns dict(o, ht, h_saved).  dt_bias [H, K] (optional) is
    added inside the softplus; gate_log2 = True takes the gate in log2 units;
    qk_l2norm = True L2-normalises q and k per token first."""
    import torch
    for name, t in (("g_raw", g_raw), ("beta", beta), ("A_log", A_log)):
        if t is None:
            raise ValueError("%s is required" % name)
    _validate(q, v, cu_seqlens, _gate_specs(g_raw, beta, A_log, h0, dt_bias),
              (("k", k), ("v", v)))
    prob, (B, T, H, K, V) = _make_prob(q, v, cu_seqlens, gate_log2, qk_l2norm)
    N = (len(prob.cu_host) - 1) if prob.cu_host is not None else B
    nc = num_chunks(prob)
    dev = q.device
    o = torch.empty_like(v) if want_o else None
    ht = torch.empty((N, H, K, V), dtype=torch.float32, device=dev) if want_ht else None
    hs = torch.empty((nc, H, K, V), dtype=q.dtype, device=dev) if want_states else None
    ws_n = workspace_size(prob, KDA_WS_FWD_REF if _entry == "kda_fwd_ref" else KDA_WS_FWD)
    ws = workspace if workspace is not None else torch.empty(max(ws_n, 1), dtype=torch.uint8,
                                                             device=dev)
    io = FwdIO(_ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta), _ptr(A_log), _ptr(h0),
               _ptr(o), _ptr(ht), _ptr(hs), _ptr(dt_bias))
    _check(getattr(load_library(), _entry)(prob.ref(), ctypes.byref(io), _ptr(ws), ws.numel(),
                                           _stream_ptr(stream)))
    return dict(o=o, ht=ht, h_saved=hs)


def kda_fwd(q, k, v, g_raw, beta, A_log, h0=None, cu_seqlens=None, want_o=True, want_ht=True,
            want_states=True, stream=None, workspace=None, dt_bias=None, gate_log2=False,
            qk_l2norm=False):
    """Production forward (chunk form), same arguments and results as kda_fwd_ref."""
    return kda_fwd_ref(q, k, v, g_raw, beta, A_log, h0, cu_seqlens, want_o, want_ht, want_states,
                       stream, workspace, dt_bias, gate_log2, qk_l2norm, _entry="kda_fwd")


class BwdPlan:
    """Pre-allocated outputs and workspace for repeated kda_bwd calls on fixed
    shapes (used by the benchmark so the timed region allocates nothing)."""

    def __init__(self, q, k, v, g_raw, beta, A_log, dO, h0=None, dht=None, h_saved=None,
                 cu_seqlens=None, want_dh0=True, want_dstates=False, dt_bias=None,
                 gate_log2=False, want_ddt_bias=None, qk_l2norm=False):
        import torch
        for name, t in (("g_raw", g_raw), ("beta", beta), ("A_log", A_log), ("dO", dO)):
            if t is None:
                raise ValueError("%s is required" % name)
        specs = _gate_specs(g_raw, beta, A_log, h0, dt_bias)
        specs.append(("dht", dht, lambda L, B, T, H, K, V, N: (N, H, K, V), torch.float32))
        _validate(q, v, cu_seqlens, specs, (("k", k), ("v", v), ("dO", dO)), h_saved=h_saved)
        self.prob, (B, T, H, K, V) = _make_prob(q, v, cu_seqlens, gate_log2, qk_l2norm)
        N = (len(self.prob.cu_host) - 1) if self.prob.cu_host is not None else B
        dev = q.device
        self.inputs = (q, k, v, g_raw, beta, A_log, dO, h0, dht, h_saved, dt_bias)
        if want_ddt_bias is None:
            want_ddt_bias = dt_bias is not None
        self.ddt_bias = (torch.empty((H, K), dtype=torch.float32, device=dev) if want_ddt_bias
                         else None)
        self.dq = torch.empty_like(q)
        self.dk = torch.empty_like(k)
        self.dv = torch.empty_like(v)
        self.dg_raw = torch.empty_like(g_raw)
        self.dbeta = torch.empty_like(beta)
        self.dA_log = torch.empty_like(A_log)
        self.dh0 = torch.empty((N, H, K, V), dtype=torch.float32, device=dev) if want_dh0 else None
        self.nc = num_chunks(self.prob)
        self.dstates = (torch.empty((self.nc, H, K, V), dtype=q.dtype, device=dev)
                        if want_dstates else None)
        ws_n = workspace_size(self.prob, KDA_WS_BWD)
        self.ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
        self.io = BwdIO(_ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta), _ptr(A_log), _ptr(h0),
                        _ptr(dO), _ptr(dht), _ptr(h_saved), _ptr(self.dq), _ptr(self.dk),
                        _ptr(self.dv), _ptr(self.dg_raw), _ptr(self.dbeta), _ptr(self.dA_log),
                        _ptr(self.dh0), _ptr(self.dstates), _ptr(dt_bias), _ptr(self.ddt_bias))

    def run(self, stream=None):
        _check(load_library().kda_bwd(self.prob.ref(), ctypes.byref(self.io), _ptr(self.ws),
                                      self.ws.numel(), _stream_ptr(stream)))

    def run_noalloc(self, stream=None):
        """The same call through kda_bwd_noalloc: the library's static device scratch
        instead of this plan's workspace (nothing is allocated)."""
        _check(load_library().kda_bwd_noalloc(self.prob.ref(), ctypes.byref(self.io),
                                              _stream_ptr(stream)))

    def outputs(self):
        return dict(dq=self.dq, dk=self.dk, dv=self.dv, dg_raw=self.dg_raw, dbeta=self.dbeta,
                    dA_log=self.dA_log, dh0=self.dh0, dstates=self.dstates,
                    ddt_bias=self.ddt_bias)


def kda_bwd(q, k, v, g_raw, beta, A_log, dO, h0=None, dht=None, h_saved=None, cu_seqlens=None,
            want_dh0=True, want_dstates=False, stream=None, dt_bias=None, gate_log2=False,
            qk_l2norm=False):
    """Backward pass.  Returns dict(dq, dk, dv, dg_raw, dbeta, dA_log, dh0, dstates,
    ddt_bias); ddt_bias is produced when dt_bias is given."""
    plan = BwdPlan(q, k, v, g_raw, beta, A_log, dO, h0, dht, h_saved, cu_seqlens, want_dh0,
                   want_dstates, dt_bias, gate_log2, qk_l2norm=qk_l2norm)
    plan.run(stream)
    return plan.outputs()


def timing_enable(on: bool = True):
    _check(load_library().kda_timing_enable(1 if on else 0))


def timing_read():
    """Per-stage (total ms, launches) since the last read, keyed by stage name."""
    n = len(STAGES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    load_library().kda_timing_read(ms, cnt, n)
    return {STAGES[i]: (ms[i], cnt[i]) for i in range(n)}
