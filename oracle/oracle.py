"""Python front end of the fp64 CPU oracle (kda_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline leg of the benchmark; never by the HIP library or its binding.

Every function takes numpy arrays in the packed token-major layout
([TT, H, D], sequence boundaries in cu_seqlens) and computes in fp64.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")          # AVX2/FMA build
_LIB_GENERIC = os.path.join(_HERE, "liboracle_generic.so")
_lib = None
# Summation order may be changed by the compiler (vectorised fp64 reductions);
# that moves results by rounding only.
_FAST = ["-O3", "-fno-math-errno", "-fassociative-math", "-fno-signed-zeros",
         "-fno-trapping-math"]


def _cpu_has_avx2() -> bool:
    try:
        flags = open("/proc/cpuinfo").read()
    except OSError:
        return False
    return " avx2" in flags and " fma" in flags


def _compile(out, extra):
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc"] + _FAST + extra + ["-fopenmp", "-fPIC", "-shared", "-o", tmp,
                                                     _SRC, "-lm"])
    os.replace(tmp, out)


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, OpenMP): an AVX2/FMA variant and a
    baseline x86-64 variant; returns the one this CPU runs."""
    for out, extra in ((_LIB, ["-march=x86-64-v3"]), (_LIB_GENERIC, [])):
        if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
            _compile(out, extra)
    return _LIB if _cpu_has_avx2() else _LIB_GENERIC


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        lib.kda_oracle_gate.argtypes = [i64, i32, i32, P, P, P, ctypes.c_double, P]
        lib.kda_oracle_l2norm.argtypes = [i64, i32, i32, P, ctypes.c_double, P, P]
        lib.kda_oracle_l2norm.restype = None
        lib.kda_oracle_l2norm_backward.argtypes = [i64, i32, i32, P, P, P, P]
        lib.kda_oracle_l2norm_backward.restype = None
        lib.kda_oracle_gate.restype = None
        lib.kda_oracle_gate_backward.argtypes = [i64, i32, i32, P, P, P, ctypes.c_double, P, P, P,
                                                 P, P]
        lib.kda_oracle_gate_backward.restype = None
        fwd = [i32, P, i32, i32, i32, P, P, P, P, P, P, i32, P, P, P, i32]
        lib.kda_oracle_forward.argtypes = fwd
        lib.kda_oracle_forward.restype = i32
        lib.kda_oracle_forward_chunked.argtypes = fwd
        lib.kda_oracle_forward_chunked.restype = i32
        lib.kda_oracle_backward.argtypes = [i32, P, i32, i32, i32, P, P, P, P, P, P, P, P, i32,
                                            P, P, P, P, P, P, P, i32]
        lib.kda_oracle_backward.restype = i32
        lib.kda_oracle_num_threads.argtypes = []
        lib.kda_oracle_num_threads.restype = i32
        _lib = lib
    return _lib


def _d(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _p(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().kda_oracle_num_threads())


def _nchunks(cu, C):
    lens = np.diff(np.asarray(cu, dtype=np.int64))
    return int(sum((int(l) + C - 1) // C for l in lens))


def gate(g_raw, A_log, dt_bias=None, log2_units=False):
    """g = unit * (-exp(A_log[h]) * softplus(g_raw + dt_bias[h])), the natural-log decay
    exponent per token and key channel; unit = ln 2 for a gate in log2 units, else 1."""
    g_raw, A_log = _d(g_raw), _d(A_log)
    TT, H, K = g_raw.shape
    g = np.empty_like(g_raw)
    db = None if dt_bias is None else _d(np.broadcast_to(dt_bias, (H, K)))
    _load().kda_oracle_gate(TT, H, K, _p(g_raw), _p(A_log), _p(db),
                            math.log(2.0) if log2_units else 1.0, _p(g))
    return g


def gate_backward(g_raw, A_log, g, dg, dt_bias=None, log2_units=False):
    """dg_raw = dg * unit * (-exp(A_log) sigmoid(g_raw + dt_bias));  dA_log[h] = sum dg * g;
    ddt_bias[h, i] = sum over tokens of dg_raw.  Returns (dg_raw, dA_log, ddt_bias)."""
    g_raw, A_log, g, dg = _d(g_raw), _d(A_log), _d(g), _d(dg)
    TT, H, K = g_raw.shape
    dg_raw = np.empty_like(g_raw)
    dA = np.empty(H, dtype=np.float64)
    ddt = np.empty((H, K), dtype=np.float64)
    db = None if dt_bias is None else _d(np.broadcast_to(dt_bias, (H, K)))
    _load().kda_oracle_gate_backward(TT, H, K, _p(g_raw), _p(A_log), _p(db),
                                     math.log(2.0) if log2_units else 1.0, _p(g), _p(dg),
                                     _p(dg_raw), _p(dA), _p(ddt))
    return dg_raw, dA, ddt


L2NORM_EPS = 1e-6


def l2norm(x, eps=L2NORM_EPS):
    """xn = x / sqrt(sum_i x_i^2 + eps) per (token, head); returns (xn, r) with r the
    reciprocal norm [TT, H]."""
    x = _d(x)
    TT, H, D = x.shape
    xn = np.empty_like(x)
    r = np.empty((TT, H))
    _load().kda_oracle_l2norm(TT, H, D, _p(x), eps, _p(xn), _p(r))
    return xn, r


def l2norm_backward(xn, r, dxn):
    """dx = r (dxn - xn (xn . dxn)) per (token, head)."""
    xn, r, dxn = _d(xn), _d(r), _d(dxn)
    TT, H, D = xn.shape
    dx = np.empty_like(xn)
    _load().kda_oracle_l2norm_backward(TT, H, D, _p(xn), _p(r), _p(dxn), _p(dx))
    return dx


def _forward(fn, q, k, v, g, beta, h0, cu, chunk, want_states, nthreads):
    q, k, v, g, beta, h0 = map(_d, (q, k, v, g, beta, h0))
    cu = np.ascontiguousarray(cu, dtype=np.int64)
    TT, H, K = q.shape
    V = v.shape[2]
    N = len(cu) - 1
    o = np.empty((TT, H, V))
    ht = np.empty((N, H, K, V))
    states = np.empty((_nchunks(cu, chunk), H, K, V)) if want_states else None
    rc = fn(N, _p(cu), H, K, V, _p(q), _p(k), _p(v), _p(g), _p(beta), _p(h0), chunk, _p(o),
            _p(ht), _p(states), nthreads)
    if rc != 0:
        raise RuntimeError("oracle forward failed: %d" % rc)
    return o, ht, states


def forward(q, k, v, g, beta, h0, cu, chunk=64, want_states=True, nthreads=0):
    """Per-token recurrence. Returns (o, ht, states at chunk starts)."""
    return _forward(_load().kda_oracle_forward, q, k, v, g, beta, h0, cu, chunk, want_states,
                    nthreads)


def forward_chunked(q, k, v, g, beta, h0, cu, chunk=64, want_states=True, nthreads=0):
    """Chunk form of the same forward (independent code path)."""
    return _forward(_load().kda_oracle_forward_chunked, q, k, v, g, beta, h0, cu, chunk,
                    want_states, nthreads)


def backward(q, k, v, g, beta, h0, dO, dht, cu, chunk=64, want_dstates=False, nthreads=0):
    """Hand-derived per-token reverse mode. Gradients w.r.t. q, k, v, g, beta, h0,
    and (optionally) dL/dS at the end of every chunk."""
    q, k, v, g, beta, h0, dO, dht = map(_d, (q, k, v, g, beta, h0, dO, dht))
    cu = np.ascontiguousarray(cu, dtype=np.int64)
    TT, H, K = q.shape
    V = v.shape[2]
    N = len(cu) - 1
    dq = np.empty((TT, H, K))
    dk = np.empty((TT, H, K))
    dv = np.empty((TT, H, V))
    dg = np.empty((TT, H, K))
    db = np.empty((TT, H))
    dh0 = np.empty((N, H, K, V))
    dst = np.empty((_nchunks(cu, chunk), H, K, V)) if want_dstates else None
    rc = _load().kda_oracle_backward(N, _p(cu), H, K, V, _p(q), _p(k), _p(v), _p(g), _p(beta),
                                     _p(h0), _p(dO), _p(dht), chunk, _p(dq), _p(dk), _p(dv),
                                     _p(dg), _p(db), _p(dh0), _p(dst), nthreads)
    if rc != 0:
        raise RuntimeError("oracle backward failed: %d" % rc)
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=db, dh0=dh0, dstates=dst)


def kda_forward(inp: dict, nthreads=0) -> dict:
    """Forward from raw inputs (same optional entries as kda_backward): o, ht and the
    states at every chunk start, by the per-token recurrence."""
    gkw = dict(dt_bias=inp.get("dt_bias"), log2_units=bool(inp.get("gate_log2", False)))
    g = gate(inp["g_raw"], inp["A_log"], **gkw)
    q, k = inp["q"], inp["k"]
    if inp.get("qk_l2norm", False):
        q, k = l2norm(q)[0], l2norm(k)[0]
    o, ht, st = forward(q, k, inp["v"], g, inp["beta"], inp["h0"], inp["cu_seqlens"],
                        chunk=inp.get("chunk", 64), want_states=True, nthreads=nthreads)
    return dict(o=o, ht=ht, states=st)


def kda_backward(inp: dict, want_dstates=False, want_states=False, nthreads=0) -> dict:
    """Full backward from raw inputs (an input dict as produced by kda_inputs):
    gate, per-token backward, gate chain rule.  Returns fp64 arrays dq, dk, dv,
    dg_raw, dA_log, dbeta, dh0, ddt_bias (+ dstates / states on request).  Optional
    entries: dt_bias [H, K] (added inside the softplus), gate_log2 (the gate is in
    log2 units: the decay per step is 2^g) and qk_l2norm (q and k are L2-normalised per
    token first; dq, dk are then w.r.t. the raw q, k)."""
    gkw = dict(dt_bias=inp.get("dt_bias"), log2_units=bool(inp.get("gate_log2", False)))
    g = gate(inp["g_raw"], inp["A_log"], **gkw)
    cu = inp["cu_seqlens"]
    q, k = inp["q"], inp["k"]
    norm = bool(inp.get("qk_l2norm", False))
    if norm:
        q, rq = l2norm(q)
        k, rk = l2norm(k)
    out = backward(q, k, inp["v"], g, inp["beta"], inp["h0"], inp["dO"],
                   inp["dht"], cu, chunk=inp.get("chunk", 64), want_dstates=want_dstates,
                   nthreads=nthreads)
    if norm:
        out["dq"] = l2norm_backward(q, rq, out["dq"])
        out["dk"] = l2norm_backward(k, rk, out["dk"])
    dg_raw, dA, ddt = gate_backward(inp["g_raw"], inp["A_log"], g, out["dg"], **gkw)
    out["dg_raw"] = dg_raw
    out["dA_log"] = dA
    out["ddt_bias"] = ddt
    out["g"] = g
    if want_states:
        o, ht, st = forward(q, k, inp["v"], g, inp["beta"], inp["h0"], cu,
                            chunk=inp.get("chunk", 64), want_states=True, nthreads=nthreads)
        out["o"], out["ht"], out["states"] = o, ht, st
    return out
