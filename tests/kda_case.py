"""Shared helpers for the GPU parity tests: upload an input dict, run the HIP
path through the C ABI, run the oracle on the same (dtype-rounded) inputs, and
compare with the metric max|gpu - ref| / max|ref| per tensor."""
from __future__ import annotations

import numpy as np

import kda_inputs as KI

TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_gpu(inp: dict):
    import torch
    dev = torch.device("cuda:0")
    act = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32

    def t(x, dt=torch.float32):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt)

    g = dict(q=t(inp["q"], act), k=t(inp["k"], act), v=t(inp["v"], act), dO=t(inp["dO"], act),
             g_raw=t(inp["g_raw"]), beta=t(inp["beta"]), A_log=t(inp["A_log"]), h0=t(inp["h0"]),
             dht=t(inp["dht"]), dt_bias=t(inp.get("dt_bias")))
    if not inp["varlen"]:
        B, T = inp["B"], inp["T"]
        for key in ("q", "k", "v", "dO", "g_raw"):
            g[key] = g[key].reshape(B, T, *g[key].shape[1:])
        g["beta"] = g["beta"].reshape(B, T, inp["H"])
    return g


def run_gpu(inp: dict, use_h_saved=True, want_dstates=True):
    import linear_attention_backward_amd as K
    import torch
    g = to_gpu(inp)
    cu = inp["cu_seqlens"] if inp["varlen"] else None
    gate = dict(dt_bias=g["dt_bias"], gate_log2=bool(inp.get("gate_log2", False)),
                qk_l2norm=bool(inp.get("qk_l2norm", False)))
    fwd = K.kda_fwd_ref(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], h0=g["h0"],
                        cu_seqlens=cu, **gate)
    out = K.kda_bwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], g["dO"],
                    h0=g["h0"], dht=g["dht"], h_saved=fwd["h_saved"] if use_h_saved else None,
                    cu_seqlens=cu, want_dstates=want_dstates, **gate)
    torch.cuda.synchronize()
    res = {}
    TT = inp["q"].shape[0]
    for key, val in list(out.items()) + [("o", fwd["o"]), ("ht", fwd["ht"]),
                                         ("h_saved", fwd["h_saved"])]:
        if val is None:
            continue
        a = val.float().cpu().numpy().astype(np.float64)
        if key in ("dq", "dk", "dv", "dg_raw", "o") and a.ndim == 4:
            a = a.reshape(TT, *a.shape[2:])
        if key == "dbeta" and a.ndim == 3:
            a = a.reshape(TT, a.shape[-1])
        res[key] = a
    return res


def rel_err(got, ref) -> float:
    den = float(np.abs(ref).max())
    num = float(np.abs(got - ref).max())
    if den == 0.0:
        return num
    return num / den


def compare(res: dict, ref: dict, keys, tol: float, heads=None, label=""):
    """Check rel_err <= tol for every key; `heads` restricts GPU tensors to the
    sampled heads (axis 1) the oracle was run on."""
    report = {}
    for key in keys:
        got = res[key]
        if heads is not None and key not in ("dA_log", "ddt_bias"):
            got = got[:, heads]
        elif heads is not None:
            got = got[heads]
        e = rel_err(got, ref[key])
        report[key] = e
    bad = {k: v for k, v in report.items() if not (v <= tol)}
    assert not bad, "%s: errors above %g: %s (all: %s)" % (label, tol, bad, report)
    return report


def oracle_for(inp: dict, heads=None, want_dstates=True, want_states=True):
    from oracle import oracle as O
    sub = KI.select_heads(inp, heads) if heads is not None else inp
    return O.kda_backward(sub, want_dstates=want_dstates, want_states=want_states)


def run_gpu_fwd(inp: dict):
    """The production forward through the C ABI: o, ht, h_saved as fp64 arrays."""
    import linear_attention_backward_amd as K
    import torch
    g = to_gpu(inp)
    cu = inp["cu_seqlens"] if inp["varlen"] else None
    fwd = K.kda_fwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], h0=g["h0"],
                    cu_seqlens=cu, dt_bias=g["dt_bias"],
                    gate_log2=bool(inp.get("gate_log2", False)),
                    qk_l2norm=bool(inp.get("qk_l2norm", False)))
    torch.cuda.synchronize()
    TT = inp["q"].shape[0]
    res = {}
    for key, val in fwd.items():
        a = val.float().cpu().numpy().astype(np.float64)
        if key == "o" and a.ndim == 4:
            a = a.reshape(TT, *a.shape[2:])
        res[key] = a
    return res


def oracle_fwd_for(inp: dict, heads=None):
    from oracle import oracle as O
    sub = KI.select_heads(inp, heads) if heads is not None else inp
    return O.kda_forward(sub)
