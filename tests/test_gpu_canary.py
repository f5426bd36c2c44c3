"""Out-of-bounds and phantom-row writes: every output of kda_bwd and kda_fwd (and the
workspace) is placed inside a larger device buffer whose guard regions before and after
hold a fixed byte pattern.  Rows past a sequence's end inside its last chunk have no
address of their own in the native [T, H, D] layout (they are the next sequence's rows,
or lie past the tensor), so a phantom-row write either corrupts a neighbour's gradient
(caught by the oracle comparison here) or lands in a guard (caught by the guard check).
The output bodies start as NaN, so an element the kernels never write fails too.
"""
import ctypes

import numpy as np
import pytest

import kda_inputs as KI
from tests import kda_case as KC

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes; keeps the body 256-byte aligned
PAT = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_backward_amd as K
    K.load_library()


class Guarded:
    """A device tensor of `shape`/`dtype` inside a guarded byte buffer."""

    def __init__(self, shape, dtype):
        import torch
        self.shape, self.dtype = tuple(shape), dtype
        self.nbytes = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.buf = torch.full((self.nbytes + 2 * GUARD,), PAT, dtype=torch.uint8, device="cuda")
        self.buf[GUARD:GUARD + self.nbytes] = 0xFF  # NaN in fp32 and bf16
        self.ptr = ctypes.c_void_p(self.buf.data_ptr() + GUARD)

    def guards_intact(self):
        g = self.buf.cpu().numpy()
        return bool(np.all(g[:GUARD] == PAT) and np.all(g[GUARD + self.nbytes:] == PAT))

    def value(self):
        body = self.buf[GUARD:GUARD + self.nbytes].view(self.dtype).reshape(self.shape)
        return body.float().cpu().numpy().astype(np.float64)


def _zero_len():
    return KI.make_inputs(KI.Workload("zero_len", 1, 0 + 70 + 0 + 5 + 64, 2, 128, 128, "bf16",
                                      1200, varlen_seqs=4, fixed_lengths=(0, 70, 0, 69),
                                      h0_std=0.3, dht_std=1.0))


def _inputs(name):
    return _zero_len() if name == "zero_len" else KI.make_inputs(KI.get_workload(name))


NAMES = ["ragged_bf16", "multi_ragged_bf16", "zero_len", "qk_norm_bf16", "ragged_fp32",
         "gate_bias_bf16"]


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("fused", [None, "1"])
def test_backward_writes_stay_in_bounds(name, fused, monkeypatch):
    """fused = "1": the state scan inside prep (which writes dU into the workspace) and
    the gradient pass that reads it; None: the path the library picks (separate
    kernels for these small cases)."""
    import torch
    import linear_attention_backward_amd as K
    if fused is not None:
        if name == "zero_len":
            pytest.skip("the scan inside prep needs a chunk in every sequence")
        monkeypatch.setenv("KDA_PREPSCAN", fused)
    inp = _inputs(name)
    print("\n[case] canary backward %s prepscan=%s" % (name, fused), flush=True)
    g = KC.to_gpu(inp)
    cu = inp["cu_seqlens"] if inp["varlen"] else None
    gate = dict(dt_bias=g["dt_bias"], gate_log2=bool(inp.get("gate_log2", False)),
                qk_l2norm=bool(inp.get("qk_l2norm", False)))
    fwd = K.kda_fwd_ref(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], h0=g["h0"],
                        cu_seqlens=cu, **gate)
    prob, (B, T, H, D, V) = K._make_prob(g["q"], g["v"], cu, gate["gate_log2"],
                                         gate["qk_l2norm"])
    N = inp["N"]
    nc = K.num_chunks(prob)
    act = g["q"].dtype
    lead = tuple(g["q"].shape[:-1])
    outs = {"dq": Guarded(lead + (D,), act), "dk": Guarded(lead + (D,), act),
            "dv": Guarded(lead + (V,), act), "dg_raw": Guarded(lead + (D,), torch.float32),
            "dbeta": Guarded(lead, torch.float32), "dA_log": Guarded((H,), torch.float32),
            "dh0": Guarded((N, H, D, V), torch.float32),
            "dstates": Guarded((nc, H, D, V), act)}
    if g["dt_bias"] is not None:
        outs["ddt_bias"] = Guarded((H, D), torch.float32)
    ws_n = K.workspace_size(prob, K.KDA_WS_BWD)
    ws = Guarded((max(ws_n, 1),), torch.uint8)
    P = K._ptr
    io = K.BwdIO(P(g["q"]), P(g["k"]), P(g["v"]), P(g["g_raw"]), P(g["beta"]), P(g["A_log"]),
                 P(g["h0"]), P(g["dO"]), P(g["dht"]), P(fwd["h_saved"]),
                 outs["dq"].ptr, outs["dk"].ptr, outs["dv"].ptr, outs["dg_raw"].ptr,
                 outs["dbeta"].ptr, outs["dA_log"].ptr, outs["dh0"].ptr, outs["dstates"].ptr,
                 P(g["dt_bias"]), outs["ddt_bias"].ptr if "ddt_bias" in outs else None)
    K._check(K.load_library().kda_bwd(prob.ref(), ctypes.byref(io), ws.ptr, ws_n,
                                      K._stream_ptr()))
    torch.cuda.synchronize()
    bad = [k for k, o in outs.items() if not o.guards_intact()]
    assert not bad and ws.guards_intact(), "writes past a buffer: %s (workspace %s)" % (
        bad, ws.guards_intact())
    TT = inp["q"].shape[0]
    res = {}
    for key, o in outs.items():
        a = o.value()
        if key in ("dq", "dk", "dv", "dg_raw"):
            a = a.reshape(TT, H, -1)
        elif key == "dbeta":
            a = a.reshape(TT, H)
        assert np.all(np.isfinite(a)), key + " has elements that were never written"
        res[key] = a
    ref = KC.oracle_for(inp)
    keys = ["dq", "dk", "dv", "dg_raw", "dbeta", "dA_log", "dh0", "dstates"]
    keys += ["ddt_bias"] if "ddt_bias" in outs else []
    KC.compare(res, ref, keys, KC.TOL[inp["dtype"]], label="canary " + name)


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("entry", ["kda_fwd", "kda_fwd_ref"])
def test_forward_writes_stay_in_bounds(name, entry):
    import torch
    import linear_attention_backward_amd as K
    inp = _inputs(name)
    print("\n[case] canary %s %s" % (entry, name), flush=True)
    g = KC.to_gpu(inp)
    cu = inp["cu_seqlens"] if inp["varlen"] else None
    gl2, qkn = bool(inp.get("gate_log2", False)), bool(inp.get("qk_l2norm", False))
    prob, (B, T, H, D, V) = K._make_prob(g["q"], g["v"], cu, gl2, qkn)
    N = inp["N"]
    nc = K.num_chunks(prob)
    act = g["q"].dtype
    outs = {"o": Guarded(tuple(g["v"].shape), act), "ht": Guarded((N, H, D, V), torch.float32),
            "h_saved": Guarded((nc, H, D, V), act)}
    ws_n = K.workspace_size(prob, K.KDA_WS_FWD if entry == "kda_fwd" else K.KDA_WS_FWD_REF)
    ws = Guarded((max(ws_n, 1),), torch.uint8)
    P = K._ptr
    io = K.FwdIO(P(g["q"]), P(g["k"]), P(g["v"]), P(g["g_raw"]), P(g["beta"]), P(g["A_log"]),
                 P(g["h0"]), outs["o"].ptr, outs["ht"].ptr, outs["h_saved"].ptr, P(g["dt_bias"]))
    K._check(getattr(K.load_library(), entry)(prob.ref(), ctypes.byref(io), ws.ptr, ws_n,
                                              K._stream_ptr()))
    torch.cuda.synchronize()
    bad = [k for k, o in outs.items() if not o.guards_intact()]
    assert not bad and ws.guards_intact(), "writes past a buffer: %s (workspace %s)" % (
        bad, ws.guards_intact())
    TT = inp["q"].shape[0]
    res = {k: o.value() for k, o in outs.items()}
    res["o"] = res["o"].reshape(TT, H, V)
    for key, a in res.items():
        assert np.all(np.isfinite(a)), key + " has elements that were never written"
    ref = KC.oracle_fwd_for(inp)
    ref["h_saved"] = ref["states"]
    KC.compare(res, ref, ["o", "ht", "h_saved"], KC.TOL[inp["dtype"]],
               label="canary %s %s" % (entry, name))
