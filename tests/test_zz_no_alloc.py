"""kda_bwd_noalloc (workspace in the library's static device scratch, nothing
allocated) against kda_bwd with a caller workspace, through the C ABI: the same kernels
on the same inputs, so the outputs must agree bit for bit (and therefore within the
parity bar).  Two calls in a row, the second on a smaller problem, so the second runs
on scratch that still holds the first call's contents; then a call without h_saved
(the in-stream state recompute also lives in the scratch) and a problem too large for
the scratch, which is rejected without a launch.
"""
import ctypes

import numpy as np
import pytest

import kda_inputs as KI
from tests import kda_case as KC

pytestmark = pytest.mark.gpu

OUTS = ("dq", "dk", "dv", "dg_raw", "dbeta", "dA_log", "dh0", "dstates")


@pytest.fixture(scope="module")
def lib():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_backward_amd as K
    lib = K.load_library()
    lib.kda_bwd_noalloc.argtypes = [ctypes.POINTER(K.Problem), ctypes.POINTER(K.BwdIO),
                                    ctypes.c_void_p]
    lib.kda_bwd_noalloc.restype = ctypes.c_int
    return lib


def _run_both(lib, name, use_h_saved=True):
    import torch
    import linear_attention_backward_amd as K
    inp = KI.make_inputs(KI.get_workload(name))
    print("\n[case] no-alloc %s h_saved=%s" % (name, use_h_saved), flush=True)
    g = KC.to_gpu(inp)
    cu = inp["cu_seqlens"] if inp["varlen"] else None
    gate = dict(dt_bias=g["dt_bias"], gate_log2=bool(inp.get("gate_log2", False)),
                qk_l2norm=bool(inp.get("qk_l2norm", False)))
    fwd = K.kda_fwd_ref(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], h0=g["h0"],
                        cu_seqlens=cu, **gate)
    hs = fwd["h_saved"] if use_h_saved else None
    ref_plan = K.BwdPlan(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], g["dO"],
                         h0=g["h0"], dht=g["dht"], h_saved=hs, cu_seqlens=cu, want_dstates=True,
                         **gate)
    ref_plan.run()
    # the same call through the no-allocation entry point, into fresh output buffers
    plan = K.BwdPlan(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], g["dO"],
                     h0=g["h0"], dht=g["dht"], h_saved=hs, cu_seqlens=cu, want_dstates=True,
                     **gate)
    for key in OUTS:  # make stale values visible
        t = getattr(plan, key)
        if t is not None:
            t.fill_(float("nan"))
    st = lib.kda_bwd_noalloc(plan.prob.ref(), ctypes.byref(plan.io), K._stream_ptr())
    assert st == 0, K.status_string(st)
    torch.cuda.synchronize()
    a, b = ref_plan.outputs(), plan.outputs()
    tol = KC.TOL[inp["dtype"]]
    for key in OUTS:
        if a[key] is None:
            continue
        x = a[key].float().cpu().numpy().astype(np.float64)
        y = b[key].float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(y)), key
        assert KC.rel_err(y, x) <= tol, key
        assert np.array_equal(a[key].view(torch.uint8 if a[key].dtype == torch.bfloat16
                                          else torch.int32).cpu().numpy(),
                              b[key].view(torch.uint8 if b[key].dtype == torch.bfloat16
                                          else torch.int32).cpu().numpy()), key


def test_noalloc_matches_kda_bwd(lib):
    _run_both(lib, "weak_decay_bf16")      # 128 chunk-heads, h0 / dht, split scans
    _run_both(lib, "ragged_bf16")          # smaller, on the scratch the first call left
    _run_both(lib, "gate_log2_fp32", use_h_saved=False)  # state recompute in the scratch


def test_noalloc_rejects_oversized(lib):
    import linear_attention_backward_amd as K
    prob = K._Prob(8, 4096, 32, 128, 128, K.KDA_DTYPE_BF16)
    io = K.BwdIO()
    io.h_saved = 256  # given: the smaller workspace, still far above the scratch
    st = lib.kda_bwd_noalloc(prob.ref(), ctypes.byref(io), None)
    assert st == -5, st
    assert "scratch" in K.status_string(st)
