"""kda_bwd and kda_fwd captured into a HIP graph (through torch.cuda.CUDAGraph) and replayed.

The library enqueues kernels only (no memory set, copy, allocation or host
synchronisation inside a call), so one call can be captured and replayed; every
replay must reproduce the eager call bit for bit (the kernels are deterministic).
Each replay follows eager work of the program's own (a second plan's eager call and
an overwrite of the graph's outputs), with a synchronisation in between, and is
checked against the eager result."""
import numpy as np
import pytest

import kda_inputs as KI
from tests import kda_case as KC

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_backward_amd as K
    K.load_library()


def _plan(inp, use_h_saved=True):
    import linear_attention_backward_amd as K
    import torch
    g = KC.to_gpu(inp)
    cu = inp["cu_seqlens"] if inp["varlen"] else None
    vk = dict(dt_bias=g["dt_bias"], gate_log2=bool(inp.get("gate_log2", False)),
              qk_l2norm=bool(inp.get("qk_l2norm", False)))
    hs = None
    if use_h_saved:
        hs = K.kda_fwd_ref(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"],
                           h0=g["h0"], cu_seqlens=cu, want_o=False, want_ht=False,
                           **vk)["h_saved"]
    torch.cuda.synchronize()
    plan = K.BwdPlan(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], g["dO"],
                     h0=g["h0"], dht=g["dht"], h_saved=hs, cu_seqlens=cu, want_dstates=True,
                     **vk)
    return plan, g


def _snapshot(plan):
    return {k: v.clone() for k, v in plan.outputs().items() if v is not None}


@pytest.mark.parametrize("name,env,use_h_saved", [
    ("tiny_fp32", {}, True),
    ("ragged_bf16", {}, True),                       # separate prep and scan kernels
    ("weak_decay_bf16", {"KDA_PREPSCAN": "1"}, True),  # the scan inside prep
    ("single_seq_bf16", {}, True),                   # split scan (groups of chunks)
    ("gate_bias_bf16", {}, False),                   # with the in-stream state recompute
    ("qk_norm_fp32", {"KDA_PREPSCAN": "1"}, False),
])
def test_graph_replay_matches_eager(name, env, use_h_saved, monkeypatch):
    import torch
    for key, val in env.items():
        monkeypatch.setenv(key, val)
    print("\n[case] graph %s env=%s h_saved=%s" % (name, env, use_h_saved), flush=True)
    inp = KI.make_inputs(KI.get_workload(name))
    plan, _ = _plan(inp, use_h_saved)
    other, _ = _plan(KI.make_inputs(KI.get_workload("tiny_fp32")))
    stream = torch.cuda.current_stream()
    plan.run(stream)
    torch.cuda.synchronize()
    ref = _snapshot(plan)

    # capture (torch wants the captured work run once on a side stream first)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        plan.run(side)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.run(torch.cuda.current_stream())
    torch.cuda.synchronize()

    for rep in range(3):
        for t in plan.outputs().values():  # eager overwrite: the replay must rewrite all
            if t is not None:
                t.fill_(float("nan"))
        other.run(stream)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for key, want in ref.items():
            got = plan.outputs()[key]
            assert torch.equal(got, want), "%s replay %d: %s differs" % (name, rep, key)
    # and the result is still the oracle's (replays reproduce a checked call)
    res = {k: v.float().cpu().numpy().astype(np.float64) for k, v in ref.items()}
    TT = inp["q"].shape[0]
    for key in ("dq", "dk", "dv", "dg_raw"):
        if res[key].ndim == 4:
            res[key] = res[key].reshape(TT, *res[key].shape[2:])
    if res["dbeta"].ndim == 3:
        res["dbeta"] = res["dbeta"].reshape(TT, -1)
    oref = KC.oracle_for(inp)
    keys = ["dq", "dk", "dv", "dg_raw", "dbeta", "dA_log", "dh0", "dstates"]
    if inp.get("dt_bias") is not None:
        keys.append("ddt_bias")
    KC.compare(res, oref, keys, KC.TOL[inp["dtype"]], label=name + " graph")


@pytest.mark.parametrize("name,env", [
    ("tiny_fp32", {}),
    ("ragged_bf16", {}),                        # per-chunk pass, then the state scan
    ("weak_decay_bf16", {"KDA_PREPSCAN": "1"}),  # the state scan inside prep
    ("single_seq_bf16", {}),                    # split scan
])
def test_graph_replay_forward(name, env, monkeypatch):
    """kda_fwd captured and replayed: o, ht and h_saved bitwise equal to the eager call."""
    import ctypes
    import linear_attention_backward_amd as K
    import torch
    for key, val in env.items():
        monkeypatch.setenv(key, val)
    print("\n[case] graph forward %s env=%s" % (name, env), flush=True)
    inp = KI.make_inputs(KI.get_workload(name))
    g = KC.to_gpu(inp)
    cu = inp["cu_seqlens"] if inp["varlen"] else None
    vk = dict(dt_bias=g["dt_bias"], gate_log2=bool(inp.get("gate_log2", False)),
              qk_l2norm=bool(inp.get("qk_l2norm", False)))
    prob = K._make_prob(g["q"], g["v"], cu, vk["gate_log2"], vk["qk_l2norm"])[0]
    ws = torch.empty(max(K.workspace_size(prob, K.KDA_WS_FWD), 1), dtype=torch.uint8,
                     device="cuda")
    res = K.kda_fwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], h0=g["h0"],
                    cu_seqlens=cu, workspace=ws, **vk)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in res.items()}
    io = K.FwdIO(*[K._ptr(x) for x in (g["q"], g["k"], g["v"], g["g_raw"], g["beta"],
                                       g["A_log"], g["h0"], res["o"], res["ht"],
                                       res["h_saved"], g["dt_bias"])])
    lib = K.load_library()

    def call(stream):
        K._check(lib.kda_fwd(prob.ref(), ctypes.byref(io), K._ptr(ws), ws.numel(),
                             K._stream_ptr(stream)))

    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        call(side)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        for t in res.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for key, want in ref.items():
            assert torch.equal(res[key], want), "%s replay %d: %s differs" % (name, rep, key)


def test_concurrent_calls_from_threads():
    """Two host threads calling kda_bwd at once, each on its own stream with its own
    workspace (the library keeps no per-call state; its only shared state, the occupancy
    cache, is locked): every result bitwise equal to the same call made alone."""
    import threading
    import torch
    plans = [_plan(KI.make_inputs(KI.get_workload(n)))[0] for n in ("ragged_bf16", "tiny_fp32")]
    refs = []
    for p in plans:
        p.run(torch.cuda.current_stream())
        torch.cuda.synchronize()
        refs.append(_snapshot(p))
    streams = [torch.cuda.Stream() for _ in plans]
    errors = []

    def work(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(8):
                    plans[i].run(streams[i])
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(plans))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for p, ref in zip(plans, refs):
        for key, want in ref.items():
            assert torch.equal(p.outputs()[key], want), key
