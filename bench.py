"""Benchmark: KDA backward tokens/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload train_bf16]

One step = one full kda_bwd call (chunk table, prep, reverse state-gradient
scan, gradient pass, dA_log reduction) on the training-shape workload
B=8, T=4096, H=32, K=V=128, bf16 activations, chunk 64, with the chunk start
states (from the reference forward) already resident in HBM.  Prints ONE JSON
line.  The CPU baseline is the fp64 oracle timed on a bounded sample of the same
workload on the host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Algorithmic bytes per token-head (bf16 activations, K = V = 128, chunk 64 unless given)
# as the measurement plan counts them for the whole path: every input read once, every
# output written once, the chunk-start state read once and the state gradient handed
# from the scan to the gradient pass once (written, then read).  Per chunk-head
# quantities are divided by 64.  Each byte is assigned to the kernel that moves it
# compulsorily: the gradient pass reads every per-token input and the two states and
# writes every per-token output; the scan writes the state-gradient hand-off; prep's
# traffic (re-reads of q, k, g_raw, beta and its own intermediates) is all overhead.
# When prep runs the scan itself (fused), the hand-off is prep's.
def kernel_bytes_per_token_head(D=128, es=2, fused=False):
    act = D * es          # one activation row
    f32row = D * 4        # one fp32 row (g_raw, dg_raw)
    state = D * D * es / 64.0   # one K x V state per chunk
    return {
        "prep": state if fused else 0.0,
        "scan": 0.0 if fused else state,                 # dS_out written
        # q, k, v, dO, g_raw, beta in; S_in and dS_out in; dq, dk, dv, dg_raw, dbeta out
        "grad": 4 * act + f32row + 4 + 2 * state + 3 * act + f32row + 4,
    }


def path_bytes_per_token_head(D=128, es=2):
    return sum(kernel_bytes_per_token_head(D, es).values())


# Algorithmic MFMA work per chunk-head (C = 64, D = K = V): seven state contractions
# (C x D x D each), eleven causal C x C x D products at half density, the 64 x 64
# inverse (2 C^3 / 3); in FLOP.
def path_flops_per_chunk_head(D=128, C=64):
    w = C * D * D * 2
    u = C * C * D * 2
    return 7 * w + 5.5 * u + 2 * C ** 3 / 3


def _code_only(text):
    """C++ source without comments and with whitespace collapsed (a comment edit does not
    change the code a profile was taken on).  The kernels hold no string literal with
    comment markers in it."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_sources_digest():
    """Digest of the device code (the .hip sources and the headers they include, comments
    and whitespace aside); the host-side API file does not change what a kernel reads or
    writes."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_backward_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(_code_only(open(os.path.join(csrc, f)).read()).encode())
    return h.hexdigest()[:16]


def _profile_json(name):
    """A committed counter summary under profiles/, only if it was taken on the current
    kernel sources."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    return d if d.get("sources") == kernel_sources_digest() else None


def load_traffic(kernel_stage):
    """HBM traffic measured by rocprofv3 counters (profiles/traffic.json), only
    if it was taken on the current kernel sources."""
    d = _profile_json("traffic.json")
    ent = None if d is None else d.get("kernels", {}).get(kernel_stage)
    return None if ent is None else ent.get("bytes_per_launch")


def load_counters(kernel_stage):
    """SQ counter ratios of one kernel (profiles/counters.json), only if they were taken
    on the current kernel sources."""
    d = _profile_json("counters.json")
    return None if d is None else d.get("kernels", {}).get(kernel_stage)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, target_s=12.0):
    """Time the fp64 oracle on whole heads of the workload (every sequence of
    each head), sized to roughly target_s seconds; scale to tokens/s.  Returns the
    record, the oracle's outputs and the heads it ran on (for the parity check)."""
    import numpy as np
    import kda_inputs as KI
    from oracle import oracle as O
    threads = O.num_threads()
    H = inp["H"]
    TT = inp["q"].shape[0]
    # probe: one head, the first sequence, its first 256 tokens
    probe = KI.select_heads(KI.select_seqs(inp, [0]), [0])
    n0 = min(256, int(probe["cu_seqlens"][-1]))
    for key in ("q", "k", "v", "dO", "g_raw", "beta"):
        probe[key] = probe[key][:n0]
    probe["cu_seqlens"] = np.array([0, n0])
    t = time.perf_counter()
    O.kda_backward(probe, nthreads=1)
    per_token_head = (time.perf_counter() - t) / n0
    units_per_head = inp["N"]
    est_per_head = per_token_head * TT / max(1, min(threads, units_per_head))
    nh = int(max(1, min(H, round(target_s / max(est_per_head, 1e-9)))))
    # keep all threads busy: whole heads, every sequence
    heads = list(range(nh))
    sub = KI.select_heads(inp, heads)
    t = time.perf_counter()
    ref = O.kda_backward(sub)
    dt = time.perf_counter() - t
    token_heads = TT * nh
    tok_s = token_heads / H / dt
    rec = {"value": tok_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": "%d of %d heads x all %d tokens (%d token-heads), fp64, %.1f s"
                     % (nh, H, TT, token_heads, dt)}
    return rec, ref, heads


def parity_report(outs, ref, heads, inp, tol):
    """max|gpu - oracle| / max|oracle| per output on the oracle's heads."""
    import numpy as np
    TT = inp["q"].shape[0]
    rep = {}
    for key in ("dq", "dk", "dv", "dg_raw", "dbeta", "dA_log", "dh0"):
        val = outs.get(key)
        if val is None or key not in ref:
            continue
        a = val.float().cpu().numpy().astype(np.float64)
        if key in ("dq", "dk", "dv", "dg_raw"):
            a = a.reshape(TT, a.shape[-2], a.shape[-1])[:, heads]
        elif key == "dbeta":
            a = a.reshape(TT, -1)[:, heads]
        elif key == "dA_log":
            a = a[heads]
        else:
            a = a[:, heads]
        den = float(np.abs(ref[key]).max())
        num = float(np.abs(a - ref[key]).max())
        rep[key] = num / den if den > 0 else num
    return {"metric": "max|gpu-oracle|/max|oracle| per output", "tol": tol,
            "heads": "%d of %d" % (len(heads), inp["H"]), "max_rel_err": rep,
            "pass": all(v <= tol for v in rep.values())}


KERNEL_STAGE = (("k_prep", "prep"), ("k_scanw", "scan"), ("k_gradf", "grad"))


def _stage_of(name):
    for key, stage in KERNEL_STAGE:
        if key in name:
            return stage
    return None


def _pmc_kib(csv_path, counter):
    """Average counter value (KiB) per dispatch of every backward kernel stage (one row of
    the rocprofv3 CSV per dispatch; the dispatches of all kernels of a stage averaged
    together)."""
    import csv
    per = {}
    for row in csv.DictReader(open(csv_path)):
        if row["Counter_Name"] != counter:
            continue
        stage = _stage_of(row["Kernel_Name"])
        if stage is None:
            continue
        per.setdefault(stage, []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in per.items()}


def _copy_kib(csv_path, counter):
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]]
    return sum(vals) / len(vals)


def summarize_profiles(fetch_csv, write_csv, calib_fetch_csv, calib_write_csv, copy_mib,
                       out_path=None):
    """Write profiles/traffic.json (or out_path) from rocprofv3 --pmc FETCH_SIZE /
    WRITE_SIZE runs of this benchmark and of its --copy-calib mode (a copy of copy_mib
    MiB): each counter is scaled by (bytes the copy moves) / (what the counter read for
    it)."""
    nbytes = copy_mib << 20
    fs = nbytes / (_copy_kib(calib_fetch_csv, "FETCH_SIZE") * 1024.0)
    ws = nbytes / (_copy_kib(calib_write_csv, "WRITE_SIZE") * 1024.0)
    fk = _pmc_kib(fetch_csv, "FETCH_SIZE")
    wk = _pmc_kib(write_csv, "WRITE_SIZE")
    out = {"sources": kernel_sources_digest(),
           "workload": "train_bf16 (B=8,T=4096,H=32,K=V=128,bf16)",
           "fetch_scale": fs, "write_scale": ws, "kernels": {}}
    for stage in sorted(set(fk) & set(wk)):
        rb = fk[stage] * 1024.0 * fs
        wb = wk[stage] * 1024.0 * ws
        out["kernels"][stage] = {"fetch_kib_raw": fk[stage], "write_kib_raw": wk[stage],
                                 "read_bytes": rb, "write_bytes": wb, "bytes_per_launch": rb + wb}
    path = out_path or os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    return out


N_XCD = 8       # GRBM_GUI_ACTIVE is reported once per XCD and summed in the CSV
CU_NUM = 256
SIMD_NUM = 1024


def summarize_counters(csvs, out_path=None):
    """Write profiles/counters.json (or out_path) from rocprofv3 --pmc CSVs of this benchmark (any split
    of the counters below over passes): per backward kernel, the profiler's own ratios
    VALU busy = SQ_ACTIVE_INST_VALU / (CUs x kernel cycles), MFMA busy =
    SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x kernel cycles), MFMA FLOP = MOPS_BF16 x 512,
    resident waves per SIMD = SQ_WAVE_CYCLES / (CUs x kernel cycles) and LDS bank-conflict
    cycles / LDS-active cycles; kernel cycles = GRBM_GUI_ACTIVE / XCDs."""
    vals = {}
    for path in csvs:
        for stage, cnt in _pmc_all(path).items():
            vals.setdefault(stage, {}).update(cnt)
    out = {"sources": kernel_sources_digest(),
           "workload": "train_bf16 (B=8,T=4096,H=32,K=V=128,bf16)", "kernels": {}}
    for stage, c in vals.items():
        if "GRBM_GUI_ACTIVE" not in c:
            continue
        cyc = c["GRBM_GUI_ACTIVE"] / N_XCD
        ent = {"kernel_cycles": cyc, "raw": c}
        if "SQ_ACTIVE_INST_VALU" in c:
            ent["valu_busy"] = c["SQ_ACTIVE_INST_VALU"] / (CU_NUM * cyc)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            ent["mfma_busy"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMD_NUM * cyc)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:
            ent["mfma_flop_per_launch"] = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
        if "SQ_WAVE_CYCLES" in c:
            ent["waves_per_simd"] = c["SQ_WAVE_CYCLES"] / (CU_NUM * cyc)
        if "SQ_LDS_BANK_CONFLICT" in c and c.get("SQ_LDS_IDX_ACTIVE"):
            ent["lds_bank_conflict_frac"] = c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"]
        out["kernels"][stage] = ent
    with open(out_path or os.path.join(ROOT, "profiles", "counters.json"), "w") as f:
        json.dump(out, f, indent=1)
    return out


def _pmc_all(csv_path):
    """Average value of every counter per dispatch of every backward kernel stage."""
    import csv
    per = {}
    for row in csv.DictReader(open(csv_path)):
        stage = _stage_of(row["Kernel_Name"])
        if stage is None:
            continue
        per.setdefault(stage, {}).setdefault(row["Counter_Name"], []).append(
            float(row["Counter_Value"]))
    return {st: {k: sum(v) / len(v) for k, v in d.items()} for st, d in per.items()}


def time_graph(torch, plan, stream, steps):
    """ms per kda_bwd call replayed from a HIP graph captured once (torch.cuda.CUDAGraph)."""
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):  # torch runs captured work once on a side stream first
        plan.run(side)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.run(torch.cuda.current_stream())
    graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def bench_forward(a, K, torch, inp, g, cu, vk, wl, variants):
    """kda_fwd timed over the whole call (chunk table, per-chunk pass, state scan), with
    the reference forward timed once beside it."""
    args = (g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"])
    kw = dict(h0=g["h0"], cu_seqlens=cu, **vk)
    stream = torch.cuda.current_stream()
    prob = K._make_prob(g["q"], g["v"], cu, vk["gate_log2"], vk["qk_l2norm"])[0]
    ws = torch.empty(max(K.workspace_size(prob, K.KDA_WS_FWD), 1), dtype=torch.uint8,
                     device="cuda")
    for _ in range(a.warmup):
        K.kda_fwd(*args, workspace=ws, **kw)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    res = K.kda_fwd(*args, workspace=ws, **kw)
    io = K.FwdIO(*[K._ptr(x) for x in (g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"],
                                       g["h0"], res["o"], res["ht"], res["h_saved"], g["dt_bias"])])
    lib = K.load_library()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(a.steps):
        K._check(lib.kda_fwd(prob.ref(), ctypes.byref(io), K._ptr(ws), ws.numel(),
                             K._stream_ptr(stream)))
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    e0.record(stream)
    K.kda_fwd_ref(*args, **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_ref = e0.elapsed_time(e1)
    tokens = int(inp["q"].shape[0])
    H, D = inp["H"], inp["K"]
    es = 2 if inp["dtype"] == "bf16" else 4
    # algorithmic bytes per token-head: q, k, v, g_raw, beta in; o and the chunk-start
    # state (K x V per 64 tokens) out
    per_th = 3 * D * es + 4 * D + 4 + D * es + D * D * es / 64
    nbytes = per_th * tokens * H
    achieved = nbytes / (ms / 1e3) / 1e9
    log("kda_fwd: %.3f ms (kda_fwd_ref %.3f ms)" % (ms, ms_ref))
    print(json.dumps({
        "metric": "KDA forward tokens/s (o, ht, chunk-start states)", "value": tokens / (ms / 1e3),
        "unit": "tokens/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": inp["dtype"],
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "H": H, "K": D, "V": inp["V"],
                   "chunk": 64, "parallelism": "single-gpu"},
        **({"variants": [k for k, v in variants.items() if v]} if any(variants.values()) else {}),
        "path_roofline": {"bound": "hbm", "algorithmic_bytes": nbytes, "achieved": achieved,
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS},
        "reference_forward_ms": ms_ref}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="train_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dt-bias", action="store_true",
                    help="method variant: a per-(head, channel) gate bias (and its gradient)")
    ap.add_argument("--gate-log2", action="store_true",
                    help="method variant: the gate in log2 units (decay 2^g)")
    ap.add_argument("--qk-l2norm", action="store_true",
                    help="method variant: q and k L2-normalised inside the method")
    ap.add_argument("--graph", action="store_true",
                    help="also time the backward step replayed from a HIP graph captured once")
    ap.add_argument("--forward", action="store_true",
                    help="time the production forward (kda_fwd: o, ht and the chunk-start "
                         "states) instead of the backward; prints its own JSON line")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times) so that "
                         "HBM counters can be scaled against a kernel of known traffic")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV",
                                                             "CALIB_FETCH_CSV", "CALIB_WRITE_CSV"),
                    help="write profiles/traffic.json from rocprofv3 counter CSVs of this "
                         "benchmark and of --copy-calib 1024 (no GPU needed)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_CSV",
                    help="write profiles/counters.json from rocprofv3 --pmc CSVs of this "
                         "benchmark (SQ busy, MFMA, occupancy and LDS counters; no GPU needed)")
    a = ap.parse_args()
    if a.summarize_counters:
        print(json.dumps(summarize_counters(a.summarize_counters), indent=1))
        return
    if a.summarize_traffic:
        print(json.dumps(summarize_profiles(*a.summarize_traffic, copy_mib=1024), indent=1))
        return
    if a.copy_calib:
        import torch
        n = a.copy_calib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "repeats": 3}))
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU; the library has no multi-GPU path (--gpus %d)" % a.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import kda_inputs as KI
    import linear_attention_backward_amd as K
    from tests import kda_case as KC

    assert torch.cuda.is_available(), "needs a GPU"
    K.load_library()
    wl = KI.get_workload(a.workload)
    t = time.perf_counter()
    inp = KI.make_inputs(wl)
    variants = dict(dt_bias=a.dt_bias, gate_log2=a.gate_log2, qk_l2norm=a.qk_l2norm)
    inp = KI.with_variants(inp, **variants)
    log("inputs generated in %.1f s" % (time.perf_counter() - t))
    g = KC.to_gpu(inp)
    cu = inp["cu_seqlens"] if inp["varlen"] else None
    vk = dict(dt_bias=g["dt_bias"], gate_log2=inp["gate_log2"], qk_l2norm=inp["qk_l2norm"])
    if a.forward:
        bench_forward(a, K, torch, inp, g, cu, vk, wl, variants)
        return
    fwd = K.kda_fwd_ref(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], h0=g["h0"],
                        cu_seqlens=cu, want_o=False, want_ht=False, **vk)
    torch.cuda.synchronize()
    plan = K.BwdPlan(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], g["dO"],
                     h0=g["h0"], dht=g["dht"], h_saved=fwd["h_saved"], cu_seqlens=cu, **vk)
    stream = torch.cuda.current_stream()
    for _ in range(a.warmup):
        plan.run(stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    # per-kernel durations: HIP events around each launch, on the launch stream, inside
    # the timed region (the library records them; read after the region)
    K.timing_enable(True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(a.steps):
        plan.run(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    st = K.timing_read()
    K.timing_enable(False)
    ms = e0.elapsed_time(e1) / a.steps
    tokens = int(inp["q"].shape[0])
    value = tokens / (ms / 1e3)
    log("kda_bwd: %.3f ms/step (wall %.3f ms/step)" % (ms, t_wall * 1e3 / a.steps))
    per = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in st.items()}
    log("per-kernel ms: " + " ".join("%s=%.3f" % kv for kv in per.items() if kv[1] > 0))

    # the same step with the last-level cache (256 MB MALL) flushed before each one by a
    # 1 GiB write; each step timed on its own
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    nf = max(3, min(a.steps, 10))
    fl = []
    for _ in range(nf):
        flush.zero_()
        e0.record(stream)
        plan.run(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        fl.append(e0.elapsed_time(e1))
    del flush
    fl.sort()
    ms_flushed = fl[len(fl) // 2]
    log("kda_bwd with the MALL flushed before each step: %.3f ms (median of %d)" % (ms_flushed, nf))

    # --graph: the same step captured once into a HIP graph and replayed (the library
    # enqueues kernels only): what a caller that replays its backward saves in launch
    # overhead
    ms_graph = None
    if a.graph:
        ms_graph = time_graph(torch, plan, stream, a.steps)
        log("kda_bwd replayed as a HIP graph: %.3f ms/step" % ms_graph)

    dom = max(("prep", "scan", "grad"), key=lambda s: per[s])
    H, D = inp["H"], inp["K"]
    es = 2 if inp["dtype"] == "bf16" else 4
    token_heads = tokens * H
    fused = st["scan"][1] == 0  # prep ran the state-gradient scan itself
    kb = kernel_bytes_per_token_head(D, es, fused)[dom] * token_heads
    achieved = kb / (per[dom] / 1e3) / 1e9
    traffic = load_traffic(dom)
    path_bytes = path_bytes_per_token_head(D, es) * token_heads
    # Which roofline binds: the path's MFMA work per algorithmic byte against the ridge
    # point (bf16 peak / HBM peak).  The MFMA work is the counted one when counters for
    # these sources are committed, else the algorithmic count.
    ctr = {st_: load_counters(st_) for st_ in (("prep", "grad") if fused
                                                else ("prep", "scan", "grad"))}
    chunk_heads = int(plan.nc) * H
    if all(c is not None for c in ctr.values()):
        flops = sum(c["mfma_flop_per_launch"] for c in ctr.values())
        flops_src = "rocprofv3 SQ_INSTS_VALU_MFMA_MOPS_BF16 (profiles/counters.json)"
    else:
        flops = path_flops_per_chunk_head(D) * chunk_heads
        flops_src = "algorithmic count"
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    intensity = flops / path_bytes
    bound = "mfma" if intensity > ridge else "hbm"
    roof = {"bound": bound, "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "algorithmic_bytes_per_launch": kb,
            "duration_ms": per[dom],
            "duration_source": "mean of HIP-event durations of the %d launches in the timed "
                               "region, on the launch stream" % a.steps,
            "bound_from": {"flop_per_byte": intensity, "ridge_flop_per_byte": ridge,
                           "flop_source": flops_src}}
    c = ctr.get(dom)
    if c is not None:
        # what holds the kernel below its roofline, from its SQ counters
        mfma_tflops = c["mfma_flop_per_launch"] / (per[dom] / 1e3) / 1e12
        roof["counters"] = {"valu_busy": c["valu_busy"], "mfma_busy": c["mfma_busy"],
                            "mfma_tflops": mfma_tflops,
                            "mfma_frac_of_bf16_peak": mfma_tflops / BF16_PEAK_TFLOPS,
                            "lds_bank_conflict_frac": c.get("lds_bank_conflict_frac"),
                            "occupancy_waves_per_simd": c.get("waves_per_simd"),
                            "hbm_frac_measured": (traffic / (per[dom] / 1e3) / 1e9 / HBM_PEAK_GBS
                                                  if traffic else None)}
        busy = {"valu-issue": c["valu_busy"], "mfma": c["mfma_busy"]}
        if traffic:
            busy["hbm"] = traffic / (per[dom] / 1e3) / 1e9 / HBM_PEAK_GBS
        roof["limiter"] = max(busy, key=busy.get)
    out = {
        "metric": "KDA backward tokens/s (H=32,K=V=128,bf16)",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp["dtype"],
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "H": H, "K": D, "V": inp["V"],
                   "chunk": 64, "h_saved": "given", "parallelism": "single-gpu",
                   "kernels": "prep with the state-gradient scan inside, gradient pass"
                   if fused else "prep, state-gradient scan, gradient pass"},
        **({"variants": [k for k, v in variants.items() if v]} if any(variants.values()) else {}),
        "roofline": roof,
        "path_roofline": {"bound": bound, "algorithmic_bytes": path_bytes,
                          "achieved": path_bytes / (ms / 1e3) / 1e9, "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": path_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS},
        "kernel_ms": per,
        "mall_flushed_ms_per_step": ms_flushed,
        **({"graph_replay_ms_per_step": ms_graph} if ms_graph is not None else {}),
    }
    if not a.no_cpu_baseline:
        rec, ref, heads = cpu_baseline(inp)
        out["cpu_baseline"] = rec
        out["parity"] = parity_report(plan.outputs(), ref, heads, inp,
                                      KC.TOL[inp["dtype"]])
        log("parity vs oracle (%s): %s" % (out["parity"]["heads"], " ".join(
            "%s=%.2e" % kv for kv in out["parity"]["max_rel_err"].items())))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
