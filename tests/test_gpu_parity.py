"""Parity of the HIP path (through the C ABI) against the fp64 oracle.

Metric per output tensor: max|gpu - ref| / max|ref|; bar 1e-4 for fp32
activations, 2e-2 for bf16 activations with fp32 accumulation.  Besides the
gradients, the reference forward's chunk-start states and outputs and the
scan's per-chunk state gradients are compared with the oracle's (the latter
pins the reverse scan alone).  Every workload, the three large ones included, is
compared on all of its heads and sequences.
"""
import numpy as np
import pytest

import kda_inputs as KI
from tests import kda_case as KC

pytestmark = pytest.mark.gpu

GRADS = ["dq", "dk", "dv", "dg_raw", "dbeta", "dA_log", "dh0"]
INTER = ["dstates", "h_saved", "o", "ht"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_backward_amd as K
    K.load_library()


def _check(name, heads=None, use_h_saved=True):
    print("\n[case] %s heads=%s h_saved=%s" % (name, heads, use_h_saved), flush=True)
    inp = KI.make_inputs(KI.get_workload(name))
    res = KC.run_gpu(inp, use_h_saved=use_h_saved)
    ref = KC.oracle_for(inp, heads)
    ref["dstates"] = ref["dstates"]
    ref["h_saved"] = ref["states"]
    tol = KC.TOL[inp["dtype"]]
    keys = GRADS + INTER + (["ddt_bias"] if inp.get("dt_bias") is not None else [])
    rep = KC.compare(res, ref, keys, tol, heads=heads, label=name)
    print("[errors] " + " ".join("%s=%.2e" % kv for kv in rep.items()), flush=True)
    return res


@pytest.mark.parametrize("name", ["tiny_fp32", "weak_decay_fp32", "ragged_fp32",
                                  "single_token_fp32"])
def test_parity_fp32(name):
    _check(name)


@pytest.mark.parametrize("name", ["single_seq_bf16", "weak_decay_bf16", "strong_decay_bf16",
                                  "ragged_bf16", "ragged_bf16_d64", "multi_ragged_bf16"])
def test_parity_bf16(name):
    _check(name)


@pytest.mark.parametrize("name", ["gate_bias_bf16", "gate_log2_fp32", "gate_log2_bf16"])
def test_gate_variants(name):
    """A per-channel gate bias inside the softplus (with its gradient, ddt_bias) and gates
    in log2 units, in the reference forward and in every backward kernel."""
    _check(name)


@pytest.mark.parametrize("name", ["qk_norm_bf16", "qk_norm_fp32", "qk_norm_bf16_d64"])
def test_qk_l2norm(name):
    """q and k L2-normalised inside the method (a pass before the kernels, the
    projection of dq, dk after them), also with log2-unit gates and a gate bias."""
    _check(name)


@pytest.mark.parametrize("name,heads", [
    ("tiny_fp32", None), ("ragged_fp32", None), ("weak_decay_fp32", None),
    ("single_token_fp32", None), ("single_seq_bf16", None), ("ragged_bf16", None),
    ("ragged_bf16_d64", None), ("multi_ragged_bf16", None), ("strong_decay_bf16", None),
    ("gate_bias_bf16", None), ("gate_log2_fp32", None), ("qk_norm_bf16", None)])
def test_forward_parity(name, heads):
    """The production forward (kda_fwd) against the oracle's per-token recurrence:
    outputs, final states and the states at every chunk start."""
    print("\n[case] forward %s heads=%s" % (name, heads), flush=True)
    inp = KI.make_inputs(KI.get_workload(name))
    res = KC.run_gpu_fwd(inp)
    ref = KC.oracle_fwd_for(inp, heads)
    ref["h_saved"] = ref["states"]
    rep = KC.compare(res, ref, ["o", "ht", "h_saved"], KC.TOL[inp["dtype"]], heads=heads,
                     label="forward " + name)
    print("[errors] " + " ".join("%s=%.2e" % kv for kv in rep.items()), flush=True)


@pytest.mark.parametrize("name", ["train_bf16", "varlen_bf16", "long_bf16", "train_bf16_d64",
                                  "train_fp32_d64"])
def test_parity_full_size(name):
    """The three large workloads at full size, and the training shape at K = V = 64 in bf16
    and fp32 (four waves per workgroup), every head and every sequence: the
    backward (with the reference forward's chunk-start states, in the launch
    configuration the benchmark times), the reference forward and the production
    forward (its split state scan on the long-context workload), all against one
    oracle run (per-token recurrence and its hand-derived reverse mode)."""
    print("\n[case] full size %s, all heads" % name, flush=True)
    inp = KI.make_inputs(KI.get_workload(name))
    res = KC.run_gpu(inp)
    fres = KC.run_gpu_fwd(inp)
    print("[gpu done] %s" % name, flush=True)
    ref = KC.oracle_for(inp)
    ref["h_saved"] = ref["states"]
    tol = KC.TOL[inp["dtype"]]
    rep = KC.compare(res, ref, GRADS + INTER, tol, label=name)
    print("[errors] " + " ".join("%s=%.2e" % kv for kv in rep.items()), flush=True)
    del res
    rep = KC.compare(fres, ref, ["o", "ht", "h_saved"], tol, label="forward " + name)
    print("[errors forward] " + " ".join("%s=%.2e" % kv for kv in rep.items()), flush=True)


@pytest.mark.parametrize("name", ["tiny_fp32", "ragged_bf16", "gate_log2_fp32", "qk_norm_fp32"])
def test_state_recompute_path(name):
    """h_saved omitted: the library recomputes the chunk states in-stream."""
    _check(name, use_h_saved=False)


def test_zero_length_sequences():
    """Packed batch with empty sequences: they own no chunk, dh0 = dht there."""
    wl = KI.Workload("zero_len", 1, 0 + 70 + 0 + 5 + 64, 2, 128, 128, "bf16", 1200, varlen_seqs=4,
                     fixed_lengths=(0, 70, 0, 69), h0_std=0.3, dht_std=1.0)
    inp = KI.make_inputs(wl)
    print("\n[case] zero_len", flush=True)
    res = KC.run_gpu(inp)
    ref = KC.oracle_for(inp)
    ref["h_saved"] = ref["states"]
    KC.compare(res, ref, GRADS + INTER, KC.TOL["bf16"], label="zero_len")


@pytest.mark.parametrize("name,mode", [("ragged_fp32", "mix"), ("ragged_bf16", "mix"),
                                       ("ragged_fp32", "zero"), ("ragged_bf16", "zero")])
def test_degenerate_beta(name, mode):
    """beta exactly 0 (the token writes nothing: S_t = Diag(exp g_t) S_{t-1}, and k_t, v_t
    have no gradient) and exactly 1 (the old value along k_t is fully replaced): on all
    tokens ("zero") or on a random third each ("mix").  Backward and production forward."""
    inp = KI.make_inputs(KI.get_workload(name))
    b = inp["beta"]
    if mode == "zero":
        b = np.zeros_like(b)
    else:
        u = np.random.default_rng(4242).integers(0, 3, size=b.shape)
        b = np.where(u == 0, 0.0, np.where(u == 1, 1.0, b)).astype(b.dtype)
    inp = dict(inp, beta=b)
    print("\n[case] degenerate beta %s %s" % (name, mode), flush=True)
    res = KC.run_gpu(inp)
    ref = KC.oracle_for(inp)
    ref["h_saved"] = ref["states"]
    tol = KC.TOL[inp["dtype"]]
    if mode == "zero":
        assert np.abs(ref["dk"]).max() == 0.0 and np.abs(ref["dv"]).max() == 0.0
    KC.compare(res, ref, GRADS + INTER, tol, label="beta %s %s" % (name, mode))
    fres = KC.run_gpu_fwd(inp)
    KC.compare(fres, ref, ["o", "ht", "h_saved"], tol, label="beta %s %s forward" % (name, mode))


@pytest.mark.parametrize("name", ["ragged_fp32", "multi_ragged_bf16"])
def test_no_decay_heads(name):
    """A_log = -inf on head 0 (g = 0 exactly: the plain delta rule) and, with three heads,
    A_log = -95 on head 1 (e^{A_log} below the fp32 normal range): finite gradients equal to
    the oracle's, dg_raw and dA_log zero on the no-decay head."""
    inp = KI.make_inputs(KI.get_workload(name))
    a = inp["A_log"].copy()
    a[0] = -np.inf
    if a.shape[0] > 2:
        a[1] = -95.0
    inp = dict(inp, A_log=a)
    print("\n[case] no-decay heads %s" % name, flush=True)
    res = KC.run_gpu(inp)
    ref = KC.oracle_for(inp)
    ref["h_saved"] = ref["states"]
    for key in GRADS:
        assert np.all(np.isfinite(res[key])), key
    assert np.abs(ref["dg_raw"][:, 0]).max() == 0.0 and ref["dA_log"][0] == 0.0
    KC.compare(res, ref, GRADS + INTER, KC.TOL[inp["dtype"]], label="no decay %s" % name)
    fres = KC.run_gpu_fwd(inp)
    KC.compare(fres, ref, ["o", "ht", "h_saved"], KC.TOL[inp["dtype"]],
               label="no decay %s forward" % name)


def test_repeatable_bitwise():
    """Two runs give bit-identical outputs (no atomics, fixed reduction order)."""
    inp = KI.make_inputs(KI.get_workload("weak_decay_bf16"))
    print("\n[case] repeat weak_decay_bf16", flush=True)
    a = KC.run_gpu(inp)
    b = KC.run_gpu(inp)
    for key in GRADS + ["dstates"]:
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("name,group", [("weak_decay_bf16", 3), ("weak_decay_fp32", 2),
                                        ("ragged_bf16", 1), ("ragged_fp32", 3),
                                        ("single_seq_bf16", 5)])
def test_split_scan(name, group, monkeypatch):
    """The state-gradient scan split into groups of a few chunks (group maps, group
    boundaries, re-scan from the boundaries) against the oracle; weak decay keeps
    the cross-group terms large."""
    monkeypatch.setenv("KDA_SCAN_GROUP", str(group))
    monkeypatch.setenv("KDA_SCANPQ", "0")
    print("\n[case] split scan %s, %d chunks per group" % (name, group), flush=True)
    _check(name)


@pytest.mark.parametrize("name,group", [("weak_decay_bf16", 3), ("weak_decay_fp32", 2),
                                        ("ragged_bf16", 1), ("ragged_bf16_d64", 2),
                                        ("multi_ragged_bf16", 1), ("single_seq_bf16", 5)])
def test_split_scan_joint_maps(name, group, monkeypatch):
    """The split scan with each group's transition and offset formed by one workgroup
    (the form chosen by itself once separate workgroups would need more than one round
    of the GPU, as on the long-context workload), forced here on small cases."""
    monkeypatch.setenv("KDA_SCAN_GROUP", str(group))
    monkeypatch.setenv("KDA_SCANPQ", "1")
    print("\n[case] split scan, joint group maps, %s, %d chunks per group" % (name, group),
          flush=True)
    _check(name)


@pytest.mark.parametrize("name,group", [("weak_decay_bf16", 3), ("ragged_fp32", 2),
                                        ("multi_ragged_bf16", 1)])
def test_joint_maps_bitwise(name, group, monkeypatch):
    """The joint and the separate group maps run the same products in the same order
    (each map's accumulation, its bf16 state tiles), so the backward's and the
    forward's results agree bit for bit between the two forms."""
    monkeypatch.setenv("KDA_SCAN_GROUP", str(group))
    inp = KI.make_inputs(KI.get_workload(name))
    print("\n[case] joint vs separate group maps, %s, %d chunks per group" % (name, group),
          flush=True)
    out = {}
    for joint in (0, 1):
        monkeypatch.setenv("KDA_SCANPQ", str(joint))
        out[joint] = (KC.run_gpu(inp), KC.run_gpu(inp, use_h_saved=False), KC.run_gpu_fwd(inp))
    keys = (GRADS + ["dstates"], GRADS + ["dstates"], ["o", "ht", "h_saved"])
    for a, b, ks in zip(out[0], out[1], keys):
        for key in ks:
            assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("name,group", [("weak_decay_bf16", 3), ("weak_decay_fp32", 2),
                                        ("ragged_bf16", 1), ("ragged_fp32", 3),
                                        ("single_seq_bf16", 5), ("gate_log2_fp32", 2)])
@pytest.mark.parametrize("joint", [0, 1])
def test_forward_split_scan(name, group, joint, monkeypatch):
    """The production forward's state scan split into groups of a few chunks (group
    maps from I and from 0, boundaries chained from h0, re-scan with outputs); the maps
    as separate workgroups (joint = 0) and both in one workgroup (joint = 1)."""
    monkeypatch.setenv("KDA_SCAN_GROUP", str(group))
    monkeypatch.setenv("KDA_SCANPQ", str(joint))
    print("\n[case] forward split scan %s, %d chunks per group, joint maps %d"
          % (name, group, joint), flush=True)
    inp = KI.make_inputs(KI.get_workload(name))
    res = KC.run_gpu_fwd(inp)
    ref = KC.oracle_fwd_for(inp)
    ref["h_saved"] = ref["states"]
    rep = KC.compare(res, ref, ["o", "ht", "h_saved"], KC.TOL[inp["dtype"]],
                     label="forward split " + name)
    print("[errors] " + " ".join("%s=%.2e" % kv for kv in rep.items()), flush=True)


def test_recompute_with_split_scans(monkeypatch):
    """Backward without h_saved and with split scans: the forward's split scan recomputes
    the chunk-start states, the backward's split scan carries dS."""
    monkeypatch.setenv("KDA_SCAN_GROUP", "2")
    print("\n[case] recompute + split scans weak_decay_fp32", flush=True)
    _check("weak_decay_fp32", use_h_saved=False)


def test_split_scan_zero_length(monkeypatch):
    monkeypatch.setenv("KDA_SCAN_GROUP", "1")
    wl = KI.Workload("zero_len", 1, 0 + 70 + 0 + 5 + 64, 2, 128, 128, "bf16", 1200, varlen_seqs=4,
                     fixed_lengths=(0, 70, 0, 69), h0_std=0.3, dht_std=1.0)
    inp = KI.make_inputs(wl)
    print("\n[case] split scan zero_len", flush=True)
    res = KC.run_gpu(inp)
    ref = KC.oracle_for(inp)
    ref["h_saved"] = ref["states"]
    KC.compare(res, ref, GRADS + INTER, KC.TOL["bf16"], label="zero_len split")
    fres = KC.run_gpu_fwd(inp)  # the production forward's split scan, empty sequences too
    KC.compare(fres, ref, ["o", "ht", "h_saved"], KC.TOL["bf16"], label="zero_len forward split")


@pytest.mark.parametrize("name,cap", [("ragged_fp32", 3), ("ragged_bf16", 3),
                                      ("ragged_bf16_d64", 2), ("weak_decay_bf16", 5),
                                      ("multi_ragged_bf16", 2), ("gate_bias_bf16", 3)])
def test_persistent_walk(name, cap, monkeypatch):
    """Prep and the gradient pass with a grid of `cap` workgroups: each workgroup walks
    many (chunk, head) items and hands the prefetched tiles of the next item over
    across ragged chunks.  Results match the oracle and, bit for bit, a run with the
    full grid (an item's arithmetic does not depend on which workgroup runs it)."""
    inp = KI.make_inputs(KI.get_workload(name))
    print("\n[case] persistent walk %s, grid capped at %d" % (name, cap), flush=True)
    # the separate prep and scan kernels in both runs (a capped grid can make the scans
    # inside prep eligible; they have capped-grid tests of their own)
    monkeypatch.setenv("KDA_PREPSCAN", "0")
    full = KC.run_gpu(inp)
    monkeypatch.setenv("KDA_GRID_CAP", str(cap))
    capped = KC.run_gpu(inp)
    ref = KC.oracle_for(inp)
    ref["h_saved"] = ref["states"]
    extra = ["ddt_bias"] if inp.get("dt_bias") is not None else []
    KC.compare(capped, ref, GRADS + INTER + extra, KC.TOL[inp["dtype"]], label=name + " capped")
    for key in GRADS + ["dstates"] + extra:
        assert np.array_equal(full[key], capped[key]), key


FUSED = ["tiny_fp32", "weak_decay_bf16", "weak_decay_fp32", "multi_ragged_bf16", "qk_norm_fp32",
         "gate_log2_bf16", "single_seq_bf16", "strong_decay_bf16", "qk_norm_bf16_d64",
         # packed sequences of different lengths (units sorted by chunk count, snake order)
         "ragged_bf16", "ragged_fp32", "ragged_bf16_d64", "gate_bias_bf16", "gate_log2_fp32",
         "qk_norm_bf16"]


@pytest.mark.parametrize("name", FUSED)
def test_prep_with_scan(name, monkeypatch):
    """Prep with the reverse state-gradient scan inside (one workgroup per (sequence,
    head) unit at a time, its chunks last to first; no Tm / PT in memory), forced on:
    gradients, per-chunk dS and dh0 against the oracle."""
    monkeypatch.setenv("KDA_PREPSCAN", "1")
    print("\n[case] prep with scan %s" % name, flush=True)
    _check(name)


@pytest.mark.parametrize("name,cap", [("weak_decay_bf16", 3), ("multi_ragged_bf16", 2),
                                      ("weak_decay_fp32", 2), ("qk_norm_fp32", 3),
                                      ("ragged_bf16", 3), ("gate_bias_bf16", 2)])
def test_prep_with_scan_capped(name, cap, monkeypatch):
    """The same with the grid capped, so that every workgroup walks several units (the
    state restarts from dht at each unit's last chunk, the next unit's inputs are fetched
    during the current unit's first chunk): oracle parity, and bit-identical results to
    the full grid and to the separate prep and scan kernels' per-chunk dS inputs."""
    monkeypatch.setenv("KDA_PREPSCAN", "1")
    inp = KI.make_inputs(KI.get_workload(name))
    print("\n[case] prep with scan %s, grid capped at %d" % (name, cap), flush=True)
    full = KC.run_gpu(inp)
    monkeypatch.setenv("KDA_GRID_CAP", str(cap))
    capped = KC.run_gpu(inp)
    ref = KC.oracle_for(inp)
    ref["h_saved"] = ref["states"]
    KC.compare(capped, ref, GRADS + INTER, KC.TOL[inp["dtype"]], label=name + " capped")
    for key in GRADS + ["dstates"]:
        assert np.array_equal(full[key], capped[key]), key


@pytest.mark.parametrize("name", FUSED)
def test_forward_with_scan(name, monkeypatch):
    """The production forward in one kernel (prep's forward mode carrying the state:
    X = Uv - W S, O = Qd S + Mqk X, S <- e^{G_T} S + Kr^T X per chunk, no per-chunk operands
    in memory), forced on for workloads with equal chunk counts per sequence: o, ht and the
    chunk-start states against the oracle's per-token recurrence."""
    monkeypatch.setenv("KDA_PREPSCAN", "1")
    print("\n[case] forward with scan %s" % name, flush=True)
    inp = KI.make_inputs(KI.get_workload(name))
    res = KC.run_gpu_fwd(inp)
    ref = KC.oracle_fwd_for(inp)
    ref["h_saved"] = ref["states"]
    rep = KC.compare(res, ref, ["o", "ht", "h_saved"], KC.TOL[inp["dtype"]],
                     label="forward with scan " + name)
    print("[errors] " + " ".join("%s=%.2e" % kv for kv in rep.items()), flush=True)


@pytest.mark.parametrize("name,cap", [("weak_decay_bf16", 3), ("multi_ragged_bf16", 2),
                                      ("qk_norm_fp32", 3), ("ragged_fp32", 2),
                                      ("gate_log2_fp32", 3)])
def test_forward_with_scan_capped(name, cap, monkeypatch):
    """The same with several units per workgroup (the state restarts from h0 at each
    unit's first chunk): oracle parity and bit-identical results to the full grid."""
    monkeypatch.setenv("KDA_PREPSCAN", "1")
    inp = KI.make_inputs(KI.get_workload(name))
    print("\n[case] forward with scan %s, grid capped at %d" % (name, cap), flush=True)
    full = KC.run_gpu_fwd(inp)
    monkeypatch.setenv("KDA_GRID_CAP", str(cap))
    capped = KC.run_gpu_fwd(inp)
    ref = KC.oracle_fwd_for(inp)
    ref["h_saved"] = ref["states"]
    KC.compare(capped, ref, ["o", "ht", "h_saved"], KC.TOL[inp["dtype"]], label=name + " capped")
    for key in ("o", "ht", "h_saved"):
        assert np.array_equal(full[key], capped[key]), key


@pytest.mark.parametrize("name", ["tiny_fp32", "weak_decay_bf16", "qk_norm_fp32", "ragged_bf16"])
def test_recompute_with_scans_in_prep(name, monkeypatch):
    """kda_bwd without h_saved with both scans inside prep: the fused forward recomputes
    the chunk-start states, the fused backward carries dS."""
    monkeypatch.setenv("KDA_PREPSCAN", "1")
    print("\n[case] recompute, scans inside prep, %s" % name, flush=True)
    _check(name, use_h_saved=False)


@pytest.mark.parametrize("wl", [
    KI.Workload("empty_batch_fp32", 2, 0, 2, 64, 64, "f32", 1300, h0_std=0.3, dht_std=1.0,
                dt_bias_std=1.0),
    KI.Workload("empty_seqs_bf16", 1, 0, 3, 128, 128, "bf16", 1301, varlen_seqs=3,
                fixed_lengths=(0, 0, 0), h0_std=0.3, dht_std=1.0, gate_log2=True,
                qk_l2norm=True),
], ids=lambda w: w.name)
@pytest.mark.parametrize("use_h_saved", [True, False])
def test_no_tokens(wl, use_h_saved):
    """No tokens at all (an empty batch, or packed sequences that are all empty): nothing
    per token to compute; dh0 = dht, ht = h0, dA_log = 0 and ddt_bias = 0, as the oracle
    gives, from the backward, the reference forward and the production forward."""
    print("\n[case] no tokens %s h_saved=%s" % (wl.name, use_h_saved), flush=True)
    inp = KI.make_inputs(wl)
    res = KC.run_gpu(inp, use_h_saved=use_h_saved)
    fres = KC.run_gpu_fwd(inp)
    ref = KC.oracle_for(inp)
    extra = ["ddt_bias"] if inp.get("dt_bias") is not None else []
    for key in ["dh0", "dA_log", "ht"] + extra:
        assert np.array_equal(res[key], ref[key]), key
    assert np.array_equal(fres["ht"], ref["ht"])
    for key in ("dq", "dk", "dv", "dg_raw", "dbeta", "o"):
        assert res[key].size == 0, key


def test_max_row_stride():
    """The largest token row the library accepts, H*K just under 2^22 (H = 32767,
    K = V = 128, bf16: an fp32 g_raw row of 16 MiB less 512 bytes), over one full chunk
    with h0 and dht: the 24-bit row-offset arithmetic of the kernels at its limit.
    Backward (fused with the scan: 32767 units), reference and production forward;
    compared with the oracle on four heads spread over the row (heads are independent)."""
    import linear_attention_backward_amd as K
    import torch
    wl = KI.Workload("max_row_bf16", 1, 64, 32767, 128, 128, "bf16", 1400, h0_std=0.3,
                     dht_std=1.0)
    print("\n[case] max row stride: H=%d K=%d T=%d" % (wl.H, wl.K, wl.T), flush=True)
    inp = KI.make_inputs(wl)
    heads = [0, 1, 16383, 32766]
    g = KC.to_gpu(inp)
    fwd = K.kda_fwd_ref(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], h0=g["h0"])
    out = K.kda_bwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], g["dO"],
                    h0=g["h0"], dht=g["dht"], h_saved=fwd["h_saved"], want_dstates=True)
    pf = K.kda_fwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], h0=g["h0"])
    torch.cuda.synchronize()
    print("[gpu done] max row stride", flush=True)
    hi = torch.tensor(heads, device="cuda")

    def pick(t, axis):
        return t.index_select(axis, hi).float().cpu().numpy().astype(np.float64)

    res = {k: pick(out[k], 2).reshape(64, len(heads), -1) for k in ("dq", "dk", "dv", "dg_raw")}
    res["dbeta"] = pick(out["dbeta"], 2).reshape(64, len(heads))
    res["dA_log"] = pick(out["dA_log"], 0)
    res["dstates"] = pick(out["dstates"], 1)
    res["dh0"] = pick(out["dh0"], 1)
    res["h_saved"] = pick(fwd["h_saved"], 1)
    res["o"] = pick(fwd["o"], 2).reshape(64, len(heads), -1)
    res["ht"] = pick(fwd["ht"], 1)
    fres = {"o": pick(pf["o"], 2).reshape(64, len(heads), -1), "ht": pick(pf["ht"], 1),
            "h_saved": pick(pf["h_saved"], 1)}
    del g, fwd, out, pf
    ref = KC.oracle_for(inp, heads)
    ref["h_saved"] = ref["states"]
    tol = KC.TOL["bf16"]
    rep = KC.compare(res, ref, ["dq", "dk", "dv", "dg_raw", "dbeta", "dA_log", "dh0",
                                "dstates", "h_saved", "o", "ht"], tol, label="max row stride")
    print("[errors] " + " ".join("%s=%.2e" % kv for kv in rep.items()), flush=True)
    KC.compare(fres, ref, ["o", "ht", "h_saved"], tol, label="max row stride forward")


@pytest.mark.parametrize("n,lo,dtype,D,env", [
    (5000, 0, "bf16", 64, {}),                       # more sequences than the fused scan orders
    (4096, 1, "f32", 64, {"KDA_PREPSCAN": "1"}),      # the most the fused scan orders
], ids=["5000_seqs_bf16", "4096_seqs_fp32_fused"])
def test_many_sequences(n, lo, dtype, D, env, monkeypatch):
    """Thousands of short packed sequences (lengths 0-99 or 1-99 tokens, empty ones
    included): the chunk table and its longest-first unit order at and past their largest
    size, the per-sequence state scans, dh0 of every sequence."""
    for key, val in env.items():
        monkeypatch.setenv(key, val)
    rng = np.random.default_rng(1500 + n)
    lens = tuple(int(x) for x in rng.integers(lo, 100, size=n))
    wl = KI.Workload("seqs%d" % n, 1, sum(lens), 2, D, D, dtype, 1500 + n, varlen_seqs=n,
                     fixed_lengths=lens, h0_std=0.3, dht_std=1.0, alog_lo=-3.0, alog_hi=1.0)
    print("\n[case] %d sequences, %d tokens, env=%s" % (n, sum(lens), env), flush=True)
    inp = KI.make_inputs(wl)
    res = KC.run_gpu(inp)
    fres = KC.run_gpu_fwd(inp)
    ref = KC.oracle_for(inp)
    ref["h_saved"] = ref["states"]
    tol = KC.TOL[dtype]
    rep = KC.compare(res, ref, GRADS + INTER, tol, label=wl.name)
    print("[errors] " + " ".join("%s=%.2e" % kv for kv in rep.items()), flush=True)
    KC.compare(fres, ref, ["o", "ht", "h_saved"], tol, label=wl.name + " forward")


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128)])
def test_extreme_decay(dtype, D):
    """A_log = 10 (e^A_log = 22026) with g_raw around 2: per-token log decays of about
    -5e4, every decay factor between two tokens underflows to 0 and the cumulative gate
    reaches -1e7 within a chunk; each token sees only its own write.  dg, dA_log and dh0
    are exactly 0 in the oracle; the kernels must not turn the huge cumulative gates into
    inf or NaN anywhere."""
    wl = KI.Workload("extreme_decay", 1, 200, 2, D, D, dtype, 1600, alog_lo=10.0, alog_hi=10.0,
                     graw_mean=2.0, h0_std=0.3, dht_std=1.0)
    print("\n[case] extreme decay %s" % dtype, flush=True)
    inp = KI.make_inputs(wl)
    res = KC.run_gpu(inp)
    fres = KC.run_gpu_fwd(inp)
    ref = KC.oracle_for(inp)
    ref["h_saved"] = ref["states"]
    tol = KC.TOL[dtype]
    for key, val in list(res.items()) + [("f_" + k, v) for k, v in fres.items()]:
        assert np.isfinite(val).all(), key
    rep = KC.compare(res, ref, GRADS + INTER, tol, label="extreme decay")
    print("[errors] " + " ".join("%s=%.2e" % kv for kv in rep.items()), flush=True)
    KC.compare(fres, ref, ["o", "ht", "h_saved"], tol, label="extreme decay forward")
