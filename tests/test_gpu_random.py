"""Seeded random combinations of shapes, gate options and launch choices, each checked
against the fp64 oracle: the backward (with the saved chunk states given or recomputed)
and the production forward.

Every case draws, from its own seed: the activation dtype and head size (fp32 K = 64,
bf16 K = 64 or 128), the head count, either a uniform batch or packed sequences (empty
ones included), the decay regime, h0 / dht present or not, the gate bias, log2-unit
gates and in-kernel q/k normalisation; and the library's launch choices through its
environment overrides: the scans inside prep or the separate kernels, split scans with
small chunk groups (joint or separate group maps), and a capped persistent grid.  The
named cases in the other test files pin each option; these mix them."""
import math

import numpy as np
import pytest

import kda_inputs as KI
from tests import kda_case as KC

pytestmark = pytest.mark.gpu

GRADS = ["dq", "dk", "dv", "dg_raw", "dbeta", "dA_log", "dh0"]
N_CASES = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_backward_amd as K
    K.load_library()


def draw_case(i: int):
    """Workload, launch overrides and h_saved choice of case i (host-side only)."""
    rng = np.random.default_rng(7000 + i)
    kind = rng.integers(3)
    dtype, D = [("f32", 64), ("bf16", 64), ("bf16", 128)][kind]
    H = int(rng.integers(1, 4))
    regime = rng.integers(3)
    alog = [(0.0, math.log(16.0)), (-6.0, -2.0), (-3.0, 1.0)][regime]
    common = dict(h0_std=float(rng.choice([0.0, 0.3])), dht_std=float(rng.choice([0.0, 1.0])),
                  alog_lo=alog[0], alog_hi=alog[1],
                  dt_bias_std=float(rng.choice([0.0, 1.0])), gate_log2=bool(rng.integers(2)),
                  qk_l2norm=bool(rng.integers(2)))
    if rng.integers(2):
        n = int(rng.integers(1, 6))
        lens = [int(x) for x in rng.integers(0, 260, size=n)]
        if rng.integers(3) == 0:  # an empty sequence somewhere
            lens[int(rng.integers(n))] = 0
        if sum(lens) == 0:
            lens[0] = 1
        wl = KI.Workload("rand%d" % i, 1, sum(lens), H, D, D, dtype, 7100 + i, varlen_seqs=n,
                         fixed_lengths=tuple(lens), **common)
    else:
        B = int(rng.integers(1, 4))
        T = int(rng.integers(1, 300))
        wl = KI.Workload("rand%d" % i, B, T, H, D, D, dtype, 7100 + i, **common)
    env = {}
    mode = rng.integers(3)
    if mode == 1:
        env["KDA_PREPSCAN"] = "0"
        if rng.integers(2):
            env["KDA_SCAN_GROUP"] = str(int(rng.integers(1, 4)))
            env["KDA_SCANPQ"] = str(i % 2)
    elif mode == 2:
        env["KDA_PREPSCAN"] = "1"
    if rng.integers(2):
        env["KDA_GRID_CAP"] = str(int(rng.integers(1, 6)))
    use_h_saved = bool(rng.integers(4) != 0)
    return wl, env, use_h_saved


def test_draws_cover_the_options():
    """The drawn cases reach every option at least once (host-side check of the draws)."""
    seen = set()
    for i in range(N_CASES):
        wl, env, hs = draw_case(i)
        seen.add(("dtype", wl.dtype, wl.K))
        seen.add(("varlen", wl.varlen_seqs > 0))
        seen.add(("bias", wl.dt_bias_std > 0))
        seen.add(("log2", wl.gate_log2))
        seen.add(("qn", wl.qk_l2norm))
        seen.add(("h_saved", hs))
        seen.add(("prepscan", env.get("KDA_PREPSCAN")))
        seen.add(("group", "KDA_SCAN_GROUP" in env))
        seen.add(("maps", env.get("KDA_SCANPQ")))
        seen.add(("cap", "KDA_GRID_CAP" in env))
    for opt in [("dtype", "f32", 64), ("dtype", "bf16", 64), ("dtype", "bf16", 128),
                ("varlen", True), ("varlen", False), ("bias", True), ("log2", True),
                ("qn", True), ("h_saved", False), ("prepscan", "0"), ("prepscan", "1"),
                ("prepscan", None), ("group", True), ("maps", "0"), ("maps", "1"), ("cap", True)]:
        assert opt in seen, opt


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i, monkeypatch):
    wl, env, use_h_saved = draw_case(i)
    print("\n[case] random %d: %s env=%s h_saved=%s" % (i, wl, env, use_h_saved), flush=True)
    for key, val in env.items():
        monkeypatch.setenv(key, val)
    inp = KI.make_inputs(wl)
    tol = KC.TOL[inp["dtype"]]
    res = KC.run_gpu(inp, use_h_saved=use_h_saved)
    ref = KC.oracle_for(inp)
    ref["h_saved"] = ref["states"]
    extra = ["ddt_bias"] if inp.get("dt_bias") is not None else []
    keys = [x for x in GRADS if x != "dA_log"] + ["dstates", "h_saved", "o", "ht"] + extra
    rep = KC.compare(res, ref, keys, tol, label="random %d" % i)
    print("[errors] " + " ".join("%s=%.2e" % kv for kv in rep.items()), flush=True)
    # dA_log[h] is one sum over the head's tokens and channels, sum dg g, whose terms
    # cancel (sum |dg g| / |sum dg g| reaches 1e2-1e4 on these draws): with one to three
    # heads the per-tensor metric is the relative error of that sum itself.  It passes
    # the per-tensor bar, or (bf16 activations, whose intermediates carry bf16 rounding)
    # the forward error bound of a sum whose terms are each within bf16 precision,
    # 2^-8 sum |dg g|.
    err = np.abs(res["dA_log"] - ref["dA_log"])
    terms = np.abs(ref["dg"] * ref["g"]).sum(axis=(0, 2))
    scale = float(np.abs(ref["dA_log"]).max())
    ok = err <= tol * (scale if scale > 0 else 1.0)  # the metric of the other outputs
    if inp["dtype"] == "bf16":
        ok |= err <= 2.0 ** -8 * terms
    print("[dA_log] err %s sum|terms| %s" % (err, terms), flush=True)
    assert ok.all(), "random %d: dA_log error %s (reference %s)" % (i, err, ref["dA_log"])
    fres = KC.run_gpu_fwd(inp)
    KC.compare(fres, ref, ["o", "ht", "h_saved"], tol, label="random %d forward" % i)
