"""The seeded input generator shared by the oracle and the HIP path (CPU only).

It holds none of the method's arithmetic, but both sides see exactly what it returns, so
its recipe is pinned here: bf16 rounding against torch's own conversion, determinism per
seed, the drawn distributions and structure (unit-norm q/k rows, beta in (0, 1), A_log in
its range, packed lengths that sum to the total with a ragged chunk), and that head and
sequence selection are plain sub-arrays of the full inputs."""
import math

import numpy as np
import pytest

import kda_inputs as KI


def test_round_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(10.0) ** rng.integers(
            -30, 30, size=100000).astype(np.float32),
        # exact ties between two bf16 values (both parities of the kept bit), signed zeros,
        # the largest finite float (rounds to inf), infinities, the smallest normal
        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0, -0.0,
                  np.finfo(np.float32).max, np.inf, -np.inf, np.finfo(np.float32).tiny],
                 dtype=np.float32)])
    got = KI.round_bf16(x)
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    nan = KI.round_bf16(np.array([np.nan], dtype=np.float32))
    assert np.isnan(nan).all()


def test_same_seed_same_inputs():
    wl = KI.get_workload("ragged_bf16")
    a, b = KI.make_inputs(wl), KI.make_inputs(wl)
    for key, val in a.items():
        if isinstance(val, np.ndarray):
            assert np.array_equal(val, b[key]), key


@pytest.mark.parametrize("name", ["tiny_fp32", "ragged_bf16", "weak_decay_bf16",
                                  "gate_bias_bf16", "qk_norm_fp32"])
def test_recipe(name):
    wl = KI.get_workload(name)
    inp = KI.make_inputs(wl)
    TT = wl.tokens
    assert inp["q"].shape == (TT, wl.H, wl.K) and inp["v"].shape == (TT, wl.H, wl.V)
    assert inp["cu_seqlens"][0] == 0 and inp["cu_seqlens"][-1] == TT
    if not wl.qk_l2norm:  # unit rows (up to the bf16 rounding of bf16 workloads)
        tol = 1e-2 if wl.dtype == "bf16" else 1e-5
        for key in ("q", "k"):
            nrm = np.linalg.norm(inp[key].astype(np.float64), axis=-1)
            assert np.abs(nrm - 1.0).max() < tol, key
    assert (inp["beta"] > 0).all() and (inp["beta"] < 1).all()
    assert (inp["A_log"] >= wl.alog_lo).all() and (inp["A_log"] <= wl.alog_hi).all()
    if wl.dtype == "bf16":  # every activation is bf16-exact
        for key in ("q", "k", "v", "dO"):
            assert np.array_equal(KI.round_bf16(inp[key]), inp[key]), key
    assert (inp["h0"] is None) == (wl.h0_std == 0) and (inp["dht"] is None) == (wl.dht_std == 0)
    assert (inp["dt_bias"] is None) == (wl.dt_bias_std == 0)


def test_varlen_lengths():
    rng = np.random.default_rng(3)
    for _ in range(50):
        n = int(rng.integers(2, 20))
        lo, hi = 64, 8192
        total = int(rng.integers(n * lo, n * hi // 4))
        lens = KI.varlen_lengths(np.random.default_rng(int(rng.integers(1 << 30))), n, total,
                                 lo, hi)
        assert int(lens.sum()) == total
        assert (lens >= lo).all() and (lens <= hi).all()
        assert any(int(x) % KI.CHUNK for x in lens)  # at least one ragged chunk
    wl = KI.get_workload("varlen_bf16")  # its lengths are the generator's first draws
    lens = KI.varlen_lengths(np.random.default_rng(wl.seed), wl.varlen_seqs, wl.tokens,
                             wl.varlen_min, wl.varlen_max)
    assert len(lens) == 16 and int(lens.sum()) == 65536


def test_selection_is_a_subarray():
    inp = KI.make_inputs(KI.get_workload("ragged_fp32"))
    sub = KI.select_heads(inp, [1])
    for key in ("q", "k", "v", "dO", "g_raw", "beta"):
        assert np.array_equal(sub[key], inp[key][:, [1]]), key
    assert np.array_equal(sub["A_log"], inp["A_log"][[1]])
    seq = KI.select_seqs(inp, [2])
    a, b = inp["cu_seqlens"][2], inp["cu_seqlens"][3]
    assert np.array_equal(seq["q"], inp["q"][a:b])
    assert list(seq["cu_seqlens"]) == [0, b - a]


def test_workload_table_matches_the_stated_shapes():
    W = KI.WORKLOADS
    assert (W["tiny_fp32"].B, W["tiny_fp32"].T, W["tiny_fp32"].H, W["tiny_fp32"].K) == (1, 256, 2, 64)
    assert (W["single_seq_bf16"].T, W["single_seq_bf16"].H, W["single_seq_bf16"].K) == (2048, 16, 128)
    assert (W["train_bf16"].B, W["train_bf16"].T, W["train_bf16"].H) == (8, 4096, 32)
    assert W["varlen_bf16"].varlen_seqs == 16 and W["varlen_bf16"].tokens == 65536
    assert (W["long_bf16"].T, W["long_bf16"].H) == (131072, 16)
    assert all(w.alog_lo == 0.0 and abs(w.alog_hi - math.log(16.0)) < 1e-12 for w in W.values())
