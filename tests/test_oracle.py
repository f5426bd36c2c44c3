"""Pins for the fp64 CPU oracle (no GPU).

Each test ties the oracle to something other than itself: a hand-worked scalar
example, closed forms of special cases, finite differences of its own forward,
an independent autograd derivative, agreement between the per-token and the
chunk forms, and library routines for the gate.  Shapes use K != V so that a
transposed operand cannot pass.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(seed, lens, H, K, V, decay=0.5, with_state=True):
    rng = np.random.default_rng(seed)
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    TT = int(cu[-1])
    N = len(lens)
    q = rng.standard_normal((TT, H, K))
    k = rng.standard_normal((TT, H, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((TT, H, V))
    g_raw = rng.standard_normal((TT, H, K))
    A_log = rng.uniform(-2.0, 0.5, size=H) + math.log(decay)
    beta = rng.uniform(0.05, 0.95, size=(TT, H))
    h0 = rng.standard_normal((N, H, K, V)) if with_state else None
    dO = rng.standard_normal((TT, H, V))
    dht = rng.standard_normal((N, H, K, V)) if with_state else None
    return dict(cu=cu, q=q, k=k, v=v, g_raw=g_raw, A_log=A_log, beta=beta, h0=h0, dO=dO,
                dht=dht)


def _loss(c, **over):
    d = dict(c)
    d.update(over)
    g = O.gate(d["g_raw"], d["A_log"], dt_bias=d.get("dt_bias"),
               log2_units=bool(d.get("gate_log2", False)))
    q, k = d["q"], d["k"]
    if d.get("qk_l2norm"):
        q, k = O.l2norm(q)[0], O.l2norm(k)[0]
    o, ht, _ = O.forward(q, k, d["v"], g, d["beta"], d["h0"], d["cu"], chunk=4,
                         want_states=False)
    L = float(np.sum(o * d["dO"]))
    if d["dht"] is not None:
        L += float(np.sum(ht * d["dht"]))
    return L


def _full_backward(c, chunk=4):
    g = O.gate(c["g_raw"], c["A_log"])
    out = O.backward(c["q"], c["k"], c["v"], g, c["beta"], c["h0"], c["dO"], c["dht"], c["cu"],
                     chunk=chunk, want_dstates=True)
    dg_raw, dA, _ = O.gate_backward(c["g_raw"], c["A_log"], g, out["dg"])
    out["dg_raw"], out["dA_log"] = dg_raw, dA
    return out


def test_scalar_worked_example():
    """K = V = 1, three tokens, every value derived by hand (golden fixture)."""
    fx = json.load(open(os.path.join(GOLDEN, "scalar_recurrence.json")))
    i, e = fx["inputs"], fx["expected"]
    T = 3
    sh = (T, 1, 1)
    q = np.full(sh, i["q"])
    k = np.full(sh, i["k"])
    v = np.asarray(i["v"]).reshape(sh)
    g = np.full(sh, math.log(i["a"]))
    beta = np.full((T, 1), i["beta"])
    h0 = np.full((1, 1, 1, 1), i["h0"])
    dO = np.asarray(i["dO"]).reshape(sh)
    dht = np.full((1, 1, 1, 1), i["dht"])
    cu = np.array([0, T])
    o, ht, _ = O.forward(q, k, v, g, beta, h0, cu)
    np.testing.assert_allclose(o.ravel(), e["o"], rtol=1e-13)
    np.testing.assert_allclose(ht.ravel(), [e["ht"]], rtol=1e-13)
    out = O.backward(q, k, v, g, beta, h0, dO, dht, cu)
    for key in ("dq", "dv", "dbeta", "dk", "dg"):
        np.testing.assert_allclose(out[key].ravel(), e[key], rtol=1e-12, err_msg=key)
    np.testing.assert_allclose(out["dh0"].ravel(), [e["dh0"]], rtol=1e-12)


def test_delta_rule_write_property():
    """beta = 1, g = 0, |k| = 1: the update writes v exactly, S_t^T k_t = v_t.
    With q_t = k_t the output o_t equals v_t."""
    rng = np.random.default_rng(3)
    T, H, K, V = 9, 2, 6, 4
    k = rng.standard_normal((T, H, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, V))
    h0 = rng.standard_normal((1, H, K, V))
    o, _, _ = O.forward(k, k, v, np.zeros((T, H, K)), np.ones((T, H)), h0, np.array([0, T]))
    np.testing.assert_allclose(o, v, atol=1e-13)


def test_zero_beta_is_pure_decay():
    """beta = 0: S_t = Diag(exp(G_t)) h0 with G the running sum of g."""
    rng = np.random.default_rng(4)
    T, H, K, V = 11, 2, 5, 3
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    v = rng.standard_normal((T, H, V))
    g = -rng.uniform(0, 0.7, size=(T, H, K))
    h0 = rng.standard_normal((1, H, K, V))
    o, ht, st = O.forward(q, k, v, g, np.zeros((T, H)), h0, np.array([0, T]), chunk=4)
    G = np.cumsum(g, axis=0)
    for t in range(T):
        S_t = np.exp(G[t])[:, :, None] * h0[0]
        np.testing.assert_allclose(o[t], np.einsum("hk,hkv->hv", q[t], S_t), atol=1e-13)
    np.testing.assert_allclose(ht[0], np.exp(G[-1])[:, :, None] * h0[0], atol=1e-13)
    np.testing.assert_allclose(st[1], np.exp(G[3])[:, :, None] * h0[0], atol=1e-13)


def test_backward_closed_form_zero_beta_zero_gate():
    """beta = 0, g = 0: S_t = h0 for every t, so
    dq_t = h0 dO_t, dh0 = dht + sum_t q_t dO_t^T, dv = 0, dk = 0,
    dbeta_t = k_t^T (dht + sum_{s>=t} q_s dO_s^T)(v_t - h0^T k_t),
    dg_t = rowsum over j of (dht + sum_{s>=t} q_s dO_s^T) . h0."""
    rng = np.random.default_rng(5)
    T, H, K, V = 7, 1, 4, 3
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    v = rng.standard_normal((T, H, V))
    h0 = rng.standard_normal((1, H, K, V))
    dO = rng.standard_normal((T, H, V))
    dht = rng.standard_normal((1, H, K, V))
    out = O.backward(q, k, v, np.zeros((T, H, K)), np.zeros((T, H)), h0, dO, dht,
                     np.array([0, T]))
    S = h0[0, 0]
    np.testing.assert_allclose(out["dq"][:, 0], dO[:, 0] @ S.T, atol=1e-12)
    np.testing.assert_allclose(out["dh0"][0, 0], dht[0, 0] + q[:, 0].T @ dO[:, 0], atol=1e-12)
    np.testing.assert_allclose(out["dv"], 0.0, atol=1e-14)
    np.testing.assert_allclose(out["dk"], 0.0, atol=1e-14)
    for t in range(T):
        M = dht[0, 0] + q[t:, 0].T @ dO[t:, 0]
        db = k[t, 0] @ M @ (v[t, 0] - S.T @ k[t, 0])
        np.testing.assert_allclose(out["dbeta"][t, 0], db, atol=1e-12)
        np.testing.assert_allclose(out["dg"][t, 0], np.sum(M * S, axis=1), atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 2, 3, 4, 16, 64, 200])
def test_chunked_forward_agrees(chunk):
    """Per-token and chunk forms agree to rounding for any chunk size, ragged tails
    included (lengths 1, 13, 64, 70)."""
    c = _rand_case(7, [1, 13, 64, 70], H=2, K=6, V=5, decay=1.0)
    g = O.gate(c["g_raw"], c["A_log"])
    o1, h1, s1 = O.forward(c["q"], c["k"], c["v"], g, c["beta"], c["h0"], c["cu"], chunk=chunk)
    o2, h2, s2 = O.forward_chunked(c["q"], c["k"], c["v"], g, c["beta"], c["h0"], c["cu"],
                                   chunk=chunk)
    scale = max(np.abs(o1).max(), 1.0)
    assert np.abs(o1 - o2).max() / scale < 1e-12
    assert np.abs(h1 - h2).max() / max(np.abs(h1).max(), 1.0) < 1e-12
    assert np.abs(s1 - s2).max() / max(np.abs(s1).max(), 1.0) < 1e-12


def test_chunked_forward_strong_decay_no_overflow():
    """Strong decay (per-token log decay of tens): the chunk form uses only
    non-positive exponents, so it stays finite and still agrees."""
    c = _rand_case(8, [130], H=1, K=4, V=3)
    c["A_log"] = np.array([math.log(16.0)])
    c["g_raw"] = c["g_raw"] + 2.0
    g = O.gate(c["g_raw"], c["A_log"])
    assert g.min() < -40
    o1, h1, _ = O.forward(c["q"], c["k"], c["v"], g, c["beta"], c["h0"], c["cu"])
    o2, h2, _ = O.forward_chunked(c["q"], c["k"], c["v"], g, c["beta"], c["h0"], c["cu"])
    assert np.all(np.isfinite(o2))
    assert np.abs(o1 - o2).max() < 1e-12 * max(1.0, np.abs(o1).max())


def test_finite_differences_all_inputs():
    """Central differences of the oracle forward (eps = 1e-6) against the
    hand-derived backward, for every scalar of q, k, v, g_raw, A_log, beta, h0
    (two sequences of lengths 5 and 9, H = 2, K = 4, V = 3)."""
    c = _rand_case(11, [5, 9], H=2, K=4, V=3)
    out = _full_backward(c)
    grads = dict(q="dq", k="dk", v="dv", g_raw="dg_raw", A_log="dA_log", beta="dbeta",
                 h0="dh0")
    eps = 1e-6
    for name, gname in grads.items():
        x = c[name]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xp[idx] += eps
            xm = x.copy()
            xm[idx] -= eps
            num[idx] = (_loss(c, **{name: xp}) - _loss(c, **{name: xm})) / (2 * eps)
        err = np.abs(num - out[gname]).max() / np.abs(num).max()
        assert err < 1e-7, (name, err)


def test_autograd_and_boundary_state_gradients():
    """An independent torch fp64 implementation of the recurrence, differentiated
    by autograd, gives the same gradients, and the same dL/dS at every chunk end
    (uses by later tokens only)."""
    torch = pytest.importorskip("torch")
    c = _rand_case(12, [7, 12], H=2, K=5, V=3)
    C = 4
    out = _full_backward(c, chunk=C)
    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    q, k, v, g_raw, A_log, beta, h0 = map(T, (c["q"], c["k"], c["v"], c["g_raw"], c["A_log"],
                                              c["beta"], c["h0"]))
    g = -torch.exp(A_log)[None, :, None] * torch.nn.functional.softplus(g_raw)
    dO = torch.tensor(c["dO"])
    dht = torch.tensor(c["dht"])
    cu = c["cu"]
    L = 0.0
    bounds = []
    for n in range(len(cu) - 1):
        for h in range(q.shape[1]):
            S = h0[n, h]
            for t in range(int(cu[n]), int(cu[n + 1])):
                kt, vt, qt = k[t, h], v[t, h], q[t, h]
                St = torch.exp(g[t, h])[:, None] * S
                St = St + beta[t, h] * torch.outer(kt, vt - St.T @ kt)
                L = L + (St.T @ qt) @ dO[t, h]
                local = t - int(cu[n])
                if (local + 1) % C == 0 or t == int(cu[n + 1]) - 1:
                    S = St * 1.0  # separate node: gradient from later tokens only
                    S.retain_grad()
                    bounds.append(((n, h, local // C), S))
                else:
                    S = St
            L = L + torch.sum(S * dht[n, h])
    L.backward()
    for name, gname in dict(q="dq", k="dk", v="dv", g_raw="dg_raw", A_log="dA_log",
                            beta="dbeta", h0="dh0").items():
        ref = locals()[name].grad.numpy()
        err = np.abs(ref - out[gname]).max() / np.abs(ref).max()
        assert err < 1e-12, (name, err)
    off = np.concatenate([[0], np.cumsum([(int(cu[i + 1] - cu[i]) + C - 1) // C
                                          for i in range(len(cu) - 1)])])
    for (n, h, ci), S in bounds:
        ref = S.grad.numpy()
        got = out["dstates"][off[n] + ci, h]
        assert np.abs(ref - got).max() < 1e-12 * max(1.0, np.abs(ref).max())


def test_gate_against_library_routines():
    """softplus against numpy's logaddexp; the gate chain rule against the
    analytic derivative of logaddexp (the logistic function from scipy)."""
    from scipy.special import expit
    rng = np.random.default_rng(13)
    g_raw = rng.standard_normal((6, 3, 4)) * 5
    A_log = rng.uniform(0, math.log(16), size=3)
    g = O.gate(g_raw, A_log)
    ref = -np.exp(A_log)[None, :, None] * np.logaddexp(0.0, g_raw)
    np.testing.assert_allclose(g, ref, rtol=1e-14)
    dg = rng.standard_normal(g.shape)
    dg_raw, dA, _ = O.gate_backward(g_raw, A_log, g, dg)
    np.testing.assert_allclose(dg_raw, dg * (-np.exp(A_log)[None, :, None] * expit(g_raw)),
                               rtol=1e-13)
    np.testing.assert_allclose(dA, np.sum(dg * ref, axis=(0, 2)), rtol=1e-12)


def test_parallel_matches_serial():
    """OpenMP over (sequence, head) units does not change results."""
    c = _rand_case(14, [30, 17, 40], H=3, K=8, V=6)
    g = O.gate(c["g_raw"], c["A_log"])
    a = O.backward(c["q"], c["k"], c["v"], g, c["beta"], c["h0"], c["dO"], c["dht"], c["cu"],
                   nthreads=1)
    b = O.backward(c["q"], c["k"], c["v"], g, c["beta"], c["h0"], c["dO"], c["dht"], c["cu"],
                   nthreads=4)
    for key in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert np.array_equal(a[key], b[key]), key


def _as_inputs(c, **over):
    d = dict(c)
    d.update(over)
    return dict(q=d["q"], k=d["k"], v=d["v"], g_raw=d["g_raw"], A_log=d["A_log"], beta=d["beta"],
                h0=d["h0"], dO=d["dO"], dht=d["dht"], cu_seqlens=d["cu"], chunk=4,
                dt_bias=d.get("dt_bias"), gate_log2=d.get("gate_log2", False),
                qk_l2norm=d.get("qk_l2norm", False))


_GRADS = ("dq", "dk", "dv", "dg_raw", "dA_log", "dbeta", "dh0")


def test_gate_variants_against_library_routines():
    """The gate map with a per-channel bias and in log2 units against numpy's
    logaddexp; its chain rule against scipy's logistic function; the bias gradient
    against numpy's sum over tokens."""
    from scipy.special import expit
    rng = np.random.default_rng(21)
    g_raw = rng.standard_normal((7, 3, 4)) * 4
    A_log = rng.uniform(-1, math.log(16), size=3)
    db = rng.standard_normal((3, 4))
    for log2_units, unit in ((False, 1.0), (True, math.log(2.0))):
        x = g_raw + db[None]
        g = O.gate(g_raw, A_log, dt_bias=db, log2_units=log2_units)
        ref = unit * (-np.exp(A_log)[None, :, None] * np.logaddexp(0.0, x))
        np.testing.assert_allclose(g, ref, rtol=1e-14)
        dg = rng.standard_normal(g.shape)
        dg_raw, dA, ddt = O.gate_backward(g_raw, A_log, g, dg, dt_bias=db, log2_units=log2_units)
        ref_raw = dg * unit * (-np.exp(A_log)[None, :, None] * expit(x))
        np.testing.assert_allclose(dg_raw, ref_raw, rtol=1e-13)
        np.testing.assert_allclose(dA, np.sum(dg * ref, axis=(0, 2)), rtol=1e-12)
        np.testing.assert_allclose(ddt, ref_raw.sum(axis=0), rtol=1e-12, atol=1e-15)


def test_log2_gate_is_a_shifted_A_log():
    """A gate in log2 units decays by 2^g = exp(g ln 2), and ln 2 e^{A_log} =
    e^{A_log + ln ln 2}: every output equals that of the natural-log gate with A_log
    shifted by ln(ln 2), gradients included (dA_log too, the shift being additive)."""
    c = _rand_case(22, [6, 11], H=2, K=4, V=3)
    a = O.kda_backward(_as_inputs(c, gate_log2=True))
    b = O.kda_backward(_as_inputs(c, A_log=c["A_log"] + math.log(math.log(2.0))))
    for name in _GRADS + ("ddt_bias",):
        np.testing.assert_allclose(a[name], b[name], rtol=1e-11, atol=1e-13, err_msg=name)


def test_dt_bias_is_a_shifted_g_raw():
    """A bias inside the softplus is the same as adding it to g_raw: every output
    agrees with the unbiased problem on g_raw + dt_bias, and ddt_bias is the sum of
    dg_raw over all tokens."""
    c = _rand_case(23, [6, 11], H=2, K=4, V=3)
    db = np.random.default_rng(24).standard_normal((2, 4))
    a = O.kda_backward(_as_inputs(c, dt_bias=db))
    b = O.kda_backward(_as_inputs(c, g_raw=c["g_raw"] + db[None]))
    for name in _GRADS:
        np.testing.assert_allclose(a[name], b[name], rtol=1e-12, atol=1e-14, err_msg=name)
    np.testing.assert_allclose(a["ddt_bias"], b["dg_raw"].sum(axis=0), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("gate_log2", [False, True])
def test_finite_differences_gate_variants(gate_log2):
    """Central differences of the oracle forward against its backward for dt_bias,
    g_raw and A_log, with a bias present and the gate in either unit."""
    c = _rand_case(25, [5, 7], H=2, K=4, V=3)
    c["dt_bias"] = np.random.default_rng(26).standard_normal((2, 4))
    c["gate_log2"] = gate_log2
    out = O.kda_backward(_as_inputs(c))
    eps = 1e-6
    for name, gname in (("dt_bias", "ddt_bias"), ("g_raw", "dg_raw"), ("A_log", "dA_log")):
        x = c[name]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xp[idx] += eps
            xm = x.copy()
            xm[idx] -= eps
            num[idx] = (_loss(c, **{name: xp}) - _loss(c, **{name: xm})) / (2 * eps)
        err = np.abs(num - out[gname]).max() / np.abs(num).max()
        assert err < 1e-7, (name, err)


def test_l2norm_against_library_routines():
    """The per-token L2 normalisation against numpy, its chain rule against torch
    autograd of the same map."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(27)
    x = rng.standard_normal((9, 3, 5)) * rng.uniform(0.01, 10, size=(9, 3, 1))
    xn, r = O.l2norm(x)
    ref = x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + O.L2NORM_EPS)
    np.testing.assert_allclose(xn, ref, rtol=1e-14)
    np.testing.assert_allclose(r, 1.0 / np.sqrt(np.sum(x * x, axis=-1) + O.L2NORM_EPS), rtol=1e-14)
    dxn = rng.standard_normal(x.shape)
    xt = torch.tensor(x, requires_grad=True)
    yt = xt * torch.rsqrt((xt * xt).sum(-1, keepdim=True) + O.L2NORM_EPS)
    (yt * torch.tensor(dxn)).sum().backward()
    np.testing.assert_allclose(O.l2norm_backward(xn, r, dxn), xt.grad.numpy(), rtol=1e-11,
                               atol=1e-14)


def test_finite_differences_qk_l2norm():
    """With q and k L2-normalised inside the method, central differences of the loss
    in the raw q and k match dq and dk (gate bias present, both gate units covered by
    the other finite-difference tests)."""
    c = _rand_case(28, [5, 7], H=2, K=4, V=3)
    c["q"] = c["q"] * 3.0
    c["k"] = c["k"] * 0.5 + 0.1
    c["qk_l2norm"] = True
    c["dt_bias"] = np.random.default_rng(29).standard_normal((2, 4))
    out = O.kda_backward(_as_inputs(c))
    eps = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("g_raw", "dg_raw"), ("beta", "dbeta")):
        x = c[name]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xp[idx] += eps
            xm = x.copy()
            xm[idx] -= eps
            num[idx] = (_loss(c, **{name: xp}) - _loss(c, **{name: xm})) / (2 * eps)
        err = np.abs(num - out[gname]).max() / np.abs(num).max()
        assert err < 1e-7, (name, err)
