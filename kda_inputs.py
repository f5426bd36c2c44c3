"""Seeded synthetic inputs for the KDA backward pass.

This module only draws and casts inputs; it holds none of the method's
arithmetic.  Both the HIP path (through its tests and benchmark) and the CPU
oracle consume the arrays it returns, so the two sides always see bit-identical
(dtype-rounded) inputs.

Recipe (the same for every workload):
  * numpy PCG64 generator, seed given per workload;
  * draw order: sequence lengths (varlen only), A_log, q, k, v, beta logits,
    g_raw, dO, h0, dht;
  * q, k ~ N(0,1) then L2-normalised per (token, head) in fp32;
  * v, dO ~ N(0,1); beta = sigmoid(N(0,1)); g_raw ~ N(0,1);
  * A_log ~ U(lo, hi) per head (default U(0, ln 16));
  * h0 ~ N(0, h0_std^2), dht ~ N(0, dht_std^2) when enabled, else absent (zero);
  * for bf16 workloads q, k, v, dO are rounded to bf16 (round to nearest even);
    g_raw, beta, A_log, h0, dht stay fp32.

Arrays are packed token-major: [TT, H, D] with TT the total token count;
a uniform batch [B, T, H, D] is the same memory as TT = B*T with sequence
boundaries cu_seqlens = [0, T, 2T, ...].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

CHUNK = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    K: int
    V: int
    dtype: str  # "f32" or "bf16"
    seed: int
    varlen_seqs: int = 0  # >0: this many packed sequences, total B*T tokens
    varlen_min: int = 64
    varlen_max: int = 8192
    h0_std: float = 0.0
    dht_std: float = 0.0
    alog_lo: float = 0.0
    alog_hi: float = math.log(16.0)
    graw_mean: float = 0.0
    fixed_lengths: Optional[tuple] = None  # explicit packed lengths
    dt_bias_std: float = 0.0  # >0: a per-(head, channel) gate bias of this scale
    gate_log2: bool = False   # gate in log2 units (decay 2^g per step)
    qk_l2norm: bool = False   # q, k normalised inside the method: drawn raw (scale 2, 0.5)

    @property
    def tokens(self) -> int:
        return self.B * self.T


# The five measured / checked workloads (chunk 64 throughout).
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 256, 2, 64, 64, "f32", 1000),
    "single_seq_bf16": Workload("single_seq_bf16", 1, 2048, 16, 128, 128, "bf16", 1001),
    "train_bf16": Workload("train_bf16", 8, 4096, 32, 128, 128, "bf16", 1002),
    "varlen_bf16": Workload("varlen_bf16", 1, 65536, 32, 128, 128, "bf16", 1003,
                            varlen_seqs=16, h0_std=0.1, dht_std=1.0),
    "long_bf16": Workload("long_bf16", 1, 131072, 16, 128, 128, "bf16", 1004),
}

# Extra checked (untimed) inputs.
EXTRA = {
    # weak decay: cross-chunk terms and the state-gradient carry matter
    "weak_decay_bf16": Workload("weak_decay_bf16", 2, 1024, 4, 128, 128, "bf16", 1101,
                                alog_lo=-6.0, alog_hi=-2.0, h0_std=0.5, dht_std=1.0),
    "weak_decay_fp32": Workload("weak_decay_fp32", 2, 512, 2, 64, 64, "f32", 1102,
                                alog_lo=-6.0, alog_hi=-2.0, h0_std=0.5, dht_std=1.0),
    # strong decay stress: per-token log decays of tens, exp(-G) would overflow
    "strong_decay_bf16": Workload("strong_decay_bf16", 1, 512, 4, 128, 128, "bf16", 1103,
                                  alog_lo=math.log(16.0), alog_hi=math.log(16.0),
                                  graw_mean=2.0),
    # ragged single sequences, lengths around the chunk size
    "ragged_bf16": Workload("ragged_bf16", 1, 1 + 63 + 64 + 65 + 200, 4, 128, 128, "bf16",
                            1104, varlen_seqs=5, fixed_lengths=(1, 63, 64, 65, 200),
                            h0_std=0.3, dht_std=1.0, alog_lo=-3.0, alog_hi=1.0),
    "ragged_fp32": Workload("ragged_fp32", 1, 1 + 63 + 64 + 65 + 200, 2, 64, 64, "f32",
                            1105, varlen_seqs=5, fixed_lengths=(1, 63, 64, 65, 200),
                            h0_std=0.3, dht_std=1.0, alog_lo=-3.0, alog_hi=1.0),
    # several sequences of a length that is not a multiple of the chunk (no cu_seqlens:
    # every sequence ends in a ragged chunk), odd head count
    "multi_ragged_bf16": Workload("multi_ragged_bf16", 3, 100, 3, 128, 128, "bf16", 1107,
                                  h0_std=0.3, dht_std=1.0, alog_lo=-3.0, alog_hi=1.0),
    # one token per sequence
    "single_token_fp32": Workload("single_token_fp32", 2, 1, 1, 64, 64, "f32", 1108,
                                  h0_std=0.5, dht_std=1.0),
    # bf16 with K = V = 64 (the other supported bf16 head size)
    "ragged_bf16_d64": Workload("ragged_bf16_d64", 1, 1 + 63 + 64 + 65 + 200, 4, 64, 64, "bf16",
                                1106, varlen_seqs=5, fixed_lengths=(1, 63, 64, 65, 200),
                                h0_std=0.3, dht_std=1.0, alog_lo=-3.0, alog_hi=1.0),
    # gate variants: a per-channel bias inside the softplus, gates in log2 units
    "gate_bias_bf16": Workload("gate_bias_bf16", 1, 1 + 63 + 64 + 65 + 200, 4, 128, 128, "bf16",
                               1109, varlen_seqs=5, fixed_lengths=(1, 63, 64, 65, 200),
                               h0_std=0.3, dht_std=1.0, alog_lo=-3.0, alog_hi=1.0,
                               dt_bias_std=1.0),
    "gate_log2_fp32": Workload("gate_log2_fp32", 1, 1 + 63 + 64 + 65 + 200, 2, 64, 64, "f32",
                               1110, varlen_seqs=5, fixed_lengths=(1, 63, 64, 65, 200),
                               h0_std=0.3, dht_std=1.0, alog_lo=-3.0, alog_hi=1.0,
                               dt_bias_std=1.0, gate_log2=True),
    "gate_log2_bf16": Workload("gate_log2_bf16", 3, 100, 3, 128, 128, "bf16", 1111,
                               h0_std=0.3, dht_std=1.0, alog_lo=-3.0, alog_hi=1.0,
                               gate_log2=True),
    # q, k L2-normalised inside the method (raw inputs of norm 2 sqrt(K) and sqrt(K) / 2)
    "qk_norm_bf16": Workload("qk_norm_bf16", 1, 1 + 63 + 64 + 65 + 200, 4, 128, 128, "bf16",
                             1112, varlen_seqs=5, fixed_lengths=(1, 63, 64, 65, 200),
                             h0_std=0.3, dht_std=1.0, alog_lo=-3.0, alog_hi=1.0,
                             qk_l2norm=True),
    "qk_norm_fp32": Workload("qk_norm_fp32", 2, 200, 2, 64, 64, "f32", 1113, h0_std=0.3,
                             dht_std=1.0, alog_lo=-3.0, alog_hi=1.0, dt_bias_std=1.0,
                             gate_log2=True, qk_l2norm=True),
    "qk_norm_bf16_d64": Workload("qk_norm_bf16_d64", 2, 130, 2, 64, 64, "bf16", 1114,
                                 h0_std=0.3, dht_std=1.0, alog_lo=-3.0, alog_hi=1.0,
                                 qk_l2norm=True),
    # the training shape with the other supported head sizes (measurement: bench.py --workload)
    "train_bf16_d64": Workload("train_bf16_d64", 8, 4096, 32, 64, 64, "bf16", 1115),
    "train_fp32_d64": Workload("train_fp32_d64", 8, 4096, 32, 64, 64, "f32", 1116),
}


def get_workload(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    return EXTRA[name]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest-even bf16, returned as fp32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already bf16-exact (as int16)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16).view(np.int16)


def varlen_lengths(rng: np.random.Generator, n: int, total: int, lo: int, hi: int) -> np.ndarray:
    """n lengths drawn U[lo, hi], rescaled to sum to `total`, rounded, clamped to
    [lo, hi]; the residual goes onto the sequences in order (still clamped)."""
    raw = rng.integers(lo, hi + 1, size=n).astype(np.float64)
    lens = np.clip(np.round(raw * (total / raw.sum())), lo, hi).astype(np.int64)
    resid = total - int(lens.sum())
    i = 0
    guard = 0
    while resid != 0:
        step = 1 if resid > 0 else -1
        cand = lens[i % n] + step
        if lo <= cand <= hi:
            lens[i % n] = cand
            resid -= step
        i += 1
        guard += 1
        if guard > 100 * n * (hi - lo + 1):
            raise ValueError("cannot fit lengths")
    if all(int(x) % CHUNK == 0 for x in lens):
        # make at least one chunk ragged: move one token between the first two
        if lens[0] - 1 >= lo and lens[1] + 1 <= hi:
            lens[0] -= 1
            lens[1] += 1
    return lens


def _l2norm(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-6))).astype(np.float32)


def make_inputs(wl: Workload) -> dict:
    rng = np.random.default_rng(wl.seed)
    TT, H, K, V = wl.tokens, wl.H, wl.K, wl.V
    if wl.varlen_seqs > 0:
        if wl.fixed_lengths is not None:
            lens = np.asarray(wl.fixed_lengths, dtype=np.int64)
            assert int(lens.sum()) == TT
        else:
            lens = varlen_lengths(rng, wl.varlen_seqs, TT, wl.varlen_min, wl.varlen_max)
        N = len(lens)
    else:
        lens = np.full(wl.B, wl.T, dtype=np.int64)
        N = wl.B
    cu = np.zeros(N + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)

    A_log = rng.uniform(wl.alog_lo, wl.alog_hi, size=H).astype(np.float32)
    q = rng.standard_normal((TT, H, K), dtype=np.float32)
    k = rng.standard_normal((TT, H, K), dtype=np.float32)
    if wl.qk_l2norm:
        q, k = q * np.float32(2.0), k * np.float32(0.5)
    else:
        q, k = _l2norm(q), _l2norm(k)
    v = rng.standard_normal((TT, H, V), dtype=np.float32)
    blog = rng.standard_normal((TT, H), dtype=np.float32)
    beta = (1.0 / (1.0 + np.exp(-blog.astype(np.float64)))).astype(np.float32)
    g_raw = rng.standard_normal((TT, H, K), dtype=np.float32)
    if wl.graw_mean != 0.0:
        g_raw = (g_raw + np.float32(wl.graw_mean)).astype(np.float32)
    dO = rng.standard_normal((TT, H, V), dtype=np.float32)
    h0 = None
    dht = None
    if wl.h0_std > 0:
        h0 = (rng.standard_normal((N, H, K, V), dtype=np.float32) * np.float32(wl.h0_std))
    if wl.dht_std > 0:
        dht = (rng.standard_normal((N, H, K, V), dtype=np.float32) * np.float32(wl.dht_std))
    dt_bias = None
    if wl.dt_bias_std > 0:  # drawn last: the other inputs do not depend on it
        dt_bias = rng.standard_normal((H, K), dtype=np.float32) * np.float32(wl.dt_bias_std)
    if wl.dtype == "bf16":
        q, k, v, dO = round_bf16(q), round_bf16(k), round_bf16(v), round_bf16(dO)
    return dict(name=wl.name, dtype=wl.dtype, B=wl.B, T=wl.T, H=H, K=K, V=V, N=N,
                chunk=CHUNK, cu_seqlens=cu, lens=lens, varlen=wl.varlen_seqs > 0,
                q=q, k=k, v=v, dO=dO, g_raw=g_raw, beta=beta, A_log=A_log, h0=h0, dht=dht,
                dt_bias=dt_bias, gate_log2=wl.gate_log2, qk_l2norm=wl.qk_l2norm)


def with_variants(inp: dict, dt_bias=False, gate_log2=False, qk_l2norm=False) -> dict:
    """The same inputs with method variants switched on: a per-(head, channel) gate bias
    ~ N(0,1) from its own seeded stream, the gate in log2 units, q/k L2-normalised inside
    the method."""
    out = dict(inp)
    if dt_bias and out.get("dt_bias") is None:
        rng = np.random.default_rng(7001)
        out["dt_bias"] = rng.standard_normal((inp["H"], inp["K"]), dtype=np.float32)
    out["gate_log2"] = bool(out.get("gate_log2", False) or gate_log2)
    out["qk_l2norm"] = bool(out.get("qk_l2norm", False) or qk_l2norm)
    return out


def select_heads(inp: dict, heads) -> dict:
    """Restrict an input dict to a subset of heads (copies)."""
    heads = list(heads)
    out = dict(inp)
    for key in ("q", "k", "v", "dO", "g_raw", "beta"):
        out[key] = np.ascontiguousarray(inp[key][:, heads])
    out["A_log"] = np.ascontiguousarray(inp["A_log"][heads])
    for key in ("h0", "dht"):
        if inp[key] is not None:
            out[key] = np.ascontiguousarray(inp[key][:, heads])
    if inp.get("dt_bias") is not None:
        out["dt_bias"] = np.ascontiguousarray(inp["dt_bias"][heads])
    out["H"] = len(heads)
    return out


def select_seqs(inp: dict, seqs) -> dict:
    """Restrict an input dict to a subset of sequences (copies, repacked)."""
    seqs = list(seqs)
    cu = inp["cu_seqlens"]
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
    out = dict(inp)
    for key in ("q", "k", "v", "dO", "g_raw", "beta"):
        out[key] = np.ascontiguousarray(inp[key][idx])
    lens = np.asarray([cu[s + 1] - cu[s] for s in seqs], dtype=np.int64)
    ncu = np.zeros(len(seqs) + 1, dtype=np.int64)
    ncu[1:] = np.cumsum(lens)
    out["cu_seqlens"] = ncu
    out["lens"] = lens
    out["N"] = len(seqs)
    for key in ("h0", "dht"):
        if inp[key] is not None:
            out[key] = np.ascontiguousarray(inp[key][seqs])
    out["varlen"] = True
    return out
