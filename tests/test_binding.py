"""The Python binding rejects malformed tensors before anything reaches the library.

CPU only: the tensors here live in host memory, so a call that passed every
shape, dtype and layout check would stop at the device check.  The library is
replaced by a stub that fails the test if it is touched, so every error below is
raised before any library call (and therefore before any launch).
"""
import pytest

torch = pytest.importorskip("torch")

import linear_attention_backward_amd as K  # noqa: E402


@pytest.fixture(autouse=True)
def _no_library(monkeypatch):
    def boom(*a, **k):
        raise AssertionError("the library was reached")
    monkeypatch.setattr(K, "load_library", boom)


B, T, H, D = 2, 70, 3, 64
NC = B * ((T + 63) // 64)


def _args(act=torch.bfloat16):
    f = torch.float32
    return dict(q=torch.zeros(B, T, H, D, dtype=act), k=torch.zeros(B, T, H, D, dtype=act),
                v=torch.zeros(B, T, H, D, dtype=act), g_raw=torch.zeros(B, T, H, D, dtype=f),
                beta=torch.zeros(B, T, H, dtype=f), A_log=torch.zeros(H, dtype=f),
                dO=torch.zeros(B, T, H, D, dtype=act), h0=torch.zeros(B, H, D, D, dtype=f),
                dht=torch.zeros(B, H, D, D, dtype=f),
                h_saved=torch.zeros(NC, H, D, D, dtype=act))


def _bwd(a):
    return K.kda_bwd(a["q"], a["k"], a["v"], a["g_raw"], a["beta"], a["A_log"], a["dO"],
                     h0=a["h0"], dht=a["dht"], h_saved=a["h_saved"],
                     dt_bias=a.get("dt_bias"))


def _fwd(a):
    return K.kda_fwd(a["q"], a["k"], a["v"], a["g_raw"], a["beta"], a["A_log"], h0=a["h0"],
                     dt_bias=a.get("dt_bias"))


@pytest.mark.parametrize("act", [torch.bfloat16, torch.float32])
def test_well_formed_host_tensors_stop_at_device_check(act):
    for call in (_bwd, _fwd):
        with pytest.raises(ValueError, match="on the GPU"):
            call(_args(act))


BAD = [
    # (what, mutate, message)
    ("g_raw bf16", lambda a: a.update(g_raw=a["g_raw"].bfloat16()), "g_raw must be"),
    ("beta fp64", lambda a: a.update(beta=a["beta"].double()), "beta must be"),
    ("A_log bf16", lambda a: a.update(A_log=a["A_log"].bfloat16()), "A_log must be"),
    ("h0 bf16", lambda a: a.update(h0=a["h0"].bfloat16()), "h0 must be"),
    ("k fp32 with bf16 q", lambda a: a.update(k=a["k"].float()), "k must be"),
    ("v fp32 with bf16 q", lambda a: a.update(v=a["v"].float()), "v must be"),
    ("fp16 activations", lambda a: [a.update({n: a[n].half()}) for n in ("q", "k", "v", "dO")],
     "bfloat16 or float32"),
    ("k shorter", lambda a: a.update(k=a["k"][:, :T - 1].contiguous()), "k must have shape"),
    ("beta with a channel axis", lambda a: a.update(beta=torch.zeros(B, T, H, 1)),
     "beta must have shape"),
    ("A_log per channel", lambda a: a.update(A_log=torch.zeros(H, D)), "A_log must have shape"),
    ("h0 one sequence short", lambda a: a.update(h0=torch.zeros(B - 1, H, D, D)),
     "h0 must have shape"),
    ("dt_bias per head only", lambda a: a.update(dt_bias=torch.zeros(H)), "dt_bias must have"),
    ("q transposed view", lambda a: a.update(q=a["q"].transpose(0, 1).contiguous()
                                            .transpose(0, 1)), "q must be contiguous"),
    ("g_raw strided", lambda a: a.update(g_raw=torch.zeros(B, T, H, 2 * D)[..., ::2]),
     "g_raw must be contiguous"),
]


@pytest.mark.parametrize("what,mutate,msg", BAD, ids=[b[0] for b in BAD])
def test_bad_argument_raises_before_library(what, mutate, msg):
    a = _args()
    mutate(a)
    for call in (_bwd, _fwd):
        with pytest.raises((ValueError, TypeError), match=msg):
            call(a)


@pytest.mark.parametrize("what,mutate,msg", [
    ("dO fp32", lambda a: a.update(dO=a["dO"].float()), "dO must be"),
    ("dht fp64", lambda a: a.update(dht=a["dht"].double()), "dht must be"),
    ("dht shape", lambda a: a.update(dht=torch.zeros(B, H, D, D + 1)), "dht must have shape"),
    ("h_saved one chunk short", lambda a: a.update(h_saved=a["h_saved"][1:].contiguous()),
     "h_saved must have shape"),
    ("h_saved fp32 with bf16 q", lambda a: a.update(h_saved=a["h_saved"].float()),
     "h_saved must be"),
], ids=["dO fp32", "dht fp64", "dht shape", "h_saved short", "h_saved fp32"])
def test_backward_only_arguments(what, mutate, msg):
    a = _args()
    mutate(a)
    with pytest.raises(ValueError, match=msg):
        _bwd(a)


def test_packed_sequences_shapes():
    """Packed [T, H, D] activations with cu_seqlens: h_saved holds one state per chunk of
    every sequence (ragged ends count as a chunk)."""
    cu = [0, 1, 66, 130]
    nc = 1 + 2 + 1
    f = torch.float32
    a = dict(q=torch.zeros(130, H, D, dtype=torch.bfloat16), g_raw=torch.zeros(130, H, D),
             beta=torch.zeros(130, H), A_log=torch.zeros(H),
             h_saved=torch.zeros(nc, H, D, D, dtype=torch.bfloat16))
    a["k"], a["v"], a["dO"] = a["q"].clone(), a["q"].clone(), a["q"].clone()
    call = lambda hs: K.kda_bwd(a["q"], a["k"], a["v"], a["g_raw"], a["beta"], a["A_log"],
                                a["dO"], h0=torch.zeros(3, H, D, D, dtype=f), h_saved=hs,
                                cu_seqlens=cu)
    with pytest.raises(ValueError, match="on the GPU"):
        call(a["h_saved"])
    with pytest.raises(ValueError, match="h_saved must have shape"):
        call(torch.zeros(nc + 1, H, D, D, dtype=torch.bfloat16))
