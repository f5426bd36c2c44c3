"""The C ABI on the CPU: the library loads, exports every function kda.h
declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import linear_attention_backward_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    return sorted(set(re.findall(r"KDA_API\s+[\w\s\*]*?\b(kda_\w+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = K.load_library()
    names = _declared()
    assert len(names) >= 8, names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings():
    assert K.abi_version() == 3
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(K.status_string(code), str) and K.status_string(code)


def _ws(prob, which=K.KDA_WS_BWD):
    n = ctypes.c_size_t(0)
    st = K.load_library().kda_workspace_size(prob.ref(), which, ctypes.byref(n))
    return st, n.value


def test_shape_validation():
    ok = K._Prob(2, 100, 4, 128, 128, K.KDA_DTYPE_BF16)
    st, n = _ws(ok)
    assert st == 0 and n > 0
    assert _ws(K._Prob(2, 100, 4, 96, 96, K.KDA_DTYPE_BF16))[0] == K.KDA_ERR_UNSUPPORTED
    assert _ws(K._Prob(2, 100, 4, 128, 64, K.KDA_DTYPE_BF16))[0] == K.KDA_ERR_UNSUPPORTED
    assert _ws(K._Prob(2, 100, 4, 128, 128, K.KDA_DTYPE_F32))[0] == K.KDA_ERR_UNSUPPORTED
    assert _ws(K._Prob(2, 100, 4, 64, 64, 7))[0] == K.KDA_ERR_UNSUPPORTED
    assert _ws(K._Prob(0, 100, 4, 64, 64, 0))[0] == K.KDA_ERR_INVALID_ARGUMENT
    assert _ws(K._Prob(1, 100, 0, 64, 64, 0))[0] == K.KDA_ERR_INVALID_ARGUMENT
    # token-head rows past 32-bit indexing
    assert _ws(K._Prob(1, 1 << 24, 127, 64, 64, 0))[0] == 0
    assert _ws(K._Prob(1, 1 << 24, 128, 64, 64, 0))[0] == K.KDA_ERR_UNSUPPORTED
    assert _ws(K._Prob(4, 1 << 22, 128, 64, 64, 0))[0] == K.KDA_ERR_UNSUPPORTED
    # a token row of fp32 (H * K * 4 bytes) at or past 2^24 bytes
    assert _ws(K._Prob(1, 64, (1 << 15) - 1, 128, 128, K.KDA_DTYPE_BF16))[0] == 0
    assert _ws(K._Prob(1, 64, 1 << 15, 128, 128, K.KDA_DTYPE_BF16))[0] == K.KDA_ERR_UNSUPPORTED
    p = K._Prob(1, 100, 4, 64, 64, 0)
    p.p.chunk = 32
    assert _ws(p)[0] == K.KDA_ERR_UNSUPPORTED
    n = ctypes.c_size_t(0)
    assert K.load_library().kda_workspace_size(ok.ref(), 5, ctypes.byref(n)) == -1
    assert _ws(K._Prob(2, 100, 4, 128, 128, K.KDA_DTYPE_BF16, gate_units=K.KDA_GATE_LOG2))[0] == 0
    bad = K._Prob(2, 100, 4, 128, 128, K.KDA_DTYPE_BF16)
    bad.p.gate_units = 2
    assert _ws(bad)[0] == K.KDA_ERR_INVALID_ARGUMENT
    bad = K._Prob(2, 100, 4, 128, 128, K.KDA_DTYPE_BF16, qk_l2norm=2)
    assert _ws(bad)[0] == K.KDA_ERR_INVALID_ARGUMENT
    # the q/k L2 norm: kda_bwd and kda_fwd normalise inside their kernels (no extra
    # workspace); the reference forward keeps normalised copies and reciprocal norms
    for which in (K.KDA_WS_BWD, K.KDA_WS_FWD):
        plain = _ws(K._Prob(2, 100, 4, 128, 128, K.KDA_DTYPE_BF16), which)[1]
        normed = _ws(K._Prob(2, 100, 4, 128, 128, K.KDA_DTYPE_BF16, qk_l2norm=1), which)[1]
        assert normed == plain, which
    ref_plain = _ws(K._Prob(2, 100, 4, 128, 128, K.KDA_DTYPE_BF16), K.KDA_WS_FWD_REF)[1]
    ref_normed = _ws(K._Prob(2, 100, 4, 128, 128, K.KDA_DTYPE_BF16, qk_l2norm=1),
                     K.KDA_WS_FWD_REF)[1]
    assert ref_normed >= ref_plain + 2 * 200 * 4 * 128 * 2 + 2 * 200 * 4 * 4
    for T in (1, 64, 1000):  # the production forward's workspace also serves kda_fwd_ref
        for qn in (0, 1):
            p = K._Prob(2, T, 4, 128, 128, K.KDA_DTYPE_BF16, qk_l2norm=qn)
            assert _ws(p, K.KDA_WS_FWD)[1] >= _ws(p, K.KDA_WS_FWD_REF)[1]


def test_cu_seqlens_validation():
    fake_dev = ctypes.c_void_p(16)  # never dereferenced: validation fails or no launch happens
    def prob(cu, T, B=1):
        p = K._Prob(B, T, 2, 64, 64, K.KDA_DTYPE_F32, cu, None)
        p.p.cu_seqlens_dev = fake_dev
        return p
    assert _ws(prob([0, 10, 100], 100))[0] == 0
    assert _ws(prob([0, 10, 100], 101))[0] == K.KDA_ERR_INVALID_ARGUMENT  # sum != T
    assert _ws(prob([0, 50, 40, 100], 100))[0] == K.KDA_ERR_INVALID_ARGUMENT  # not monotone
    assert _ws(prob([1, 10, 100], 100))[0] == K.KDA_ERR_INVALID_ARGUMENT  # cu[0] != 0
    assert _ws(prob([0, 10, 100], 100, B=2))[0] == K.KDA_ERR_INVALID_ARGUMENT
    host_only = K._Prob(1, 100, 2, 64, 64, 0, [0, 10, 100], None)
    assert _ws(host_only)[0] == K.KDA_ERR_INVALID_ARGUMENT  # host copy without device copy


def test_num_chunks_and_workspace_monotone():
    nc = ctypes.c_int64(0)
    p = K._Prob(1, 1 + 63 + 64 + 65 + 0, 2, 64, 64, 0, [0, 1, 64, 128, 193, 193], None)
    p.p.cu_seqlens_dev = ctypes.c_void_p(16)
    assert K.load_library().kda_num_chunks(p.ref(), ctypes.byref(nc)) == 0
    assert nc.value == 1 + 1 + 1 + 2 + 0
    sizes = [_ws(K._Prob(1, T, 4, 128, 128, 1))[1] for T in (64, 128, 1000, 4096)]
    assert sizes == sorted(sizes)
    assert _ws(K._Prob(1, 64, 4, 128, 128, 1), K.KDA_WS_FWD)[1] <= sizes[0]


def test_bwd_rejects_bad_calls_without_launching():
    lib = K.load_library()
    p = K._Prob(1, 64, 2, 64, 64, K.KDA_DTYPE_F32)
    # NULL io
    assert lib.kda_bwd(p.ref(), None, None, 0, None) == K.KDA_ERR_INVALID_ARGUMENT
    io = K.BwdIO()
    assert lib.kda_bwd(p.ref(), ctypes.byref(io), None, 0, None) == K.KDA_ERR_INVALID_ARGUMENT
    # misaligned pointer
    al = 256
    for f in ("q", "k", "v", "g_raw", "beta", "A_log", "dO", "dq", "dk", "dv", "dg_raw", "dbeta",
              "dA_log"):
        setattr(io, f, al)
    io.q = 258
    assert lib.kda_bwd(p.ref(), ctypes.byref(io), None, 0, None) == K.KDA_ERR_INVALID_ARGUMENT
    io.q = 256
    io.dt_bias = 264  # the gate bias is read in 16-byte pieces
    assert lib.kda_bwd(p.ref(), ctypes.byref(io), None, 0, None) == K.KDA_ERR_INVALID_ARGUMENT
    io.dt_bias = None
    io.ddt_bias = 258
    assert lib.kda_bwd(p.ref(), ctypes.byref(io), None, 0, None) == K.KDA_ERR_INVALID_ARGUMENT
    io.ddt_bias = None
    # workspace too small
    assert lib.kda_bwd(p.ref(), ctypes.byref(io), ctypes.c_void_p(256), 16, None) == \
        K.KDA_ERR_WORKSPACE_TOO_SMALL
    assert lib.kda_fwd_ref(p.ref(), None, None, 0, None) == K.KDA_ERR_INVALID_ARGUMENT


def test_binding_raises_on_error():
    with pytest.raises(K.KdaError):
        K._check(K.KDA_ERR_UNSUPPORTED)


def test_aliasing_rejected_without_launching():
    """Outputs may not overlap inputs, other outputs or the workspace (every call below
    is rejected during validation, so none of these fake addresses is ever used)."""
    lib = K.load_library()
    p = K._Prob(1, 64, 2, 64, 64, K.KDA_DTYPE_F32)
    st, need = _ws(p)
    assert st == 0
    base, step = 1 << 32, 1 << 28
    fields = ("q", "k", "v", "g_raw", "beta", "A_log", "dO", "dq", "dk", "dv", "dg_raw",
              "dbeta", "dA_log", "dh0", "h0", "dht")
    ws = base + len(fields) * step

    def io_with(**over):
        io = K.BwdIO()
        for i, f in enumerate(fields):
            setattr(io, f, base + i * step)
        for f, val in over.items():
            setattr(io, f, val)
        return io

    addr = {f: base + i * step for i, f in enumerate(fields)}
    for over in (dict(dq=addr["q"]),                       # output on an input
                 dict(dv=addr["dO"] + 4096),               # partly on an input
                 dict(dk=addr["dq"]),                      # two outputs
                 dict(dA_log=addr["dbeta"] + 16),
                 dict(dh0=addr["h0"]),
                 dict(dg_raw=ws),                          # output in the workspace
                 dict(beta=ws + 256)):                     # input in the workspace
        io = io_with(**over)
        assert lib.kda_bwd(p.ref(), ctypes.byref(io), ctypes.c_void_p(ws), need, None) == \
            K.KDA_ERR_INVALID_ARGUMENT, over
    fio = K.FwdIO()
    for i, f in enumerate(("q", "k", "v", "g_raw", "beta", "A_log", "h0", "o", "ht",
                           "h_saved")):
        setattr(fio, f, base + i * step)
    fio.o = fio.v  # the output o on the input v
    st, need_f = _ws(p, K.KDA_WS_FWD)
    for entry in ("kda_fwd", "kda_fwd_ref"):
        assert getattr(lib, entry)(p.ref(), ctypes.byref(fio), ctypes.c_void_p(ws), need_f,
                                   None) == K.KDA_ERR_INVALID_ARGUMENT, entry


def test_noalloc_rejects_oversized_without_launching():
    """kda_bwd_noalloc refuses a problem whose workspace exceeds its static scratch
    before it looks anything up on a device."""
    lib = K.load_library()
    io = K.BwdIO()
    io.h_saved = 256
    big = K._Prob(8, 4096, 32, 128, 128, K.KDA_DTYPE_BF16)
    assert lib.kda_bwd_noalloc(big.ref(), ctypes.byref(io), None) == K.KDA_ERR_SCRATCH_TOO_SMALL
    assert "scratch" in K.status_string(K.KDA_ERR_SCRATCH_TOO_SMALL)
    assert lib.kda_bwd_noalloc(big.ref(), None, None) == K.KDA_ERR_INVALID_ARGUMENT
    bad = K._Prob(8, 4096, 32, 96, 96, K.KDA_DTYPE_BF16)
    assert lib.kda_bwd_noalloc(bad.ref(), ctypes.byref(io), None) == K.KDA_ERR_UNSUPPORTED
