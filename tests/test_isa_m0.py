"""The global -> LDS copies set M0 in inline asm without telling the compiler (listing M0
as clobbered is rejected by the backend), so they rely on the compiler keeping nothing in
M0 in these kernels.  This test checks that invariant on the library's own gfx950 code
objects after every build: the only instructions that name M0 are the copy sequence
`s_mov_b32 m0, s<n>; s_nop 0; global_load_lds_dwordx4`, every global_load_lds is the
third instruction of such a sequence, and no instruction that reads M0 implicitly
appears at all (relative moves, messages, GWS and ordered counts, LDS-append/consume,
interpolation, lane-addressed LDS).  A compiler or source change that breaks it fails
here instead of corrupting tiles silently.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "linear_attention_backward_amd", "libkda.so")
OBJDUMP = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "llvm-objdump")

# instructions that read M0 without naming it
IMPLICIT_M0 = re.compile(r"^(s_movrel|v_movrel|s_sendmsg|ds_gws|ds_ordered_count|ds_append|"
                         r"ds_consume|v_interp|ds_read_addtid|ds_write_addtid|s_ttracedata|"
                         r"buffer_load_lds|buffer_store_lds|global_load_lds|s_buffer_load_lds)")


def _instructions(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("libkda.so not built")
    if not os.path.exists(OBJDUMP):
        pytest.skip("llvm-objdump not available")
    lib = tmp_path / "libkda.so"
    shutil.copy(LIB, lib)
    subprocess.run([OBJDUMP, "--offloading", str(lib)], cwd=tmp_path, check=True,
                   capture_output=True)
    objs = sorted(p for p in os.listdir(tmp_path) if p.endswith("gfx950"))
    assert objs, "no gfx950 code object in libkda.so"
    out = {}
    for o in objs:
        dis = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", str(tmp_path / o)],
                             capture_output=True, text=True, check=True).stdout
        ins = []
        for line in dis.splitlines():
            line = line.split("//")[0].strip()
            if not line or line.endswith(":") or line.startswith("Disassembly"):
                continue
            ins.append(line)
        out[o] = ins
    return out


def test_m0_only_in_copy_sequences(tmp_path):
    copies = 0
    for obj, ins in _instructions(tmp_path).items():
        for i, text in enumerate(ins):
            op = text.split()[0]
            names_m0 = re.search(r"\bm0\b", text) is not None
            if op.startswith("global_load_lds"):
                assert i >= 2 and re.fullmatch(r"s_mov_b32 m0, s\d+", ins[i - 2]) and \
                    ins[i - 1] == "s_nop 0", "%s: unguarded %s at %d" % (obj, text, i)
                copies += 1
                continue
            if names_m0:
                assert re.fullmatch(r"s_mov_b32 m0, s\d+", text) and i + 2 < len(ins) and \
                    ins[i + 1] == "s_nop 0" and ins[i + 2].startswith("global_load_lds"), \
                    "%s: M0 used outside a copy sequence: %s" % (obj, text)
                continue
            assert not IMPLICIT_M0.match(op), "%s: implicit M0 reader %s" % (obj, text)
    assert copies > 0, "no global -> LDS copies found (the check would be vacuous)"
