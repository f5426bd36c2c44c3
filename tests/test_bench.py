"""The benchmark's measurement arithmetic (CPU only): algorithmic bytes per token-head,
the profile digest's insensitivity to comments, and the HBM-traffic and SQ-counter
summaries computed from rocprofv3-style CSVs (synthetic rows with known answers)."""
import csv
import json

import pytest

import bench


def test_algorithmic_bytes_per_token_head():
    # bf16, K = V = 128: q, k, v, dO (4 x 256 B) + g_raw (512 B) + beta (4 B) in, S_in and
    # dS_out (2 x 32 KiB per 64 tokens = 2 x 512 B), dq, dk, dv (3 x 256 B) + dg_raw (512 B)
    # + dbeta (4 B) out
    k = bench.kernel_bytes_per_token_head(128, 2, fused=True)
    assert k["grad"] == 4 * 256 + 512 + 4 + 2 * 512 + 3 * 256 + 512 + 4 == 3848
    assert k["prep"] == 512 and bench.kernel_bytes_per_token_head(128, 2)["scan"] == 512
    assert bench.path_bytes_per_token_head(128, 2) == 3848 + 512
    # the per-chunk MFMA count: 7 state contractions, 5.5 causal C x C x D, the inverse
    assert bench.path_flops_per_chunk_head(128, 64) == 7 * 64 * 128 * 128 * 2 + \
        5.5 * 64 * 64 * 128 * 2 + 2 * 64 ** 3 / 3


def test_code_only_ignores_comments_and_whitespace():
    a = "int x = 1; // one\n/* block\n comment */ float  y;\n"
    b = "int x = 1;\n\n  float y;   // changed comment\n"
    assert bench._code_only(a) == bench._code_only(b) == "int x = 1; float y;"
    assert bench._code_only("a = b;") != bench._code_only("a = c;")


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for r in rows:
            wr.writerow(dict(zip(["Kernel_Name", "Counter_Name", "Counter_Value"], r)))


GRAD = "_ZN3kda7k_gradfIDF16bLi128ELb0ELb0ELb1EEEvPKNS_9ChunkInfoEii"
PREP = "_ZN3kda6k_prepIDF16bLi128ELb0ELb0ELb0ELb1EEEvPKNS_9ChunkInfo"


def test_traffic_summary(tmp_path):
    # a 1 MiB copy that reads FETCH = 512 KiB (scale 2) and WRITE = 1024 KiB (scale 1)
    _write_csv(tmp_path / "cf.csv", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0)] * 3)
    _write_csv(tmp_path / "cw.csv", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0)] * 3)
    _write_csv(tmp_path / "f.csv", [(GRAD, "FETCH_SIZE", 100.0), (GRAD, "FETCH_SIZE", 300.0),
                                    (PREP, "FETCH_SIZE", 50.0), ("other", "FETCH_SIZE", 9e9)])
    _write_csv(tmp_path / "w.csv", [(GRAD, "WRITE_SIZE", 40.0), (PREP, "WRITE_SIZE", 10.0)])
    out = bench.summarize_profiles(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                   str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), 1,
                                   out_path=str(tmp_path / "traffic.json"))
    assert out["fetch_scale"] == 2.0 and out["write_scale"] == 1.0
    g = out["kernels"]["grad"]
    assert g["read_bytes"] == 200.0 * 1024 * 2 and g["write_bytes"] == 40.0 * 1024
    assert g["bytes_per_launch"] == g["read_bytes"] + g["write_bytes"]
    assert out["kernels"]["prep"]["read_bytes"] == 50.0 * 1024 * 2
    assert json.load(open(tmp_path / "traffic.json"))["sources"] == bench.kernel_sources_digest()


def test_counter_summary(tmp_path):
    cyc = 1000.0
    _write_csv(tmp_path / "sq.csv", [
        (GRAD, "GRBM_GUI_ACTIVE", cyc * bench.N_XCD),
        (GRAD, "SQ_ACTIVE_INST_VALU", 0.5 * bench.CU_NUM * cyc),
        (GRAD, "SQ_VALU_MFMA_BUSY_CYCLES", 0.1 * bench.SIMD_NUM * cyc),
        (GRAD, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1000.0),
        (GRAD, "SQ_WAVE_CYCLES", 2.0 * bench.CU_NUM * cyc)])
    _write_csv(tmp_path / "lds.csv", [(GRAD, "SQ_LDS_BANK_CONFLICT", 30.0),
                                      (GRAD, "SQ_LDS_IDX_ACTIVE", 100.0)])
    out = bench.summarize_counters([str(tmp_path / "sq.csv"), str(tmp_path / "lds.csv")],
                                   out_path=str(tmp_path / "counters.json"))
    g = out["kernels"]["grad"]
    assert g["kernel_cycles"] == cyc
    assert g["valu_busy"] == pytest.approx(0.5) and g["mfma_busy"] == pytest.approx(0.1)
    assert g["waves_per_simd"] == pytest.approx(2.0)
    assert g["mfma_flop_per_launch"] == 512000.0
    assert g["lds_bank_conflict_frac"] == pytest.approx(0.3)


def test_gpu_count_other_than_one_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
