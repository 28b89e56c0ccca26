"""Host-side checks of bench.py (no GPU): the one-GPU guard, the parsing of
rocprofv3 counter files, the copy-probe calibration of HBM traffic, and the
per-source-hash lookup of the stored traffic record."""
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

pytestmark = pytest.mark.cpu

HEADER = ("Correlation_Id,Dispatch_Id,Agent_Id,Queue_Id,Process_Id,Thread_Id,Grid_Size,"
          "Kernel_Id,Kernel_Name,Workgroup_Size,LDS_Block_Size,Scratch_Size,VGPR_Count,"
          "Accum_VGPR_Count,SGPR_Count,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n")


def write_counters(folder, rows):
    os.makedirs(os.path.join(folder, "host"), exist_ok=True)
    with open(os.path.join(folder, "host", "p_counter_collection.csv"), "w") as f:
        f.write(HEADER)
        for i, (kernel, counter, value) in enumerate(rows):
            f.write(f'{i},{i},"Agent 1",1,1,1,64,1,"{kernel}",64,0,0,8,0,8,'
                    f'"{counter}",{value},0,1\n')


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counter_mean_over_matching_dispatches(tmp_path):
    d = tmp_path / "af"
    write_counters(str(d), [("void attn_fwd_fast16<128>", "FETCH_SIZE", 100.0),
                            ("void attn_fwd_fast16<128>", "FETCH_SIZE", 300.0),
                            ("elementwise_copy", "FETCH_SIZE", 7.0),
                            ("void attn_fwd_fast16<128>", "WRITE_SIZE", 5.0)])
    assert bench.pmc_per_dispatch(str(d), "FETCH_SIZE", lambda k: "attn_fwd" in k) == 200.0
    assert bench.pmc_per_dispatch(str(d), "FETCH_SIZE", lambda k: "attn_fwd" not in k) == 7.0
    with pytest.raises(SystemExit):
        bench.pmc_per_dispatch(str(d), "GRBM_COUNT", lambda k: True)


def test_record_and_lookup_traffic(tmp_path, monkeypatch):
    src = tmp_path / "kernels.hip"
    src.write_text("int v = 1; // kernel source v1\n")
    traffic = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    mib = 64
    copy_bytes = (mib << 20) // (4 * 16384) * 16384 * 4
    # the copy reads half its bytes by FETCH_SIZE and all of them by WRITE_SIZE
    write_counters(str(tmp_path / "cf"), [("copy", "FETCH_SIZE", copy_bytes / 2048.0)])
    write_counters(str(tmp_path / "cw"), [("copy", "WRITE_SIZE", copy_bytes / 1024.0)])
    write_counters(str(tmp_path / "af"), [("attn_fwd_fast16", "FETCH_SIZE", 1000.0)])
    write_counters(str(tmp_path / "aw"), [("attn_fwd_fast16", "WRITE_SIZE", 250.0)])
    args = types.SimpleNamespace(workload="bf16_b1h32_s16384_d128_causal", copy_mib=mib,
                                 record_traffic=[str(tmp_path / x) for x in ("af", "aw", "cf", "cw")])
    assert bench.record_traffic(args) == 0
    rec = json.loads(traffic.read_text())["bf16_b1h32_s16384_d128_causal"]
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["read_bytes"] == 2 * 1000 * 1024
    assert rec["write_bytes"] == 250 * 1024
    assert bench.stored_traffic("bf16_b1h32_s16384_d128_causal") == 2 * 1000 * 1024 + 250 * 1024
    # an edit of comments only keeps the record; a changed kernel invalidates it
    src.write_text("int v = 1;   // the same code, another comment\n")
    assert bench.stored_traffic("bf16_b1h32_s16384_d128_causal") == 2 * 1000 * 1024 + 250 * 1024
    src.write_text("int v = 2; // kernel source v2\n")
    assert bench.stored_traffic("bf16_b1h32_s16384_d128_causal") is None
    assert bench.stored_traffic("no_such_workload") is None


@pytest.mark.parametrize("S_q", [2048, 4096, 16384])
def test_sample_rows_visit_every_row_position_of_a_wave(S_q):
    """The full-size row samples see each of the 32 row positions of a wave
    (a wave owns 32 consecutive query rows), and the stride-67 subsample of
    the 16k fp8 test does too."""
    from tiled_scaled_dot_amd.workloads import sample_rows

    samples = [sample_rows(S_q)] + ([sample_rows(S_q, stride=67)] if S_q >= 67 * 32 else [])
    for rows in samples:
        assert {r % 32 for r in rows} == set(range(32))
        assert {0, 1, S_q - 1} <= set(rows)
        assert all(0 <= r < S_q for r in rows) and rows == sorted(set(rows))


def test_counter_summary_clock_and_busy_fractions(tmp_path, capsys):
    """GRBM_COUNT summed over 8 XCDs over a 1 ms dispatch of 1.5e6 cycles per
    XCD is a 1500 MHz clock; the MFMA busy and MOPS counters turn into the
    pipe's busy fraction and the rate against the peak at that clock."""
    d = tmp_path / "pmc"
    os.makedirs(d / "host")
    with open(d / "host" / "p_agent_info.csv", "w") as f:
        f.write("Agent_Type,Num_Xcc,Simd_Count,Array_Count\nCPU,1,0,0\nGPU,8,1024,32\n")
    cycles = 1.5e6
    counters = {"GRBM_COUNT": 8 * cycles, "GRBM_GUI_ACTIVE": 8 * cycles * 0.9,
                "SQ_VALU_MFMA_BUSY_CYCLES": 1024 * cycles * 0.5,
                "SQ_BUSY_CYCLES": 32 * cycles * 0.8,
                "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1024 * cycles * 0.5 * 2}
    with open(d / "host" / "p_counter_collection.csv", "w") as f:
        f.write(HEADER)
        for disp in (1, 2):
            for name, value in counters.items():
                f.write(f'{disp},{disp},"Agent 1",1,1,1,64,1,"attn_fwd_fast16",64,0,0,8,0,8,'
                        f'"{name}",{value},0,1000000\n')
    assert bench.counter_summary(str(d), skip=1) == 0
    r = json.loads(capsys.readouterr().out)["attn_fwd_fast16"]
    assert r["dispatches"] == 1 and r["mean_ns"] == 1000000
    assert r["clock_mhz"] == pytest.approx(1500.0)
    assert r["gui_active"] == pytest.approx(0.9)
    assert r["mfma_busy"] == pytest.approx(0.5)
    assert r["sq_busy"] == pytest.approx(0.8)
    # half of 1024 SIMDs x 1024 FLOP/clk at 1.5 GHz
    assert r["mfma_tflops_bf16"] == pytest.approx(1024 * 1024 * 1.5e9 * 0.5 / 1e12, rel=1e-3)
    assert r["pct_of_bf16_peak_at_clock"] == pytest.approx(50.0 * 2516.6 / 2516.58, rel=1e-3)


def test_trace_summary_back_to_back_window(tmp_path, capsys):
    """The trace summary averages every dispatch and, separately, the last N
    (the back-to-back block bench.py times), in start-time order."""
    d = tmp_path / "trace" / "host"
    os.makedirs(d)
    with open(d / "s_kernel_trace.csv", "w") as f:
        f.write("Kind,Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp,Grid_Size_X,"
                "Workgroup_Size_X\n")
        # rows out of order on purpose; durations 400 (first), then 100, 100, 200, 200
        for i, (start, dur) in enumerate([(50, 200), (0, 400), (10, 100), (60, 200), (20, 100)]):
            f.write(f"KERNEL_DISPATCH,{i},attn_fwd_fast16,{start},{start + dur},1024,512\n")
    assert bench.trace_summary(str(tmp_path / "trace"), last=2) == 0
    r = json.loads(capsys.readouterr().out)["attn_fwd_fast16"]
    assert r["dispatches"] == 5 and r["mean_ns"] == 200
    assert r["min_ns"] == 100 and r["max_ns"] == 400
    assert r["mean_ns_last_2"] == 200
    assert r["workgroups"] == 2 and r["threads"] == 512
