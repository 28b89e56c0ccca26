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
