"""Host-side tools that need no GPU: the HBM-byte summariser that turns
rocprofv3 FETCH_SIZE / WRITE_SIZE runs into the per-launch traffic bench.py
reports, and the build's check for kernel launch stubs."""

import csv
import json
import os
import subprocess

import pytest

from exact_tiled_attention_13_amd import build as build_mod
from exact_tiled_attention_13_amd import traffic

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_run(root, stage, counter, rows):
    d = os.path.join(root, f"pmc_{stage}_{counter}")
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for disp, kernel, value in rows:
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": kernel, "Counter_Name": counter,
                        "Counter_Value": value})


def _fake_profile(root):
    """Copy: FETCH_SIZE reads half of the 262144 KiB copied, WRITE_SIZE all of
    it; a fill kernel in the same run must be ignored. Each attention stage:
    three launches of its kernel (one split over two counter instances, as
    rocprofv3 reports per-XCD blocks), plus a forward launch in the backward
    stages that must be ignored."""
    copy = "__amd_rocclr_copyBuffer"
    _write_run(root, "copy", "FETCH_SIZE", [(1, "__amd_rocclr_fillBufferAligned", 0.0)]
               + [(i, copy, 131072.0) for i in (2, 3, 4)])
    _write_run(root, "copy", "WRITE_SIZE", [(1, "__amd_rocclr_fillBufferAligned", 262144.0)]
               + [(i, copy, 262144.0) for i in (2, 3, 4)])
    values = {"fwd": (1000.0, 300.0), "bwd_dq_prep": (2000.0, 400.0), "bwd_dkdv": (3000.0, 600.0)}
    for stage, (kernel, _) in traffic.STAGES.items():
        f, w = values[stage]
        for counter, v in (("FETCH_SIZE", f), ("WRITE_SIZE", w)):
            rows = [(1, "void fa::fwd_bf16_kernel<128, false, 8>(fa::FwdArgs)", 99999.0)] if stage != "fwd" else []
            name = f"void {kernel}(fa::Args)"
            rows += [(2, name, v / 2), (2, name, v / 2), (3, name, v), (4, name, v)]
            _write_run(root, stage, counter, rows)
    return values


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path):
    values = _fake_profile(str(tmp_path))
    s = traffic.summarise(str(tmp_path))
    assert s["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert s["calibration"]["write_scale"] == pytest.approx(1.0)
    for stage, (kernel, name) in traffic.STAGES.items():
        e = s["kernels"][name]
        f, w = values[stage]
        assert e["fetch_kib"] == pytest.approx(f)
        assert e["write_kib"] == pytest.approx(w)
        assert e["hbm_bytes"] == pytest.approx(1024.0 * (2.0 * f + w))
        assert e["source_sha256"] == traffic.kernel_source_hash(name)
        assert e["kernel"] == kernel.split("::")[1]


def test_traffic_cli_writes_json(tmp_path):
    _fake_profile(str(tmp_path))
    out = tmp_path / "t.json"
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    subprocess.run(["python3", "-m", "exact_tiled_attention_13_amd.traffic", str(tmp_path), "--out", str(out)],
                   check=True, cwd=root, capture_output=True)
    d = json.loads(out.read_text())
    assert set(d["kernels"]) == {name for _, name in traffic.STAGES.values()}


def test_traffic_missing_run_is_an_error(tmp_path):
    with pytest.raises(FileNotFoundError):
        traffic.summarise(str(tmp_path))


def test_source_hash_separates_forward_and_backward():
    hf, hb = traffic.kernel_source_hash("fwd_noncausal"), traffic.kernel_source_hash("bwd_dq_prep_noncausal")
    assert len(hf) == 64 and len(hb) == 64 and hf != hb
    assert traffic.kernel_source_hash("bwd_dkdv_noncausal") == hb


def test_stub_check_passes_on_the_built_library():
    if not os.path.exists(build_mod.LIB):
        pytest.skip("library not built")
    build_mod._check_stubs(build_mod.LIB)
