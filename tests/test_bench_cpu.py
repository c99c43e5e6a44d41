"""Host-side logic of bench.py: the single-GPU guard and the traffic summary
written from rocprofv3 counter CSVs (synthetic CSVs here, no GPU)."""

import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_csv(d, counter, dispatches):
    """dispatches: list of (kernel name, [per-instance values]) in dispatch order."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        for i, (name, vals) in enumerate(dispatches, 1):
            for v in vals:  # one row per counter instance; the writer sums them
                row = {k: 0 for k in FIELDS}
                row.update(Dispatch_Id=i, Kernel_Name=name, Counter_Name=counter,
                           Counter_Value=f"{v:.6f}")
                w.writerow(row)


def test_traffic_summary_scales_by_the_copy(tmp_path, monkeypatch):
    bench = load_bench()
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    calls = ["quant_act_M1", "forward_M1"]
    probe = tmp_path / "probe.json"
    probe.write_text(json.dumps(dict(workload="gemv_k2048_n2048", calls=calls,
                                     copy_bytes=bench.COPY_BYTES, copy_kernel="neg")))
    kib = bench.COPY_BYTES / 1024
    setup = ("void at::native::fill_kernel(int)", [5.0])
    # the counters read the copy at half (fetch) and twice (write) its true size
    fetch = [setup, ("void bl::quant_rows_kernel<0, false, false>(int)", [3.0, 1.0]),
             ("void bl::gemv_valu_kernel<1, 4, 1>(int)", [512.0, 512.0]),
             setup, ("void at::native::neg_kernel(int)", [kib / 4, kib / 4])]
    # a torch kernel between the step and the copy is skipped
    write = [setup, ("void bl::quant_rows_kernel<0, false, false>(int)", [2.0]),
             ("void bl::gemv_valu_kernel<1, 4, 1>(int)", [16.0]), setup,
             ("void at::native::neg_kernel(int)", [2 * kib])]
    write_csv(tmp_path / "f", "FETCH_SIZE", fetch)
    write_csv(tmp_path / "w", "WRITE_SIZE", write)
    args = type("A", (), dict(traffic_write=[str(probe), str(tmp_path / "f"), str(tmp_path / "w")],
                              workload=1))()
    bench.traffic_write(args)
    out = (tmp_path / "traffic_gemv_k2048_n2048.md").read_text()
    assert f"source_digest: {bench.kernel_source_digest()}" in out
    # forward: 1024 KiB fetched x 2 + 16 KiB written x 0.5
    assert bench.read_traffic("gemv_k2048_n2048", "forward_M1") == pytest.approx(
        1024 * 1024 * 2 + 16 * 1024 * 0.5, rel=1e-5)
    assert bench.read_traffic("gemv_k2048_n2048", "quant_act_M1") == pytest.approx(
        4 * 1024 * 2 + 2 * 1024 * 0.5, rel=1e-5)
    # a summary taken on other kernel sources is not used
    (tmp_path / "traffic_gemv_k2048_n2048.md").write_text(
        out.replace(bench.kernel_source_digest(), "0" * 16))
    assert bench.read_traffic("gemv_k2048_n2048", "forward_M1") is None


def test_traffic_summary_rejects_a_run_without_the_copy(tmp_path, monkeypatch):
    bench = load_bench()
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    probe = tmp_path / "probe.json"
    probe.write_text(json.dumps(dict(workload="gemv_k2048_n2048", calls=["forward_M1"],
                                     copy_bytes=bench.COPY_BYTES, copy_kernel="neg")))
    rows = [("void bl::gemv_valu_kernel<1, 4, 1>(int)", [1.0]), ("void other(int)", [1.0])]
    write_csv(tmp_path / "f", "FETCH_SIZE", rows)
    write_csv(tmp_path / "w", "WRITE_SIZE", rows)
    args = type("A", (), dict(traffic_write=[str(probe), str(tmp_path / "f"), str(tmp_path / "w")],
                              workload=1))()
    with pytest.raises(SystemExit):
        bench.traffic_write(args)


def test_kernel_labels_follow_the_dispatch():
    """The roofline line names the kernel the library's dispatch picks."""
    bench = load_bench()
    # 1-bit: the LDS decode kernel from 5 tokens, and from 2 at K >= 4096
    assert bench.forward1_kernel(16, 4096) == "decode_lds_kernel"
    assert bench.forward1_kernel(4, 4096) == "decode_lds_kernel"
    assert bench.forward1_kernel(4, 2048) == "gemv1_kernel"
    assert bench.forward1_kernel(1, 8192) == "gemv1_kernel"
    # base-3: one pass on MFMA for 2..16 tokens whose staged block fits
    # 144 KB (16 tokens: K = 8960 fits, K = 8976 does not)
    assert bench.forward3_kernel(16, 8960) == "gemv3_mfma_kernel"
    assert bench.forward3_kernel(16, 8976) == "gemv3_kernel"
    assert bench.forward3_kernel(1, 4096) == "gemv3_kernel"
    assert bench.forward3_kernel(2, 4096) == "gemv3_mfma_kernel"
    assert bench.forward3_kernel(17, 1024) == "gemv3_kernel"
    # 2-bit: GEMV for one token, the LDS decode kernel at decode sizes, GEMM
    assert bench.forward_kernel(1, 4096, 11008) == "gemv_valu_kernel"
    assert bench.forward_kernel(16, 4096, 11008) == "decode_lds_kernel"


def test_traffic_digest_covers_existing_sources():
    bench = load_bench()
    csrc = os.path.join(ROOT, "bitlinear_rmsnorm_absmax_amd", "csrc")
    for f in bench.TRAFFIC_SOURCES:
        assert os.path.exists(os.path.join(csrc, f)), f
    d = bench.kernel_source_digest()
    assert len(d) == 16 and d == bench.kernel_source_digest()
