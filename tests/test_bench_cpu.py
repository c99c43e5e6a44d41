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
    assert bench.forward1_kernel(16, 4096, 11008) == "decode_lds_kernel"
    assert bench.forward1_kernel(4, 4096, 11008) == "decode_lds_kernel"
    assert bench.forward1_kernel(4, 2048, 11008) == "gemv1_kernel"
    assert bench.forward1_kernel(1, 8192, 28672) == "decode_lds_kernel"
    assert bench.forward1_kernel(1, 8192, 4096) == "gemv1_kernel"
    assert bench.forward1_kernel(1, 2048, 2048) == "gemv1_kernel"
    # base-3: one pass on MFMA for 2..16 tokens whose staged block fits
    # 144 KB (16 tokens: K = 8960 fits, K = 8976 does not)
    assert bench.forward3_kernel(16, 8960) == "gemv3_mfma_kernel"
    assert bench.forward3_kernel(16, 8976) == "gemv3_kernel"
    assert bench.forward3_kernel(1, 4096) == "gemv3_kernel"
    assert bench.forward3_kernel(2, 4096) == "gemv3_mfma_kernel"
    assert bench.forward3_kernel(17, 1024) == "gemv3_kernel"
    # 2-bit: GEMV for one token on small shapes, the LDS decode kernel at decode
    # sizes (one token too on long rows over many row tiles), GEMM
    assert bench.forward_kernel(1, 2048, 2048) == "gemv_valu_kernel"
    assert bench.forward_kernel(1, 2560, 6912) == "gemv_valu_kernel"
    assert bench.forward_kernel(1, 4096, 11008) == "decode_lds_kernel"
    assert bench.forward_kernel(1, 8192, 28672) == "decode_lds_kernel"
    # one token quantised inside the kernel: MFMA decode on long rows, else VALU
    assert bench.quant_forward_kernel(1, 8192, 28672) == "decode_lds_kernel"
    assert bench.quant_forward_kernel(1, 4096, 11008) == "decode_lds_kernel"
    assert bench.quant_forward_kernel(1, 2048, 2048) == "quant_gemv_kernel"
    assert bench.quant_forward_kernel(1, 2560, 13824) == "quant_gemv_kernel"
    assert bench.forward_kernel(16, 4096, 11008) == "decode_lds_kernel"
    assert bench.forward_kernel(64, 8192, 28672) == "gemm_pair_kernel"
    assert bench.forward_kernel(512, 2560, 2560) == "gemm_pair_kernel"
    assert bench.forward_kernel(512, 6912, 2560) == "gemm_pair_kernel"
    assert bench.forward_kernel(512, 8192, 28672) == "gemm_dma_kernel"   # 128 x 256 tiles
    assert bench.forward_kernel(2048, 4096, 11008) == "gemm_dma_kernel"
    assert bench.forward_kernel(512, 2560, 13824) == "gemm_dma_kernel"   # 128 x 128 tiles


def test_traffic_digest_covers_every_library_source():
    bench = load_bench()
    csrc = os.path.join(ROOT, "bitlinear_rmsnorm_absmax_amd", "csrc")
    srcs = bench._library_sources()
    assert set(srcs) == {f for f in os.listdir(csrc) if f.endswith((".hip", ".h", ".cpp"))}
    assert "gemm_dma.hip" in srcs and "api.cpp" in srcs and "mfma_epilogue.h" in srcs
    d = bench.kernel_source_digest()
    assert len(d) == 16 and d == bench.kernel_source_digest()


def test_mfma_counters_give_utilisation(tmp_path, monkeypatch):
    """The MFMA pass: ops = MOPS x 512, utilisation = busy cycles per SIMD
    (summed over the 1024 SIMDs / 1024) / (dispatch duration x 2.4 GHz)."""
    bench = load_bench()
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    calls = ["quant_act_M512", "forward_M512"]
    probe = tmp_path / "probe.json"
    probe.write_text(json.dumps(dict(workload="sweep_k8192_n28672", calls=calls,
                                     copy_bytes=bench.COPY_BYTES, copy_kernel="neg",
                                     info={"forward_M512": dict(ops=240518168576, alg_bytes=1)})))
    kib = bench.COPY_BYTES / 1024
    seq = [("void bl::quant_rows_kernel<0, false, false>(int)", [1.0]),
           ("void bl::gemm_dma_kernel<1, 4, 4, 2, 3, 1>(int)", [1.0]),
           ("void at::native::neg_kernel(int)", [kib])]
    write_csv(tmp_path / "f", "FETCH_SIZE", seq)
    write_csv(tmp_path / "w", "WRITE_SIZE", seq)
    d = tmp_path / "m"
    os.makedirs(d)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        rows = [(1, "void bl::quant_rows_kernel<0, false, false>(int)", "SQ_INSTS_VALU_MFMA_MOPS_I8", [0.0]),
                (1, "void bl::quant_rows_kernel<0, false, false>(int)", "SQ_VALU_MFMA_BUSY_CYCLES", [0.0]),
                (1, "void bl::quant_rows_kernel<0, false, false>(int)", "GRBM_GUI_ACTIVE", [10.0, 10.0]),
                (2, "void bl::gemm_dma_kernel<1, 4, 4, 2, 3, 1>(int)", "SQ_INSTS_VALU_MFMA_MOPS_I8",
                 [240518168576 / 512 / 2] * 2),
                (2, "void bl::gemm_dma_kernel<1, 4, 4, 2, 3, 1>(int)", "SQ_VALU_MFMA_BUSY_CYCLES", [61440.0] * 1024),
                (2, "void bl::gemm_dma_kernel<1, 4, 4, 2, 3, 1>(int)", "GRBM_GUI_ACTIVE", [1000.0, 990.0]),
                (3, "void at::native::neg_kernel(int)", "SQ_INSTS_VALU_MFMA_MOPS_I8", [0.0]),
                (3, "void at::native::neg_kernel(int)", "SQ_VALU_MFMA_BUSY_CYCLES", [0.0]),
                (3, "void at::native::neg_kernel(int)", "GRBM_GUI_ACTIVE", [5.0])]
        for did, name, cn, vals in rows:
            for v in vals:
                row = {k: 0 for k in FIELDS}
                row.update(Dispatch_Id=did, Kernel_Name=name, Counter_Name=cn, Counter_Value=f"{v:.6f}",
                           Start_Timestamp=1000000, End_Timestamp=1000000 + (51200 if did == 2 else 1000))
                w.writerow(row)
    args = type("A", (), dict(traffic_write=[str(probe), str(tmp_path / "f"), str(tmp_path / "w"), str(d)],
                              workload=5))()
    bench.traffic_write(args)
    # 61440 busy cycles per SIMD / (51.2 us x 2400 cycles per us) = 0.5
    assert bench.read_mfma_util("sweep_k8192_n28672", "forward_M512") == pytest.approx(0.5)
    assert bench.read_mfma_util("sweep_k8192_n28672", "quant_act_M512") is None
    text = (tmp_path / "traffic_sweep_k8192_n28672.md").read_text()
    assert "| forward_M512 | 2.405e+11 | 2.405e+11 |" in text


def test_trace_phases_split_calls_that_share_a_kernel(tmp_path, monkeypatch):
    """Two calls of one step run the same kernel at the same grid (one and
    eight tokens on the decode kernel): their timed-steps and in-step
    dispatches are reported together, and each call's back-to-back graph and
    per-launch pairs on their own, in bench order."""
    import argparse
    import math
    bench = load_bench()
    import workloads
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    wid, steps, warmup, per_launch = 5, 4, 2, 3
    wl = workloads.WORKLOADS[wid]
    ncopy = max(1, math.ceil(bench.ROTATE_BYTES / (wl.N * wl.K // 4)))
    reps = max(1, math.ceil(steps / ncopy))
    kern = "void bl::decode_lds_kernel<16, 2, 2, false, 1, 2, 1>(int)"
    seq = [(kern, 5.0)] * 2 + [(kern, 6.0)] * (2 * warmup) + [(kern, 10.0)] * (2 * steps) + \
        [(kern, 12.0)] * (2 * steps)
    for own in (20.0, 30.0):
        seq += [(kern, 99.0)] * ncopy + [(kern, own)] * (reps * ncopy) + \
            [(kern, own + 1.0)] * per_launch
    seq += [("void bl::floor_stream_read_kernel(int)", 1.0), ("void bl::floor_empty_kernel(int)", 1.0)]
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Workgroup_Size_X"])
        t = 0
        for name, us in seq:
            w.writerow([name, t, t + int(us * 1000), 114688, 512])
            t += int(us * 1000) + 100
    args = argparse.Namespace(trace_summary=(str(d), "python3 bench.py"), workload=wid, configs=[],
                              steps=steps, sub_steps=steps, warmup=warmup, per_launch=per_launch)
    bench.trace_summary(args)
    text = (tmp_path / f"kernels_{wl.name}.md").read_text()
    rows = {}
    for ln in text.splitlines():
        cols = ln.split("|")
        if ln.startswith("| ") and "decode_lds" in ln and len(cols) > 7:
            rows[cols[4].strip()] = cols[5:7]
    assert rows["timed steps (2 calls)"][0].strip() == str(2 * steps)
    assert float(rows["timed steps (2 calls)"][1]) == 10.0
    assert rows["in-step events (2 calls)"][0].strip() == str(2 * steps)
    assert float(rows["in-step events (2 calls)"][1]) == 12.0
    assert float(rows["back-to-back (call 1 of 2)"][1]) == 20.0
    assert float(rows["per-launch events (call 1 of 2)"][1]) == 21.0
    assert float(rows["back-to-back (call 2 of 2)"][1]) == 30.0
    assert float(rows["per-launch events (call 2 of 2)"][1]) == 31.0
