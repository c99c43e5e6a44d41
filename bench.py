#!/usr/bin/env python3
"""Throughput of the ternary BitLinear hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

A step is one pass of the path over one batch of synthetic input: for every
token count M of the workload, the activation quantisation
(bitlinear_quant_act) followed by the ternary product with rescale
(bitlinear_forward); for the GLU workload the whole RMSNorm+quant -> gate ->
up -> SiLU*up+requant -> down chain.  Weight packing is offline and outside
the step.

Inputs are seeded synthetic draws (workloads.py), resident in HBM before the
timed region.  The packed weights rotate through at least 512 MB of copies so
that consecutive steps cannot be served from the 256 MB Infinity Cache.
The K timed steps are one replay of a HIP graph holding all K of them, so
host launch overhead does not pace the GPU.  Per-call kernel durations come from a second
pass: for each call of the step, a HIP graph of that call alone, once per
weight copy, replayed between two HIP events on the stream the kernels run on;
the dominant forward call gives the roofline.

Prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, published
ROTATE_BYTES = 512 * 10 ** 6   # twice the Infinity Cache
COPY_BYTES = 256 * 2 ** 20     # calibration copy of the traffic counters
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--no-rotate", action="store_true", help="one weight copy (warm cache)")
    ap.add_argument("--eager", action="store_true", help="time eager launches, no graphs")
    ap.add_argument("--unfused", action="store_true",
                    help="the separate calls: one-token steps as bitlinear_quant_act + "
                         "bitlinear_forward instead of bitlinear_quant_forward, and the GLU's "
                         "gate and up as two products + bitlinear_silu_mul_quant instead of "
                         "one product on the stacked weights + bitlinear_silu_mul_quant_acc")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the oracle CPU baseline (0 = skip)")
    ap.add_argument("--op", choices=("layer", "ternarize", "binary", "grouped", "base3"),
                    default="layer",
                    help="layer: the BitLinear step (default); ternarize: absmean "
                         "ternarisation + packing of fp32 weights of the workload's shape; "
                         "binary: the step on 1-bit Sign(W - alpha) weights "
                         "(bitlinear_quant_act + bitlinear_forward1 per token count); "
                         "grouped: the step with --groups group scales along K "
                         "(bitlinear_quant_act_grouped + bitlinear_forward_grouped); "
                         "base3: the step on 1.6-bit base-3 packed weights "
                         "(bitlinear_quant_act + bitlinear_forward3)")
    ap.add_argument("--groups", type=int, default=4, help="group count of --op grouped")
    ap.add_argument("--traffic-probe", metavar="JSON",
                    help="launch every call of one step once, then a plain copy kernel of "
                         f"{COPY_BYTES} bytes, write the launch order to JSON and exit "
                         "(run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--traffic-write", nargs=3, metavar=("JSON", "FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn the two counter runs of --traffic-probe into "
                         "profiles/traffic_<workload>.md")
    return ap.parse_args()


def forward1_kernel(M: int, K: int) -> str:
    """The kernel bitlinear_forward1 runs for M tokens (its dispatch, for the
    bench shapes: K % 256 == 0 and the activation block fits LDS)."""
    return "decode_lds_kernel" if M >= 5 or (M >= 2 and K >= 4096) else "gemv1_kernel"


def forward3_kernel(M: int, K: int) -> str:
    """The kernel bitlinear_forward3 runs for M tokens (its dispatch)."""
    steps = (-(-K // 80) + 3) // 4
    fits = M * (20 * steps + 1) * 16 <= 144 * 1024
    return "gemv3_mfma_kernel" if 2 <= M <= 16 and fits else "gemv3_kernel"


def forward_kernel(M: int, K: int, N: int) -> str:
    """Kernel that bitlinear_forward picks (the library's dispatch)."""
    if M == 1:
        return "gemv_valu_kernel"
    lds_fits = K % 256 == 0 and ((M * K + 1023) // 1024) * 1024 + 16384 + 128 <= 160 * 1024
    if (5 <= M <= 16 or (2 <= M <= 4 and K >= 4096)) and lds_fits:
        return "decode_lds_kernel"
    if M <= 16 or (M <= 32 and not (-(-N // 128) >= 128 and K % 256 == 0)):
        return "skinny_mfma_kernel"
    if K % 128 != 0:
        return "gemm_mfma_kernel"
    if M >= 256 and -(-M // 128) * -(-N // 256) >= 256:
        return "gemm_pipe_kernel"   # 128 x 256 tiles
    if -(-M // 64) * -(-N // 128) <= 256 and K % 256 == 0:
        return "gemm_dma_kernel"    # 64 x 128 tiles, two or three K groups
    return "gemm_pipe_kernel"       # 128 x 128 tiles


# ----------------------------------------------------------------------------- timers

class RunAll:
    """Runs every call; records how often each call occurs per step."""

    def __init__(self):
        self.calls = {}
        self.info = {}

    def __call__(self, name, M=0, N=0, K=0, wbytes=0, xbytes=0, kernel=None):
        self.calls[name] = self.calls.get(name, 0) + 1
        if wbytes:
            # algorithmic bytes of one forward launch: packed W + x_q + gamma + y
            # (+ the unquantised activations read by a fused call)
            self.info[name] = dict(alg_bytes=wbytes + M * K + 4 * M + 4 * M * N + xbytes,
                                   ops=2 * M * N * K, wbytes=wbytes, M=M, N=N, K=K,
                                   kernel=kernel or forward_kernel(M, K, N))
        return True


class RunOne:
    """Runs only the call `name`; the first run records the start event."""

    def __init__(self, torch, name):
        self.torch = torch
        self.name = name
        self.e0 = torch.cuda.Event(enable_timing=True)
        self.e1 = torch.cuda.Event(enable_timing=True)
        self.started = False

    def __call__(self, name, *a, **kw):
        if name != self.name:
            return False
        if not self.started:
            self.e0.record(self.torch.cuda.current_stream())
            self.started = True
        return True

    def avg_us(self, launches):
        self.e1.record(self.torch.cuda.current_stream())
        self.torch.cuda.synchronize()
        return self.e0.elapsed_time(self.e1) * 1e3 / launches


# ----------------------------------------------------------------------------- plan

class Layer:
    """One packed weight matrix (with rotation copies) on the GPU."""

    def __init__(self, torch, bl, dev, w: np.ndarray, beta, rotate: bool):
        self.N, self.K = w.shape
        self.beta = float(beta)
        packed, _ = bl.pack_weights(torch.from_numpy(w).to(dev))
        self.wbytes = packed.numel() * 4
        self.copies = [packed]
        if rotate:
            n = max(1, math.ceil(ROTATE_BYTES / self.wbytes))
            self.copies += [packed.clone() for _ in range(n - 1)]


def build_plan(args, torch, bl, dev):
    """Returns (ops, meta, keepalive): ops(step_idx, timer) launches one step."""
    wid = args.workload
    wl = workloads.WORKLOADS[wid]
    rotate = not args.no_rotate
    lib = bl.lib

    def stream():
        return torch.cuda.current_stream(dev).cuda_stream

    def check(st):
        if st != 0:
            raise RuntimeError(bl.last_error())

    def fused(M, K, N):
        # bitlinear_quant_forward runs as one kernel for one token, K % 64 == 0,
        # K <= 16384, N <= 16384 (--unfused times the two calls instead)
        return not args.unfused and M == 1 and K % 64 == 0 and K <= 16384 and N <= 16384

    meta = {"workload": wl.name, "K": wl.K, "N": wl.N, "M": list(wl.ms)}
    if wl.glu_f:
        wg, wu, wd = workloads.glu_weights(wid)
        bg, bu, bd = workloads.glu_betas(wid)
        # default: gate and up as one product on the stacked weights [W_gate; W_up]
        # writing int32 accumulators, then bitlinear_silu_mul_quant_acc (one weight
        # stream and one launch for both projections; every stage bit-identical to
        # the separate calls); --unfused runs the separate calls
        stacked = not args.unfused
        if stacked:
            layers = [Layer(torch, bl, dev, np.concatenate([wg, wu], axis=0), 1.0, rotate),
                      Layer(torch, bl, dev, wd, bd, rotate)]
        else:
            layers = [Layer(torch, bl, dev, w, b, rotate) for w, b in ((wg, bg), (wu, bu), (wd, bd))]
        ncopy = min(len(L.copies) for L in layers)
        D, Fh = wl.K, wl.glu_f
        gain = torch.ones(D, dtype=torch.float32, device=dev)
        bufs = []
        for M in wl.ms:
            x = torch.from_numpy(workloads.workload_activations(wid, M)).to(dev)
            bufs.append(dict(
                M=M, x=x, q=torch.empty((M, D), dtype=torch.int8, device=dev),
                g=torch.empty(M, device=dev), yg=torch.empty((M, Fh), device=dev),
                yu=torch.empty((M, Fh), device=dev),
                acc_gu=torch.empty((M, 2 * Fh), dtype=torch.int32, device=dev),
                hq=torch.empty((M, Fh), dtype=torch.int8, device=dev),
                gh=torch.empty(M, device=dev), y=torch.empty((M, D), device=dev)))

        def ops(step, run):
            c = step % ncopy
            for b in bufs:
                M = b["M"]
                if stacked:
                    L = layers[0]
                    if fused(M, D, 2 * Fh):
                        if run(f"quant_forward_rms_gateup_M{M}", M, L.N, L.K, L.wbytes,
                               4 * M * D + 4 * D, "quant_gemv_kernel"):
                            check(lib.bitlinear_quant_forward(
                                b["x"].data_ptr(), bl.F32, M, D, gain.data_ptr(), wl.rms_eps,
                                L.copies[c].data_ptr(), 2 * Fh, 1.0, b["q"].data_ptr(),
                                b["g"].data_ptr(), None, b["acc_gu"].data_ptr(), stream()))
                    else:
                        if run(f"quant_act_rms_M{M}"):
                            check(lib.bitlinear_quant_act(b["x"].data_ptr(), bl.F32, M, D,
                                                          gain.data_ptr(), wl.rms_eps,
                                                          b["q"].data_ptr(), b["g"].data_ptr(),
                                                          stream()))
                        if run(f"forward_gateup_M{M}", M, L.N, L.K, L.wbytes):
                            check(lib.bitlinear_forward(b["q"].data_ptr(), b["g"].data_ptr(), M, D,
                                                        L.copies[c].data_ptr(), 2 * Fh, 1.0, None,
                                                        b["acc_gu"].data_ptr(), stream()))
                    if run(f"silu_mul_quant_acc_M{M}"):
                        check(lib.bitlinear_silu_mul_quant_acc(
                            b["acc_gu"].data_ptr(), b["g"].data_ptr(), M, Fh, bg, bu, None,
                            b["hq"].data_ptr(), b["gh"].data_ptr(), stream()))
                else:
                    if run(f"quant_act_rms_M{M}"):
                        check(lib.bitlinear_quant_act(b["x"].data_ptr(), bl.F32, M, D,
                                                      gain.data_ptr(), wl.rms_eps, b["q"].data_ptr(),
                                                      b["g"].data_ptr(), stream()))
                    for nm, L, out in (("gate", layers[0], b["yg"]), ("up", layers[1], b["yu"])):
                        if run(f"forward_{nm}_M{M}", M, L.N, L.K, L.wbytes):
                            check(lib.bitlinear_forward(b["q"].data_ptr(), b["g"].data_ptr(), M, D,
                                                        L.copies[c].data_ptr(), Fh, L.beta,
                                                        out.data_ptr(), None, stream()))
                    if run(f"silu_mul_quant_M{M}"):
                        check(lib.bitlinear_silu_mul_quant(b["yg"].data_ptr(), b["yu"].data_ptr(), M,
                                                           Fh, None, b["hq"].data_ptr(),
                                                           b["gh"].data_ptr(), stream()))
                L = layers[-1]
                if run(f"forward_down_M{M}", M, L.N, L.K, L.wbytes):
                    check(lib.bitlinear_forward(b["hq"].data_ptr(), b["gh"].data_ptr(), M, Fh,
                                                L.copies[c].data_ptr(), D, L.beta, b["y"].data_ptr(),
                                                None, stream()))

        meta.update(weight_bytes_per_step=sum(L.wbytes for L in layers) * len(wl.ms),
                    weight_copies=ncopy,
                    ops_per_step=sum(2 * M * (2 * D * Fh + Fh * D) for M in wl.ms))
        return ops, meta, (layers, bufs, gain)

    w = workloads.workload_weights(wid)
    L = Layer(torch, bl, dev, w, workloads.workload_beta(wid), rotate)
    K, N = wl.K, wl.N
    bufs = []
    for M in wl.ms:
        xa = workloads.workload_activations(wid, M)
        if wl.act == "normal_bf16":
            x, dt = torch.from_numpy(xa).to(dev).view(torch.bfloat16), bl.BF16
        else:
            x, dt = torch.from_numpy(xa).to(dev), bl.F32
        bufs.append(dict(M=M, x=x, dt=dt, q=torch.empty((M, K), dtype=torch.int8, device=dev),
                         g=torch.empty(M, device=dev), y=torch.empty((M, N), device=dev)))

    def ops(step, run):
        wptr = L.copies[step % len(L.copies)].data_ptr()
        for b in bufs:
            M = b["M"]
            if fused(M, K, N):
                xb = M * K * (2 if b["dt"] == bl.BF16 else 4)
                if run(f"quant_forward_M{M}", M, N, K, L.wbytes, xb, "quant_gemv_kernel"):
                    check(lib.bitlinear_quant_forward(b["x"].data_ptr(), b["dt"], M, K, None, 0.0,
                                                      wptr, N, L.beta, b["q"].data_ptr(),
                                                      b["g"].data_ptr(), b["y"].data_ptr(), None,
                                                      stream()))
                continue
            if run(f"quant_act_M{M}"):
                check(lib.bitlinear_quant_act(b["x"].data_ptr(), b["dt"], M, K, None, 0.0,
                                              b["q"].data_ptr(), b["g"].data_ptr(), stream()))
            if run(f"forward_M{M}", M, N, K, L.wbytes):
                check(lib.bitlinear_forward(b["q"].data_ptr(), b["g"].data_ptr(), M, K, wptr, N,
                                            L.beta, b["y"].data_ptr(), None, stream()))

    meta.update(weight_bytes_per_step=L.wbytes * len(wl.ms), weight_copies=len(L.copies),
                ops_per_step=sum(2 * M * N * K for M in wl.ms))
    return ops, meta, (L, bufs)


# ----------------------------------------------------------------------------- traffic

# The sources of the calls whose traffic is recorded (the decode step: the
# quantiser, the fused one-token call, the skinny dispatch and the LDS decode
# kernel) with the shared headers and the ABI's dispatch.
TRAFFIC_SOURCES = ("api.cpp", "device_common.h", "internal.h", "quant_rows.h", "quant_act.hip",
                   "quant_gemv.hip", "skinny_mfma.hip", "decode_lds.hip", "gemv_valu.hip")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bitlinear_rmsnorm_absmax_amd", "csrc")
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload_name: str, call: str):
    """HBM bytes per launch of `call` from the committed counter summary
    profiles/traffic_<workload>.md, only if it was taken on the current kernel
    sources (else None)."""
    path = os.path.join(PROFILES, f"traffic_{workload_name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source_digest:\s*(\w+)", text)
    m_val = re.search(rf"traffic_bytes_per_launch\[{re.escape(call)}\]:\s*([0-9.eE+]+)", text)
    if not m_src or not m_val or m_src.group(1) != kernel_source_digest():
        return None
    return float(m_val.group(1))


def traffic_probe(args, torch, ops, dev):
    """One eager step (every call once, in step order), then the calibration
    copy: an elementwise kernel that reads COPY_BYTES and writes COPY_BYTES."""
    src = torch.zeros(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    seq = []
    ops(0, lambda name, *a, **kw: seq.append(name) or True)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    with open(args.traffic_probe, "w") as f:
        json.dump(dict(workload=workloads.WORKLOADS[args.workload].name, calls=seq,
                       copy_bytes=COPY_BYTES, copy_kernel="neg"), f)


def _counter_rows(d: str, counter: str):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {d}, found {files}")
    per = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            did = int(r["Dispatch_Id"])
            name, v = per.get(did, (r["Kernel_Name"], 0.0))
            per[did] = (name, v + float(r["Counter_Value"]))
    return [per[k] for k in sorted(per)]


def traffic_write(args):
    """profiles/traffic_<workload>.md from the FETCH_SIZE and WRITE_SIZE runs of
    --traffic-probe: the last dispatches of each run are the probe's step and
    its copy; the counters (KiB per dispatch) are scaled by what they read for
    the copy of known size."""
    probe_json, fdir, wdir = args.traffic_write
    probe = json.load(open(probe_json))
    calls = probe["calls"]

    def pick(rows):
        """(library dispatches of the probe's step, the calibration copy)"""
        copies = [i for i, (name, _) in enumerate(rows) if "neg" in name]
        if not copies:
            raise SystemExit("counter run holds no calibration copy")
        lib = [r for r in rows[:copies[-1]] if "bl::" in r[0]][-len(calls):]
        if len(lib) != len(calls):
            raise SystemExit(f"counter run holds {len(lib)} library dispatches, "
                             f"the probe made {len(calls)}")
        for call, (name, _) in zip(calls, lib):
            want = ("quant_gemv" if call.startswith("quant_forward") else
                    "quant_rows" if call.startswith(("quant", "silu")) else "_kernel")
            if want not in name or (call.startswith("forward") and "quant_rows" in name):
                raise SystemExit(f"dispatch {name} does not match call {call}")
        return lib, rows[copies[-1]]

    fr, fcopy = pick(_counter_rows(fdir, "FETCH_SIZE"))
    wr, wcopy = pick(_counter_rows(wdir, "WRITE_SIZE"))
    cb = probe["copy_bytes"]
    f_scale = cb / (fcopy[1] * 1024)
    w_scale = cb / (wcopy[1] * 1024)
    wl = next(w for w in workloads.WORKLOADS.values() if w.name == probe["workload"])
    lines = [f"# HBM traffic per launch: {wl.name}", "",
             "Counters: rocprofv3 `--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE` (KiB per dispatch), "
             "each in its own run of the probe; commands (from the repository root, "
             "`cd /tmp && export TMPDIR=/tmp` first):", "",
             "```",
             f"python3 bench.py --workload {args.workload} --traffic-probe gpurun_out/probe.json",
             f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o run -- "
             f"python3 bench.py --workload {args.workload} --traffic-probe gpurun_out/probe.json",
             f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o run -- "
             f"python3 bench.py --workload {args.workload} --traffic-probe gpurun_out/probe.json",
             f"python3 bench.py --workload {args.workload} --traffic-write gpurun_out/probe.json "
             "gpurun_out/pmc_fetch gpurun_out/pmc_write",
             "```", "",
             f"Calibration: an elementwise negation of {cb} bytes (reads {cb}, writes {cb}) "
             f"reads FETCH_SIZE {fcopy[1]:.0f} KiB and WRITE_SIZE {wcopy[1]:.0f} KiB; "
             f"scale factors {f_scale:.4f} (fetch) and {w_scale:.4f} (write).", "",
             "| call | kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled bytes |",
             "|---|---|---:|---:|---:|"]
    vals = []
    for call, (fk, fv), (wk, wv) in zip(calls, fr, wr):
        if fk != wk:
            raise SystemExit(f"dispatch mismatch between the runs: {fk} / {wk}")
        b = fv * 1024 * f_scale + wv * 1024 * w_scale
        short = fk.replace("(anonymous namespace)::", "").replace("void ", "")
        short = short[:short.index(">(") + 1] if ">(" in short else short.split("(")[0]
        lines.append(f"| {call} | `{short}` | {fv:.0f} | {wv:.0f} | {b:.4g} |")
        vals.append((call, b))
    lines += ["", f"source_digest: {kernel_source_digest()}", ""]
    lines += [f"traffic_bytes_per_launch[{c}]: {b:.6g}" for c, b in vals]
    path = os.path.join(PROFILES, f"traffic_{wl.name}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


# ----------------------------------------------------------------------------- cpu baseline

def cpu_baseline(args, seconds: float):
    """The oracle (plain C loops, OpenMP over outputs) on the same workload,
    whole steps, for about ``seconds`` of CPU time."""
    import oracle
    wid = args.workload
    wl = workloads.WORKLOADS[wid]
    if wl.glu_f:
        wg, wu, wd = workloads.glu_weights(wid)
        betas = workloads.glu_betas(wid)
        gain = np.ones(wl.K, np.float32)
        xs = [workloads.workload_activations(wid, M) for M in wl.ms]
        wbytes = (wg.size + wu.size + wd.size) // 4 * len(wl.ms)

        def step():
            for x in xs:
                oracle.glu(x, wg, wu, wd, betas, gain, wl.rms_eps)
        desc = "GLU chain"
    else:
        w = workloads.workload_weights(wid)
        beta = workloads.workload_beta(wid)
        xs = []
        for M in wl.ms:
            x = workloads.workload_activations(wid, M)
            xs.append(oracle.bf16_to_f32(x) if wl.act == "normal_bf16" else x)
        rows = w.shape[0]
        # large workloads: a bounded slice of output rows (same K, same M sweep)
        est = sum(x.shape[0] for x in xs) * w.size * 1.5e-9  # ~1.5 ns per MAC and thread
        if est / max(oracle.num_threads(), 1) > seconds:
            rows = max(64, int(rows * seconds * oracle.num_threads() / est / 3))
            w = np.ascontiguousarray(w[:rows])
        wbytes = w.size // 4 * len(wl.ms)

        def step():
            for x in xs:
                q, g = oracle.quant_act(x)
                oracle.forward(q, g, w, beta)
        desc = f"whole steps over {rows} of {wl.N} output rows"
    n = 0
    t0 = time.perf_counter()
    while True:
        step()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or el / n * (n + 1) > 3 * seconds:
            break
    return dict(value=round(wbytes * n / el / 1e9, 4), unit="packed-W GB/s",
                cores=oracle.num_threads(), kind="oracle",
                sample=f"{n} x ({desc}), M={list(wl.ms)}, {el:.1f} s")


# ----------------------------------------------------------------------------- ternarize

def bench_ternarize(args, torch, bl, dev):
    """bitlinear_ternarize on seeded fp32 weights N(0, 0.02^2) of the workload's
    [N][K]: one call per step (row sums, ordered total, codes + packing)."""
    wl = workloads.WORKLOADS[args.workload]
    N, K = wl.N, wl.K
    W = (workloads.rng_for(args.workload, 30).standard_normal((N, K)) * 0.02).astype(np.float32)
    Wd = torch.from_numpy(W).to(dev)
    packed = torch.empty((N, K // 16), dtype=torch.int32, device=dev)
    beta = torch.empty((1,), dtype=torch.float32, device=dev)
    beta64 = torch.empty((1,), dtype=torch.float64, device=dev)

    def call():
        st = bl.lib.bitlinear_ternarize(Wd.data_ptr(), N, K, packed.data_ptr(), None,
                                        beta.data_ptr(), beta64.data_ptr(),
                                        torch.cuda.current_stream(dev).cuda_stream)
        if st != 0:
            raise RuntimeError(bl.last_error())

    call()
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    alg = 8 * N * K + N * K // 4   # W read twice (row sums, codes) + packed words written
    gbs = alg / (us * 1e-6) / 1e9
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < args.cpu_seconds / 2 or n == 0:
            oracle.ternarize(W)
            n += 1
        el = time.perf_counter() - t0
        cpu = dict(value=round(4 * N * K * n / el / 1e9, 4), unit="fp32-W GB/s", cores=1,
                   kind="oracle", sample=f"{n} x oracle.ternarize on [{N}][{K}], {el:.1f} s")
    line = {
        "metric": "absmean ternarisation + packing: fp32-W GB/s",
        "value": round(4 * N * K / (us * 1e-6) / 1e9, 2),
        "unit": "fp32-W GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"ternarize_{wl.name}", "N": N, "K": K,
                   "timing": "hip_graph_per_step"},
        "roofline": dict(bound="hbm", achieved=round(gbs, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None,
                         call="bitlinear_ternarize", avg_launch_us=round(us, 3),
                         alg_bytes_per_launch=alg),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


# ----------------------------------------------------------------------------- 1-bit step

def bench_binary(args, torch, bl, dev):
    """The decode step of the workload on 1-bit weights: seeded fp32 W
    N(0.003, 0.02^2) binarised on the GPU (Sign(W - alpha), beta = mean |W|),
    then per token count quant + bitlinear_forward1; weights rotate through
    >= 512 MB of copies; steps are HIP graph replays."""
    wl = workloads.WORKLOADS[args.workload]
    N, K = wl.N, wl.K
    W = (workloads.rng_for(args.workload, 31).standard_normal((N, K)) * 0.02 + 0.003).astype(np.float32)
    packed1, _, _, _, beta, _ = bl.binarize(torch.from_numpy(W).to(dev))
    beta = float(beta.item())
    cpu = binary_cpu_baseline(args, W, beta, args.cpu_seconds) if args.cpu_seconds > 0 else None
    del W
    wbytes = N * K // 8
    copies = [packed1] + [packed1.clone() for _ in range(max(1, math.ceil(ROTATE_BYTES / wbytes)) - 1)]
    bufs = []
    for M in [m for m in wl.ms if m <= 16]:   # decode token counts; more tokens take the 2-bit path
        x = torch.from_numpy(workloads.workload_activations(args.workload, M)).to(dev)
        bufs.append(dict(M=M, x=x, q=torch.empty((M, K), dtype=torch.int8, device=dev),
                         g=torch.empty(M, device=dev), y=torch.empty((M, N), device=dev)))
    lib = bl.lib

    def stream():
        return torch.cuda.current_stream(dev).cuda_stream

    def ops(step, only=None):
        w = copies[step % len(copies)].data_ptr()
        for b in bufs:
            M = b["M"]
            if only in (None, f"quant_act_M{M}"):
                assert lib.bitlinear_quant_act(b["x"].data_ptr(), bl.F32, M, K, None, 0.0,
                                               b["q"].data_ptr(), b["g"].data_ptr(), stream()) == 0
            if only in (None, f"forward1_M{M}"):
                assert lib.bitlinear_forward1(b["q"].data_ptr(), b["g"].data_ptr(), M, K, w, N, beta,
                                              b["y"].data_ptr(), None, stream()) == 0

    def graph(only=None):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream(device=dev)
        with torch.cuda.graph(g, stream=s):
            for c in range(len(copies)):
                ops(c, only)
        return g

    def time_graph(g, per_replay):
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, math.ceil(args.steps / len(copies)))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * per_replay)

    ops(0)
    torch.cuda.synchronize()
    us_step = time_graph(graph(), len(copies))
    per_call = {}
    for b in bufs:
        M = b["M"]
        for name in (f"quant_act_M{M}", f"forward1_M{M}"):
            per_call[name] = dict(avg_us=round(time_graph(graph(name), len(copies)), 3))
        alg = wbytes + M * K + 4 * M + 4 * M * N
        per_call[f"forward1_M{M}"].update(alg_bytes=alg, packed_w_GBs=round(
            wbytes / (per_call[f"forward1_M{M}"]["avg_us"] * 1e-6) / 1e9, 1))
    dom = max((k for k in per_call if k.startswith("forward1")), key=lambda k: per_call[k]["avg_us"])
    d = per_call[dom]
    gbs = d["alg_bytes"] / (d["avg_us"] * 1e-6) / 1e9
    line = {
        "metric": "BitLinear 1-bit weights: packed-W GB/s",
        "value": round(wbytes * len(bufs) / (us_step * 1e-6) / 1e9, 2),
        "unit": "packed-W GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us_step * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": f"binary_{wl.name}", "M": [b["M"] for b in bufs], "K": K, "N": N,
                   "weight_copies": len(copies), "timing": "hip_graph_per_step"},
        "roofline": dict(bound="hbm", achieved=round(gbs, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None, call=dom,
                         kernel=forward1_kernel(int(dom.split("M")[-1]), K),
                         avg_launch_us=d["avg_us"],
                         alg_bytes_per_launch=d["alg_bytes"]),
        "cpu_baseline": cpu,
        "per_call": per_call,
    }
    print(json.dumps(line), flush=True)


def binary_cpu_baseline(args, W, beta, seconds):
    """The oracle's quantisation + product on the oracle's own binarisation of
    the same W, whole decode steps over a bounded slice of output rows."""
    import oracle
    wl = workloads.WORKLOADS[args.workload]
    ms = [m for m in wl.ms if m <= 16]
    xs = [workloads.workload_activations(args.workload, M) for M in ms]
    est = sum(ms) * W.size * 1.5e-9
    rows = W.shape[0]
    if est / max(oracle.num_threads(), 1) > seconds:
        rows = max(64, int(rows * seconds * oracle.num_threads() / est / 3))
    w, _ = oracle.binarize(np.ascontiguousarray(W[:rows]))
    n = 0
    t0 = time.perf_counter()
    while True:
        for x in xs:
            q, g = oracle.quant_act(x)
            oracle.forward(q, g, w, beta)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or el / n * (n + 1) > 3 * seconds:
            break
    return dict(value=round(w.size // 8 * len(ms) * n / el / 1e9, 4), unit="packed-W GB/s",
                cores=oracle.num_threads(), kind="oracle",
                sample=f"{n} x (decode steps over {rows} of {W.shape[0]} output rows, +-1 weights "
                       f"unpacked), M={ms}, {el:.1f} s")


# ----------------------------------------------------------------------------- grouped step

def bench_grouped(args, torch, bl, dev):
    """The decode step of the workload with group scales: the workload's ternary
    weights split into G groups of K/G input columns (group-major, packed),
    per-group betas U(0.01, 0.05); per token count bitlinear_quant_act_grouped
    + bitlinear_forward_grouped; weights rotate through >= 512 MB of copies;
    the timed steps are one graph replay."""
    wl = workloads.WORKLOADS[args.workload]
    N, K, G = wl.N, wl.K, args.groups
    KG = K // G
    w = workloads.workload_weights(args.workload)
    wg = np.ascontiguousarray(w.reshape(N, G, KG).transpose(1, 0, 2)).reshape(G * N, KG)
    packed, _ = bl.pack_weights(torch.from_numpy(wg).to(dev))
    packed = packed.view(G, N, KG // 16)
    beta = workloads.rng_for(args.workload, 32).uniform(0.01, 0.05, G).astype(np.float32)
    beta_d = torch.from_numpy(beta).to(dev)
    wbytes = N * K // 4
    copies = [packed] + [packed.clone() for _ in range(max(1, math.ceil(ROTATE_BYTES / wbytes)) - 1)]
    bufs = []
    for M in [m for m in wl.ms if m <= 64]:
        x = torch.from_numpy(workloads.workload_activations(args.workload, M)).to(dev)
        bufs.append(dict(M=M, x=x, q=torch.empty((G, M, KG), dtype=torch.int8, device=dev),
                         g=torch.empty((G, M), device=dev), y=torch.empty((M, N), device=dev),
                         acc=torch.empty((G, M, N), dtype=torch.int32, device=dev)))
    lib = bl.lib

    def stream():
        return torch.cuda.current_stream(dev).cuda_stream

    def ops(step, only=None):
        wp = copies[step % len(copies)].data_ptr()
        for b in bufs:
            M = b["M"]
            if only in (None, f"quant_act_grouped_M{M}"):
                assert lib.bitlinear_quant_act_grouped(b["x"].data_ptr(), bl.F32, M, K, G, None, 0.0,
                                                       b["q"].data_ptr(), b["g"].data_ptr(), stream()) == 0
            if only in (None, f"forward_grouped_M{M}"):
                acc = None if lib.bitlinear_forward_grouped_one_launch(M, K, G, N) else b["acc"].data_ptr()
                assert lib.bitlinear_forward_grouped(b["q"].data_ptr(), b["g"].data_ptr(), M, K, G, wp,
                                                     N, beta_d.data_ptr(), b["y"].data_ptr(),
                                                     acc, stream()) == 0

    s = torch.cuda.Stream(device=dev)

    def graph(first, count, only=None):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(first, first + count):
                ops(i, only)
        return g

    def time_graph(g, per_replay):
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / per_replay

    ops(0)
    torch.cuda.synchronize()
    graph(0, args.warmup).replay()
    us_step = time_graph(graph(args.warmup, args.steps), args.steps)
    per_call = {}
    for b in bufs:
        M = b["M"]
        for name in (f"quant_act_grouped_M{M}", f"forward_grouped_M{M}"):
            per_call[name] = dict(avg_us=round(time_graph(graph(0, len(copies), name), len(copies)), 3))
        alg = wbytes + M * K + 4 * G * M + 4 * M * N
        per_call[f"forward_grouped_M{M}"].update(alg_bytes=alg, packed_w_GBs=round(
            wbytes / (per_call[f"forward_grouped_M{M}"]["avg_us"] * 1e-6) / 1e9, 1))
    dom = max((k for k in per_call if k.startswith("forward")), key=lambda k: per_call[k]["avg_us"])
    d = per_call[dom]
    gbs = d["alg_bytes"] / (d["avg_us"] * 1e-6) / 1e9
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        xs = [workloads.workload_activations(args.workload, b["M"]) for b in bufs]
        est = sum(b["M"] for b in bufs) * w.size * 1.5e-9
        rows = N
        if est / max(oracle.num_threads(), 1) > args.cpu_seconds:
            rows = max(64, int(N * args.cpu_seconds * oracle.num_threads() / est / 3))
        wr = np.ascontiguousarray(w[:rows])
        n = 0
        t0 = time.perf_counter()
        while True:
            for x in xs:
                q, g = oracle.quant_act_grouped(x, G)
                oracle.forward_grouped(q, g, wr, beta)
            n += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or el / n * (n + 1) > 3 * args.cpu_seconds:
                break
        cpu = dict(value=round(wr.size // 4 * len(xs) * n / el / 1e9, 4), unit="packed-W GB/s",
                   cores=oracle.num_threads(), kind="oracle",
                   sample=f"{n} x (decode steps over {rows} of {N} output rows, G={G}), "
                          f"M={[b['M'] for b in bufs]}, {el:.1f} s")
    line = {
        "metric": f"BitLinear with {G} group scales along K: packed-W GB/s",
        "value": round(wbytes * len(bufs) / (us_step * 1e-6) / 1e9, 2),
        "unit": "packed-W GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us_step * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": f"grouped{G}_{wl.name}", "M": [b["M"] for b in bufs], "K": K, "N": N,
                   "G": G, "weight_copies": len(copies), "timing": "hip_graph_of_all_timed_steps"},
        "roofline": dict(bound="hbm", achieved=round(gbs, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None, call=dom,
                         kernel=("decode_lds_kernel (groups in the epilogue)"
                                 if lib.bitlinear_forward_grouped_one_launch(int(dom.split("M")[-1]), K, G, N)
                                 else f"{G} group products + group_sum_kernel"),
                         avg_launch_us=d["avg_us"],
                         alg_bytes_per_launch=d["alg_bytes"]),
        "cpu_baseline": cpu,
        "per_call": per_call,
    }
    print(json.dumps(line), flush=True)


# ----------------------------------------------------------------------------- base-3 step

def bench_base3(args, torch, bl, dev):
    """The decode step of the workload on base-3 packed weights (1.6 bits per
    weight): the workload's ternary weights packed by bitlinear_pack_weights3,
    per token count bitlinear_quant_act + bitlinear_forward3; weights rotate
    through >= 512 MB of copies; the timed steps are one graph replay."""
    wl = workloads.WORKLOADS[args.workload]
    N, K = wl.N, wl.K
    beta = float(workloads.workload_beta(args.workload))
    w = workloads.workload_weights(args.workload)
    packed3, _ = bl.pack_weights3(torch.from_numpy(w).to(dev))
    wbytes = packed3.numel() * 4
    copies = [packed3] + [packed3.clone() for _ in range(max(1, math.ceil(ROTATE_BYTES / wbytes)) - 1)]
    bufs = []
    for M in [m for m in wl.ms if m <= 16]:
        x = torch.from_numpy(workloads.workload_activations(args.workload, M)).to(dev)
        bufs.append(dict(M=M, x=x, q=torch.empty((M, K), dtype=torch.int8, device=dev),
                         g=torch.empty(M, device=dev), y=torch.empty((M, N), device=dev)))
    lib = bl.lib

    def stream():
        return torch.cuda.current_stream(dev).cuda_stream

    def ops(step, only=None):
        wp = copies[step % len(copies)].data_ptr()
        for b in bufs:
            M = b["M"]
            if only in (None, f"quant_act_M{M}"):
                assert lib.bitlinear_quant_act(b["x"].data_ptr(), bl.F32, M, K, None, 0.0,
                                               b["q"].data_ptr(), b["g"].data_ptr(), stream()) == 0
            if only in (None, f"forward3_M{M}"):
                assert lib.bitlinear_forward3(b["q"].data_ptr(), b["g"].data_ptr(), M, K, wp, N, beta,
                                              b["y"].data_ptr(), None, stream()) == 0

    s = torch.cuda.Stream(device=dev)

    def graph(first, count, only=None):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(first, first + count):
                ops(i, only)
        return g

    def time_graph(g, per_replay):
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / per_replay

    ops(0)
    torch.cuda.synchronize()
    graph(0, args.warmup).replay()
    us_step = time_graph(graph(args.warmup, args.steps), args.steps)
    per_call = {}
    for b in bufs:
        M = b["M"]
        for name in (f"quant_act_M{M}", f"forward3_M{M}"):
            per_call[name] = dict(avg_us=round(time_graph(graph(0, len(copies), name), len(copies)), 3))
        alg = wbytes + M * K + 4 * M + 4 * M * N
        per_call[f"forward3_M{M}"].update(alg_bytes=alg, packed_w_GBs=round(
            wbytes / (per_call[f"forward3_M{M}"]["avg_us"] * 1e-6) / 1e9, 1))
    dom = max((k for k in per_call if k.startswith("forward")), key=lambda k: per_call[k]["avg_us"])
    d = per_call[dom]
    gbs = d["alg_bytes"] / (d["avg_us"] * 1e-6) / 1e9
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        xs = [workloads.workload_activations(args.workload, b["M"]) for b in bufs]
        est = sum(b["M"] for b in bufs) * w.size * 1.5e-9
        rows = N
        if est / max(oracle.num_threads(), 1) > args.cpu_seconds:
            rows = max(64, int(N * args.cpu_seconds * oracle.num_threads() / est / 3))
        p3, _ = oracle.pack3(np.ascontiguousarray(w[:rows]))
        n = 0
        t0 = time.perf_counter()
        while True:
            wr = oracle.unpack3(p3, K)  # the oracle reads the packed bytes each step
            for x in xs:
                q, g = oracle.quant_act(x)
                oracle.forward(q, g, wr, beta)
            n += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or el / n * (n + 1) > 3 * args.cpu_seconds:
                break
        cpu = dict(value=round(p3.size * len(xs) * n / el / 1e9, 4), unit="packed-W GB/s",
                   cores=oracle.num_threads(), kind="oracle",
                   sample=f"{n} x (unpack + decode steps over {rows} of {N} output rows), "
                          f"M={[b['M'] for b in bufs]}, {el:.1f} s")
    line = {
        "metric": "BitLinear on 1.6-bit base-3 weights: packed-W GB/s",
        "value": round(wbytes * len(bufs) / (us_step * 1e-6) / 1e9, 2),
        "unit": "packed-W GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us_step * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": f"base3_{wl.name}", "M": [b["M"] for b in bufs], "K": K, "N": N,
                   "weight_bytes": wbytes, "weight_copies": len(copies),
                   "timing": "hip_graph_of_all_timed_steps"},
        "roofline": dict(bound="hbm", achieved=round(gbs, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None, call=dom,
                         kernel=forward3_kernel(int(dom.split("M")[-1]), K), avg_launch_us=d["avg_us"],
                         alg_bytes_per_launch=d["alg_bytes"]),
        "cpu_baseline": cpu,
        "per_call": per_call,
    }
    print(json.dumps(line), flush=True)


# ----------------------------------------------------------------------------- main

def main():
    args = parse()
    if args.traffic_write:
        traffic_write(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path is a "
              "single-GPU kernel set and this build launches no multi-GPU run.", file=sys.stderr)
        sys.exit(2)
    if os.environ.get("WORLD_SIZE", "1") not in ("", "1"):
        print("bench.py is single-process; WORLD_SIZE > 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import bitlinear_rmsnorm_absmax_amd as bl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.op == "ternarize":
        bench_ternarize(args, torch, bl, dev)
        return
    if args.op == "binary":
        bench_binary(args, torch, bl, dev)
        return
    if args.op == "grouped":
        bench_grouped(args, torch, bl, dev)
        return
    if args.op == "base3":
        bench_base3(args, torch, bl, dev)
        return
    if args.traffic_probe:
        args.no_rotate = True
    ops, meta, keep = build_plan(args, torch, bl, dev)
    if args.traffic_probe:
        traffic_probe(args, torch, ops, dev)
        return
    rec = RunAll()
    ops(0, rec)  # first launch of every kernel; records the calls of a step
    torch.cuda.synchronize()
    print(f"# workload {meta['workload']}: M={meta['M']} K={meta['K']} N={meta['N']}, "
          f"{meta['weight_copies']} weight copies", file=sys.stderr, flush=True)

    ncopy = meta["weight_copies"]
    s = torch.cuda.Stream(device=dev)

    def steps_graph(first, count):
        """One HIP graph of `count` consecutive steps (step i uses weight copy
        i mod ncopy): a single replay launches them all, so the host does not
        pace the GPU between steps."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(first, first + count):
                ops(i, RunAll())
        return g

    def run_steps(first, count):
        if count <= 0:
            return
        if args.eager:
            for i in range(first, first + count):
                ops(i, RunAll())
        else:
            steps_graph(first, count).replay()

    run_steps(0, args.warmup)
    timed = None if args.eager else steps_graph(args.warmup, args.steps)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    if timed is not None:
        timed.replay()
    else:
        run_steps(args.warmup, args.steps)
    e1.record()
    torch.cuda.synchronize()
    del timed
    ms_step = e0.elapsed_time(e1) / args.steps
    print(f"# timed {args.steps} steps: {ms_step * 1e3:.2f} us/step", file=sys.stderr, flush=True)

    # per-call durations: each call launched back to back, one launch per
    # weight copy, replayed from one HIP graph (eager: from the host)
    kern = {}
    for name, per_step in rec.calls.items():
        if args.eager:
            t = RunOne(torch, name)
            for i in range(args.steps):
                ops(args.warmup + i, t)
            avg = t.avg_us(args.steps * per_step)
        else:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for c in range(ncopy):
                    ops(c, lambda n, *a, **kw: n == name)
            reps = max(1, math.ceil(args.steps / ncopy))
            g.replay()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            avg = e0.elapsed_time(e1) * 1e3 / (reps * ncopy * per_step)
            del g
        kern[name] = dict(avg_us=avg, per_step=per_step, **rec.info.get(name, {}))
    print("# per-call GPU time (us): " + ", ".join(f"{k} {v['avg_us']:.2f}" for k, v in kern.items()),
          file=sys.stderr, flush=True)

    fwd = {k: v for k, v in kern.items() if "alg_bytes" in v}
    dom = max(fwd, key=lambda k: fwd[k]["avg_us"] * fwd[k]["per_step"])
    d = fwd[dom]
    traffic = read_traffic(meta["workload"], dom)
    if d["M"] >= 512:
        tops = d["ops"] / (d["avg_us"] * 1e-6) / 1e12
        roof = dict(bound="mfma", achieved=round(tops, 2), peak=INT8_PEAK_TOPS, unit="TOP/s",
                    frac=round(tops / INT8_PEAK_TOPS, 4), traffic=traffic)
    else:
        gbs = d["alg_bytes"] / (d["avg_us"] * 1e-6) / 1e9
        roof = dict(bound="hbm", achieved=round(gbs, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(gbs / HBM_PEAK_GBS, 4), traffic=traffic)
    roof.update(call=dom, kernel=d["kernel"], avg_launch_us=round(d["avg_us"], 3),
                alg_bytes_per_launch=d["alg_bytes"], ops_per_launch=d["ops"])

    cpu = cpu_baseline(args, args.cpu_seconds) if args.cpu_seconds > 0 else None

    value = meta["weight_bytes_per_step"] / (ms_step * 1e-3) / 1e9
    per_call = {}
    for k, v in kern.items():
        e = dict(avg_us=round(v["avg_us"], 3), per_step=v["per_step"])
        if "alg_bytes" in v:
            e.update(kernel=v["kernel"],
                     packed_w_GBs=round(v["wbytes"] / (v["avg_us"] * 1e-6) / 1e9, 1),
                     alg_GBs=round(v["alg_bytes"] / (v["avg_us"] * 1e-6) / 1e9, 1),
                     int8_eq_TOPS=round(v["ops"] / (v["avg_us"] * 1e-6) / 1e12, 2))
        per_call[k] = e
    line = {
        "metric": "BitLinear ternary GEMV/GEMM: packed-W GB/s (% HBM peak), int8-eq TOPS",
        "value": round(value, 2),
        "unit": "packed-W GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": meta["workload"], "M": meta["M"], "K": meta["K"], "N": meta["N"],
                   "weight_copies": meta["weight_copies"],
                   "timing": "eager" if args.eager else "hip_graph_of_all_timed_steps",
                   "fusion": "separate calls" if args.unfused else
                   "one-token quant_forward; GLU gate+up stacked",
                   "int8_eq_TOPS_per_step": round(meta["ops_per_step"] / (ms_step * 1e-3) / 1e12, 3),
                   "hbm_frac_per_step": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_call": per_call,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
