#!/usr/bin/env python3
"""Throughput of the ternary BitLinear hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5] [--configs 1,2,3,4]

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
host launch overhead does not pace the GPU.  Per-call durations come from
three further passes: the in-step durations (the same K steps once more,
eager, queued behind a spin kernel so that they run back to back, with a
timing event between consecutive calls on their stream; HIP graphs here do
not time events recorded inside them), the back-to-back time (a HIP graph of
that call alone, once per weight copy, replayed between two events), and
per-launch durations (each launch of the call alone between two events):
mean, median, p10 and p90.  The dominant forward call's back-to-back time
gives the roofline (the fraction from its in-step durations rides along: a
long MFMA kernel runs cooler between the memory-bound calls of a step, while
every in-step duration also carries an event's cost of a few microseconds);
the floors are an empty launch and a read-only pass over the same weight
bytes.
The headline workload is the large-shape sweep (K=8192, N=28672, M in
{1, 8, 64, 512}); the other four workloads are measured the same way into the
line's "configs" record.

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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=5, choices=sorted(workloads.WORKLOADS),
                    help="the headline workload (default 5: the large-shape sweep K=8192 "
                         "N=28672, M in {1, 8, 64, 512}, the largest that fits one GPU)")
    ap.add_argument("--configs", default="1,2,3,4",
                    type=lambda v: [] if v in ("", "none") else [int(c) for c in v.split(",")],
                    help="workloads measured as sub-records under 'configs' (none: skip)")
    ap.add_argument("--sub-steps", type=int, default=50, help="timed steps of each sub-record")
    ap.add_argument("--per-launch", type=int, default=50,
                    help="event-bracketed launches per call for the per-launch statistics")
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
    ap.add_argument("--trace-summary", nargs=2, metavar=("TRACE_DIR", "COMMAND"),
                    help="no GPU: write profiles/kernels_<workload>.md from a rocprofv3 "
                         "--kernel-trace run of COMMAND (a bench.py command line with the same "
                         "step, warmup, per-launch and config arguments as this one)")
    ap.add_argument("--traffic-write", nargs="+", metavar="PATH",
                    help="no GPU: JSON FETCH_DIR WRITE_DIR [MFMA_DIR]: turn the counter runs of "
                         "--traffic-probe into profiles/traffic_<workload>.md")
    return ap.parse_args()


def forward1_kernel(M: int, K: int, N: int) -> str:
    """The kernel bitlinear_forward1 runs for M tokens (its dispatch, for the
    bench shapes, whose activation block fits LDS)."""
    one_token = M == 1 and K >= 4096 and K % 1024 == 0 and N // 64 >= 150
    decode = (M >= 5 or (M >= 2 and K >= 4096) or one_token) and K % 512 == 0
    return "decode_lds_kernel" if decode else "gemv1_kernel"


def forward3_kernel(M: int, K: int) -> str:
    """The kernel bitlinear_forward3 runs for M tokens (its dispatch)."""
    steps = (-(-K // 80) + 3) // 4
    fits = M * (20 * steps + 1) * 16 <= 144 * 1024
    return "gemv3_mfma_kernel" if 2 <= M <= 16 and fits else "gemv3_kernel"


def quant_forward_kernel(M: int, K: int, N: int) -> str:
    """Kernel of bitlinear_quant_forward when it runs as one launch (one
    token): the MFMA decode kernel on long rows over many row tiles, else the
    VALU fused kernel."""
    lds_fits = ((M * K + 1023) // 1024) * 1024 + 16384 + 128 <= 160 * 1024
    decode = M == 1 and K >= 4096 and K % 512 == 0 and N // 64 >= 150 and lds_fits
    return "decode_lds_kernel" if decode else "quant_gemv_kernel"


def forward_kernel(M: int, K: int, N: int) -> str:
    """Kernel that bitlinear_forward picks (the library's dispatch)."""
    lds_fits = K % 256 == 0 and ((M * K + 1023) // 1024) * 1024 + 16384 + 128 <= 160 * 1024
    if M == 1:
        one_token_decode = K >= 4096 and K % 512 == 0 and N // 64 >= 150 and lds_fits
        return "decode_lds_kernel" if one_token_decode else "gemv_valu_kernel"
    if (5 <= M <= 16 or (2 <= M <= 4 and K >= 4096)) and lds_fits:
        return "decode_lds_kernel"
    if M <= 16 or (M <= 32 and not (-(-N // 128) >= 128 and K % 256 == 0)):
        return "skinny_mfma_kernel"
    if K % 128 != 0:
        return "gemm_mfma_kernel"
    # the LDS-ring kernel: 128 x 256 tiles (M >= 256 and at least 256 such
    # tiles); at most 256 tiles of 64 x 128 with K % 256 == 0: the two K
    # groups sharing each weight copy (gemm_pair_kernel); else 128 x 128
    wide = -(-M // 128) * -(-N // 256)
    tiles64 = -(-M // 64) * -(-N // 128)
    if not (M >= 256 and wide >= 256) and tiles64 <= 256 and K % 256 == 0:
        return "gemm_pair_kernel"
    return "gemm_dma_kernel"


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


def build_plan(args, torch, bl, dev, wid):
    """Returns (ops, meta, keepalive): ops(step_idx, timer) launches one step."""
    wl = workloads.WORKLOADS[wid]
    rotate = not args.no_rotate
    lib = bl.lib

    def stream():
        return torch.cuda.current_stream(dev).cuda_stream

    def check(st):
        if st != 0:
            raise RuntimeError(bl.last_error())

    def fused(M, K, N):
        # bitlinear_quant_forward as one kernel (one token; --unfused times the
        # two calls instead)
        return not args.unfused and lib.bitlinear_quant_forward_one_launch(M, K, N) == 1

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
                               4 * M * D + 4 * D, quant_forward_kernel(M, D, 2 * Fh)):
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

        operands = {}
        for b in bufs:
            M = b["M"]
            if stacked:
                operands[f"forward_gateup_M{M}"] = (b["q"], layers[0].copies[0], M, D, 2 * Fh)
            else:
                operands[f"forward_gate_M{M}"] = (b["q"], layers[0].copies[0], M, D, Fh)
                operands[f"forward_up_M{M}"] = (b["q"], layers[1].copies[0], M, D, Fh)
            operands[f"forward_down_M{M}"] = (b["hq"], layers[-1].copies[0], M, Fh, D)
        meta.update(weight_bytes_per_step=sum(L.wbytes for L in layers) * len(wl.ms),
                    weight_copies=ncopy, operands=operands,
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
                if run(f"quant_forward_M{M}", M, N, K, L.wbytes, xb, quant_forward_kernel(M, K, N)):
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
                ops_per_step=sum(2 * M * N * K for M in wl.ms),
                operands={f"forward_M{b['M']}": (b["q"], L.copies[0], b["M"], K, N) for b in bufs})
    return ops, meta, (L, bufs)


# ----------------------------------------------------------------------------- traffic

# The traffic summaries are valid only for the kernel sources they were taken
# on: every source file of the library (kernels, shared headers, the ABI's
# dispatch) enters the digest.
def _library_sources():
    csrc = os.path.join(ROOT, "bitlinear_rmsnorm_absmax_amd", "csrc")
    return sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".h", ".cpp")))


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bitlinear_rmsnorm_absmax_amd", "csrc")
    for f in _library_sources():
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


def read_mfma_util(workload_name: str, call: str):
    """Matrix-pipe utilisation of `call` from the committed counter summary,
    only if it was taken on the current kernel sources (else None)."""
    path = os.path.join(PROFILES, f"traffic_{workload_name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source_digest:\s*(\w+)", text)
    m_val = re.search(rf"mfma_util\[{re.escape(call)}\]:\s*([0-9.eE+]+)", text)
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
    rec = RunAll()

    def run(name, *a, **kw):
        seq.append(name)
        return rec(name, *a, **kw)
    ops(0, run)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    info = {k: dict(ops=v["ops"], alg_bytes=v["alg_bytes"]) for k, v in rec.info.items()}
    with open(args.traffic_probe, "w") as f:
        json.dump(dict(workload=workloads.WORKLOADS[args.workload].name, calls=seq,
                       copy_bytes=COPY_BYTES, copy_kernel="neg", info=info), f)


def _counter_rows(d: str, counter: str, reduce: str = "sum"):
    """[(kernel name, value)] per dispatch, in dispatch order: the counter's
    instances summed, or (reduce="duration") the dispatch's duration in
    microseconds from its timestamps."""
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
            name, v = per.get(did, (r["Kernel_Name"], None))
            if reduce == "duration":
                v = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
            else:
                x = float(r["Counter_Value"])
                v = x if v is None else v + x
            per[did] = (name, v)
    return [per[k] for k in sorted(per)]


# SQ_VALU_MFMA_BUSY_CYCLES counts, per SIMD, the cycles its matrix pipe is
# occupied: one 32x32x32 int8 MFMA (65536 operations) occupies it 32 cycles,
# so the busy cycles are the operations / 2048 per SIMD, independent of
# stalls; the utilisation is those cycles over the dispatch's duration at the
# 2.4 GHz peak engine clock (GRBM_GUI_ACTIVE is recorded too; under counter
# collection it also counts the collection's own cycles).
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_I8", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
SIMD_NUM = 256 * 4
PEAK_CLOCK_MHZ = 2400.0


def traffic_write(args):
    """profiles/traffic_<workload>.md from the FETCH_SIZE and WRITE_SIZE runs of
    --traffic-probe: the last dispatches of each run are the probe's step and
    its copy; the counters (KiB per dispatch) are scaled by what they read for
    the copy of known size."""
    probe_json, fdir, wdir = args.traffic_write[:3]
    mdir = args.traffic_write[3] if len(args.traffic_write) > 3 else None
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
            if call.startswith("quant_forward"):
                ok = "quant_gemv" in name or "decode_lds" in name
            elif call.startswith(("quant", "silu")):
                ok = any(k in name for k in ("quant_rows", "quant_split", "quant_f32"))
            else:
                ok = "_kernel" in name and "quant_" not in name
            if not ok:
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
             *([f"rocprofv3 --pmc {' '.join(MFMA_COUNTERS)} --output-format csv -d "
                f"gpurun_out/pmc_mfma -o run -- python3 bench.py --workload {args.workload} "
                "--traffic-probe gpurun_out/probe.json"] if mdir else []),
             f"python3 bench.py --workload {args.workload} --traffic-write gpurun_out/probe.json "
             "gpurun_out/pmc_fetch gpurun_out/pmc_write" + (" gpurun_out/pmc_mfma" if mdir else ""),
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
    mvals = []
    if mdir:
        mo = pick(_counter_rows(mdir, MFMA_COUNTERS[0]))[0]
        mb = pick(_counter_rows(mdir, MFMA_COUNTERS[1]))[0]
        md = pick(_counter_rows(mdir, MFMA_COUNTERS[1], "duration"))[0]
        info = probe.get("info", {})
        lines += ["", "MFMA counters (third run of the probe: `--pmc " + " ".join(MFMA_COUNTERS) +
                  "`): int8 MFMA operations (SQ_INSTS_VALU_MFMA_MOPS_I8 x 512, against the "
                  "algorithmic 2*M*N*K; decode kernels pad M to their 16-row MFMA tile), the "
                  "matrix pipe's busy cycles per SIMD (SQ_VALU_MFMA_BUSY_CYCLES summed over "
                  f"{SIMD_NUM} SIMDs / {SIMD_NUM}: operations / 2048 per SIMD, independent of "
                  "stalls), the dispatch's duration in the same run, and the utilisation: busy "
                  f"cycles / (duration x {PEAK_CLOCK_MHZ / 1000:.1f} GHz peak clock).", "",
                  "| call | MFMA ops | 2*M*N*K | busy cycles per SIMD | duration us | MFMA util at peak clock |",
                  "|---|---:|---:|---:|---:|---:|"]
        for call, (_, ops), (_, busy), (_, dur) in zip(calls, mo, mb, md):
            if ops <= 0:
                continue
            alg = info.get(call, {}).get("ops", 0)
            per_simd = busy / SIMD_NUM
            util = per_simd / (dur * PEAK_CLOCK_MHZ) if dur > 0 else 0.0
            lines.append(f"| {call} | {ops * 512:.4g} | {alg:.4g} | {per_simd:.4g} | {dur:.2f} | "
                         f"{100 * util:.1f} % |")
            mvals.append((call, util))
    lines += ["", f"source_digest: {kernel_source_digest()}", ""]
    lines += [f"traffic_bytes_per_launch[{c}]: {b:.6g}" for c, b in vals]
    lines += [f"mfma_util[{c}]: {u:.4f}" for c, u in mvals]
    path = os.path.join(PROFILES, f"traffic_{wl.name}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


# ----------------------------------------------------------------------------- trace summary

def _phase_counts(wid, steps, warmup, per_launch, ncopy):
    """Launches of one call in a bench run, in order: the first step, the
    warmup graph, the timed graph, the in-step event pass (the timed steps
    again, eager, an event between consecutive calls), the back-to-back graph
    (its first replay, then the timed replays) and the per-launch event
    pairs."""
    reps = max(1, math.ceil(steps / ncopy))
    return [("first", 1), ("warmup", warmup), ("timed steps", steps), ("in-step events", steps),
            ("back-to-back first", ncopy), ("back-to-back", reps * ncopy),
            ("per-launch events", per_launch)]


def trace_summary(args):
    """profiles/kernels_<workload>.md from a `rocprofv3 --kernel-trace --stats`
    run of bench.py: per kernel and grid, every dispatch's duration (mean,
    median, p10, p90) and, where the count matches one workload's launch
    pattern, the same split by bench phase."""
    import csv
    import glob
    d, cmd = args.trace_summary
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one kernel_trace.csv under {d}, found {files}")
    rows = list(csv.DictReader(open(files[0])))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    # each workload's measurement ends with its floor kernels, so the runs of
    # floor dispatches cut the trace into the workloads, in bench order
    wids = [args.workload] + [c for c in args.configs if c != args.workload]
    wi, in_floor = 0, False
    groups = {}
    for r in rows:
        name = r["Kernel_Name"].replace("(anonymous namespace)::", "").replace("void ", "")
        name = name[:name.index(">(") + 1] if ">(" in name else name.split("(")[0]
        is_floor = "floor_" in name
        if in_floor and not is_floor and "bl::" in name:
            wi += 1
        in_floor = is_floor or (in_floor and "bl::" not in name)
        w = wids[min(wi, len(wids) - 1)]
        key = (workloads.WORKLOADS[w].name, name, int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)

    def stats(v):
        a = np.array(v)
        return (f"{len(a)} | {a.mean():.2f} | {np.median(a):.2f} | "
                f"{np.percentile(a, 10):.2f} | {np.percentile(a, 90):.2f}")

    def pattern(wid, count):
        """the launch pattern of the k calls of workload wid that share one
        kernel and grid, with `count` dispatches in all: (label, dispatches)
        in trace order.  The steps launch the k calls in turn (first step,
        warmup and timed graphs and the in-step pass hold k dispatches a
        step); then each call has its own back-to-back graph and per-launch
        pairs, one call after the other."""
        head = wid == args.workload
        steps = args.steps if head else args.sub_steps
        warm = args.warmup if head else max(2, args.warmup // 4)
        # the weight copies the bench rotates through for this workload
        # (packed bytes of the largest weight matrix; GLU: the stacked gate
        # and up rows), tried first, so that a count two readings fit is
        # read with the right one
        wl = workloads.WORKLOADS[wid]
        rows = 2 * wl.glu_f if wl.glu_f else wl.N
        expect = max(1, math.ceil(ROTATE_BYTES / (rows * wl.K // 4)))
        tries = [(k, expect) for k in range(1, 5)] + \
            [(k, n) for k in range(1, 5) for n in range(1, 1024) if n != expect]
        for k, ncopy in tries:
            pat = _phase_counts(wid, steps, warm, args.per_launch, ncopy)
            if count % k or sum(c for _, c in pat) != count // k:
                continue
            if k == 1:
                return pat
            shared = [(lab if lab not in ("timed steps", "in-step events") else f"{lab} ({k} calls)",
                       k * c) for lab, c in pat[:4]]
            own = [(f"{lab} (call {j + 1} of {k})", c) for j in range(k) for lab, c in pat[4:]]
            return shared + own
        return None

    lines = [f"# Kernel trace: `{cmd}`", "",
             "Command (repository root; `cd /tmp && export TMPDIR=/tmp` first, paths relative to "
             "the repository):", "", "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/trace -o bench -- "
             f"{cmd}",
             f"python3 bench.py --trace-summary gpurun_out/trace \"{cmd}\"", "```", "",
             "Durations in microseconds from the kernel trace (end - start of each dispatch), per "
             "workload (in bench order; each one's floor kernels close it), kernel and grid size.", "",
             "| workload | kernel | grid | workgroup | dispatches | mean | median | p10 | p90 |",
             "|---|---|---:|---:|---:|---:|---:|---:|---:|"]
    order = sorted(groups.items(), key=lambda kv: (wids.index(next(
        w for w in wids if workloads.WORKLOADS[w].name == kv[0][0])), -sum(kv[1])))
    for (wname, name, grid, wg), v in order:
        if "bl::" not in name:
            continue
        lines.append(f"| {wname} | `{name}` | {grid} | {wg} | {stats(v)} |")
    lines += ["", "By bench phase (library calls of the measured steps: the timed steps graph, "
              "the in-step event pass (the same steps, eager, an event between consecutive "
              "calls), the back-to-back graph of each call alone that bench.py's avg_launch_us "
              "comes from, and the per-launch event pairs):", "",
              "| workload | kernel | grid | phase | dispatches | mean | median | p10 | p90 |",
              "|---|---|---:|---|---:|---:|---:|---:|---:|"]
    for (wname, name, grid, wg), v in order:
        if "bl::" not in name or "floor_" in name:
            continue
        wid = next(w for w in wids if workloads.WORKLOADS[w].name == wname)
        pat = pattern(wid, len(v))
        if pat is None:
            continue
        i = 0
        for lab, c in pat:
            if lab.startswith(("timed steps", "in-step events", "back-to-back", "per-launch events")) \
                    and not lab.startswith("back-to-back first") and c > 0:
                lines.append(f"| {wname} | `{name}` | {grid} | {lab} | {stats(v[i:i + c])} |")
            i += c
    out = os.path.join(PROFILES, f"kernels_{workloads.WORKLOADS[args.workload].name}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


# ----------------------------------------------------------------------------- cpu baseline

def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wid: int, seconds: float, threads: int = 0):
    """The oracle (plain C loops, OpenMP over outputs) on the same workload,
    whole steps, for about ``seconds`` of CPU time; ``threads`` > 0 pins the
    oracle's thread count (1: the one-core timing), 0 leaves it at the
    host's cores."""
    import oracle
    wl = workloads.WORKLOADS[wid]
    default_threads = oracle.num_threads()
    if threads > 0:
        oracle.set_num_threads(threads)
    try:
        nthr = oracle.num_threads()
        if wl.glu_f:
            wg, wu, wd = workloads.glu_weights(wid)
            betas = workloads.glu_betas(wid)
            gain = np.ones(wl.K, np.float32)
            ms = list(wl.ms) if threads != 1 else [m for m in wl.ms if m == 1]
            xs = [workloads.workload_activations(wid, M) for M in ms]
            wbytes = (wg.size + wu.size + wd.size) // 4 * len(ms)

            def step():
                for x in xs:
                    oracle.glu(x, wg, wu, wd, betas, gain, wl.rms_eps)
            desc = "GLU chain"
        else:
            w = workloads.workload_weights(wid)
            beta = workloads.workload_beta(wid)
            ms = list(wl.ms)
            xs = []
            for M in ms:
                x = workloads.workload_activations(wid, M)
                xs.append(oracle.bf16_to_f32(x) if wl.act == "normal_bf16" else x)
            rows = w.shape[0]
            # large workloads: a bounded slice of output rows (same K, same M sweep)
            est = sum(x.shape[0] for x in xs) * w.size * 1.5e-9  # ~1.5 ns per MAC and thread
            if est / max(nthr, 1) > seconds:
                rows = max(64, int(rows * seconds * nthr / est / 3))
                w = np.ascontiguousarray(w[:rows])
            wbytes = w.size // 4 * len(ms)

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
    finally:
        oracle.set_num_threads(default_threads)
    return dict(value=round(wbytes * n / el / 1e9, 4), unit="packed-W GB/s",
                cores=nthr, kind="oracle", cpu_model=cpu_model(),
                host_cores=len(os.sched_getaffinity(0)),
                sample=f"{n} x ({desc}), M={ms}, {el:.1f} s")


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
                         kernel=forward1_kernel(int(dom.split("M")[-1]), K, N),
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


# ----------------------------------------------------------------------------- timing

SPIN_CYCLES = 20_000_000   # ~8-10 ms of shader clock: the host queues all launches meanwhile


def launch_stats(torch, s, launch, n):
    """Per-launch durations of ``launch(i)``, i = 0..n-1: each launch sits
    between two timing events on stream ``s``; a spin kernel ahead of them
    holds the stream until the host has queued every launch, so the GPU runs
    them back to back and each event pair brackets exactly one launch (the
    events also keep consecutive launches from overlapping).  Returns mean,
    median, p10, p90 in microseconds."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        torch.cuda._sleep(SPIN_CYCLES)
        for i in range(n):
            ev[i][0].record(s)
            launch(i)
            ev[i][1].record(s)
    torch.cuda.synchronize()
    d = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return dict(avg_us=float(d.mean()), median_us=float(np.median(d)),
                p10_us=float(np.percentile(d, 10)), p90_us=float(np.percentile(d, 90)),
                launches=n)


def in_step_stats(torch, s, ops, first, count, chunk=20):
    """Per-call durations inside whole steps: steps first .. first+count-1
    launched again in step order on stream ``s`` (the timed steps' weight
    copies and call sequence), with one timing event between consecutive
    calls, so each call's duration is the time between the events around it.
    The steps go in chunks of ``chunk``, each queued behind a spin kernel so
    that the GPU runs its calls back to back, as in the timed graph.  Returns
    {call: [durations in us]} and the per-step sums of the durations."""
    durs, sums = {}, []
    torch.cuda.synchronize()
    for c0 in range(first, first + count, chunk):
        marks = []

        def mark(name, *a, **kw):
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(s)
            marks.append((name, ev))
            return True

        with torch.cuda.stream(s):
            torch.cuda._sleep(SPIN_CYCLES)
            for i in range(c0, min(c0 + chunk, first + count)):
                ops(i, mark)
                mark(None)  # closes the step's last call; the next step's first mark is not used
        torch.cuda.synchronize()
        step = 0.0
        for (name, e0), (_, e1) in zip(marks, marks[1:]):
            if name is None:
                sums.append(step)
                step = 0.0
                continue
            us = e0.elapsed_time(e1) * 1e3
            durs.setdefault(name, []).append(us)
            step += us
    return durs, sums


def floors(torch, bl, dev, s, nbytes, n=50, mfma=None):
    """The empty-launch floor and a read-only pass over ``nbytes`` (weight
    copies rotated as the layer's own calls rotate them); with ``mfma`` =
    (x_q, w_packed, M, K, N) of a product, also the register-only MFMA floor
    of that product (bitlinear_floor_mfma on its own operands)."""
    lib = bl.lib
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    nb = nbytes // 16 * 16
    copies = max(1, math.ceil(ROTATE_BYTES / max(nb, 1)))
    buf = torch.empty((copies, nb), dtype=torch.uint8, device=dev)
    buf.fill_(0x5A)

    def empty(i):
        if lib.bitlinear_floor_empty(torch.cuda.current_stream(dev).cuda_stream) != 0:
            raise RuntimeError(bl.last_error())

    def read(i):
        if lib.bitlinear_floor_stream_read(buf[i % copies].data_ptr(), nb, sink.data_ptr(),
                                           torch.cuda.current_stream(dev).cuda_stream) != 0:
            raise RuntimeError(bl.last_error())

    def b2b(fn):
        """back-to-back: one graph of one launch per copy, replayed between events"""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for c in range(copies):
                fn(c)
        reps = max(1, math.ceil(n / copies))
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * copies)

    read(0)
    e = launch_stats(torch, s, empty, n)
    r = launch_stats(torch, s, read, n)
    eb, rb = b2b(empty), b2b(read)
    del buf
    out = dict(empty_launch_b2b_us=round(eb, 3), stream_read_b2b_us=round(rb, 3),
               empty_launch_event_us=round(e["median_us"], 3),
               stream_read_event_us=round(r["median_us"], 3),
               stream_read_bytes=nb,
               stream_read_GBs=round(nb / (rb * 1e-6) / 1e9, 1),
               stream_read_frac_of_peak=round(nb / (rb * 1e-6) / 1e9 / HBM_PEAK_GBS, 4))
    if mfma is not None and mfma[3] % 128 == 0:
        q, w, M, K, N = mfma

        def mf(i):
            if lib.bitlinear_floor_mfma(q.data_ptr(), M, K, w.data_ptr(), N, sink.data_ptr(),
                                        torch.cuda.current_stream(dev).cuda_stream) != 0:
                raise RuntimeError(bl.last_error())

        mf(0)
        mb = b2b(mf)
        tops = 2 * M * N * K / (mb * 1e-6) / 1e12
        out.update(mfma_floor_b2b_us=round(mb, 3), mfma_floor_TOPS=round(tops, 1),
                   mfma_floor_frac_of_peak=round(tops / INT8_PEAK_TOPS, 4),
                   mfma_floor_shape=[M, K, N])
    return out


def measure_workload(args, torch, bl, dev, wid, steps, warmup, per_launch, headline):
    """One workload: the K-step graph time, every call's back-to-back time
    (a graph of that call alone, once per weight copy) and its per-launch
    event-bracketed durations, the dominant forward call's roofline and the
    same-byte floors.  Returns a dict (the bench line's body)."""
    ops, meta, keep = build_plan(args, torch, bl, dev, wid)
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

    if args.eager:
        for i in range(warmup):
            ops(i, RunAll())
    elif warmup > 0:
        steps_graph(0, warmup).replay()
    timed = None if args.eager else steps_graph(warmup, steps)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    if timed is not None:
        timed.replay()
    else:
        for i in range(warmup, warmup + steps):
            ops(i, RunAll())
    e1.record()
    torch.cuda.synchronize()
    del timed
    ms_step = e0.elapsed_time(e1) / steps
    print(f"# timed {steps} steps: {ms_step * 1e3:.2f} us/step", file=sys.stderr, flush=True)
    # the durations of the calls inside the steps: the timed steps once more,
    # eager, with an event between consecutive calls
    ins, ins_sums = in_step_stats(torch, s, ops, warmup, steps)

    kern = {}
    for name, per_step in rec.calls.items():
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for c in range(ncopy):
                ops(c, lambda n, *a, **kw: n == name)
        reps = max(1, math.ceil(steps / ncopy))
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        b2b = e0.elapsed_time(e1) * 1e3 / (reps * ncopy * per_step)
        del g
        st = launch_stats(torch, s, lambda i, name=name: ops(i, lambda n, *a, **kw: n == name),
                          per_launch)
        st = {k: v / per_step if k.endswith("_us") else v for k, v in st.items()}
        d_in = np.array(ins[name])
        kern[name] = dict(b2b_us=b2b, per_step=per_step, **st, **rec.info.get(name, {}),
                          in_step=dict(mean_us=float(d_in.mean()), median_us=float(np.median(d_in)),
                                       p10_us=float(np.percentile(d_in, 10)),
                                       p90_us=float(np.percentile(d_in, 90)), launches=len(d_in)))
    print("# per-call GPU time (us, in-step mean | per-launch mean | back-to-back): " +
          ", ".join(f"{k} {v['in_step']['mean_us']:.2f} | {v['avg_us']:.2f} | {v['b2b_us']:.2f}"
                    for k, v in kern.items()),
          file=sys.stderr, flush=True)

    fwd = {k: v for k, v in kern.items() if "alg_bytes" in v}
    dom = max(fwd, key=lambda k: fwd[k]["b2b_us"] * fwd[k]["per_step"])
    d = fwd[dom]
    floor = floors(torch, bl, dev, s, d["wbytes"], per_launch,
                   mfma=meta["operands"].get(dom) if d["M"] >= 512 else None)
    traffic = read_traffic(meta["workload"], dom)
    roof = roofline_of(d, traffic, floor)
    if roof["bound"] == "mfma":
        roof["mfma_util_counter"] = read_mfma_util(meta["workload"], dom)
    per_call = {}
    for k, v in kern.items():
        e = dict(avg_us=round(v["b2b_us"], 3), per_step=v["per_step"],
                 in_step_events={a: (round(b, 3) if a.endswith("_us") else b)
                                 for a, b in v["in_step"].items()},
                 per_launch_events=dict(mean_us=round(v["avg_us"], 3),
                                        median_us=round(v["median_us"], 3),
                                        p10_us=round(v["p10_us"], 3), p90_us=round(v["p90_us"], 3)))
        if "alg_bytes" in v:
            r = roofline_of(v, read_traffic(meta["workload"], k), None)
            us = v["b2b_us"]
            e.update(kernel=v["kernel"],
                     packed_w_GBs=round(v["wbytes"] / (us * 1e-6) / 1e9, 1),
                     alg_GBs=round(v["alg_bytes"] / (us * 1e-6) / 1e9, 1),
                     int8_eq_TOPS=round(v["ops"] / (us * 1e-6) / 1e12, 2),
                     bound=r["bound"], frac=r["frac"])
        per_call[k] = e
    value = meta["weight_bytes_per_step"] / (ms_step * 1e-3) / 1e9
    del keep
    torch.cuda.empty_cache()
    return dict(
        value=round(value, 2), ms_per_step=round(ms_step, 5), steps=steps, warmup=warmup,
        config={"workload": meta["workload"], "M": meta["M"], "K": meta["K"], "N": meta["N"],
                "weight_copies": meta["weight_copies"],
                "in_step_sum_us": round(float(np.mean(ins_sums)), 3),
                "timing": "eager" if args.eager else "hip_graph_of_all_timed_steps",
                "fusion": "separate calls" if args.unfused else
                "one-token quant_forward; GLU gate+up stacked",
                "int8_eq_TOPS_per_step": round(meta["ops_per_step"] / (ms_step * 1e-3) / 1e12, 3),
                "hbm_frac_per_step": round(value / HBM_PEAK_GBS, 4)},
        roofline=roof, floor=floor, per_call=per_call)


def roofline_of(d, traffic, floor):
    """Roofline of one forward call from its average launch duration, the
    back-to-back time (HIP events around a graph of that call's launches on
    its stream, divided by the launch count): int8 MFMA for 512 tokens and
    more (2*M*N*K ops), HBM bytes otherwise (packed W + x_q + gamma + y, + the
    fp32/bf16 rows a fused call reads).  The same fraction from the in-step
    event pass (the call between the other calls of the timed steps, where a
    long MFMA kernel runs cooler and so faster than back to back, but each
    duration also carries an event's own cost of about 3-4 us) and the
    per-launch event statistics ride along."""
    us, ins = d["b2b_us"], d["in_step"]["mean_us"]
    if d["M"] >= 512:
        tops = d["ops"] / (us * 1e-6) / 1e12
        roof = dict(bound="mfma", achieved=round(tops, 2), peak=INT8_PEAK_TOPS, unit="TOP/s",
                    frac=round(tops / INT8_PEAK_TOPS, 4), traffic=traffic,
                    frac_in_step=round(d["ops"] / (ins * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4))
        if floor and "mfma_floor_b2b_us" in floor:
            roof["frac_of_mfma_floor"] = round(floor["mfma_floor_b2b_us"] / us, 4)
    else:
        gbs = d["alg_bytes"] / (us * 1e-6) / 1e9
        roof = dict(bound="hbm", achieved=round(gbs, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(gbs / HBM_PEAK_GBS, 4), traffic=traffic,
                    frac_in_step=round(d["alg_bytes"] / (ins * 1e-6) / 1e9 / HBM_PEAK_GBS, 4))
        if floor:
            roof["frac_of_stream_read"] = round(floor["stream_read_b2b_us"] / us, 4)
    roof.update(call=None, kernel=d["kernel"], avg_launch_us=round(us, 3),
                in_step_events={a: (round(b, 3) if a.endswith("_us") else b)
                                for a, b in d["in_step"].items()},
                per_launch_events=dict(mean_us=round(d["avg_us"], 3),
                                       median_us=round(d["median_us"], 3),
                                       p10_us=round(d["p10_us"], 3), p90_us=round(d["p90_us"], 3),
                                       launches=d["launches"]),
                alg_bytes_per_launch=d["alg_bytes"], ops_per_launch=d["ops"])
    return roof


# ----------------------------------------------------------------------------- main

METRIC = "BitLinear ternary GEMV/GEMM: packed-W GB/s (% HBM peak), int8-eq TOPS"


def main():
    args = parse()
    if args.traffic_write:
        traffic_write(args)
        return
    if args.trace_summary:
        trace_summary(args)
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
        ops, meta, keep = build_plan(args, torch, bl, dev, args.workload)
        traffic_probe(args, torch, ops, dev)
        return

    head = measure_workload(args, torch, bl, dev, args.workload, args.steps, args.warmup,
                            args.per_launch, True)
    dom = max((k for k, v in head["per_call"].items() if "kernel" in v),
              key=lambda k: head["per_call"][k]["avg_us"] * head["per_call"][k]["per_step"])
    head["roofline"]["call"] = dom
    sub = {}
    for wid in args.configs:
        if wid == args.workload:
            continue
        r = measure_workload(args, torch, bl, dev, wid, args.sub_steps, max(2, args.warmup // 4),
                             args.per_launch, False)
        r["roofline"]["call"] = max((k for k, v in r["per_call"].items() if "kernel" in v),
                                    key=lambda k: r["per_call"][k]["avg_us"] *
                                    r["per_call"][k]["per_step"])
        if wid in (1, 2, 4) and args.cpu_seconds > 0:
            r["cpu_baseline_1core"] = cpu_baseline(wid, min(3.0, args.cpu_seconds), threads=1)
        sub[str(wid)] = r
    cpu = cpu_baseline(args.workload, args.cpu_seconds) if args.cpu_seconds > 0 else None
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "packed-W GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "floor": head["floor"],
        "cpu_baseline": cpu,
        "per_call": head["per_call"],
        "configs": sub,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
