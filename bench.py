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
Timed steps are replays of HIP graphs (one per weight copy), so host launch
overhead does not pace the GPU.  Per-call kernel durations come from a second
pass that launches each call of the step back to back `steps` times between
two HIP events on its stream; the dominant forward call gives the roofline.

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
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--no-rotate", action="store_true", help="one weight copy (warm cache)")
    ap.add_argument("--eager", action="store_true", help="time eager launches, no graphs")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the oracle CPU baseline (0 = skip)")
    return ap.parse_args()


def forward_kernel(M: int, K: int) -> str:
    """Kernel that bitlinear_forward picks for M (the library's dispatch)."""
    if M <= 2:
        return "gemv_valu_kernel"
    if M <= 32:
        return "skinny_mfma_kernel"
    return "gemm_dma_kernel" if K % 128 == 0 else "gemm_mfma_kernel"


# ----------------------------------------------------------------------------- timers

class RunAll:
    """Runs every call; records how often each call occurs per step."""

    def __init__(self):
        self.calls = {}
        self.info = {}

    def __call__(self, name, M=0, N=0, K=0, wbytes=0):
        self.calls[name] = self.calls.get(name, 0) + 1
        if wbytes:
            # algorithmic bytes of one forward launch: packed W + x_q + gamma + y
            self.info[name] = dict(alg_bytes=wbytes + M * K + 4 * M + 4 * M * N,
                                   ops=2 * M * N * K, wbytes=wbytes, M=M, N=N, K=K,
                                   kernel=forward_kernel(M, K))
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

    meta = {"workload": wl.name, "K": wl.K, "N": wl.N, "M": list(wl.ms)}
    if wl.glu_f:
        wg, wu, wd = workloads.glu_weights(wid)
        bg, bu, bd = workloads.glu_betas(wid)
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
                hq=torch.empty((M, Fh), dtype=torch.int8, device=dev),
                gh=torch.empty(M, device=dev), y=torch.empty((M, D), device=dev)))

        def ops(step, run):
            c = step % ncopy
            for b in bufs:
                M = b["M"]
                if run(f"quant_act_rms_M{M}"):
                    check(lib.bitlinear_quant_act(b["x"].data_ptr(), bl.F32, M, D, gain.data_ptr(),
                                                  wl.rms_eps, b["q"].data_ptr(), b["g"].data_ptr(),
                                                  stream()))
                for nm, L, out in (("gate", layers[0], b["yg"]), ("up", layers[1], b["yu"])):
                    if run(f"forward_{nm}_M{M}", M, L.N, L.K, L.wbytes):
                        check(lib.bitlinear_forward(b["q"].data_ptr(), b["g"].data_ptr(), M, D,
                                                    L.copies[c].data_ptr(), Fh, L.beta,
                                                    out.data_ptr(), None, stream()))
                if run(f"silu_mul_quant_M{M}"):
                    check(lib.bitlinear_silu_mul_quant(b["yg"].data_ptr(), b["yu"].data_ptr(), M, Fh,
                                                       None, b["hq"].data_ptr(), b["gh"].data_ptr(),
                                                       stream()))
                L = layers[2]
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

def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bitlinear_rmsnorm_absmax_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
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


# ----------------------------------------------------------------------------- main

def main():
    args = parse()
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
    ops, meta, keep = build_plan(args, torch, bl, dev)
    rec = RunAll()
    ops(0, rec)  # first launch of every kernel; records the calls of a step
    torch.cuda.synchronize()
    print(f"# workload {meta['workload']}: M={meta['M']} K={meta['K']} N={meta['N']}, "
          f"{meta['weight_copies']} weight copies", file=sys.stderr, flush=True)

    ncopy = meta["weight_copies"]
    graphs = None
    if not args.eager:
        graphs = []
        s = torch.cuda.Stream(device=dev)
        for c in range(ncopy):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                ops(c, RunAll())
            graphs.append(g)
        torch.cuda.synchronize()

    def run(i):
        if graphs is not None:
            graphs[i % ncopy].replay()
        else:
            ops(i, RunAll())

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        run(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    print(f"# timed {args.steps} steps: {ms_step * 1e3:.2f} us/step", file=sys.stderr, flush=True)

    # per-call durations: each call launched back to back `steps` times
    kern = {}
    for name, per_step in rec.calls.items():
        t = RunOne(torch, name)
        for i in range(args.steps):
            ops(args.warmup + i, t)
        kern[name] = dict(avg_us=t.avg_us(args.steps * per_step), per_step=per_step,
                          **rec.info.get(name, {}))
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
                   "timing": "eager" if args.eager else "hip_graph_per_step",
                   "int8_eq_TOPS_per_step": round(meta["ops_per_step"] / (ms_step * 1e-3) / 1e12, 3),
                   "hbm_frac_per_step": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_call": per_call,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
