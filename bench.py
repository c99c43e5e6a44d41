#!/usr/bin/env python3
"""Throughput of the ternary BitLinear hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

A step is one pass of the path over one batch of synthetic input: per token
count M of the workload, the activation quantisation (bitlinear_quant_act)
followed by the ternary product with rescale (bitlinear_forward); for the GLU
workload the whole RMSNorm+quant -> gate -> up -> SiLU*up+requant -> down
chain.  Weight packing is offline and outside the step.

Inputs are seeded synthetic draws (workloads.py) resident in HBM before the
timed region.  The packed weights rotate through at least 512 MB of copies so
that consecutive steps cannot be served from the 256 MB Infinity Cache.
Timed steps are replays of HIP graphs (one per weight copy) so host launch
overhead does not pace the GPU; a second pass launches the same steps eagerly
with HIP events around every kernel call on its stream to obtain each
kernel's average duration for the roofline figure.

Prints ONE JSON line (rank 0, N=1).
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
    """Returns (ops, meta): ops(step_idx, timer) launches one step."""
    wid = args.workload
    wl = workloads.WORKLOADS[wid]
    rotate = not args.no_rotate
    lib = bl.lib
    F32, BF16 = bl.F32, bl.BF16

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
                yu=torch.empty((M, Fh), device=dev), hq=torch.empty((M, Fh), dtype=torch.int8, device=dev),
                gh=torch.empty(M, device=dev), y=torch.empty((M, D), device=dev)))

        def ops(step, timer):
            c = step % ncopy
            for b in bufs:
                M = b["M"]
                with timer("quant_act_rms"):
                    check(lib.bitlinear_quant_act(b["x"].data_ptr(), F32, M, D, gain.data_ptr(),
                                                  wl.rms_eps, b["q"].data_ptr(), b["g"].data_ptr(), stream()))
                for L, out in ((layers[0], b["yg"]), (layers[1], b["yu"])):
                    with timer(f"forward_M{M}", L.wbytes, M, L.N, L.K):
                        check(lib.bitlinear_forward(b["q"].data_ptr(), b["g"].data_ptr(), M, D,
                                                    L.copies[c].data_ptr(), Fh, L.beta,
                                                    out.data_ptr(), None, stream()))
                with timer("silu_mul_quant"):
                    check(lib.bitlinear_silu_mul_quant(b["yg"].data_ptr(), b["yu"].data_ptr(), M, Fh,
                                                       None, b["hq"].data_ptr(), b["gh"].data_ptr(),
                                                       stream()))
                L = layers[2]
                with timer(f"forward_M{M}", L.wbytes, M, L.N, L.K):
                    check(lib.bitlinear_forward(b["hq"].data_ptr(), b["gh"].data_ptr(), M, Fh,
                                                L.copies[c].data_ptr(), D, L.beta, b["y"].data_ptr(),
                                                None, stream()))

        meta.update(weight_bytes_per_step=sum(L.wbytes for L in layers) * len(wl.ms),
                    weight_copies=ncopy, ops_per_step=sum(2 * M * (2 * D * Fh + Fh * D) for M in wl.ms))
        return ops, meta, (layers, bufs)

    w = workloads.workload_weights(wid)
    L = Layer(torch, bl, dev, w, workloads.workload_beta(wid), rotate)
    K, N = wl.K, wl.N
    bufs = []
    for M in wl.ms:
        xa = workloads.workload_activations(wid, M)
        if wl.act == "normal_bf16":
            x = torch.from_numpy(xa).to(dev).view(torch.bfloat16)
            dt = BF16
        else:
            x = torch.from_numpy(xa).to(dev)
            dt = F32
        bufs.append(dict(M=M, x=x, dt=dt, q=torch.empty((M, K), dtype=torch.int8, device=dev),
                         g=torch.empty(M, device=dev), y=torch.empty((M, N), device=dev)))

    def ops(step, timer):
        wptr = L.copies[step % len(L.copies)].data_ptr()
        for b in bufs:
            M = b["M"]
            with timer("quant_act"):
                check(lib.bitlinear_quant_act(b["x"].data_ptr(), b["dt"], M, K, None, 0.0,
                                              b["q"].data_ptr(), b["g"].data_ptr(), stream()))
            with timer(f"forward_M{M}", L.wbytes, M, N, K):
                check(lib.bitlinear_forward(b["q"].data_ptr(), b["g"].data_ptr(), M, K, wptr, N,
                                            L.beta, b["y"].data_ptr(), None, stream()))

    meta.update(weight_bytes_per_step=L.wbytes * len(wl.ms), weight_copies=len(L.copies),
                ops_per_step=sum(2 * M * N * K for M in wl.ms))
    return ops, meta, (L, bufs)


# ----------------------------------------------------------------------------- timing

class NullTimer:
    def __call__(self, name, *a):
        return self

    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


class EventTimer:
    """HIP events on the launching stream around every call."""

    def __init__(self, torch):
        self.torch = torch
        self.pending = []
        self.info = {}

    def __call__(self, name, wbytes=0, M=0, N=0, K=0):
        self._name = name
        if wbytes:
            # algorithmic bytes of one forward launch: packed W + x_q + gamma + y
            self.info[name] = dict(alg_bytes=wbytes + M * K + 4 * M + 4 * M * N,
                                   ops=2 * M * N * K, wbytes=wbytes)
        return self

    def __enter__(self):
        s = self.torch.cuda.current_stream()
        self._e0 = self.torch.cuda.Event(enable_timing=True)
        self._e0.record(s)
        return self

    def __exit__(self, *a):
        e1 = self.torch.cuda.Event(enable_timing=True)
        e1.record(self.torch.cuda.current_stream())
        self.pending.append((self._name, self._e0, e1))
        return False

    def summary(self):
        self.torch.cuda.synchronize()
        out = {}
        for name, e0, e1 in self.pending:
            d = out.setdefault(name, [])
            d.append(e0.elapsed_time(e1) * 1e3)  # us
        return {k: dict(n=len(v), avg_us=float(np.mean(v)), med_us=float(np.median(v)),
                        total_us=float(np.sum(v)), **self.info.get(k, {})) for k, v in out.items()}


# ----------------------------------------------------------------------------- traffic

def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bitlinear_rmsnorm_absmax_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload_name: str):
    """HBM bytes per launch of the dominant kernel from a committed counter
    summary (profiles/traffic_<workload>.md), only if it was taken on the
    current kernel sources."""
    path = os.path.join(PROFILES, f"traffic_{workload_name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source_digest:\s*(\w+)", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
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
        wbytes = w.size // 4 * len(wl.ms)
        rows = w.shape[0]
        # large workloads: a bounded slice of output rows (same K, same M sweep)
        est = sum(x.shape[0] for x in xs) * w.size * 1e-9  # ~1 ns per MAC and thread
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
    torch.cuda.synchronize()
    print(f"# workload {meta['workload']}: M={meta['M']} K={meta['K']} N={meta['N']}, "
          f"{meta['weight_copies']} weight copies", file=sys.stderr, flush=True)

    ncopy = meta["weight_copies"]
    null = NullTimer()
    graphs = None
    if not args.eager:
        # one graph per weight copy; step i replays graph i % ncopy
        ops(0, null)  # first eager launch initialises every kernel
        torch.cuda.synchronize()
        graphs = []
        s = torch.cuda.Stream(device=dev)
        for c in range(ncopy):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                ops(c, null)
            graphs.append(g)
        torch.cuda.synchronize()

    def run(i):
        if graphs is not None:
            graphs[i % ncopy].replay()
        else:
            ops(i, null)

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        run(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    print(f"# timed {args.steps} steps: {ms_step * 1e3:.2f} us/step (wall {wall * 1e3 / args.steps:.2f})",
          file=sys.stderr, flush=True)

    # per-kernel durations: the same steps launched eagerly, events on the stream
    timer = EventTimer(torch)
    for i in range(args.steps):
        ops(args.warmup + i, timer)
    kern = timer.summary()
    print("# per-call GPU time (us): " + ", ".join(f"{k} {v['avg_us']:.2f}" for k, v in kern.items()),
          file=sys.stderr, flush=True)

    fwd = {k: v for k, v in kern.items() if k.startswith("forward_")}
    dom_name = max(fwd, key=lambda k: fwd[k]["total_us"])
    # roofline over every forward launch of the step (same kernel family)
    alg = sum(v["alg_bytes"] * v["n"] for v in fwd.values())
    dur = sum(v["total_us"] for v in fwd.values())
    achieved = alg / (dur * 1e-6) / 1e9
    wl = workloads.WORKLOADS[args.workload]
    mfma_bound = max(wl.ms) >= 512
    value = meta["weight_bytes_per_step"] / (ms_step * 1e-3) / 1e9
    traffic = read_traffic(meta["workload"])
    roof = dict(bound="hbm", achieved=round(achieved, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                kernel="bitlinear_forward (" + ", ".join(sorted(fwd)) + ")",
                avg_launch_us=round(dur / sum(v["n"] for v in fwd.values()), 3))
    if mfma_bound:
        ops_all = sum(v["ops"] * v["n"] for v in fwd.values())
        tops = ops_all / (dur * 1e-6) / 1e12
        roof = dict(bound="mfma", achieved=round(tops, 2), peak=INT8_PEAK_TOPS, unit="TOP/s",
                    frac=round(tops / INT8_PEAK_TOPS, 4), traffic=traffic,
                    kernel="bitlinear_forward (" + ", ".join(sorted(fwd)) + ")",
                    avg_launch_us=round(dur / sum(v["n"] for v in fwd.values()), 3))

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(args, args.cpu_seconds)

    per_call = {k: dict(avg_us=round(v["avg_us"], 3),
                        **({"packed_w_GBs": round(v["wbytes"] / (v["avg_us"] * 1e-6) / 1e9, 1),
                            "int8_eq_TOPS": round(v["ops"] / (v["avg_us"] * 1e-6) / 1e12, 2)}
                           if "wbytes" in v else {}))
                for k, v in kern.items()}
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
