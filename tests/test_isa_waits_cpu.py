"""The hand-counted vector-memory waits of the ring GEMM and the decode kernel,
checked in the gfx950 assembly that the library's own flags produce.

Both kernels copy global memory straight into LDS (global_load_lds) and wait
for those copies with an explicit ``s_waitcnt vmcnt(n)`` whose n is the number
of vector-memory instructions issued after them.  That count is right only if
the compiler emits exactly the expected loads, in program order, and adds no
wait of its own.  This test compiles the two sources (hipcc, host only, no
GPU) and checks, for every instantiation:

- ring GEMM (``gemm_dma_kernel`` and its two-group form ``gemm_pair_kernel``):
  the steady-state loop -- the one that
  copies, waits, meets at a barrier and multiplies -- holds exactly one
  vector-memory wait, and its count equals the copies the loop issues per
  step times STAGES - 2 (the steps issued after the one the wave multiplies
  next stay in flight while it waits: one with three stages, two with four);
- decode with the token quantised in the kernel: the first wait for the
  row's chunks leaves the first batch of weight loads (issued after them)
  in flight;
- decode (``decode_lds_kernel``): every wait that publishes the activation
  block (a vmcnt wait followed by the barrier after the copies' barrier, with
  no multiply in between) counts exactly the weight loads issued between the
  two barriers, so the copies -- older -- have landed and the weights may
  still be in flight; and no other wait sits between the two barriers, which
  would hold the weight loads back until the copies have landed.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bitlinear_rmsnorm_absmax_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not installed")


def _asm(src, tmp_path):
    import sys
    sys.path.insert(0, ROOT)
    from bitlinear_rmsnorm_absmax_amd import build as lib_build
    flags = [f for f in lib_build.HIP_FLAGS if f not in ("-shared", "-fPIC")]
    out = str(tmp_path / (os.path.basename(src) + ".s"))
    cmd = ["hipcc", *flags, "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           "-o", out, os.path.join(CSRC, src)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read()


def _functions(asm, name_part):
    """{mangled name: instruction lines} of the kernels whose name contains name_part."""
    out = {}
    for m in re.finditer(r"^(_Z\S+):", asm, re.M):
        name = m.group(1)
        if name_part not in name:
            continue
        end = asm.find("s_endpgm", m.end())
        out[name] = [l.split(";")[0].strip() for l in asm[m.end():end].splitlines()]
    return out


def _vmcnt(line):
    m = re.match(r"s_waitcnt\b.*\bvmcnt\((\d+)\)", line)
    return int(m.group(1)) if m else None


def _loops(lines):
    """(label, body lines) of every loop: from a label to the last branch back to it."""
    loops = []
    for i, l in enumerate(lines):
        m = re.match(r"(\.LBB\w+):$", l)
        if not m:
            continue
        back = [k for k in range(i + 1, len(lines))
                if re.match(r"s_c?branch\w*\s+" + re.escape(m.group(1)) + r"$", lines[k])]
        if back:
            loops.append((m.group(1), lines[i:back[-1] + 1]))
    return loops


def test_ring_gemm_waits_match_its_copies(tmp_path):
    asm = _asm("gemm_dma.hip", tmp_path)
    funcs = _functions(asm, "gemm_dma_kernel")
    assert funcs, "no gemm_dma_kernel instantiation found"
    pair = _functions(asm, "gemm_pair_kernel")
    assert pair, "no gemm_pair_kernel instantiation found"
    funcs.update(pair)
    for name, lines in funcs.items():
        steady = [(lab, body) for lab, body in _loops(lines)
                  if any(l.startswith("global_load_lds") for l in body)
                  and any(l.startswith("s_barrier") for l in body)
                  and any(l.startswith("v_mfma") for l in body)]
        assert len(steady) == 1, f"{name}: {len(steady)} steady-state loops"
        body = steady[0][1]
        waits = [_vmcnt(l) for l in body if _vmcnt(l) is not None]
        copies = sum(l.startswith("global_load_lds") for l in body)
        others = [l for l in body if re.match(r"(global|buffer|flat)_(load|store|atomic)", l)
                  and not l.startswith("global_load_lds")]
        # gemm_dma_kernel<WM, WN, TM, TN, STAGES> / gemm_pair_kernel<STAGES, P>:
        # STAGES - 2 later steps stay in flight while the wave waits for the
        # step it multiplies next
        m = re.search(r"gemm_dma_kernelILi\d+ELi\d+ELi\d+ELi\d+ELi(\d+)E", name) or \
            re.search(r"gemm_pair_kernelILi(\d+)E", name)
        stages = int(m.group(1))
        assert waits == [(stages - 2) * copies], (
            f"{name}: waits {waits} in the loop, {copies} copies a step, {stages} stages")
        assert not others, f"{name}: other vector-memory instructions in the loop: {others[:3]}"


def _fused(name):
    """decode_lds_kernel<..., FQ, FRMS>: FQ != 0 quantises one token in the kernel"""
    m = re.search(r"ELi(\d+)ELb[01]EEEv", name)
    return m is not None and int(m.group(1)) != 0


def test_decode_publish_waits_match_its_weight_loads(tmp_path):
    funcs = _functions(_asm("decode_lds.hip", tmp_path), "decode_lds_kernel")
    assert funcs, "no decode_lds_kernel instantiation found"
    assert any(_fused(n) for n in funcs) and any(not _fused(n) for n in funcs)
    for name, lines in funcs.items():
        if _fused(name):
            # the row's chunk loads, a barrier, the first weight batch; the
            # waits for the cached chunks must leave that batch in flight
            b = next(i for i, l in enumerate(lines) if l.startswith("s_barrier"))
            assert any(re.match(r"global_load_dword", l) for l in lines[:b]), f"{name}: no row loads"
            k = b + 1
            while k < len(lines) and not lines[k].startswith(("s_waitcnt", "s_cbranch", ".LBB")):
                k += 1
            weights = sum(bool(re.match(r"global_load_dword", l)) for l in lines[b + 1:k])
            assert weights > 0, f"{name}: no weight loads after the row loads"
            first = next(_vmcnt(l) for l in lines[k:] if _vmcnt(l) is not None)
            assert first >= weights, f"{name}: vmcnt({first}) waits for the {weights} weight loads"
            continue
        barriers = [i for i, l in enumerate(lines) if l.startswith("s_barrier")]
        checked = 0
        for b in barriers:
            # a publishing wait: the last vmcnt wait before this barrier, with
            # no other instruction that touches vector memory in between
            w = b - 1
            while w >= 0 and _vmcnt(lines[w]) is None and not lines[w].startswith(("s_barrier", ".LBB")):
                w -= 1
            if w < 0 or _vmcnt(lines[w]) is None or _vmcnt(lines[w]) == 0:
                continue
            # back to the copies' barrier, or to the label that starts this
            # branch of the code (a branch of its own may hold the publish)
            prev = w - 1
            while prev >= 0 and not lines[prev].startswith(("s_barrier", ".LBB")):
                prev -= 1
            if prev < 0:
                continue
            span = lines[prev + 1:w]
            # the barrier after the multiplies waits only as far as it needs
            # (the loads past the last chunk may stay in flight): not a publish
            if any(l.startswith(("global_load_lds", "v_mfma")) for l in span):
                continue
            loads = sum(bool(re.match(r"global_load_dword", l)) for l in span)
            if loads == 0:  # e.g. the wait after the stream's last batch
                continue
            assert loads == _vmcnt(lines[w]), (
                f"{name}: wait vmcnt({_vmcnt(lines[w])}) after {loads} weight loads")
            # and no earlier wait there: one would hold the weight loads back
            # until the activation copies have landed
            early = [l for l in span if _vmcnt(l) is not None]
            assert not early, f"{name}: {early} before the weight loads"
            checked += 1
        assert checked >= 1, f"{name}: no publishing wait found"
