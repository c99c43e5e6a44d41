"""ctypes binding of ``libbitlinear.so`` (argument marshalling only).

Torch tensors supply device memory and the current HIP stream; every step of
the computation runs in the library's kernels.  Importing this module fails
loudly when the library has not been built -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbitlinear.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "bitlinear.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_HIP, ERR_VALUE = range(7)
F32, BF16 = 0, 1
PATH_AUTO, PATH_GEMV, PATH_SKINNY, PATH_GEMM = range(4)
MAX_K = 131072

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_f32 = ctypes.c_float

_SIGNATURES = {
    "bitlinear_quant_act": [_vp, ctypes.c_int, _i64, _i64, _vp, _f32, _vp, _vp, _vp],
    "bitlinear_pack_weights": [_vp, _i64, _i64, _vp, _vp, _vp],
    "bitlinear_forward": [_vp, _vp, _i64, _i64, _vp, _i64, _f32, _vp, _vp, _vp],
    "bitlinear_forward_path": [_vp, _vp, _i64, _i64, _vp, _i64, _f32, _vp, _vp, ctypes.c_int, _vp],
    "bitlinear_quant_forward": [_vp, ctypes.c_int, _i64, _i64, _vp, _f32, _vp, _i64, _f32, _vp, _vp,
                                _vp, _vp, _vp],
    "bitlinear_silu_mul_quant": [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp],
    "bitlinear_silu_mul_quant_acc": [_vp, _vp, _i64, _i64, _f32, _f32, _vp, _vp, _vp, _vp],
    "bitlinear_ternarize": [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp],
    "bitlinear_binarize": [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "bitlinear_pack_weights1": [_vp, _i64, _i64, _vp, _vp, _vp],
    "bitlinear_forward1": [_vp, _vp, _i64, _i64, _vp, _i64, _f32, _vp, _vp, _vp],
    "bitlinear_quant_act_grouped": [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _f32, _vp, _vp, _vp],
    "bitlinear_forward_grouped": [_vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp],
    "bitlinear_ternarize_grouped": [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp],
    "bitlinear_forward_grouped_one_launch": [_i64, _i64, _i64, _i64],
    "bitlinear_quant_forward_one_launch": [_i64, _i64, _i64],
    "bitlinear_pack_weights3": [_vp, _i64, _i64, _vp, _vp, _vp],
    "bitlinear_forward3": [_vp, _vp, _i64, _i64, _vp, _i64, _f32, _vp, _vp, _vp],
    "bitlinear_floor_empty": [_vp],
    "bitlinear_floor_stream_read": [_vp, _i64, _vp, _vp],
    "bitlinear_floor_mfma": [_vp, _i64, _i64, _vp, _i64, _vp, _vp],
    "bitlinear_last_error": [],
    "bitlinear_abi_version": [],
}


class BitLinearError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.bitlinear_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def declared_symbols() -> list:
    """Entry points declared in include/bitlinear.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(bitlinear_\w+)\s*\(", text, re.M)))


def last_error() -> str:
    return lib.bitlinear_last_error().decode()


def abi_version() -> int:
    return int(lib.bitlinear_abi_version())


def _check(status: int) -> None:
    if status != OK:
        raise BitLinearError(status, last_error())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtypes, shape=None) -> None:
    """Checks dtype, shape (exact, when given) and contiguity.  Every buffer
    the library reads or writes goes through this before its pointer is
    passed, so a short or mistyped buffer raises here instead of being read or
    written past its end on the device; _gpu() then checks the devices."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _gpu(**tensors) -> None:
    """Every given tensor (None entries skipped) is a GPU tensor, all on one device."""
    first = None
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor")
        if first is None:
            first = (name, t.device)
        elif t.device != first[1]:
            raise ValueError(f"{name} is on {t.device}, {first[0]} on {first[1]}")


def _mat(t: torch.Tensor, name: str, dtypes) -> None:
    """A 2-D input matrix."""
    if isinstance(t, torch.Tensor) and t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    _dev(t, name, dtypes)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def quant_act(x: torch.Tensor, rms_gain: Optional[torch.Tensor] = None, rms_eps: float = 1e-6,
              out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Per-token absmax int8 quantisation of x [M][K] (fp32 or bf16), optionally
    after RMSNorm with gain ``rms_gain`` [K].  Returns (x_q int8, gamma fp32)."""
    _mat(x, "x", (torch.float32, torch.bfloat16))
    M, K = x.shape
    if rms_gain is not None:
        _dev(rms_gain, "rms_gain", (torch.float32,), (K,))
    if out is None:
        x_q = torch.empty((M, K), dtype=torch.int8, device=x.device)
        gamma = torch.empty((M,), dtype=torch.float32, device=x.device)
    else:
        x_q, gamma = out
        _dev(x_q, "x_q", (torch.int8,), (M, K))
        _dev(gamma, "gamma", (torch.float32,), (M,))
    dt = BF16 if x.dtype == torch.bfloat16 else F32
    _gpu(x=x, rms_gain=rms_gain, x_q=x_q, gamma=gamma)
    _check(lib.bitlinear_quant_act(x.data_ptr(), dt, M, K, _ptr(rms_gain), float(rms_eps),
                                   x_q.data_ptr(), gamma.data_ptr(), _stream(x)))
    return x_q, gamma


def pack_weights(w: torch.Tensor, check: bool = True):
    """Ternary int8 [N][K] -> packed words [N][K/16] (int32 storage of the
    uint32 words).  With ``check`` the count of non-ternary entries is read
    back and a ValueError raised if it is not zero."""
    _mat(w, "w", (torch.int8,))
    N, K = w.shape
    packed = torch.empty((N, K // 16), dtype=torch.int32, device=w.device)
    bad = torch.zeros((1,), dtype=torch.int32, device=w.device)
    _gpu(w=w, packed=packed, bad=bad)
    _check(lib.bitlinear_pack_weights(w.data_ptr(), N, K, packed.data_ptr(), bad.data_ptr(),
                                      _stream(w)))
    if check:
        nbad = int(bad.item())
        if nbad:
            raise ValueError(f"{nbad} weight entries are not in {{-1, 0, +1}}")
    return packed, bad


def forward(x_q: torch.Tensor, gamma: torch.Tensor, w_packed: torch.Tensor, beta: float,
            path: int = PATH_AUTO, want_acc: bool = False,
            out: Optional[torch.Tensor] = None, acc_out: Optional[torch.Tensor] = None,
            acc_only: bool = False):
    """y [M][N] = BitLinear(x_q, gamma; w_packed, beta).  Returns y, or
    (y, acc) with ``want_acc``; with ``acc_only`` only the int32 accumulators
    are computed and returned."""
    _mat(x_q, "x_q", (torch.int8,))
    M, K = x_q.shape
    _dev(gamma, "gamma", (torch.float32,), (M,))
    _mat(w_packed, "w_packed", (torch.int32, torch.uint32))
    N = w_packed.shape[0]
    if w_packed.shape[1] * 16 != K:
        raise ValueError(f"w_packed has {w_packed.shape[1]} words per row, K={K} needs {K // 16}")
    if out is not None and not acc_only:
        _dev(out, "out", (torch.float32,), (M, N))
    if acc_out is not None:
        _dev(acc_out, "acc_out", (torch.int32,), (M, N))
    y = None if acc_only else (out if out is not None else
                               torch.empty((M, N), dtype=torch.float32, device=x_q.device))
    acc = acc_out
    if (want_acc or acc_only) and acc is None:
        acc = torch.empty((M, N), dtype=torch.int32, device=x_q.device)
    _gpu(x_q=x_q, gamma=gamma, w_packed=w_packed, y=y, acc=acc)
    _check(lib.bitlinear_forward_path(x_q.data_ptr(), gamma.data_ptr(), M, K, w_packed.data_ptr(),
                                      N, float(beta), _ptr(y), _ptr(acc), int(path),
                                      _stream(x_q)))
    if acc_only:
        return acc
    return (y, acc) if want_acc else y


def quant_forward(x: torch.Tensor, w_packed: torch.Tensor, beta: float,
                  rms_gain: Optional[torch.Tensor] = None, rms_eps: float = 1e-6,
                  want_acc: bool = False,
                  out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                  acc_only: bool = False):
    """quant_act then forward in one call (one kernel for a single token):
    returns (y, x_q, gamma), or (y, x_q, gamma, acc) with ``want_acc``, or
    (acc, x_q, gamma) with ``acc_only``.  ``out`` = (y, x_q, gamma) buffers."""
    _mat(x, "x", (torch.float32, torch.bfloat16))
    _mat(w_packed, "w_packed", (torch.int32, torch.uint32))
    M, K = x.shape
    N = w_packed.shape[0]
    if w_packed.shape[1] * 16 != K:
        raise ValueError(f"w_packed has {w_packed.shape[1]} words per row, K={K} needs {K // 16}")
    if rms_gain is not None:
        _dev(rms_gain, "rms_gain", (torch.float32,), (K,))
    if out is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
        x_q = torch.empty((M, K), dtype=torch.int8, device=x.device)
        gamma = torch.empty((M,), dtype=torch.float32, device=x.device)
    else:
        y, x_q, gamma = out
        if not acc_only:
            _dev(y, "y", (torch.float32,), (M, N))
        _dev(x_q, "x_q", (torch.int8,), (M, K))
        _dev(gamma, "gamma", (torch.float32,), (M,))
    if acc_only:
        y = None
    acc = torch.empty((M, N), dtype=torch.int32, device=x.device) if want_acc or acc_only else None
    dt = BF16 if x.dtype == torch.bfloat16 else F32
    _gpu(x=x, w_packed=w_packed, rms_gain=rms_gain, y=y, x_q=x_q, gamma=gamma, acc=acc)
    _check(lib.bitlinear_quant_forward(x.data_ptr(), dt, M, K, _ptr(rms_gain), float(rms_eps),
                                       w_packed.data_ptr(), N, float(beta), x_q.data_ptr(),
                                       gamma.data_ptr(), _ptr(y), _ptr(acc), _stream(x)))
    if acc_only:
        return acc, x_q, gamma
    return (y, x_q, gamma, acc) if want_acc else (y, x_q, gamma)


def silu_mul_quant_acc(acc_gu: torch.Tensor, gamma: torch.Tensor, beta_gate: float,
                       beta_up: float, want_h: bool = False):
    """GLU glue from the int32 accumulators [M][2F] of the stacked gate + up
    product -> (h_q, gamma_h[, h])."""
    _mat(acc_gu, "acc_gu", (torch.int32,))
    M, F2 = acc_gu.shape
    _dev(gamma, "gamma", (torch.float32,), (M,))
    if F2 % 2:
        raise ValueError(f"acc_gu has {F2} columns, expected 2F")
    F = F2 // 2
    h_q = torch.empty((M, F), dtype=torch.int8, device=acc_gu.device)
    g = torch.empty((M,), dtype=torch.float32, device=acc_gu.device)
    h = torch.empty((M, F), dtype=torch.float32, device=acc_gu.device) if want_h else None
    _gpu(acc_gu=acc_gu, gamma=gamma, h_q=h_q, gamma_h=g, h=h)
    _check(lib.bitlinear_silu_mul_quant_acc(acc_gu.data_ptr(), gamma.data_ptr(), M, F,
                                            float(beta_gate), float(beta_up), _ptr(h),
                                            h_q.data_ptr(), g.data_ptr(), _stream(acc_gu)))
    return (h_q, g, h) if want_h else (h_q, g)


def silu_mul_quant(gate: torch.Tensor, up: torch.Tensor, want_h: bool = False):
    """h = SiLU(gate) * up (float64 inside, fp32 out) -> (h_q, gamma_h[, h])."""
    _mat(gate, "gate", (torch.float32,))
    M, F = gate.shape
    _dev(up, "up", (torch.float32,), (M, F))
    h_q = torch.empty((M, F), dtype=torch.int8, device=gate.device)
    g = torch.empty((M,), dtype=torch.float32, device=gate.device)
    h = torch.empty((M, F), dtype=torch.float32, device=gate.device) if want_h else None
    _gpu(gate=gate, up=up, h_q=h_q, gamma_h=g, h=h)
    _check(lib.bitlinear_silu_mul_quant(gate.data_ptr(), up.data_ptr(), M, F, _ptr(h),
                                        h_q.data_ptr(), g.data_ptr(), _stream(gate)))
    return (h_q, g, h) if want_h else (h_q, g)


def ternarize(W: torch.Tensor, want_codes: bool = False):
    """Absmean ternarisation of fp32 weights [N][K] -> (packed int32 [N][K/16],
    beta fp32 [1], beta64 float64 [1][, codes int8 [N][K]]), all on W's device."""
    _mat(W, "W", (torch.float32,))
    N, K = W.shape
    dev = W.device
    packed = torch.empty((N, K // 16), dtype=torch.int32, device=dev)
    beta = torch.empty((1,), dtype=torch.float32, device=dev)
    beta64 = torch.empty((1,), dtype=torch.float64, device=dev)
    codes = torch.empty((N, K), dtype=torch.int8, device=dev) if want_codes else None
    _gpu(W=W, packed=packed, beta=beta, beta64=beta64, codes=codes)
    _check(lib.bitlinear_ternarize(W.data_ptr(), N, K, packed.data_ptr(), _ptr(codes),
                                   beta.data_ptr(), beta64.data_ptr(), _stream(W)))
    return (packed, beta, beta64, codes) if want_codes else (packed, beta, beta64)


def binarize(W: torch.Tensor):
    """Sign(W - alpha) of fp32 weights [N][K] -> (packed1 int32 [N][K/32],
    codes int8 [N][K], alpha fp32 [1], alpha64 float64 [1], beta fp32 [1],
    beta64 float64 [1]) on W's device (beta = mean |W|)."""
    _mat(W, "W", (torch.float32,))
    N, K = W.shape
    dev = W.device
    packed1 = torch.empty((N, K // 32), dtype=torch.int32, device=dev)
    codes = torch.empty((N, K), dtype=torch.int8, device=dev)
    sc = [torch.empty((1,), dtype=t, device=dev)
          for t in (torch.float32, torch.float64, torch.float32, torch.float64)]
    _gpu(W=W, packed1=packed1, codes=codes, alpha=sc[0])
    _check(lib.bitlinear_binarize(W.data_ptr(), N, K, packed1.data_ptr(), codes.data_ptr(),
                                  *(t.data_ptr() for t in sc), _stream(W)))
    return (packed1, codes, *sc)


def pack_weights1(w: torch.Tensor, check: bool = True):
    """+-1 int8 [N][K] -> (1-bit packed int32 [N][K/32], bad-count int32 [1])."""
    _mat(w, "w", (torch.int8,))
    N, K = w.shape
    packed1 = torch.empty((N, K // 32), dtype=torch.int32, device=w.device)
    bad = torch.zeros((1,), dtype=torch.int32, device=w.device)
    _gpu(w=w, packed1=packed1, bad=bad)
    _check(lib.bitlinear_pack_weights1(w.data_ptr(), N, K, packed1.data_ptr(), bad.data_ptr(),
                                       _stream(w)))
    if check:
        n_bad = int(bad.item())
        if n_bad:
            raise ValueError(f"{n_bad} weight entries are not -1 or +1")
    return packed1, bad


def forward1(x_q: torch.Tensor, gamma: torch.Tensor, w_packed1: torch.Tensor, beta: float,
             want_acc: bool = False):
    """BitLinear on 1-bit weights -> y [M][N] (and acc with ``want_acc``)."""
    _mat(x_q, "x_q", (torch.int8,))
    M, K = x_q.shape
    _dev(gamma, "gamma", (torch.float32,), (M,))
    _mat(w_packed1, "w_packed1", (torch.int32, torch.uint32))
    N = w_packed1.shape[0]
    if w_packed1.shape[1] * 32 != K:
        raise ValueError(f"w_packed1 has {w_packed1.shape[1]} words per row, K={K} needs {K // 32}")
    y = torch.empty((M, N), dtype=torch.float32, device=x_q.device)
    acc = torch.empty((M, N), dtype=torch.int32, device=x_q.device) if want_acc else None
    _gpu(x_q=x_q, gamma=gamma, w_packed1=w_packed1, y=y, acc=acc)
    _check(lib.bitlinear_forward1(x_q.data_ptr(), gamma.data_ptr(), M, K, w_packed1.data_ptr(), N,
                                  float(beta), y.data_ptr(), _ptr(acc), _stream(x_q)))
    return (y, acc) if want_acc else y


def quant_act_grouped(x: torch.Tensor, groups: int, rms_gain: Optional[torch.Tensor] = None,
                      rms_eps: float = 1e-6):
    """Group quantisation of x [M][K] (fp32 or bf16): G runs of K/G inputs per
    token, each with its own absmax scale.  Returns (x_q int8 [G][M][K/G],
    gamma fp32 [G][M])."""
    _mat(x, "x", (torch.float32, torch.bfloat16))
    M, K = x.shape
    G = int(groups)
    if G < 1 or K % G:
        raise ValueError(f"K={K} is not a multiple of G={G}")
    if rms_gain is not None:
        _dev(rms_gain, "rms_gain", (torch.float32,), (K,))
    x_q = torch.empty((G, M, K // G), dtype=torch.int8, device=x.device)
    gamma = torch.empty((G, M), dtype=torch.float32, device=x.device)
    dt = BF16 if x.dtype == torch.bfloat16 else F32
    _gpu(x=x, rms_gain=rms_gain, x_q=x_q, gamma=gamma)
    _check(lib.bitlinear_quant_act_grouped(x.data_ptr(), dt, M, K, G, _ptr(rms_gain),
                                           float(rms_eps), x_q.data_ptr(), gamma.data_ptr(),
                                           _stream(x)))
    return x_q, gamma


def forward_grouped(x_q: torch.Tensor, gamma: torch.Tensor, w_packed: torch.Tensor,
                    beta: torch.Tensor, want_acc: bool = True):
    """Grouped BitLinear: x_q int8 [G][M][KG], gamma [G][M], w_packed
    [G][N][KG/16], beta fp32 [G] on the device -> (y fp32 [M][N], acc int32
    [G][M][N]), or y alone with ``want_acc=False`` (the accumulators are then
    still allocated when the shape needs them as the group products' home)."""
    if isinstance(x_q, torch.Tensor) and x_q.dim() != 3:
        raise ValueError(f"x_q must be 3-D [G][M][KG], got shape {tuple(x_q.shape)}")
    _dev(x_q, "x_q", (torch.int8,))
    G, M, KG = x_q.shape
    _dev(gamma, "gamma", (torch.float32,), (G, M))
    _dev(w_packed, "w_packed", (torch.int32, torch.uint32))
    _dev(beta, "beta", (torch.float32,), (G,))
    if w_packed.dim() != 3 or w_packed.shape[0] != G or w_packed.shape[2] * 16 != KG:
        raise ValueError(f"w_packed shape {tuple(w_packed.shape)} does not match x_q {tuple(x_q.shape)}")
    N = w_packed.shape[1]
    y = torch.empty((M, N), dtype=torch.float32, device=x_q.device)
    acc = None
    if want_acc or not lib.bitlinear_forward_grouped_one_launch(M, G * KG, G, N):
        acc = torch.empty((G, M, N), dtype=torch.int32, device=x_q.device)
    _gpu(x_q=x_q, gamma=gamma, w_packed=w_packed, beta=beta, y=y, acc=acc)
    _check(lib.bitlinear_forward_grouped(x_q.data_ptr(), gamma.data_ptr(), M, G * KG, G,
                                         w_packed.data_ptr(), N, beta.data_ptr(), y.data_ptr(),
                                         _ptr(acc), _stream(x_q)))
    return (y, acc) if want_acc else y


def ternarize_grouped(W_grouped: torch.Tensor, want_codes: bool = False):
    """Absmean ternarisation per weight group of fp32 W_grouped [G][N][KG] ->
    (packed int32 [G][N][KG/16], beta fp32 [G], beta64 float64 [G][, codes
    int8 [G][N][KG]])."""
    if isinstance(W_grouped, torch.Tensor) and W_grouped.dim() != 3:
        raise ValueError(f"W_grouped must be 3-D [G][N][KG], got shape {tuple(W_grouped.shape)}")
    _dev(W_grouped, "W_grouped", (torch.float32,))
    G, N, KG = W_grouped.shape
    dev = W_grouped.device
    packed = torch.empty((G, N, KG // 16), dtype=torch.int32, device=dev)
    beta = torch.empty((G,), dtype=torch.float32, device=dev)
    beta64 = torch.empty((G,), dtype=torch.float64, device=dev)
    codes = torch.empty((G, N, KG), dtype=torch.int8, device=dev) if want_codes else None
    _gpu(W_grouped=W_grouped, packed=packed, beta=beta, beta64=beta64, codes=codes)
    _check(lib.bitlinear_ternarize_grouped(W_grouped.data_ptr(), N, G * KG, G, packed.data_ptr(),
                                           _ptr(codes), beta.data_ptr(), beta64.data_ptr(),
                                           _stream(W_grouped)))
    return (packed, beta, beta64, codes) if want_codes else (packed, beta, beta64)


def pack_weights3(w: torch.Tensor, check: bool = True):
    """Ternary int8 [N][K] -> base-3 packed bytes as int32 words [N][4*ceil(K/80)]
    (1.6 bits per weight), and the bad-count int32 [1]."""
    _mat(w, "w", (torch.int8,))
    N, K = w.shape
    packed3 = torch.empty((N, 4 * ((K + 79) // 80)), dtype=torch.int32, device=w.device)
    bad = torch.zeros((1,), dtype=torch.int32, device=w.device)
    _gpu(w=w, packed3=packed3, bad=bad)
    _check(lib.bitlinear_pack_weights3(w.data_ptr(), N, K, packed3.data_ptr(), bad.data_ptr(),
                                       _stream(w)))
    if check:
        n_bad = int(bad.item())
        if n_bad:
            raise ValueError(f"{n_bad} weight entries are not ternary")
    return packed3, bad


def forward3(x_q: torch.Tensor, gamma: torch.Tensor, w_packed3: torch.Tensor, beta: float,
             want_acc: bool = False):
    """BitLinear on base-3 weights -> y [M][N] (and acc with ``want_acc``)."""
    _mat(x_q, "x_q", (torch.int8,))
    M, K = x_q.shape
    _dev(gamma, "gamma", (torch.float32,), (M,))
    _mat(w_packed3, "w_packed3", (torch.int32, torch.uint32))
    N = w_packed3.shape[0]
    if w_packed3.shape[1] != 4 * ((K + 79) // 80):
        raise ValueError(f"w_packed3 has {w_packed3.shape[1]} words per row, K={K} needs "
                         f"{4 * ((K + 79) // 80)}")
    y = torch.empty((M, N), dtype=torch.float32, device=x_q.device)
    acc = torch.empty((M, N), dtype=torch.int32, device=x_q.device) if want_acc else None
    _gpu(x_q=x_q, gamma=gamma, w_packed3=w_packed3, y=y, acc=acc)
    _check(lib.bitlinear_forward3(x_q.data_ptr(), gamma.data_ptr(), M, K, w_packed3.data_ptr(), N,
                                  float(beta), y.data_ptr(), _ptr(acc), _stream(x_q)))
    return (y, acc) if want_acc else y


def bitlinear(x: torch.Tensor, w_packed: torch.Tensor, beta: float,
              rms_gain: Optional[torch.Tensor] = None, rms_eps: float = 1e-6):
    """Whole layer from fp32 / bf16 activations: quantise then multiply."""
    x_q, gamma = quant_act(x, rms_gain, rms_eps)
    return forward(x_q, gamma, w_packed, beta)


def glu(x: torch.Tensor, w_gate, w_up, w_down, betas, rms_gain, rms_eps: float = 1e-6,
        path: int = PATH_AUTO, stages: bool = False):
    """MatMul-free GLU channel mixer: RMSNorm+quant -> gate, up -> SiLU(gate)*up
    -> requant -> down.  With ``stages`` every intermediate is returned."""
    x_q, gamma = quant_act(x, rms_gain, rms_eps)
    y_gate, acc_gate = forward(x_q, gamma, w_gate, betas[0], path, want_acc=stages)
    y_up, acc_up = forward(x_q, gamma, w_up, betas[1], path, want_acc=stages)
    h_q, gamma_h, h = silu_mul_quant(y_gate, y_up, want_h=stages)
    y, acc_down = forward(h_q, gamma_h, w_down, betas[2], path, want_acc=stages)
    if not stages:
        return y
    return dict(q=x_q, gamma=gamma, acc_gate=acc_gate, y_gate=y_gate, acc_up=acc_up, y_up=y_up,
                h=h, h_q=h_q, gamma_h=gamma_h, acc_down=acc_down, y=y)
