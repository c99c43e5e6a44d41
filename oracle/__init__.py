"""CPU oracle of the ternary BitLinear layer: TEST INFRASTRUCTURE ONLY.

A ctypes wrapper around ``bitlinear_oracle.c`` (plain C loops restating the
published formulas).  Only ``tests/``, the smoke check and the CPU-baseline leg
of the benchmark may import this package; the HIP library and its Python
binding never do.

Every function takes and returns NumPy arrays (C-contiguous).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitlinear_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib: Optional[ctypes.CDLL] = None

_c_p = ctypes.c_void_p
_i64 = ctypes.c_int64


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        # ORACLE_LIB: another build of the same source (the sanitizer run of
        # the pin tests loads an AddressSanitizer / UBSan build through it)
        path = os.environ.get("ORACLE_LIB", _LIB_PATH)
        if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(path)
        sig = {
            "oracle_bf16_to_f32": [_c_p, _i64, _c_p],
            "oracle_quant_act": [_c_p, _i64, _i64, _c_p, _c_p],
            "oracle_rmsnorm_quant_act": [_c_p, _c_p, ctypes.c_float, _i64, _i64, _c_p, _c_p],
            "oracle_rmsnorm_quant_act_literal": [_c_p, _c_p, ctypes.c_float, _i64, _i64,
                                                 _c_p, _c_p],
            "oracle_pack": [_c_p, _i64, _i64, _c_p],
            "oracle_unpack": [_c_p, _i64, _i64, _c_p],
            "oracle_accumulate": [_c_p, _i64, _i64, _c_p, _i64, _c_p],
            "oracle_rescale": [_c_p, _c_p, _i64, _i64, ctypes.c_float, _c_p],
            "oracle_silu_mul": [_c_p, _c_p, _i64, _c_p],
            "oracle_ternarize": [_c_p, _i64, _i64, _c_p],
            "oracle_binarize": [_c_p, _i64, _i64, _c_p],
            "oracle_pack1": [_c_p, _i64, _i64, _c_p],
            "oracle_unpack1": [_c_p, _i64, _i64, _c_p],
            "oracle_quant_act_grouped": [_c_p, _c_p, ctypes.c_float, _i64, _i64, _i64, _c_p,
                                         _c_p],
            "oracle_pack3": [_c_p, _i64, _i64, _c_p],
            "oracle_unpack3": [_c_p, _i64, _i64, _c_p],
            "oracle_num_threads": [],
            "oracle_set_num_threads": [ctypes.c_int],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
        lib.oracle_pack.restype = ctypes.c_int64
        lib.oracle_accumulate.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.restype = None
        lib.oracle_ternarize.restype = ctypes.c_double
        lib.oracle_binarize.restype = ctypes.c_double
        lib.oracle_pack1.restype = ctypes.c_int64
        lib.oracle_unpack1.restype = None
        lib.oracle_pack3.restype = ctypes.c_int64
        lib.oracle_unpack3.restype = None
        for name in ("oracle_bf16_to_f32", "oracle_quant_act", "oracle_rmsnorm_quant_act",
                     "oracle_quant_act_grouped",
                     "oracle_rmsnorm_quant_act_literal", "oracle_unpack", "oracle_rescale",
                     "oracle_silu_mul"):
            getattr(lib, name).restype = None
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    _load().oracle_bf16_to_f32(_p(b), b.size, _p(out))
    return out


def quant_act(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token absmax int8 quantisation of fp32 x [M][K] -> (q, gamma)."""
    x = _c(x, np.float32)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    g = np.empty((M,), dtype=np.float32)
    _load().oracle_quant_act(_p(x), M, K, _p(q), _p(g))
    return q, g


def rmsnorm_quant_act(x: np.ndarray, gain: np.ndarray, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    x = _c(x, np.float32)
    gain = _c(gain, np.float32)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    g = np.empty((M,), dtype=np.float32)
    _load().oracle_rmsnorm_quant_act(_p(x), _p(gain), float(np.float32(eps)), M, K, _p(q), _p(g))
    return q, g


def quant_act_grouped(x: np.ndarray, groups: int, gain: Optional[np.ndarray] = None,
                      eps: float = 1e-6) -> Tuple[np.ndarray, np.ndarray]:
    """Group quantisation (unite.ai article, Gruppenquantisierung): fp32 x
    [M][K] -> (q int8 [G][M][K/G], gamma fp32 [G][M]), each run of K/G inputs
    of each token with its own absmax scale; optional RMSNorm gain."""
    x = _c(x, np.float32)
    M, K = x.shape
    G = int(groups)
    if G < 1 or K % G:
        raise ValueError("K must be a positive multiple of the group count")
    q = np.empty((G, M, K // G), dtype=np.int8)
    g = np.empty((G, M), dtype=np.float32)
    gp = None
    if gain is not None:
        gain = _c(gain, np.float32)
        gp = _p(gain)
    _load().oracle_quant_act_grouped(_p(x), gp, float(np.float32(eps)), M, K, G, _p(q), _p(g))
    return q, g


def rmsnorm_quant_act_literal(x: np.ndarray, gain: np.ndarray, eps: float):
    x = _c(x, np.float32)
    gain = _c(gain, np.float32)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    g = np.empty((M,), dtype=np.float64)
    _load().oracle_rmsnorm_quant_act_literal(_p(x), _p(gain), float(np.float32(eps)), M, K,
                                             _p(q), _p(g))
    return q, g


def pack(w: np.ndarray) -> Tuple[np.ndarray, int]:
    """Ternary int8 [N][K] (K % 16 == 0) -> (uint32 [N][K/16], #invalid)."""
    w = _c(w, np.int8)
    N, K = w.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    out = np.empty((N, K // 16), dtype=np.uint32)
    bad = _load().oracle_pack(_p(w), N, K, _p(out))
    return out, int(bad)


def ternarize(W: np.ndarray) -> Tuple[np.ndarray, float]:
    """fp32 weights [N][K] -> (ternary int8 [N][K], beta as a Python float =
    the float64 mean |W|, pairwise-summed); absmean rule of the datacamp
    article."""
    W = _c(W, np.float32)
    N, K = W.shape
    w = np.empty((N, K), dtype=np.int8)
    beta = _load().oracle_ternarize(_p(W), N, K, _p(w))
    return w, float(beta)


def binarize(W: np.ndarray) -> Tuple[np.ndarray, float]:
    """fp32 weights [N][K] -> (+-1 int8 [N][K], alpha = float64 mean of W);
    Sign(W - alpha) with Sign(0) = -1 (unite.ai article, weight binarisation)."""
    W = _c(W, np.float32)
    N, K = W.shape
    w = np.empty((N, K), dtype=np.int8)
    alpha = _load().oracle_binarize(_p(W), N, K, _p(w))
    return w, float(alpha)


def pack1(w: np.ndarray) -> Tuple[np.ndarray, int]:
    """+-1 int8 [N][K] (K % 32 == 0) -> (uint32 [N][K/32], #entries not +-1)."""
    w = _c(w, np.int8)
    N, K = w.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    out = np.empty((N, K // 32), dtype=np.uint32)
    bad = _load().oracle_pack1(_p(w), N, K, _p(out))
    return out, int(bad)


def unpack1(packed: np.ndarray, K: int) -> np.ndarray:
    packed = _c(packed, np.uint32)
    N = packed.shape[0]
    w = np.empty((N, K), dtype=np.int8)
    _load().oracle_unpack1(_p(packed), N, K, _p(w))
    return w


def pack3(w: np.ndarray) -> Tuple[np.ndarray, int]:
    """Ternary int8 [N][K] (K % 16 == 0) -> (base-3 bytes uint8
    [N][ceil(K/80)*16], #entries outside {-1, 0, 1})."""
    w = _c(w, np.int8)
    N, K = w.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    out = np.empty((N, (K + 79) // 80 * 16), dtype=np.uint8)
    bad = _load().oracle_pack3(_p(w), N, K, _p(out))
    return out, int(bad)


def unpack3(packed: np.ndarray, K: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    N = packed.shape[0]
    w = np.empty((N, K), dtype=np.int8)
    _load().oracle_unpack3(_p(packed), N, K, _p(w))
    return w


def unpack(packed: np.ndarray, K: int) -> np.ndarray:
    packed = _c(packed, np.uint32)
    N = packed.shape[0]
    w = np.empty((N, K), dtype=np.int8)
    _load().oracle_unpack(_p(packed), N, K, _p(w))
    return w


def accumulate(q: np.ndarray, w: np.ndarray) -> np.ndarray:
    """acc [M][N] int32 = q [M][K] . w [N][K]^T (exact)."""
    q = _c(q, np.int8)
    w = _c(w, np.int8)
    M, K = q.shape
    N, K2 = w.shape
    if K != K2:
        raise ValueError("K mismatch")
    acc = np.empty((M, N), dtype=np.int32)
    if _load().oracle_accumulate(_p(q), M, K, _p(w), N, _p(acc)):
        raise OverflowError("accumulator does not fit int32")
    return acc


def rescale(acc: np.ndarray, gamma: np.ndarray, beta: float) -> np.ndarray:
    acc = _c(acc, np.int32)
    gamma = _c(gamma, np.float32)
    M, N = acc.shape
    y = np.empty((M, N), dtype=np.float32)
    _load().oracle_rescale(_p(acc), _p(gamma), M, N, float(np.float32(beta)), _p(y))
    return y


def forward(q: np.ndarray, gamma: np.ndarray, w: np.ndarray, beta: float):
    """BitLinear on quantised activations -> (y fp32 [M][N], acc int32 [M][N])."""
    acc = accumulate(q, w)
    return rescale(acc, gamma, beta), acc


def forward_grouped(q: np.ndarray, gamma: np.ndarray, w: np.ndarray, beta: np.ndarray):
    """Grouped BitLinear (unite.ai article, Gruppenquantisierung, with
    3. BitLinear-Betrieb per group): q int8 [G][M][K/G], gamma [G][M], ternary
    w int8 [N][K] (group g = columns g*K/G .. (g+1)*K/G), beta [G] ->
    (y fp32 [M][N], acc int32 [G][M][N]).  acc[g] is group g's exact product;
    y = sum over g of acc[g] * beta[g] * gamma[g] / 128 in float64, rounded
    once to fp32."""
    q = _c(q, np.int8)
    G, M, KG = q.shape
    w = _c(w, np.int8)
    N = w.shape[0]
    if w.shape[1] != G * KG:
        raise ValueError("K mismatch")
    gamma = _c(gamma, np.float32).reshape(G, M)
    beta = _c(beta, np.float32).reshape(G)
    acc = np.empty((G, M, N), dtype=np.int32)
    y64 = np.zeros((M, N), dtype=np.float64)
    for g in range(G):
        acc[g] = accumulate(q[g], w[:, g * KG:(g + 1) * KG])
        y64 += acc[g].astype(np.float64) * float(beta[g]) * gamma[g].astype(np.float64)[:, None] / 128.0
    return y64.astype(np.float32), acc


def ternarize_grouped(W: np.ndarray, groups: int) -> Tuple[np.ndarray, np.ndarray]:
    """Absmean ternarisation per group of K/G input columns (datacamp article's
    absmean rule applied per group, unite.ai article, Gruppenquantisierung):
    fp32 W [N][K] -> (ternary int8 [N][K], beta float64 [G]); group g's beta
    is the pairwise float64 mean |W| over the row-major entries of its
    N x K/G block."""
    W = _c(W, np.float32)
    N, K = W.shape
    G = int(groups)
    if G < 1 or K % G:
        raise ValueError("K must be a positive multiple of the group count")
    KG = K // G
    w = np.empty((N, K), dtype=np.int8)
    betas = np.empty(G, dtype=np.float64)
    for g in range(G):
        wg, betas[g] = ternarize(np.ascontiguousarray(W[:, g * KG:(g + 1) * KG]))
        w[:, g * KG:(g + 1) * KG] = wg
    return w, betas


def silu_mul(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    gate = _c(gate, np.float32)
    up = _c(up, np.float32)
    h = np.empty(gate.shape, dtype=np.float64)
    _load().oracle_silu_mul(_p(gate), _p(up), gate.size, _p(h))
    return h


def bitlinear(x: np.ndarray, w: np.ndarray, beta: float, rms_gain=None, rms_eps: float = 1e-6):
    """Whole layer from fp32 activations: quantise (optionally after RMSNorm)
    then the ternary product and rescale.  Returns (y, acc, q, gamma)."""
    if rms_gain is None:
        q, g = quant_act(x)
    else:
        q, g = rmsnorm_quant_act(x, rms_gain, rms_eps)
    y, acc = forward(q, g, w, beta)
    return y, acc, q, g


def glu(x: np.ndarray, w_gate, w_up, w_down, betas, rms_gain, rms_eps: float = 1e-6):
    """MatMul-free GLU channel mixer: RMSNorm+quant -> gate, up -> SiLU(gate)*up
    (float64, rounded to fp32) -> requant -> down.  Returns a dict of stages."""
    q, g = rmsnorm_quant_act(x, rms_gain, rms_eps)
    y_gate, acc_gate = forward(q, g, w_gate, betas[0])
    y_up, acc_up = forward(q, g, w_up, betas[1])
    h64 = silu_mul(y_gate, y_up)
    h = h64.astype(np.float32)
    h_q, g_h = quant_act(h)
    y_down, acc_down = forward(h_q, g_h, w_down, betas[2])
    return dict(q=q, gamma=g, acc_gate=acc_gate, y_gate=y_gate, acc_up=acc_up, y_up=y_up,
                h64=h64, h=h, h_q=h_q, gamma_h=g_h, acc_down=acc_down, y=y_down)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's parallel loops (started from this thread)."""
    _load().oracle_set_num_threads(int(n))
