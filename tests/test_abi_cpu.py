"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/bitlinear.h, and rejects bad arguments with the documented
status before anything is launched."""

import ctypes
import subprocess

import pytest

import bitlinear_rmsnorm_absmax_amd as bl
from bitlinear_rmsnorm_absmax_amd import _lib

F = ctypes.c_float
FAKE = 0x10000  # a 16-byte aligned non-NULL address; never dereferenced on error paths


def test_every_declared_symbol_is_exported():
    declared = bl.declared_symbols()
    assert set(declared) == {
        "bitlinear_quant_act", "bitlinear_pack_weights", "bitlinear_forward",
        "bitlinear_forward_path", "bitlinear_quant_forward", "bitlinear_silu_mul_quant",
        "bitlinear_silu_mul_quant_acc",
        "bitlinear_ternarize",
        "bitlinear_binarize", "bitlinear_pack_weights1", "bitlinear_forward1",
        "bitlinear_quant_act_grouped", "bitlinear_forward_grouped", "bitlinear_ternarize_grouped",
        "bitlinear_forward_grouped_one_launch", "bitlinear_quant_forward_one_launch", "bitlinear_pack_weights3", "bitlinear_forward3",
        "bitlinear_floor_empty", "bitlinear_floor_stream_read", "bitlinear_floor_mfma",
        "bitlinear_last_error", "bitlinear_abi_version"}
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared:
        assert name in exported, name
        assert hasattr(bl.lib, name)


def test_abi_version():
    assert bl.abi_version() == 1


def _fwd(xq=FAKE, g=FAKE, M=1, K=16, w=FAKE, N=1, beta=1.0, y=FAKE, acc=None, path=0):
    return bl.lib.bitlinear_forward_path(xq, g, M, K, w, N, F(beta), y, acc, path, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(xq=None), bl.ERR_NULL, "x_q is NULL"),
    (dict(g=None), bl.ERR_NULL, "gamma is NULL"),
    (dict(w=None), bl.ERR_NULL, "w_packed is NULL"),
    (dict(y=None), bl.ERR_NULL, "y is NULL"),
    (dict(M=-1), bl.ERR_SHAPE, "M=-1"),
    (dict(N=-5), bl.ERR_SHAPE, "N=-5"),
    (dict(K=24), bl.ERR_SHAPE, "multiple of 16"),
    (dict(K=131072 + 16), bl.ERR_SHAPE, "K=131088"),
    (dict(xq=FAKE + 4), bl.ERR_ALIGN, "x_q is not 16-byte aligned"),
    (dict(w=FAKE + 8), bl.ERR_ALIGN, "w_packed is not 16-byte aligned"),
    (dict(y=FAKE + 2), bl.ERR_ALIGN, "y is not 4-byte aligned"),
    (dict(acc=FAKE + 1), bl.ERR_ALIGN, "acc is not 4-byte aligned"),
    (dict(path=7), bl.ERR_VALUE, "unknown path"),
    (dict(path=-1), bl.ERR_VALUE, "unknown path"),
    (dict(beta=float("inf")), bl.ERR_VALUE, "beta"),
    (dict(beta=float("nan")), bl.ERR_VALUE, "beta"),
    (dict(M=5, path=1), bl.ERR_VALUE, "GEMV path takes M <= 4"),
    (dict(M=65, path=2), bl.ERR_VALUE, "skinny path takes M <= 64"),
])
def test_forward_rejects(kw, status, msg):
    assert _fwd(**kw) == status
    assert msg in bl.last_error()


def test_forward_empty_work_is_ok_without_pointers():
    assert _fwd(xq=None, g=None, w=None, y=None, M=0) == bl.OK
    assert _fwd(xq=None, g=None, w=None, y=None, N=0) == bl.OK
    assert bl.last_error() == ""
    # plain entry point shares the validation
    assert bl.lib.bitlinear_forward(None, None, 0, 16, None, 3, F(1.0), None, None, None) == bl.OK


def _quant(x=FAKE, dt=0, M=1, K=16, gain=None, eps=1e-6, q=FAKE, g=FAKE):
    return bl.lib.bitlinear_quant_act(x, dt, M, K, gain, F(eps), q, g, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(x=None), bl.ERR_NULL, "x is NULL"),
    (dict(q=None), bl.ERR_NULL, "x_q is NULL"),
    (dict(g=None), bl.ERR_NULL, "gamma is NULL"),
    (dict(dt=2), bl.ERR_DTYPE, "unknown dtype"),
    (dict(K=8), bl.ERR_SHAPE, "multiple of 16"),
    (dict(M=-2), bl.ERR_SHAPE, "M=-2"),
    (dict(x=FAKE + 4), bl.ERR_ALIGN, "x is not 16-byte aligned"),
    (dict(gain=FAKE + 4), bl.ERR_ALIGN, "rms_gain is not 16-byte aligned"),
    (dict(gain=FAKE, eps=-1.0), bl.ERR_VALUE, "rms_eps"),
    (dict(gain=FAKE, eps=float("nan")), bl.ERR_VALUE, "rms_eps"),
])
def test_quant_rejects(kw, status, msg):
    assert _quant(**kw) == status
    assert msg in bl.last_error()


def test_quant_empty_is_ok():
    assert _quant(x=None, q=None, g=None, M=0) == bl.OK


def _qfwd(x=FAKE, dt=0, M=1, K=64, gain=None, eps=1e-6, w=FAKE, N=1, beta=1.0, q=FAKE, g=FAKE,
          y=FAKE, acc=None):
    return bl.lib.bitlinear_quant_forward(x, dt, M, K, gain, F(eps), w, N, F(beta), q, g, y, acc,
                                          None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(x=None), bl.ERR_NULL, "x is NULL"),
    (dict(q=None), bl.ERR_NULL, "x_q is NULL"),
    (dict(g=None), bl.ERR_NULL, "gamma is NULL"),
    (dict(w=None), bl.ERR_NULL, "w_packed is NULL"),
    (dict(y=None), bl.ERR_NULL, "y is NULL"),
    (dict(dt=3), bl.ERR_DTYPE, "unknown dtype"),
    (dict(K=40), bl.ERR_SHAPE, "multiple of 16"),
    (dict(K=131072 + 16), bl.ERR_SHAPE, "K=131088"),
    (dict(M=-1), bl.ERR_SHAPE, "M=-1"),
    (dict(N=-3), bl.ERR_SHAPE, "N=-3"),
    (dict(x=FAKE + 8), bl.ERR_ALIGN, "x is not 16-byte aligned"),
    (dict(q=FAKE + 4), bl.ERR_ALIGN, "x_q is not 16-byte aligned"),
    (dict(w=FAKE + 4), bl.ERR_ALIGN, "w_packed is not 16-byte aligned"),
    (dict(y=FAKE + 2), bl.ERR_ALIGN, "y is not 4-byte aligned"),
    (dict(acc=FAKE + 2), bl.ERR_ALIGN, "acc is not 4-byte aligned"),
    (dict(gain=FAKE + 4), bl.ERR_ALIGN, "rms_gain is not 16-byte aligned"),
    (dict(gain=FAKE, eps=float("inf")), bl.ERR_VALUE, "rms_eps"),
    (dict(beta=float("nan")), bl.ERR_VALUE, "beta"),
])
def test_quant_forward_rejects(kw, status, msg):
    assert _qfwd(**kw) == status
    assert msg in bl.last_error()


def _sacc(acc=FAKE, g=FAKE, M=1, F=16, bg=1.0, bu=1.0, h=None, q=FAKE, gh=FAKE):
    return bl.lib.bitlinear_silu_mul_quant_acc(acc, g, M, F, ctypes.c_float(bg), ctypes.c_float(bu),
                                               h, q, gh, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(acc=None), bl.ERR_NULL, "acc_gu is NULL"),
    (dict(g=None), bl.ERR_NULL, "gamma is NULL"),
    (dict(q=None), bl.ERR_NULL, "h_q is NULL"),
    (dict(gh=None), bl.ERR_NULL, "gamma_h is NULL"),
    (dict(F=40), bl.ERR_SHAPE, "multiple of 16"),
    (dict(M=-1), bl.ERR_SHAPE, "M=-1"),
    (dict(bg=float("nan")), bl.ERR_VALUE, "beta_gate and beta_up"),
    (dict(bu=float("inf")), bl.ERR_VALUE, "beta_gate and beta_up"),
    (dict(acc=FAKE + 4), bl.ERR_ALIGN, "acc_gu is not 16-byte aligned"),
    (dict(h=FAKE + 4), bl.ERR_ALIGN, "h is not 16-byte aligned"),
])
def test_silu_mul_quant_acc_rejects(kw, status, msg):
    assert _sacc(**kw) == status
    assert msg in bl.last_error()


def test_forward_y_optional_only_with_acc():
    # y may be NULL when acc is given; both NULL is an error
    assert _fwd(y=None, acc=None) == bl.ERR_NULL
    assert "y is NULL" in bl.last_error()
    assert _fwd(y=FAKE + 2, acc=FAKE) == bl.ERR_ALIGN
    assert "y is not 4-byte aligned" in bl.last_error()


def test_quant_forward_empty_is_ok():
    assert _qfwd(x=None, q=None, g=None, w=None, y=None, M=0) == bl.OK
    assert bl.last_error() == ""


@pytest.mark.parametrize("args,status,msg", [
    ((None, 1, 16, FAKE, None), bl.ERR_NULL, "w is NULL"),
    ((FAKE, 1, 16, None, None), bl.ERR_NULL, "w_packed is NULL"),
    ((FAKE, 1, 40, FAKE, None), bl.ERR_SHAPE, "multiple of 16"),
    ((FAKE, -1, 16, FAKE, None), bl.ERR_SHAPE, "N=-1"),
    ((FAKE + 1, 1, 16, FAKE, None), bl.ERR_ALIGN, "w is not 16-byte aligned"),
    ((FAKE, 1, 16, FAKE, FAKE + 2), bl.ERR_ALIGN, "bad_count"),
])
def test_pack_rejects(args, status, msg):
    assert bl.lib.bitlinear_pack_weights(*args, None) == status
    assert msg in bl.last_error()


@pytest.mark.parametrize("args,status,msg", [
    ((None, FAKE, 1, 16, None, FAKE, FAKE), bl.ERR_NULL, "gate is NULL"),
    ((FAKE, None, 1, 16, None, FAKE, FAKE), bl.ERR_NULL, "up is NULL"),
    ((FAKE, FAKE, 1, 16, None, None, FAKE), bl.ERR_NULL, "h_q is NULL"),
    ((FAKE, FAKE, 1, 16, None, FAKE, None), bl.ERR_NULL, "gamma_h is NULL"),
    ((FAKE, FAKE, 1, 20, None, FAKE, FAKE), bl.ERR_SHAPE, "F=20"),
    ((FAKE, FAKE, 1, 16, FAKE + 4, FAKE, FAKE), bl.ERR_ALIGN, "h is not 16-byte aligned"),
])
def test_silu_mul_quant_rejects(args, status, msg):
    assert bl.lib.bitlinear_silu_mul_quant(*args, None) == status
    assert msg in bl.last_error()


def test_error_text_is_thread_local():
    import threading
    assert _fwd(M=-1) == bl.ERR_SHAPE
    seen = {}

    def other():
        seen["before"] = bl.last_error()
        _quant(dt=9)
        seen["after"] = bl.last_error()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["before"] == "" and "dtype" in seen["after"]
    assert "M=-1" in bl.last_error()


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError, match="GPU tensor"):
        bl.quant_act(torch.zeros(2, 16))


def _tern(W=FAKE, N=1, K=32, packed=FAKE, codes=None, beta=FAKE, beta64=FAKE):
    return bl.lib.bitlinear_ternarize(W, N, K, packed, codes, beta, beta64, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(W=None), bl.ERR_NULL, "W is NULL"),
    (dict(packed=None), bl.ERR_NULL, "w_packed is NULL"),
    (dict(beta=None), bl.ERR_NULL, "beta is NULL"),
    (dict(beta64=None), bl.ERR_NULL, "beta64 is NULL"),
    (dict(beta=None, N=0), bl.ERR_NULL, "beta is NULL"),
    (dict(K=16), bl.ERR_SHAPE, "must be 0 or >= 32"),
    (dict(K=40), bl.ERR_SHAPE, "multiple of 16"),
    (dict(K=131072 + 16), bl.ERR_SHAPE, "K=131088"),
    (dict(N=-3), bl.ERR_SHAPE, "N=-3"),
    (dict(W=FAKE + 4), bl.ERR_ALIGN, "W is not 16-byte aligned"),
    (dict(packed=FAKE + 8), bl.ERR_ALIGN, "w_packed is not 16-byte aligned"),
    (dict(codes=FAKE + 4), bl.ERR_ALIGN, "w_ternary is not 16-byte aligned"),
    (dict(beta64=FAKE + 4), bl.ERR_ALIGN, "beta64 is not 8-byte aligned"),
])
def test_ternarize_rejects(kw, status, msg):
    assert _tern(**kw) == status
    assert msg in bl.last_error()


def _bin(W=FAKE, N=1, K=64, p1=FAKE, codes=FAKE, a=FAKE, a64=FAKE, b=FAKE, b64=FAKE):
    return bl.lib.bitlinear_binarize(W, N, K, p1, codes, a, a64, b, b64, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(W=None), bl.ERR_NULL, "W is NULL"),
    (dict(codes=None), bl.ERR_NULL, "w_codes is NULL"),
    (dict(p1=None), bl.ERR_NULL, "w_packed1 is NULL"),
    (dict(a64=None, N=0), bl.ERR_NULL, "alpha64 is NULL"),
    (dict(b=None), bl.ERR_NULL, "beta is NULL"),
    (dict(K=48), bl.ERR_SHAPE, "multiple of 32"),
    (dict(codes=FAKE + 8), bl.ERR_ALIGN, "w_codes is not 16-byte aligned"),
    (dict(a64=FAKE + 4), bl.ERR_ALIGN, "alpha64 is not 8-byte aligned"),
])
def test_binarize_rejects(kw, status, msg):
    assert _bin(**kw) == status
    assert msg in bl.last_error()


@pytest.mark.parametrize("args,status,msg", [
    ((None, 1, 32, FAKE, None), bl.ERR_NULL, "w is NULL"),
    ((FAKE, 1, 32, None, None), bl.ERR_NULL, "w_packed1 is NULL"),
    ((FAKE, 1, 16, FAKE, None), bl.ERR_SHAPE, "multiple of 32"),
    ((FAKE + 4, 1, 32, FAKE, None), bl.ERR_ALIGN, "w is not 16-byte aligned"),
    ((FAKE, 1, 32, FAKE, FAKE + 1), bl.ERR_ALIGN, "bad_count"),
])
def test_pack1_rejects(args, status, msg):
    assert bl.lib.bitlinear_pack_weights1(*args, None) == status
    assert msg in bl.last_error()


def _fwd1(xq=FAKE, g=FAKE, M=1, K=64, w=FAKE, N=1, beta=1.0, y=FAKE, acc=None):
    return bl.lib.bitlinear_forward1(xq, g, M, K, w, N, F(beta), y, acc, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(xq=None), bl.ERR_NULL, "x_q is NULL"),
    (dict(w=None), bl.ERR_NULL, "w_packed1 is NULL"),
    (dict(y=None), bl.ERR_NULL, "y is NULL"),
    (dict(K=32), bl.ERR_SHAPE, "multiple of 64"),
    (dict(beta=float("inf")), bl.ERR_VALUE, "beta is not finite"),
    (dict(w=FAKE + 4), bl.ERR_ALIGN, "w_packed1 is not 8-byte aligned"),
    (dict(M=-1), bl.ERR_SHAPE, "M=-1"),
])
def test_forward1_rejects(kw, status, msg):
    assert _fwd1(**kw) == status
    assert msg in bl.last_error()


def _qg(x=FAKE, dt=0, M=2, K=128, G=2, gain=None, eps=1e-6, xq=FAKE, g=FAKE):
    return bl.lib.bitlinear_quant_act_grouped(x, dt, M, K, G, gain, F(eps), xq, g, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(G=0), bl.ERR_SHAPE, "G=0"),
    (dict(G=3), bl.ERR_SHAPE, "runs of a multiple of 16"),
    (dict(K=96, G=4), bl.ERR_SHAPE, "runs of a multiple of 16"),
    (dict(x=None), bl.ERR_NULL, "x is NULL"),
    (dict(xq=None), bl.ERR_NULL, "x_q is NULL"),
    (dict(g=None), bl.ERR_NULL, "gamma is NULL"),
    (dict(dt=5), bl.ERR_DTYPE, "dtype"),
    (dict(gain=FAKE, eps=-1.0), bl.ERR_VALUE, "rms_eps"),
    (dict(gain=FAKE + 4), bl.ERR_ALIGN, "rms_gain"),
])
def test_quant_grouped_rejects(kw, status, msg):
    assert _qg(**kw) == status
    assert msg in bl.last_error()


def _fg(xq=FAKE, g=FAKE, M=2, K=256, G=2, w=FAKE, N=3, beta=FAKE, y=FAKE, acc=FAKE):
    return bl.lib.bitlinear_forward_grouped(xq, g, M, K, G, w, N, beta, y, acc, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(G=0), bl.ERR_SHAPE, "G=0"),
    (dict(K=256, G=3), bl.ERR_SHAPE, "runs of a multiple of 64"),
    (dict(K=128, G=4), bl.ERR_SHAPE, "runs of a multiple of 64"),
    (dict(K=24), bl.ERR_SHAPE, "multiple of 16"),
    (dict(acc=None, M=33), bl.ERR_NULL, "acc is NULL"),
    (dict(acc=FAKE + 2), bl.ERR_ALIGN, "acc is not 4-byte aligned"),
    (dict(beta=None), bl.ERR_NULL, "beta is NULL"),
    (dict(y=None), bl.ERR_NULL, "y is NULL"),
    (dict(w=FAKE + 8), bl.ERR_ALIGN, "w_packed is not 16-byte aligned"),
    (dict(M=-1), bl.ERR_SHAPE, "M=-1"),
])
def test_forward_grouped_rejects(kw, status, msg):
    assert _fg(**kw) == status
    assert msg in bl.last_error()


def test_grouped_empty_work_is_ok_without_pointers():
    assert _fg(M=0, xq=None, g=None, w=None, beta=None, y=None, acc=None) == bl.OK
    assert _fg(N=0, xq=None, g=None, w=None, beta=None, y=None, acc=None) == bl.OK
    assert _qg(M=0, x=None, xq=None, g=None) == bl.OK


def _tg(W=FAKE, N=4, K=256, G=2, wp=FAKE, codes=None, b=FAKE, b64=FAKE):
    return bl.lib.bitlinear_ternarize_grouped(W, N, K, G, wp, codes, b, b64, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(G=0), bl.ERR_SHAPE, "G=0"),
    (dict(K=192, G=2), bl.ERR_SHAPE, "runs of a multiple of 64"),
    (dict(W=None), bl.ERR_NULL, "W_grouped is NULL"),
    (dict(wp=None), bl.ERR_NULL, "w_packed is NULL"),
    (dict(b=None), bl.ERR_NULL, "beta is NULL"),
    (dict(b64=FAKE + 4), bl.ERR_ALIGN, "beta64"),
    (dict(codes=FAKE + 8), bl.ERR_ALIGN, "w_ternary"),
])
def test_ternarize_grouped_rejects(kw, status, msg):
    assert _tg(**kw) == status
    assert msg in bl.last_error()


def test_quant_forward_one_launch_query():
    q = bl.lib.bitlinear_quant_forward_one_launch
    assert q(1, 4096, 11008) == 1
    assert q(1, 16384, 16384) == 1
    assert q(1, 64, 1) == 1
    assert q(1, 8192, 28672) == 1         # long rows over many row tiles: the MFMA decode kernel
    assert q(1, 20480, 28672) == 1        # longer than the VALU kernel's LDS copy: MFMA decode
    assert q(1, 2048, 28672) == 0         # past 16384 rows with short rows: the two calls
    assert q(1, 4352, 20000) == 0         # K % 512 != 0 past 16384 rows: the two calls
    assert q(1, 16448, 40) == 0           # the codes of a longer token do not fit the LDS copy
    assert q(1, 1040, 77) == 0            # K not a multiple of 64
    assert q(2, 4096, 1000) == 0          # several tokens
    assert q(1, 0, 10) == 0 and q(1, 64, 0) == 0 and q(1, 64, -1) == 0


def test_grouped_one_launch_query():
    q = bl.lib.bitlinear_forward_grouped_one_launch
    assert q(16, 4096, 4, 11008) == 1
    assert q(1, 2048, 2, 333) == 1
    assert q(17, 4096, 4, 11008) == 0     # more tokens than the decode kernel takes
    assert q(4, 512, 4, 1000) == 0        # runs of 128 inputs: not whole 256-chunks
    assert q(4, 4096, 1, 1000) == 0       # one group is the ungrouped product
    assert q(4, 3072, 3, 1000) == 0       # 3 groups: no K split divides into them


@pytest.mark.parametrize("args,status,msg", [
    ((FAKE, 4, 24, FAKE, None), bl.ERR_SHAPE, "multiple of 16"),
    ((None, 4, 32, FAKE, None), bl.ERR_NULL, "w is NULL"),
    ((FAKE, 4, 32, None, None), bl.ERR_NULL, "w_packed3 is NULL"),
    ((FAKE, 4, 32, FAKE + 4, None), bl.ERR_ALIGN, "w_packed3"),
    ((FAKE, 4, 32, FAKE, FAKE + 2), bl.ERR_ALIGN, "bad_count"),
    ((FAKE, -2, 32, FAKE, None), bl.ERR_SHAPE, "N=-2"),
])
def test_pack3_rejects(args, status, msg):
    assert bl.lib.bitlinear_pack_weights3(*args, None) == status
    assert msg in bl.last_error()


def _f3(xq=FAKE, g=FAKE, M=1, K=160, w=FAKE, N=1, beta=1.0, y=FAKE, acc=None):
    return bl.lib.bitlinear_forward3(xq, g, M, K, w, N, F(beta), y, acc, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(K=24), bl.ERR_SHAPE, "multiple of 16"),
    (dict(w=FAKE + 8), bl.ERR_ALIGN, "w_packed3"),
    (dict(xq=None), bl.ERR_NULL, "x_q is NULL"),
    (dict(y=None), bl.ERR_NULL, "y is NULL"),
    (dict(beta=float("nan")), bl.ERR_VALUE, "beta"),
    (dict(acc=FAKE + 1), bl.ERR_ALIGN, "acc"),
])
def test_forward3_rejects(kw, status, msg):
    assert _f3(**kw) == status
    assert msg in bl.last_error()


# ------------------------------------------------------------------ binding buffer checks

def _t(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


@pytest.mark.parametrize("call,msg", [
    # caller-supplied outputs of the wrong length or dtype are refused before any pointer
    # reaches the library (CPU tensors: the shape check runs before the device check)
    (lambda t: bl.quant_act(_t((2, 32), t.float32), out=(_t((2, 16), t.int8), _t((2,), t.float32))),
     "x_q has shape (2, 16), expected (2, 32)"),
    (lambda t: bl.quant_act(_t((2, 32), t.float32), out=(_t((2, 32), t.int8), _t((1,), t.float32))),
     "gamma has shape (1,), expected (2,)"),
    (lambda t: bl.quant_act(_t((2, 32), t.float32), out=(_t((2, 32), t.uint8), _t((2,), t.float32))),
     "x_q has dtype"),
    (lambda t: bl.quant_act(_t((2, 32), t.float32), rms_gain=_t((16,), t.float32)),
     "rms_gain has shape (16,), expected (32,)"),
    (lambda t: bl.forward(_t((3, 32), t.int8), _t((2,), t.float32), _t((5, 2), t.int32), 1.0),
     "gamma has shape (2,), expected (3,)"),
    (lambda t: bl.forward(_t((3, 32), t.int8), _t((3,), t.float32), _t((5, 2), t.int32), 1.0,
                          out=_t((3, 4), t.float32)),
     "out has shape (3, 4), expected (3, 5)"),
    (lambda t: bl.forward(_t((3, 32), t.int8), _t((3,), t.float32), _t((5, 2), t.int32), 1.0,
                          acc_out=_t((3, 5), t.float32)),
     "acc_out has dtype"),
    (lambda t: bl.forward(_t((3, 32), t.int8), _t((3,), t.float32), _t((5, 2), t.int32), 1.0,
                          acc_out=_t((2, 5), t.int32)),
     "acc_out has shape (2, 5), expected (3, 5)"),
    (lambda t: bl.quant_forward(_t((1, 32), t.float32), _t((5, 2), t.int32), 1.0,
                                out=(_t((1, 4), t.float32), _t((1, 32), t.int8), _t((1,), t.float32))),
     "y has shape (1, 4), expected (1, 5)"),
    (lambda t: bl.quant_forward(_t((1, 32), t.float32), _t((5, 2), t.int32), 1.0,
                                rms_gain=_t((33,), t.float32)),
     "rms_gain has shape (33,), expected (32,)"),
    (lambda t: bl.silu_mul_quant(_t((2, 32), t.float32), _t((2, 16), t.float32)),
     "up has shape (2, 16), expected (2, 32)"),
    (lambda t: bl.silu_mul_quant_acc(_t((2, 64), t.int32), _t((3,), t.float32), 1.0, 1.0),
     "gamma has shape (3,), expected (2,)"),
    (lambda t: bl.forward1(_t((2, 64), t.int8), _t((1,), t.float32), _t((4, 2), t.int32), 1.0),
     "gamma has shape (1,), expected (2,)"),
    (lambda t: bl.forward3(_t((2, 80), t.int8), _t((4,), t.float32), _t((4, 4), t.int32), 1.0),
     "gamma has shape (4,), expected (2,)"),
    (lambda t: bl.forward_grouped(_t((2, 3, 64), t.int8), _t((2, 2), t.float32),
                                  _t((2, 5, 4), t.int32), _t((2,), t.float32)),
     "gamma has shape (2, 2), expected (2, 3)"),
    (lambda t: bl.forward_grouped(_t((2, 3, 64), t.int8), _t((2, 3), t.float32),
                                  _t((2, 5, 4), t.int32), _t((3,), t.float32)),
     "beta has shape (3,), expected (2,)"),
    (lambda t: bl.forward(_t((3, 2, 16), t.int8), _t((3,), t.float32), _t((5, 1), t.int32), 1.0),
     "x_q must be 2-D"),
])
def test_binding_rejects_mis_sized_buffers(call, msg):
    import torch
    with pytest.raises(ValueError, match=msg.replace("(", r"\(").replace(")", r"\)")):
        call(torch)


def test_binding_refuses_host_tensors_of_the_right_shape():
    import torch
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        bl.quant_act(torch.zeros((2, 32), dtype=torch.float32))


def test_row_count_limit_keeps_launcher_arithmetic_in_int():
    """N is capped at 2^30 so every launcher's int rounding of N up to a tile
    width, and every row index plus a tile offset, stays below INT_MAX."""
    lim = 1 << 30
    for fn in ("bitlinear_forward_path",):
        # at the limit: nothing to do with M = 0, so validation passes without a launch
        assert _fwd(xq=None, g=None, w=None, y=None, M=0, N=lim) == bl.OK
        assert _fwd(M=0, N=lim + 1) == bl.ERR_SHAPE
        assert f"N={lim + 1}" in bl.last_error()
    assert bl.lib.bitlinear_pack_weights(FAKE, lim + 1, 16, FAKE, None, None) == bl.ERR_SHAPE
    assert bl.lib.bitlinear_forward1(FAKE, FAKE, 0, 64, FAKE, lim + 1, F(1.0), FAKE, None,
                                     None) == bl.ERR_SHAPE
    assert bl.lib.bitlinear_forward3(FAKE, FAKE, 0, 16, FAKE, lim + 1, F(1.0), FAKE, None,
                                     None) == bl.ERR_SHAPE
    assert bl.lib.bitlinear_quant_forward(FAKE, 0, 0, 64, None, F(0.0), FAKE, lim + 1, F(1.0), FAKE,
                                          FAKE, FAKE, None, None) == bl.ERR_SHAPE


def test_floor_stream_read_rejects():
    assert bl.lib.bitlinear_floor_stream_read(FAKE, 24, FAKE, None) == bl.ERR_SHAPE
    assert bl.lib.bitlinear_floor_stream_read(FAKE, -16, FAKE, None) == bl.ERR_SHAPE
    assert bl.lib.bitlinear_floor_stream_read(None, 32, FAKE, None) == bl.ERR_NULL
    assert bl.lib.bitlinear_floor_stream_read(FAKE + 8, 32, FAKE, None) == bl.ERR_ALIGN
    assert bl.lib.bitlinear_floor_stream_read(FAKE, 32, None, None) == bl.ERR_NULL
    assert bl.lib.bitlinear_floor_stream_read(None, 0, None, None) == bl.OK


def test_floor_mfma_rejects():
    f = bl.lib.bitlinear_floor_mfma
    assert f(FAKE, 512, 200, FAKE, 256, FAKE, None) == bl.ERR_SHAPE      # K not a multiple of 128
    assert f(FAKE, 512, 8192 + 16, FAKE, 256, FAKE, None) == bl.ERR_SHAPE
    assert f(FAKE, -1, 128, FAKE, 256, FAKE, None) == bl.ERR_SHAPE
    assert f(FAKE, 512, 128, FAKE, (1 << 30) + 1, FAKE, None) == bl.ERR_SHAPE
    assert f(FAKE, 512, 262144, FAKE, 256, FAKE, None) == bl.ERR_SHAPE
    assert f(None, 512, 128, FAKE, 256, FAKE, None) == bl.ERR_NULL
    assert f(FAKE, 512, 128, None, 256, FAKE, None) == bl.ERR_NULL
    assert f(FAKE, 512, 128, FAKE, 256, None, None) == bl.ERR_NULL
    assert f(FAKE + 8, 512, 128, FAKE, 256, FAKE, None) == bl.ERR_ALIGN
    assert f(FAKE, 512, 128, FAKE + 4, 256, FAKE, None) == bl.ERR_ALIGN
    assert f(FAKE, 65535 * 128, 128, FAKE, 1 << 30, FAKE, None) == bl.ERR_SHAPE  # > 2^31-1 tiles
    assert f(None, 0, 128, None, 256, None, None) == bl.OK                # nothing to launch
    assert f(None, 512, 0, None, 256, None, None) == bl.OK
