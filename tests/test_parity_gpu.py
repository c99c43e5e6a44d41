"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bar: bit-exact int8 codes, gamma (no-norm path), packed words and int32
accumulators; fp32 outputs within 1e-6 relative (y_ref = 0 forces y = 0).
Every input comes from workloads.py; every expected value from oracle/.
"""

import ctypes
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import GOLDEN

pytestmark = pytest.mark.gpu

bl = pytest.importorskip("bitlinear_rmsnorm_absmax_amd")

REL = 1e-6
PATHS = {"gemv": bl.PATH_GEMV, "skinny": bl.PATH_SKINNY, "gemm": bl.PATH_GEMM, "auto": bl.PATH_AUTO}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return torch.device("cuda:0")


def to_dev(a, dev, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(dev)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_y_close(y, y_ref):
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    err = np.abs(y - y_ref)
    bad = err > REL * np.abs(y_ref)
    assert not bad.any(), f"{bad.sum()} outputs beyond 1e-6 rel; worst {err[bad].max()}"


class Guard:
    """An output buffer with sentinel-filled guard bands before and after it
    (and a sentinel-filled interior): `t` is the output view, `check()` asserts
    that no kernel stored outside it.  The bands are 4 KiB, a multiple of 256,
    so `t` keeps the allocator's alignment."""

    PAD = 4096
    FILL = 0xA5

    def __init__(self, shape, dtype, dev):
        n = int(np.prod(shape, dtype=np.int64)) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.buf = torch.full((2 * self.PAD + n,), self.FILL, dtype=torch.uint8, device=dev)
        self.t = self.buf[self.PAD:self.PAD + n].view(dtype).view(shape)

    def check(self, what=""):
        torch.cuda.synchronize()
        head = self.buf[:self.PAD].cpu().numpy()
        tail = self.buf[self.PAD + self.n:].cpu().numpy()
        assert (head == self.FILL).all(), f"{what}: store before the output ({int((head != self.FILL).sum())} bytes)"
        assert (tail == self.FILL).all(), f"{what}: store past the output ({int((tail != self.FILL).sum())} bytes)"


def stream():
    return torch.cuda.current_stream().cuda_stream


def gpu_pack(w, dev):
    """Packs on the GPU into a guarded buffer (checked before returning)."""
    N, K = w.shape
    wd = to_dev(w, dev)
    gp = Guard((N, K // 16), torch.int32, dev)
    bad = torch.zeros(1, dtype=torch.int32, device=dev)
    st = bl.lib.bitlinear_pack_weights(wd.data_ptr(), N, K, gp.t.data_ptr(), bad.data_ptr(), stream())
    assert st == 0, bl.last_error()
    gp.check("pack")
    assert int(host(bad)[0]) == 0
    return gp.t


def run_forward(x_f32, w, beta, dev, path=bl.PATH_AUTO, rms=False):
    """GPU quant + pack + forward into guarded outputs; checks the guard bands
    and returns host arrays (q, gamma, y, acc)."""
    M, K = x_f32.shape
    N = w.shape[0]
    xd = to_dev(x_f32, dev)
    gain = torch.ones(K, dtype=torch.float32, device=dev) if rms else None
    gq, gg = Guard((M, K), torch.int8, dev), Guard((M,), torch.float32, dev)
    q, g = bl.quant_act(xd, gain, out=(gq.t, gg.t))
    wp = gpu_pack(w, dev)
    gy, ga = Guard((M, N), torch.float32, dev), Guard((M, N), torch.int32, dev)
    y, acc = bl.forward(q, g, wp, beta, path=path, want_acc=True, out=gy.t, acc_out=ga.t)
    for gd, nm in ((gq, "x_q"), (gg, "gamma"), (gy, "y"), (ga, "acc")):
        gd.check(f"{nm} M={M} N={N} K={K} path={path}")
    return host(q), host(g), host(y), host(acc)


# ------------------------------------------------------------------ worked example

def test_worked_example_on_gpu(dev):
    gd = json.load(open(os.path.join(GOLDEN, "worked_4x4.json")))
    # pad K = 4 -> 16 with zero activations and zero weights (changes nothing)
    x = np.zeros((3, 16), np.float32)
    x[:, :4] = gd["x"]
    w = np.zeros((4, 16), np.int8)
    w[:, :4] = gd["W"]
    for name, path in PATHS.items():
        q, g, y, acc = run_forward(x, w, gd["beta"], dev, path)
        np.testing.assert_array_equal(q[:, :4], gd["q"])
        np.testing.assert_array_equal(g, gd["gamma"])
        np.testing.assert_array_equal(acc, gd["acc"], err_msg=name)
        np.testing.assert_array_equal(y, np.array(gd["y"], np.float32), err_msg=name)


# ------------------------------------------------------------------ quantisation

QUANT_CASES = [
    ("f32", 1, 2048, "normal_f32"), ("f32", 16, 4096, "normal_f32"), ("f32", 7, 1040, "normal_f32"),
    ("f32", 3, 16, "normal_f32"), ("f32", 2, 131072, "normal_f32"), ("bf16", 5, 4096, "normal_bf16"),
    ("f32", 9, 8192, "student_t3"), ("f32", 300, 4160, "normal_f32"), ("bf16", 33, 2576, "normal_bf16"),
]


@pytest.mark.parametrize("dt,M,K,act", QUANT_CASES)
def test_quant_act_bit_exact(dev, dt, M, K, act):
    x, _, _ = workloads.random_case(100 + M, M, 1, K, act=act)
    x = x.copy()
    x[0, :] = 0  # an all-zero token
    if dt == "bf16":
        xf = oracle.bf16_to_f32(x)
        xd = to_dev(x, dev, torch.bfloat16)
    else:
        xf = x
        xd = to_dev(x, dev)
    q_ref, g_ref = oracle.quant_act(xf)
    gq, gg = Guard((M, K), torch.int8, dev), Guard((M,), torch.float32, dev)
    q, g = bl.quant_act(xd, out=(gq.t, gg.t))
    gq.check(f"x_q M={M} K={K}")
    gg.check(f"gamma M={M} K={K}")
    np.testing.assert_array_equal(host(q), q_ref)
    np.testing.assert_array_equal(host(g), g_ref)


@pytest.mark.parametrize("M,K", [(1, 8192), (8, 8192), (64, 8192), (127, 4096), (4, 4096)])
def test_split_quantiser_matches_one_workgroup_rows(dev, M, K):
    """Few long rows run P workgroups per row; a stacked batch of 128 rows or
    more runs one workgroup per row.  The same rows quantised both ways (with
    and without RMSNorm) give the same codes and bit-identical gamma."""
    x = workloads.workload_activations(5, M, K) if K == 8192 else \
        workloads.random_case(230 + M, M, 1, K)[0]
    pad = np.zeros((128, K), np.float32)
    pad[:M] = x
    gain = to_dev(workloads.rng_for(231, K).uniform(0.5, 2.0, K).astype(np.float32), dev)
    for gn in (None, gain):
        q1, g1 = bl.quant_act(to_dev(x, dev), gn, 1e-6)
        q2, g2 = bl.quant_act(to_dev(pad, dev), gn, 1e-6)
        np.testing.assert_array_equal(host(q1), host(q2)[:M])
        np.testing.assert_array_equal(host(g1).view(np.uint32), host(g2)[:M].view(np.uint32))


@pytest.mark.parametrize("M,K,gain_kind", [(1, 2560, "unit"), (512, 2560, "unit"), (6, 1040, "rand"),
                                           (3, 8192, "unit"), (2, 131072, "rand")])
def test_rmsnorm_quant(dev, M, K, gain_kind):
    x, _, _ = workloads.random_case(200 + M, M, 1, K)
    rng = workloads.rng_for(201, M, K)
    gain = np.ones(K, np.float32) if gain_kind == "unit" else \
        rng.uniform(0.5, 2.0, K).astype(np.float32)
    q_ref, g_ref = oracle.rmsnorm_quant_act(x, gain, 1e-6)
    q, g = bl.quant_act(to_dev(x, dev), to_dev(gain, dev), 1e-6)
    np.testing.assert_array_equal(host(q), q_ref)
    assert_y_close(host(g), g_ref)


def _near_half_integer_rows(K):
    """Rows whose entries sit within 1e-7..2.5e-4 of a code boundary
    (x / gamma * 128 near k + 0.5), the absmax first; and rows with a tiny
    gamma, one of them subnormal."""
    rng = workloads.rng_for(1400, K)
    eps_set = np.array([0.0, 1e-7, -1e-7, 1e-6, -1e-6, 1e-5, -1e-5, 2.5e-5, -2.5e-5,
                        1e-4, -1e-4, 2.4e-4, -2.4e-4])
    rows = []
    for g0 in (1.0, 3.0, 0.7071067, 123.456, 2.5e-3):
        k = rng.integers(-128, 128, K - 1)
        e = rng.choice(eps_set, K - 1)
        x = np.clip((np.float64(np.float32(g0)) * (k + 0.5 + e) / 128.0).astype(np.float32),
                    -np.float32(g0), np.float32(g0))
        rows.append(np.concatenate([[np.float32(g0)], x]))
    for g0 in (1e-35, 3e-39):
        x = (np.float32(g0) * rng.uniform(-1, 1, K)).astype(np.float32)
        x[0] = np.float32(g0)
        rows.append(x)
    return np.array(rows, np.float32)


def test_quant_codes_near_half_integers(dev):
    """Codes decided by the correctly rounded division at its hardest inputs,
    in the row quantiser, the grouped quantiser and the fused one-token kernel."""
    K = 4096
    x = _near_half_integer_rows(K)
    q_ref, g_ref = oracle.quant_act(x)
    q, g = bl.quant_act(to_dev(x, dev))
    np.testing.assert_array_equal(host(q), q_ref)
    np.testing.assert_array_equal(host(g), g_ref)
    qg_ref, gg_ref = oracle.quant_act_grouped(x, 4)
    qg, gg = bl.quant_act_grouped(to_dev(x, dev), 4)
    np.testing.assert_array_equal(host(qg), qg_ref)
    np.testing.assert_array_equal(host(gg), gg_ref)
    wp = gpu_pack(workloads.ternary(workloads.rng_for(1401), 300, K, workloads.TERNARY_UNIFORM), dev)
    for r in range(x.shape[0]):
        _, q1, g1 = bl.quant_forward(to_dev(x[r:r + 1], dev), wp, 0.25)
        np.testing.assert_array_equal(host(q1)[0], q_ref[r])
        assert host(g1)[0] == g_ref[r]


def test_quant_empty_shapes(dev):
    q, g = bl.quant_act(torch.zeros((0, 64), device=dev))
    assert q.shape == (0, 64)
    g = torch.full((3,), 5.0, device=dev)
    q = torch.empty((3, 0), dtype=torch.int8, device=dev)
    bl.quant_act(torch.zeros((3, 0), device=dev), out=(q, g))
    assert not host(g).any()


# ------------------------------------------------------------------ packing

@pytest.mark.parametrize("N,K", [(1, 16), (33, 1040), (64, 4096), (100, 48), (7, 131072)])
def test_pack_bit_exact(dev, N, K):
    w = workloads.ternary(workloads.rng_for(300, N, K), N, K)
    ref, bad_ref = oracle.pack(w)
    packed, bad = bl.pack_weights(to_dev(w, dev))
    np.testing.assert_array_equal(host(packed).view(np.uint32), ref)
    assert int(host(bad)[0]) == bad_ref == 0


def test_pack_counts_invalid(dev):
    w = workloads.ternary(workloads.rng_for(301), 40, 64)
    w[3, 5] = 2
    w[39, 63] = -128
    w[0, 0] = 100
    ref, bad_ref = oracle.pack(w)
    packed, bad = bl.pack_weights(to_dev(w, dev), check=False)
    np.testing.assert_array_equal(host(packed).view(np.uint32), ref)
    assert int(host(bad)[0]) == bad_ref == 3
    with pytest.raises(ValueError, match="3 weight entries"):
        bl.pack_weights(to_dev(w, dev))


# ------------------------------------------------------------------ forward, small shapes

FWD_CASES = []
for _M in (1, 2, 3, 4):
    for _N, _K in ((1, 16), (17, 48), (1000, 1040), (2048, 2048), (300, 4096)):
        FWD_CASES.append(("gemv", _M, _N, _K))
# few rows over long K: the vector GEMV splits each row group's units over 2
# or 4 waves (ragged and unaligned rows, a last slice with a single unit)
for _M in (1, 3):
    for _N, _K in ((300, 4112), (2560, 6912), (100, 16400), (5, 12288), (7, 12352)):
        FWD_CASES.append(("gemv", _M, _N, _K))
for _M in (1, 5, 16, 17, 33, 64):
    for _N, _K in ((1, 16), (17, 48), (1000, 1040), (2048, 2048), (300, 4160)):
        FWD_CASES.append(("skinny", _M, _N, _K))
for _M in (1, 64, 100, 257):
    for _N, _K in ((1, 16), (17, 48), (1000, 1040), (130, 2048), (300, 4160)):
        FWD_CASES.append(("gemm", _M, _N, _K))
for _M in (1, 8, 31, 40, 96):
    FWD_CASES.append(("auto", _M, 777, 2112))
# 17..32 tokens over >= 128 column tiles of 128 take the GEMM's 64-row tiles
FWD_CASES += [("auto", 17, 16385, 256), ("auto", 32, 16400, 512), ("auto", 24, 16256, 768)]


@pytest.mark.parametrize("path,M,N,K", FWD_CASES)
def test_forward_parity(dev, path, M, N, K):
    x, w, beta = workloads.random_case(400 + M * 7 + N, M, N, K,
                                       table=workloads.TERNARY_HALF_ZERO if N % 2 else
                                       workloads.TERNARY_UNIFORM)
    x = x.copy()
    if M > 2:
        x[1] = 0.0  # zero token: gamma = 0, y = 0
    q, g, y, acc = run_forward(x, w, beta, dev, PATHS[path])
    q_ref, g_ref = oracle.quant_act(x)
    np.testing.assert_array_equal(q, q_ref)
    y_ref, acc_ref = oracle.forward(q_ref, g_ref, w, beta)
    np.testing.assert_array_equal(acc, acc_ref)
    assert_y_close(y, y_ref)


# The GEMM takes 128 x 256 tiles on its ring loop once M >= 256 and
# there are at least 256 such tiles: ragged M and N, and 1, 2, 3 and 5 K steps
# of 128 (the prologue's re-reads past the end, and an odd ring rotation).
WIDE_GEMM_CASES = [(257, 22053, 128), (256, 32769, 256), (300, 22016, 384), (384, 22016, 640)]


# At most 256 tiles of 64 x 128 and K % 256 == 0: 64-row tiles whose two K
# groups share each weight copy (ragged M, a last row tile with one row,
# ragged N).  K % 512 == 0 up to 8192: two steps a group per stage (1, 2, 3,
# 5, 7, 9 and 16 stages; 17 tokens over 129 column tiles; two full row
# tiles); otherwise one step a group in four stages (1, 3, 27, 34, 35, 36 and
# 40 step pairs; 18 tiles, not a multiple of the eight XCDs).
SMALL_TILE_GEMM_CASES = [(64, 3000, 2560), (65, 1000, 768), (96, 2000, 1536), (300, 700, 1536),
                         (512, 257, 256), (65, 300, 9216), (100, 1000, 4608), (300, 1536, 6912),
                         (37, 3000, 8192), (100, 2000, 8704), (70, 1100, 10240), (40, 700, 512),
                         (50, 1500, 8960), (17, 16400, 1024), (128, 1000, 3584)]


@pytest.mark.parametrize("M,N,K", SMALL_TILE_GEMM_CASES)
def test_gemm_small_tiles_parity(dev, M, N, K):
    assert -(-M // 64) * -(-N // 128) <= 256 and K % 256 == 0
    x, w, beta = workloads.random_case(950 + M + K, M, N, K, table=workloads.TERNARY_HALF_ZERO)
    x = x.copy()
    x[M - 1] = 0.0  # zero token in the last row tile
    q, g, y, acc = run_forward(x, w, beta, dev, bl.PATH_GEMM)
    q_ref, g_ref = oracle.quant_act(x)
    np.testing.assert_array_equal(q, q_ref)
    y_ref, acc_ref = oracle.forward(q_ref, g_ref, w, beta)
    np.testing.assert_array_equal(acc, acc_ref)
    assert_y_close(y, y_ref)


# Neither of the above (K % 256 == 128, or more than 256 tiles of 64 x 128):
# 128 x 128 tiles on the ring loop.
MID_GEMM_CASES = [(100, 1000, 640), (200, 8300, 256), (129, 4200, 384), (255, 2100, 1152)]


@pytest.mark.parametrize("M,N,K", MID_GEMM_CASES)
def test_gemm_mid_tiles_parity(dev, M, N, K):
    t64 = -(-M // 64) * -(-N // 128)
    assert (t64 > 256 or K % 256 != 0) and not (M >= 256 and -(-M // 128) * -(-N // 256) >= 256)
    x, w, beta = workloads.random_case(970 + M + K, M, N, K, table=workloads.TERNARY_UNIFORM)
    q, g, y, acc = run_forward(x, w, beta, dev, bl.PATH_GEMM)
    q_ref, g_ref = oracle.quant_act(x)
    np.testing.assert_array_equal(q, q_ref)
    y_ref, acc_ref = oracle.forward(q_ref, g_ref, w, beta)
    np.testing.assert_array_equal(acc, acc_ref)
    assert_y_close(y, y_ref)


@pytest.mark.parametrize("M,N,K", WIDE_GEMM_CASES)
def test_gemm_wide_tiles_parity(dev, M, N, K):
    assert -(-M // 128) * -(-N // 256) >= 256
    x, w, beta = workloads.random_case(900 + M + K, M, N, K, table=workloads.TERNARY_UNIFORM)
    x = x.copy()
    x[M - 2] = 0.0  # zero token in the last row tile
    q, g, y, acc = run_forward(x, w, beta, dev, bl.PATH_GEMM)
    q_ref, g_ref = oracle.quant_act(x)
    np.testing.assert_array_equal(q, q_ref)
    y_ref, acc_ref = oracle.forward(q_ref, g_ref, w, beta)
    np.testing.assert_array_equal(acc, acc_ref)
    assert_y_close(y, y_ref)


# The skinny path sends 5..16 tokens (2..4 at K >= 4096) with K % 256 == 0 to
# the LDS-staged decode kernel.  Cases cover its four workgroup widths (column
# tiles of 16: < 400, >= 400, >= 800, >= 1600 tiles, and the old boundaries
# 320, 640, 1280), ragged N, the largest K whose activation block fits in LDS
# at 16 tokens (9216), and a zero token.  The streamed form (more than four
# 256-chunks per wave, batches of two) runs with an odd number of batches and
# a half-live last batch at (16, 333, 9216), (8, 25600, 6912) and
# (5, 12800, 8704), with an even number and a half-live last batch at the last.
DECODE_LDS_CASES = [(5, 1000, 256), (7, 5200, 512), (12, 10300, 1024), (16, 20500, 768),
                    (16, 333, 9216), (9, 2570, 2560), (13, 40, 4096), (6, 17, 256),
                    (2, 3000, 8192), (3, 700, 6912), (4, 129, 6144),
                    (8, 6401, 512), (11, 12800, 256), (9, 25700, 512), (4, 11008, 4096),
                    (2, 6500, 4096), (3, 40, 4096), (8, 25600, 6912), (5, 12800, 8704),
                    # two K parts per tile (up to 8 tokens, K % 512 == 0) on each
                    # workgroup width (128, 64 and 32 rows), with ragged row tails
                    (8, 25700, 1024), (3, 26000, 2048), (8, 9700, 512), (6, 150, 1536),
                    (7, 9631, 2560),
                    # one token on the decode kernel (K >= 4096, K % 512 == 0, N / 64 >= 150)
                    (1, 9700, 4096), (1, 25700, 4608), (1, 9631, 5120),
                    # 9..16 tokens as two token groups on two-part tiles (K % 512 == 0,
                    # N / 64 >= 150), 128- and 64-row workgroups, ragged row tails
                    (16, 25700, 2048), (13, 9650, 1536), (10, 12800, 4608)]


@pytest.mark.parametrize("M,N,K", DECODE_LDS_CASES)
def test_decode_lds_parity(dev, M, N, K):
    x, w, beta = workloads.random_case(700 + M + N, M, N, K, table=workloads.TERNARY_HALF_ZERO)
    x = x.copy()
    if M > 1:
        x[1] = 0.0
    q, g, y, acc = run_forward(x, w, beta, dev, bl.PATH_SKINNY)
    q_ref, g_ref = oracle.quant_act(x)
    np.testing.assert_array_equal(q, q_ref)
    y_ref, acc_ref = oracle.forward(q_ref, g_ref, w, beta)
    np.testing.assert_array_equal(acc, acc_ref)
    assert_y_close(y, y_ref)


@pytest.mark.parametrize("M,N,K", [(16, 700, 9216), (8, 700, 9216), (16, 9650, 4608)])
def test_decode_lds_extreme_codes(dev, M, N, K):
    q = np.full((M, K), 127, np.int8)
    q[1::2] = -127
    w = np.ones((N, K), np.int8)
    w[1::3] = -1
    g = np.linspace(0.5, 2.0, M).astype(np.float32)
    packed, _ = bl.pack_weights(to_dev(w, dev))
    y, acc = bl.forward(to_dev(q, dev), to_dev(g, dev), packed, 0.03, path=bl.PATH_SKINNY,
                        want_acc=True)
    y_ref, acc_ref = oracle.forward(q, g, w, np.float32(0.03))
    np.testing.assert_array_equal(host(acc), acc_ref)
    assert np.abs(acc_ref).max() == 127 * K
    assert_y_close(host(y), y_ref)


def test_paths_agree_bitwise(dev):
    x, w, beta = workloads.random_case(500, 4, 640, 4096)
    outs = [run_forward(x, w, beta, dev, p) for p in (bl.PATH_GEMV, bl.PATH_SKINNY, bl.PATH_GEMM)]
    for o in outs[1:]:
        np.testing.assert_array_equal(o[3], outs[0][3])
        np.testing.assert_array_equal(o[2], outs[0][2])


def test_forward_extreme_values_and_max_k(dev):
    K = 131072
    q = np.full((2, K), 127, np.int8)
    q[1] = -127
    g = np.array([3.0, 0.5], np.float32)
    w = np.ones((3, K), np.int8)
    w[1] = -1
    w[2, ::2] = 0
    wp = gpu_pack(w, dev)
    y_ref, acc_ref = oracle.forward(q, g, w, 0.02)
    for p in (bl.PATH_GEMV, bl.PATH_SKINNY, bl.PATH_GEMM):
        y, acc = bl.forward(to_dev(q, dev), to_dev(g, dev), wp, 0.02, path=p, want_acc=True)
        np.testing.assert_array_equal(host(acc), acc_ref)
        assert_y_close(host(y), y_ref)
    assert acc_ref[0, 0] == 127 * K


def test_forward_empty_and_k0(dev):
    y = bl.forward(torch.zeros((0, 32), dtype=torch.int8, device=dev),
                   torch.zeros((0,), device=dev),
                   torch.zeros((5, 2), dtype=torch.int32, device=dev), 0.5)
    assert y.shape == (0, 5)
    y, acc = bl.forward(torch.zeros((3, 0), dtype=torch.int8, device=dev),
                        torch.ones((3,), device=dev),
                        torch.zeros((4, 0), dtype=torch.int32, device=dev), 0.5, want_acc=True)
    assert not host(y).any() and not host(acc).any()


def test_misaligned_tensor_is_rejected(dev):
    buf = torch.zeros(64 + 1, dtype=torch.int8, device=dev)
    xq = buf[1:].view(4, 16)
    with pytest.raises(bl.BitLinearError) as ei:
        bl.forward(xq, torch.ones(4, device=dev), torch.zeros((2, 1), dtype=torch.int32, device=dev), 1.0)
    assert ei.value.status == bl.ERR_ALIGN


# ------------------------------------------------------------------ full-size workloads

def _freivalds(acc, q, w, seed):
    """acc @ v == q @ (w^T v) in exact int64, for two independent random
    vectors v with entries in {-3..-1, 1..3}: no entry is 0, so a single
    wrong accumulator always changes its row's sum."""
    rng = workloads.rng_for(600, seed)
    for _ in range(2):
        v = (rng.integers(1, 4, size=w.shape[0]) * rng.choice([-1, 1], size=w.shape[0])).astype(np.int64)
        u = np.zeros(w.shape[1], np.int64)
        for r0 in range(0, w.shape[0], 2048):
            u += v[r0:r0 + 2048] @ w[r0:r0 + 2048].astype(np.int64)
        lhs = acc.astype(np.int64) @ v
        rhs = q.astype(np.int64) @ u
        np.testing.assert_array_equal(lhs, rhs)


def _workload_case(wid, M):
    wl = workloads.WORKLOADS[wid]
    x = workloads.workload_activations(wid, M)
    xf = oracle.bf16_to_f32(x) if wl.act == "normal_bf16" else x
    return wl, x, xf


@pytest.mark.parametrize("wid,M", [(1, 1), (2, 1), (2, 4), (2, 16), (5, 1), (5, 8), (5, 64)])
def test_workload_full_parity(dev, wid, M):
    wl, x, xf = _workload_case(wid, M)
    w = workloads.workload_weights(wid)
    beta = workloads.workload_beta(wid)
    q, g, y, acc = run_forward(xf, w, beta, dev)
    q_ref, g_ref = oracle.quant_act(xf)
    np.testing.assert_array_equal(q, q_ref)
    np.testing.assert_array_equal(g, g_ref)
    y_ref, acc_ref = oracle.forward(q_ref, g_ref, w, beta)
    np.testing.assert_array_equal(acc, acc_ref)
    assert_y_close(y, y_ref)
    assert np.abs(acc).max() <= 127 * wl.K


@pytest.mark.parametrize("wid,M", [(3, 2048), (5, 512)])
def test_workload_large_m_full(dev, wid, M):
    """The two GEMM-sized workloads at full size, every output element by
    element against the oracle (the oracle's int64 accumulation over unpacked
    weights; about 92 G and 120 G multiply-adds on the host's cores), from the
    activations as the bench feeds them (bf16 bits for the prefill workload),
    into guarded outputs; a checksum with two nonzero random vectors on top."""
    wl, x, xf = _workload_case(wid, M)
    w = workloads.workload_weights(wid)
    beta = workloads.workload_beta(wid)
    N, K = w.shape
    xd = to_dev(x, dev, torch.bfloat16) if wl.act == "normal_bf16" else to_dev(x, dev)
    gq, gg = Guard((M, K), torch.int8, dev), Guard((M,), torch.float32, dev)
    q, g = bl.quant_act(xd, out=(gq.t, gg.t))
    wp = gpu_pack(w, dev)
    gy, ga = Guard((M, N), torch.float32, dev), Guard((M, N), torch.int32, dev)
    y, acc = bl.forward(q, g, wp, beta, want_acc=True, out=gy.t, acc_out=ga.t)
    for gd, nm in ((gq, "x_q"), (gg, "gamma"), (gy, "y"), (ga, "acc")):
        gd.check(nm)
    q, g, y, acc = host(q), host(g), host(y), host(acc)
    print(f"workload {wid} M={M}: device done, oracle running", flush=True)
    q_ref, g_ref = oracle.quant_act(xf)
    np.testing.assert_array_equal(q, q_ref)
    np.testing.assert_array_equal(g, g_ref)
    y_ref, acc_ref = oracle.forward(q_ref, g_ref, w, beta)
    np.testing.assert_array_equal(acc, acc_ref)
    assert_y_close(y, y_ref)
    assert np.abs(acc).max() <= 127 * wl.K
    _freivalds(acc, q_ref, w, wid)


# ------------------------------------------------------------------ GLU (workload 4)

@pytest.mark.parametrize("M", [1, 512])
def test_glu_stagewise(dev, M):
    wl = workloads.WORKLOADS[4]
    x = workloads.workload_activations(4, M)
    wg, wu, wd = workloads.glu_weights()
    betas = workloads.glu_betas()
    gain = np.ones(wl.K, np.float32)
    ref = oracle.glu(x, wg, wu, wd, betas, gain, wl.rms_eps)

    packs = [gpu_pack(w, dev) for w in (wg, wu, wd)]
    st = bl.glu(to_dev(x, dev), *packs, betas, to_dev(gain, dev), wl.rms_eps, stages=True)
    st = {k: host(v) for k, v in st.items()}

    np.testing.assert_array_equal(st["q"], ref["q"])
    assert_y_close(st["gamma"], ref["gamma"])
    # (i) gate and up accumulators exact, their outputs within 1e-6
    for nm in ("gate", "up"):
        np.testing.assert_array_equal(st[f"acc_{nm}"], ref[f"acc_{nm}"])
    for nm in ("gate", "up"):
        assert_y_close(st[f"y_{nm}"], ref[f"y_{nm}"])
    # (ii) h: float64 SiLU*up rounded once to fp32 on both sides; the device's
    # exp may differ from the host's in the last bit, so h is held to 1e-6
    assert_y_close(st["h"], ref["h64"])
    n_h_diff = int((st["h"] != ref["h"]).sum())
    # (iii) the requantisation is exact on the device's own h: codes and gamma_h
    # bit-identical to the oracle's quantiser applied to h_gpu
    hq_ref, gh_ref = oracle.quant_act(st["h"])
    np.testing.assert_array_equal(st["h_q"], hq_ref)
    np.testing.assert_array_equal(st["gamma_h"].view(np.uint32), gh_ref.view(np.uint32))
    # (iv) the down projection is exact on the device's own codes
    y_down_ref, acc_down_ref = oracle.forward(st["h_q"], st["gamma_h"], wd, betas[2])
    np.testing.assert_array_equal(st["acc_down"], acc_down_ref)
    assert_y_close(st["y"], y_down_ref)
    # (v) report how many codes differ from the oracle's own chain (h from the
    # host's exp); they may differ only where h sits within rounding distance of
    # a half-integer step
    t_ref = ref["h"].astype(np.float64) / ref["gamma_h"][:, None].astype(np.float64) * 128.0
    dist = np.abs(t_ref - (np.floor(t_ref) + 0.5))
    diff = st["h_q"].astype(np.int32) - ref["h_q"].astype(np.int32)
    assert np.abs(diff).max() <= 1
    assert (dist[diff != 0] < 1e-3).all()
    assert_y_close(st["gamma_h"], ref["gamma_h"])
    print(f"GLU M={M}: h differs from fl32(h_ref) at {n_h_diff} entries, "
          f"h_q codes differ from the oracle chain at {int((diff != 0).sum())}")


@pytest.mark.parametrize("F", [16, 4096, 4112, 6912, 16384, 20000])
def test_silu_quant_row_widths(dev, F):
    """SiLU(gate) * up and its quantisation across the row widths of the
    quantiser: 256 threads up to 4096 elements, 512 beyond (one chunk per
    thread up to 8192, values kept in registers up to 16384, re-read past
    that).  h agrees with the oracle's float64 product rounded to fp32 within
    one ulp (the device and host exp may differ in the last bit); the codes
    and gamma are exact on the device's own h."""
    rng = workloads.rng_for(1990, F)
    M = 3
    gate = (3.0 * rng.standard_normal((M, F))).astype(np.float32)
    up = rng.standard_normal((M, F)).astype(np.float32)
    gate[1, F // 2] = 40.0  # a large product sets gamma of row 1
    gd_, ud_ = to_dev(gate, dev), to_dev(up, dev)
    gh, ghq, gg = (Guard((M, F), torch.float32, dev), Guard((M, F), torch.int8, dev),
                   Guard((M,), torch.float32, dev))
    st = bl.lib.bitlinear_silu_mul_quant(gd_.data_ptr(), ud_.data_ptr(), M, F, gh.t.data_ptr(),
                                         ghq.t.data_ptr(), gg.t.data_ptr(), stream())
    assert st == 0, bl.last_error()
    for gdd, nm in ((gh, "h"), (ghq, "h_q"), (gg, "gamma_h")):
        gdd.check(f"silu_mul_quant {nm} F={F}")
    h_q, g, h = ghq.t, gg.t, host(gh.t)
    h_ref = oracle.silu_mul(gate, up).astype(np.float32)
    ulp = np.spacing(np.abs(h_ref)).astype(np.float64)
    assert (np.abs(h.astype(np.float64) - h_ref.astype(np.float64)) <= ulp).all()
    q_ref, g_ref = oracle.quant_act(h)
    np.testing.assert_array_equal(host(h_q), q_ref)
    np.testing.assert_array_equal(host(g).view(np.uint32), g_ref.view(np.uint32))


@pytest.mark.parametrize("M", [1, 33, 512])
def test_glu_stacked_matches_stagewise(dev, M):
    """Gate and up as one product on the stacked weights [W_gate; W_up] that
    writes only accumulators (M = 1: fused with the RMSNorm quantisation), then
    bitlinear_silu_mul_quant_acc: every stage bit-identical to the stage-wise
    chain, which test_glu_stagewise pins to the oracle."""
    wl = workloads.WORKLOADS[4]
    x = workloads.workload_activations(4, M)
    wg, wu, wd = workloads.glu_weights()
    betas = workloads.glu_betas()
    F = wg.shape[0]
    gain = to_dev(np.ones(wl.K, np.float32), dev)
    pg, pu, pd = (gpu_pack(w, dev) for w in (wg, wu, wd))
    xd = to_dev(x, dev)
    st = {k: host(v) for k, v in bl.glu(xd, pg, pu, pd, betas, gain, wl.rms_eps,
                                         stages=True).items()}
    gu = torch.cat([pg, pu], dim=0).contiguous()
    if M == 1:
        acc_gu, q, g = bl.quant_forward(xd, gu, 1.0, rms_gain=gain, rms_eps=wl.rms_eps,
                                        acc_only=True)
    else:
        q, g = bl.quant_act(xd, gain, wl.rms_eps)
        acc_gu = bl.forward(q, g, gu, 1.0, acc_only=True)
    h_q, g_h, h = bl.silu_mul_quant_acc(acc_gu, g, betas[0], betas[1], want_h=True)
    y = bl.forward(h_q, g_h, pd, betas[2])
    acc_gu = host(acc_gu)
    np.testing.assert_array_equal(host(q), st["q"])
    np.testing.assert_array_equal(host(g).view(np.uint32), st["gamma"].view(np.uint32))
    np.testing.assert_array_equal(acc_gu[:, :F], st["acc_gate"])
    np.testing.assert_array_equal(acc_gu[:, F:], st["acc_up"])
    np.testing.assert_array_equal(host(h).view(np.uint32), st["h"].view(np.uint32))
    np.testing.assert_array_equal(host(h_q), st["h_q"])
    np.testing.assert_array_equal(host(g_h).view(np.uint32), st["gamma_h"].view(np.uint32))
    np.testing.assert_array_equal(host(y).view(np.uint32), st["y"].view(np.uint32))


def test_forward_accumulators_only(dev):
    x, w, beta = workloads.random_case(1200, 40, 300, 512)
    q, g = bl.quant_act(to_dev(x, dev))
    wp = gpu_pack(w, dev)
    for path in (bl.PATH_SKINNY, bl.PATH_GEMM, bl.PATH_AUTO):
        acc = bl.forward(q, g, wp, beta, path=path, acc_only=True)
        y2, acc2 = bl.forward(q, g, wp, beta, path=path, want_acc=True)
        np.testing.assert_array_equal(host(acc), host(acc2))
    acc_k0 = bl.forward(torch.zeros((3, 0), dtype=torch.int8, device=dev),
                        torch.zeros(3, device=dev), torch.zeros((5, 0), dtype=torch.int32, device=dev),
                        1.0, acc_only=True)
    assert acc_k0.shape == (3, 5) and not host(acc_k0).any()


def test_glu_down_projection_on_oracle_codes(dev):
    """The down projection (K = 6912) on the oracle's own requantised h."""
    wl = workloads.WORKLOADS[4]
    x = workloads.workload_activations(4, 512)
    wg, wu, wd = workloads.glu_weights()
    betas = workloads.glu_betas()
    ref = oracle.glu(x, wg, wu, wd, betas, np.ones(wl.K, np.float32), wl.rms_eps)
    y, acc = bl.forward(to_dev(ref["h_q"], dev), to_dev(ref["gamma_h"], dev), gpu_pack(wd, dev),
                        betas[2], want_acc=True)
    np.testing.assert_array_equal(host(acc), ref["acc_down"])
    assert_y_close(host(y), ref["y"])


# ------------------------------------------------------------------ absmean ternarisation

def _ternarize_check(W, dev):
    Wd = to_dev(W, dev)
    packed, beta, beta64, codes = bl.ternarize(Wd, want_codes=True)
    w_ref, b_ref = oracle.ternarize(W)
    assert float(host(beta64)[0]) == b_ref                       # same ordered double sum
    assert host(beta)[0] == np.float32(b_ref)
    np.testing.assert_array_equal(host(codes), w_ref)
    ref_packed, bad = oracle.pack(w_ref)
    assert bad == 0
    np.testing.assert_array_equal(host(packed).view(np.uint32), ref_packed)
    return w_ref, b_ref, packed, beta


@pytest.mark.parametrize("N,K,dist", [
    # 1 to 3 level passes of the pairwise reduction; (65, 64) is the first size
    # with a level pass (65 groups of 64), (1, 80) the smallest scratch margin
    (1, 32, "normal"), (1, 80, "normal"), (65, 64, "normal"), (37, 48, "normal"),
    (100, 4096, "normal"), (33, 112, "student_t3"),
    (2570, 2560, "normal"), (11008, 4096, "normal"), (64, 256, "scaled_ternary")])
def test_ternarize_parity(dev, N, K, dist):
    rng = workloads.rng_for(950, N, K)
    if dist == "normal":
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    elif dist == "student_t3":
        W = (rng.standard_t(3, (N, K)) * 0.05).astype(np.float32)
    else:
        T = workloads.ternary(rng, N, K, workloads.TERNARY_HALF_ZERO)
        W = T.astype(np.float32) * np.float32(0.75)
    w_ref, _, _, _ = _ternarize_check(W, dev)
    if dist == "scaled_ternary":
        np.testing.assert_array_equal(w_ref, T)


def test_ternarize_ties_on_gpu(dev):
    # the hand-derived 2 x 16 example, repeated along K (same mean): ties at beta/2 -> 0
    g = json.load(open(os.path.join(GOLDEN, "ternarize_2x16.json")))
    W = np.concatenate([np.array(g["W"], np.float32)] * 2, axis=1)
    w_ref, b_ref, _, _ = _ternarize_check(W, dev)
    assert b_ref == g["beta"]
    np.testing.assert_array_equal(w_ref, np.concatenate([np.array(g["codes"], np.int8)] * 2, axis=1))


def test_ternarize_empty(dev):
    for shape in ((0, 64), (5, 0)):
        W = torch.zeros(shape, dtype=torch.float32, device=dev)
        packed, beta, beta64 = bl.ternarize(W)
        assert float(host(beta)[0]) == 0.0 and float(host(beta64)[0]) == 0.0


def test_ternarize_then_forward(dev):
    # fp weights -> ternary + beta on the GPU -> the layer, against the oracle chain
    rng = workloads.rng_for(951, 1)
    N, K, M = 640, 2048, 6
    W = (rng.standard_normal((N, K)) * 0.03).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w_ref, b_ref, packed, beta = _ternarize_check(W, dev)
    q, g = bl.quant_act(to_dev(x, dev))
    y, acc = bl.forward(q, g, packed, float(host(beta)[0]), want_acc=True)
    q_ref, g_ref = oracle.quant_act(x)
    y_ref, acc_ref = oracle.forward(q_ref, g_ref, w_ref, np.float32(b_ref))
    np.testing.assert_array_equal(host(acc), acc_ref)
    assert_y_close(host(y), y_ref)



# ------------------------------------------------------------------ 1-bit weights

def _binarize_check(W, dev):
    packed1, codes, alpha, alpha64, beta, beta64 = bl.binarize(to_dev(W, dev))
    w_ref, a_ref = oracle.binarize(W)
    _, b_ref = oracle.ternarize(W)                 # beta = the absmean of the same tree
    assert float(host(alpha64)[0]) == a_ref
    assert host(alpha)[0] == np.float32(a_ref)
    assert float(host(beta64)[0]) == b_ref
    assert host(beta)[0] == np.float32(b_ref)
    np.testing.assert_array_equal(host(codes), w_ref)
    p_ref, bad = oracle.pack1(w_ref)
    assert bad == 0
    np.testing.assert_array_equal(host(packed1).view(np.uint32), p_ref)
    return w_ref, packed1, codes, float(host(beta)[0])


@pytest.mark.parametrize("N,K", [(1, 32), (3, 96), (257, 512), (1000, 4096), (11008, 4096)])
def test_binarize_parity(dev, N, K):
    rng = workloads.rng_for(960, N, K)
    W = (rng.standard_normal((N, K)) * 0.02 + 0.003).astype(np.float32)
    _binarize_check(W, dev)


def test_binarize_ties_on_gpu(dev):
    g = json.load(open(os.path.join(GOLDEN, "binarize_2x32.json")))
    W = np.array(g["W"], np.float32)
    w_ref, packed1, _, _ = _binarize_check(W, dev)
    np.testing.assert_array_equal(w_ref, np.array(g["codes"], np.int8))
    np.testing.assert_array_equal(host(packed1).view(np.uint32), np.array(g["packed"], np.uint32))


def test_pack_weights1_parity(dev):
    rng = workloads.rng_for(961, 1)
    w = np.where(rng.random((300, 640)) < 0.5, 1, -1).astype(np.int8)
    packed1, _ = bl.pack_weights1(to_dev(w, dev))
    np.testing.assert_array_equal(host(packed1).view(np.uint32), oracle.pack1(w)[0])
    w[5, 9] = 0
    w[7, 1] = 2
    _, bad = bl.pack_weights1(to_dev(w, dev), check=False)
    assert int(host(bad)[0]) == 2


# 1 token, 2..4 tokens below K = 4096, and K % 512 != 0: vector-ALU kernel;
# 5..16 tokens (2..4 from K = 4096) with K % 512 == 0: the LDS-staged MFMA kernel
# in its 1-bit form (all four workgroup widths, one and several load units a
# wave, an odd number of batches at K = 6656 with 1600 tiles); 17 and 20 tokens:
# several vector-ALU passes
@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (2, 17, 192), (3, 1000, 4096), (4, 333, 2560),
                                   (5, 640, 1024), (9, 100, 64), (1, 11008, 4096),
                                   (7, 5200, 512), (12, 10300, 1024), (16, 20500, 768),
                                   (16, 20500, 1536), (8, 25600, 6656), (6, 700, 9216),
                                   (16, 333, 8192), (17, 200, 512), (20, 96, 320),
                                   (4, 11008, 4096), (2, 6500, 8192), (3, 40, 4096),
                                   # two K parts per tile (M <= 8, K % 1024 == 0) on
                                   # 128-row workgroups; one tile a wave on 128-row groups
                                   (8, 25700, 2048), (9, 25700, 1024),
                                   # one token on the decode kernel (K >= 4096,
                                   # K % 1024 == 0, N / 64 >= 150)
                                   (1, 9700, 4096), (1, 25700, 5120)])
def test_forward1_parity(dev, M, N, K):
    rng = workloads.rng_for(962, M, N, K)
    w = np.where(rng.random((N, K)) < 0.5, 1, -1).astype(np.int8)
    x = rng.standard_normal((M, K)).astype(np.float32)
    if M > 2:
        x[1] = 0.0
    q, g = bl.quant_act(to_dev(x, dev))
    packed1, _ = bl.pack_weights1(to_dev(w, dev))
    gy, ga = Guard((M, N), torch.float32, dev), Guard((M, N), torch.int32, dev)
    st = bl.lib.bitlinear_forward1(q.data_ptr(), g.data_ptr(), M, K, packed1.data_ptr(), N,
                                   ctypes.c_float(0.02), gy.t.data_ptr(), ga.t.data_ptr(), stream())
    assert st == 0, bl.last_error()
    gy.check(f"forward1 y M={M} N={N} K={K}")
    ga.check(f"forward1 acc M={M} N={N} K={K}")
    y, acc = gy.t, ga.t
    q_ref, g_ref = oracle.quant_act(x)
    np.testing.assert_array_equal(host(q), q_ref)
    y_ref, acc_ref = oracle.forward(q_ref, g_ref, w, np.float32(0.02))
    np.testing.assert_array_equal(host(acc), acc_ref)
    assert_y_close(host(y), y_ref)


def test_binarize_then_both_forward_paths(dev):
    # fp weights -> +-1 codes on the GPU -> the 1-bit decode product and the
    # 2-bit path (codes packed by bitlinear_pack_weights) agree bit for bit
    rng = workloads.rng_for(963, 1)
    N, K, M = 700, 2048, 3
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    w_ref, packed1, codes, beta = _binarize_check(W, dev)
    q, g = bl.quant_act(to_dev(rng.standard_normal((M, K)).astype(np.float32), dev))
    y1, acc1 = bl.forward1(q, g, packed1, beta, want_acc=True)
    packed2, _ = bl.pack_weights(codes)
    y2, acc2 = bl.forward(q, g, packed2, beta, want_acc=True)
    np.testing.assert_array_equal(host(acc1), host(acc2))
    np.testing.assert_array_equal(host(y1), host(y2))
    y_ref, acc_ref = oracle.forward(host(q), host(g), w_ref, np.float32(beta))
    np.testing.assert_array_equal(host(acc1), acc_ref)


# ------------------------------------------------------------------ group quantisation

def grouped_bound(acc_ref, beta, gamma_ref):
    """|y - y_ref| bound of the grouped sum: each group term has two fp32
    roundings, the G terms are added in fp32 (G - 1 roundings) and y_ref is
    rounded once, so (G + 2) u times the sum of |terms| (u = 2^-24), with
    one u of slack."""
    G = acc_ref.shape[0]
    terms = np.abs(acc_ref.astype(np.float64) * beta.astype(np.float64)[:, None, None]
                   * gamma_ref.astype(np.float64)[:, :, None] / 128.0)
    return (G + 3) * 2.0 ** -24 * terms.sum(axis=0)


def group_major(a, G):
    """[R][K] -> [G][R][K/G] (group g = columns g*K/G .. (g+1)*K/G)."""
    R, K = a.shape
    return np.ascontiguousarray(a.reshape(R, G, K // G).transpose(1, 0, 2))


def pack_grouped(w, G, dev):
    N, K = w.shape
    packed, bad = bl.pack_weights(to_dev(group_major(w, G).reshape(G * N, K // G), dev))
    assert int(host(bad)[0]) == 0
    return packed.view(G, N, K // (16 * G))


@pytest.mark.parametrize("M,K,G,src", [
    (5, 1024, 4, "f32"), (3, 4096, 16, "f32"), (7, 2560, 5, "f32"), (1, 64, 4, "f32"),
    (2, 512, 2, "bf16"), (4, 2560, 4, "rms"), (9, 4096, 8, "rms"), (300, 1024, 2, "f32")])
def test_quant_grouped_parity(dev, M, K, G, src):
    rng = workloads.rng_for(970, M, K, G)
    x = (rng.standard_t(3, (M, K)) * 2.0).astype(np.float32)
    x[:, 7] *= 50.0
    if src == "bf16":
        bits = workloads.f32_to_bf16_bits(x)
        xd = to_dev(bits, dev, torch.bfloat16)
        x_ref = oracle.bf16_to_f32(bits)
    else:
        xd = to_dev(x, dev)
        x_ref = x
    gain = (rng.random(K) + 0.5).astype(np.float32) if src == "rms" else None
    q, g = bl.quant_act_grouped(xd, G, None if gain is None else to_dev(gain, dev), 1e-6)
    q_ref, g_ref = oracle.quant_act_grouped(x_ref, G, gain, 1e-6)
    np.testing.assert_array_equal(host(q), q_ref)
    if gain is None:
        np.testing.assert_array_equal(host(g), g_ref)
    else:
        assert_y_close(host(g), g_ref)


@pytest.mark.parametrize("M,K,G,N", [
    (1, 4096, 4, 1000), (4, 4096, 4, 700), (16, 4096, 4, 2000), (5, 2048, 2, 333),
    (33, 1024, 4, 517), (100, 2560, 5, 300), (2, 512, 8, 129), (1, 256, 1, 64),
    (8, 8192, 8, 600), (3, 4096, 2, 20480), (16, 2048, 8, 5000), (12, 4096, 4, 11008)])
def test_forward_grouped_parity(dev, M, K, G, N):
    rng = workloads.rng_for(971, M, K, G, N)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = workloads.ternary(rng, N, K, workloads.TERNARY_UNIFORM)
    beta = rng.uniform(0.01, 0.05, G).astype(np.float32)
    q_ref, g_ref = oracle.quant_act_grouped(x, G)
    y_ref, acc_ref = oracle.forward_grouped(q_ref, g_ref, w, beta)
    qd, gd_, wpg, bd = to_dev(q_ref, dev), to_dev(g_ref, dev), pack_grouped(w, G, dev), to_dev(beta, dev)
    gy, ga = Guard((M, N), torch.float32, dev), Guard((G, M, N), torch.int32, dev)
    st = bl.lib.bitlinear_forward_grouped(qd.data_ptr(), gd_.data_ptr(), M, K, G, wpg.data_ptr(), N,
                                          bd.data_ptr(), gy.t.data_ptr(), ga.t.data_ptr(), stream())
    assert st == 0, bl.last_error()
    gy.check(f"forward_grouped y M={M} K={K} G={G} N={N}")
    ga.check(f"forward_grouped acc M={M} K={K} G={G} N={N}")
    y, acc = gy.t, ga.t
    np.testing.assert_array_equal(host(acc), acc_ref)
    err = np.abs(host(y).astype(np.float64) - y_ref.astype(np.float64))
    assert (err <= grouped_bound(acc_ref, beta, g_ref)).all()


def test_forward_grouped_one_group_is_forward(dev):
    rng = workloads.rng_for(972, 1)
    M, K, N = 6, 1024, 300
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = workloads.ternary(rng, N, K, workloads.TERNARY_HALF_ZERO)
    q, g = bl.quant_act(to_dev(x, dev))
    wp = gpu_pack(w, dev)
    y1, acc1 = bl.forward(q, g, wp, 0.03, want_acc=True)
    y, acc = bl.forward_grouped(q.view(1, M, K), g.view(1, M), wp.view(1, N, K // 16),
                                torch.tensor([0.03], dtype=torch.float32, device=dev))
    np.testing.assert_array_equal(host(acc)[0], host(acc1))
    np.testing.assert_array_equal(host(y), host(y1))


@pytest.mark.parametrize("N,K,G", [(300, 1024, 4), (64, 4096, 16), (1000, 2560, 5), (7, 128, 2)])
def test_ternarize_grouped_parity(dev, N, K, G):
    rng = workloads.rng_for(973, N, K, G)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, :K // G] *= 3.0  # groups with different scales
    packed, beta, beta64, codes = bl.ternarize_grouped(to_dev(group_major(W, G), dev), want_codes=True)
    w_ref, b_ref = oracle.ternarize_grouped(W, G)
    np.testing.assert_array_equal(host(codes), group_major(w_ref, G))
    np.testing.assert_array_equal(host(beta64), b_ref)
    np.testing.assert_array_equal(host(beta), b_ref.astype(np.float32))
    p_ref, bad = oracle.pack(group_major(w_ref, G).reshape(G * N, K // G))
    assert bad == 0
    np.testing.assert_array_equal(host(packed).view(np.uint32).reshape(G * N, -1), p_ref)


def test_grouped_chain(dev):
    # fp weights and activations -> grouped ternarisation and quantisation ->
    # grouped product, all on the GPU, against the oracle chain
    rng = workloads.rng_for(974, 1)
    M, K, G, N = 9, 4096, 4, 1500
    W = (rng.standard_normal((N, K)) * 0.03).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    packed, beta, _ = bl.ternarize_grouped(to_dev(group_major(W, G), dev))
    q, g = bl.quant_act_grouped(to_dev(x, dev), G)
    y, acc = bl.forward_grouped(q, g, packed, beta)
    w_ref, b_ref = oracle.ternarize_grouped(W, G)
    q_ref, g_ref = oracle.quant_act_grouped(x, G)
    y_ref, acc_ref = oracle.forward_grouped(q_ref, g_ref, w_ref, b_ref.astype(np.float32))
    np.testing.assert_array_equal(host(q), q_ref)
    np.testing.assert_array_equal(host(acc), acc_ref)
    err = np.abs(host(y).astype(np.float64) - y_ref.astype(np.float64))
    assert (err <= grouped_bound(acc_ref, b_ref.astype(np.float32), g_ref)).all()


def test_grouped_empty(dev):
    q, g = bl.quant_act_grouped(torch.zeros((0, 256), device=dev), 4)
    assert q.shape == (4, 0, 64)
    q, g = bl.quant_act_grouped(torch.zeros((3, 256), device=dev), 4)
    assert not host(q).any() and not host(g).any()


def test_forward_grouped_without_acc(dev):
    # the one-launch decode path takes acc = NULL and gives the same y
    rng = workloads.rng_for(975, 1)
    M, K, G, N = 16, 4096, 4, 3000
    assert bl.lib.bitlinear_forward_grouped_one_launch(M, K, G, N) == 1
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = workloads.ternary(rng, N, K, workloads.TERNARY_HALF_ZERO)
    beta = to_dev(rng.uniform(0.01, 0.05, G).astype(np.float32), dev)
    q, g = bl.quant_act_grouped(to_dev(x, dev), G)
    wp = pack_grouped(w, G, dev)
    y1, _ = bl.forward_grouped(q, g, wp, beta)
    y2 = bl.forward_grouped(q, g, wp, beta, want_acc=False)
    np.testing.assert_array_equal(host(y2), host(y1))


# ------------------------------------------------------------------ base-3 weights

@pytest.mark.parametrize("N,K", [(1, 16), (3, 96), (300, 4096), (64, 2560), (33, 6912), (7, 1040)])
def test_pack3_parity(dev, N, K):
    w = workloads.ternary(workloads.rng_for(980, N, K), N, K, workloads.TERNARY_UNIFORM)
    packed3, bad = bl.pack_weights3(to_dev(w, dev))
    p_ref, bad_ref = oracle.pack3(w)
    assert bad_ref == 0
    np.testing.assert_array_equal(host(packed3).view(np.uint8), p_ref)


def test_pack3_counts_bad_entries(dev):
    w = workloads.ternary(workloads.rng_for(980, 1), 5, 160, workloads.TERNARY_UNIFORM)
    w[2, 17] = 2
    w[4, 159] = -7
    packed3, bad = bl.pack_weights3(to_dev(w, dev), check=False)
    p_ref, bad_ref = oracle.pack3(w)
    assert int(host(bad)[0]) == bad_ref == 2
    np.testing.assert_array_equal(host(packed3).view(np.uint8), p_ref)


@pytest.mark.parametrize("M,K,N", [(1, 4096, 1000), (4, 4096, 700), (16, 2560, 513), (3, 6912, 200),
                                   (1, 16, 7), (5, 96, 33), (9, 1040, 100), (2, 8192, 300),
                                   # one pass on MFMA with the activations staged in LDS:
                                   # ragged K (not a multiple of 80 or 320) and N, a K of one
                                   # 16-byte group, every tile width (N = 13000, 6912, 1000
                                   # pick 4, 2, 1 tiles of 16 columns a workgroup), the
                                   # largest staged block at 16 tokens (K = 8960) and the
                                   # first K past it (back to the passes)
                                   (6, 4096, 1000), (7, 16, 5), (8, 11008, 257), (11, 6912, 95),
                                   (13, 2048, 31), (15, 4000, 64), (16, 8960, 70), (16, 8976, 70),
                                   (3, 2048, 25600), (16, 4096, 13000), (4, 4096, 6912), (4, 4096, 11008),
                                   (1, 2560, 6912), (2, 336, 17)])
def test_forward3_parity(dev, M, K, N):
    rng = workloads.rng_for(981, M, K, N)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, 3] *= 40.0
    w = workloads.ternary(rng, N, K, workloads.TERNARY_HALF_ZERO)
    q_ref, g_ref = oracle.quant_act(x)
    y_ref, acc_ref = oracle.forward(q_ref, g_ref, w, np.float32(0.021))
    packed3, _ = bl.pack_weights3(to_dev(w, dev))
    qd, gd_ = to_dev(q_ref, dev), to_dev(g_ref, dev)
    gy, ga = Guard((M, N), torch.float32, dev), Guard((M, N), torch.int32, dev)
    st = bl.lib.bitlinear_forward3(qd.data_ptr(), gd_.data_ptr(), M, K, packed3.data_ptr(), N,
                                   ctypes.c_float(0.021), gy.t.data_ptr(), ga.t.data_ptr(), stream())
    assert st == 0, bl.last_error()
    gy.check(f"forward3 y M={M} K={K} N={N}")
    ga.check(f"forward3 acc M={M} K={K} N={N}")
    y, acc = gy.t, ga.t
    np.testing.assert_array_equal(host(acc), acc_ref)
    assert_y_close(host(y), y_ref)


def test_forward3_matches_the_2bit_layout(dev):
    rng = workloads.rng_for(982, 1)
    M, K, N = 4, 4096, 2000
    w = workloads.ternary(rng, N, K, workloads.TERNARY_UNIFORM)
    q, g = bl.quant_act(to_dev(rng.standard_normal((M, K)).astype(np.float32), dev))
    y2, acc2 = bl.forward(q, g, gpu_pack(w, dev), 0.03, want_acc=True)
    packed3, _ = bl.pack_weights3(to_dev(w, dev))
    y3, acc3 = bl.forward3(q, g, packed3, 0.03, want_acc=True)
    np.testing.assert_array_equal(host(acc3), host(acc2))
    np.testing.assert_array_equal(host(y3), host(y2))


# ------------------------------------------------------------------ edge cases of the widened rows

def test_grouped_rms_bf16_chain(dev):
    # bf16 activations with RMSNorm through the grouped quantiser, then the
    # grouped product (G-launch path: M = 33 > 16)
    rng = workloads.rng_for(990, 1)
    M, K, G, N = 33, 2048, 4, 700
    bits = workloads.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    gain = (rng.random(K) + 0.5).astype(np.float32)
    w = workloads.ternary(rng, N, K, workloads.TERNARY_UNIFORM)
    beta = rng.uniform(0.01, 0.05, G).astype(np.float32)
    q, g = bl.quant_act_grouped(to_dev(bits, dev, torch.bfloat16), G, to_dev(gain, dev), 1e-6)
    q_ref, g_ref = oracle.quant_act_grouped(oracle.bf16_to_f32(bits), G, gain, 1e-6)
    np.testing.assert_array_equal(host(q), q_ref)
    assert_y_close(host(g), g_ref)
    y, acc = bl.forward_grouped(q, g, pack_grouped(w, G, dev), to_dev(beta, dev))
    # the product is checked against the oracle on the GPU's own gamma (its
    # RMSNorm gamma may differ from the oracle's within the 1e-6 tolerance)
    y_ref, acc_ref = oracle.forward_grouped(q_ref, host(g), w, beta)
    np.testing.assert_array_equal(host(acc), acc_ref)
    err = np.abs(host(y).astype(np.float64) - y_ref.astype(np.float64))
    assert (err <= grouped_bound(acc_ref, beta, host(g))).all()


def test_grouped_longest_k_one_launch(dev):
    rng = workloads.rng_for(990, 2)
    M, K, G, N = 1, 131072, 8, 96
    assert bl.lib.bitlinear_forward_grouped_one_launch(M, K, G, N) == 1
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = workloads.ternary(rng, N, K, workloads.TERNARY_HALF_ZERO)
    beta = rng.uniform(0.01, 0.05, G).astype(np.float32)
    q_ref, g_ref = oracle.quant_act_grouped(x, G)
    y_ref, acc_ref = oracle.forward_grouped(q_ref, g_ref, w, beta)
    qd, gd_, wpg, bd = to_dev(q_ref, dev), to_dev(g_ref, dev), pack_grouped(w, G, dev), to_dev(beta, dev)
    gy, ga = Guard((M, N), torch.float32, dev), Guard((G, M, N), torch.int32, dev)
    st = bl.lib.bitlinear_forward_grouped(qd.data_ptr(), gd_.data_ptr(), M, K, G, wpg.data_ptr(), N,
                                          bd.data_ptr(), gy.t.data_ptr(), ga.t.data_ptr(), stream())
    assert st == 0, bl.last_error()
    gy.check(f"forward_grouped y M={M} K={K} G={G} N={N}")
    ga.check(f"forward_grouped acc M={M} K={K} G={G} N={N}")
    y, acc = gy.t, ga.t
    np.testing.assert_array_equal(host(acc), acc_ref)
    err = np.abs(host(y).astype(np.float64) - y_ref.astype(np.float64))
    assert (err <= grouped_bound(acc_ref, beta, g_ref)).all()


def test_forward_grouped_empty(dev):
    q = torch.zeros((4, 0, 64), dtype=torch.int8, device=dev)
    g = torch.zeros((4, 0), dtype=torch.float32, device=dev)
    wp = torch.zeros((4, 5, 4), dtype=torch.int32, device=dev)
    y, acc = bl.forward_grouped(q, g, wp, torch.ones(4, device=dev))
    assert y.shape == (0, 5) and acc.shape == (4, 0, 5)


def test_base3_longest_k_and_single_row(dev):
    rng = workloads.rng_for(990, 3)
    for M, K, N in ((3, 131072, 5), (1, 4096, 1)):
        x = rng.standard_normal((M, K)).astype(np.float32)
        w = workloads.ternary(rng, N, K, workloads.TERNARY_UNIFORM)
        q_ref, g_ref = oracle.quant_act(x)
        y_ref, acc_ref = oracle.forward(q_ref, g_ref, w, np.float32(0.02))
        packed3, _ = bl.pack_weights3(to_dev(w, dev))
        np.testing.assert_array_equal(host(packed3).view(np.uint8), oracle.pack3(w)[0])
        y, acc = bl.forward3(to_dev(q_ref, dev), to_dev(g_ref, dev), packed3, 0.02, want_acc=True)
        np.testing.assert_array_equal(host(acc), acc_ref)
        assert_y_close(host(y), y_ref)


def test_base3_empty(dev):
    y = bl.forward3(torch.zeros((0, 160), dtype=torch.int8, device=dev),
                    torch.zeros(0, device=dev), torch.zeros((3, 8), dtype=torch.int32, device=dev), 0.5)
    assert y.shape == (0, 3)


# ------------------------------------------------------------------ fused quantise + forward

# One token with K % 64 == 0, K <= 16384 and N <= 16384 runs as one kernel
# (workgroups of 4, 8 or 16 waves by N: 4096, 8192 and 16384 rows are the
# widest of each); the other cases (K not a multiple of 64, K past 16384, N
# past 16384, several tokens) as the two calls.
QFWD_CASES = [(1, 64, 1, "f32", None), (1, 2048, 1000, "bf16", "unit"),
              (1, 4096, 11008, "f32", "rand"), (1, 8192, 17, "bf16", None),
              (1, 16384, 300, "f32", "rand"), (1, 2560, 6912, "f32", "unit"),
              (1, 1024, 4096, "f32", None), (1, 1024, 4097, "bf16", None),
              (1, 512, 8193, "f32", "unit"), (1, 512, 16384, "f32", None),
              (1, 256, 16385, "f32", None), (1, 8192, 28672, "f32", None),
              (1, 4096, 16385, "bf16", "unit"),
              # one token quantised inside the MFMA decode kernel (K >= 4096,
              # K % 512 == 0, N / 64 >= 150): fp32 and bf16 rows, with and
              # without RMSNorm, 128- and 64-row workgroups, rows past the
              # quantiser's register cache (K > 8192), ragged row tails
              (1, 8192, 25700, "bf16", "rand"), (1, 4608, 9631, "f32", "rand"),
              (1, 12288, 9700, "f32", None), (1, 20480, 9650, "bf16", None),
              (1, 5120, 26000, "f32", "unit"),
              (1, 16448, 40, "f32", None), (1, 1040, 77, "bf16", "rand"),
              (3, 4096, 500, "bf16", "rand"), (16, 2560, 700, "f32", None),
              # 2..4 tokens on the LDS decode route (K >= 4096) at every tile
              # width (N = 1000, 11008, 13000, 25600 pick 1, 2, 4, 8 tiles of
              # 16 columns), one output column, and K = 3840 (skinny kernel)
              (2, 4096, 1000, "f32", None), (4, 4096, 11008, "f32", None),
              (3, 4096, 13000, "bf16", None), (2, 8192, 25600, "bf16", None),
              (4, 4096, 1, "f32", None), (3, 5120, 77, "f32", None),
              (3, 5632, 300, "f32", None), (4, 3840, 500, "f32", None)]


@pytest.mark.parametrize("M,K,N,dt,gain_kind", QFWD_CASES)
def test_quant_forward_parity(dev, M, K, N, dt, gain_kind):
    act = "normal_bf16" if dt == "bf16" else "normal_f32"
    x, w, beta = workloads.random_case(1100 + K + N, M, N, K, act=act,
                                       table=workloads.TERNARY_HALF_ZERO)
    if M >= 3:
        x = x.copy()
        x[1] = 0  # a zero token: gamma = 0, codes 0
    xf = oracle.bf16_to_f32(x) if dt == "bf16" else x
    xd = to_dev(x, dev, torch.bfloat16) if dt == "bf16" else to_dev(x, dev)
    rng = workloads.rng_for(1101, K)
    gain = None if gain_kind is None else (np.ones(K, np.float32) if gain_kind == "unit" else
                                           rng.uniform(0.5, 2.0, K).astype(np.float32))
    gd = None if gain is None else to_dev(gain, dev)
    wp = gpu_pack(w, dev)
    outs = dict(y=Guard((M, N), torch.float32, dev), q=Guard((M, K), torch.int8, dev),
                g=Guard((M,), torch.float32, dev), acc=Guard((M, N), torch.int32, dev))
    decode_one = M == 1 and K >= 4096 and K % 512 == 0 and N // 64 >= 150
    one = decode_one or (M == 1 and K % 64 == 0 and K <= 16384 and N <= 16384)
    assert bl.lib.bitlinear_quant_forward_one_launch(M, K, N) == int(one)
    st = bl.lib.bitlinear_quant_forward(
        xd.data_ptr(), bl.BF16 if dt == "bf16" else bl.F32, M, K, None if gd is None else gd.data_ptr(),
        ctypes.c_float(1e-6), wp.data_ptr(), N, ctypes.c_float(float(beta)), outs["q"].t.data_ptr(),
        outs["g"].t.data_ptr(), outs["y"].t.data_ptr(), outs["acc"].t.data_ptr(), stream())
    assert st == 0, bl.last_error()
    for nm, gdd in outs.items():
        gdd.check(f"quant_forward {nm} M={M} K={K} N={N}")
    y, q, g, acc = (host(outs[k].t) for k in ("y", "q", "g", "acc"))
    if gain is None:
        q_ref, g_ref = oracle.quant_act(xf)
        np.testing.assert_array_equal(g, g_ref)
    else:
        q_ref, g_ref = oracle.rmsnorm_quant_act(xf, gain, 1e-6)
        assert_y_close(g, g_ref)
    np.testing.assert_array_equal(q, q_ref)
    y_ref, acc_ref = oracle.forward(q_ref, g, w, beta)
    np.testing.assert_array_equal(acc, acc_ref)
    assert_y_close(y, y_ref)
    # bit-identical to bitlinear_quant_act followed by bitlinear_forward
    q2, g2 = bl.quant_act(xd, gd, 1e-6)
    y2, acc2 = bl.forward(q2, g2, wp, beta, want_acc=True)
    np.testing.assert_array_equal(q, host(q2))
    np.testing.assert_array_equal(g.view(np.uint32), host(g2).view(np.uint32))
    np.testing.assert_array_equal(acc, host(acc2))
    np.testing.assert_array_equal(y.view(np.uint32), host(y2).view(np.uint32))


@pytest.mark.parametrize("N", [333, 9700])  # VALU fused kernel; MFMA decode kernel
def test_quant_forward_zero_token_and_extremes(dev, N):
    K = 4096
    assert bl.lib.bitlinear_quant_forward_one_launch(1, K, N) == 1
    w = workloads.ternary(workloads.rng_for(1102), N, K, workloads.TERNARY_UNIFORM)
    w[0, :] = 1
    w[1, :] = -1
    wp = gpu_pack(w, dev)
    y, q, g = bl.quant_forward(torch.zeros((1, K), device=dev), wp, 0.5)
    assert not host(q).any() and host(g)[0] == 0.0 and not host(y).any()
    # one large entry: gamma = |x_max|, its code 127, the rest 0 or small
    x = np.zeros((1, K), np.float32)
    x[0, 5] = -3.0e30
    x[0, 9] = 1.0e29
    y, q, g, acc = (host(t) for t in bl.quant_forward(to_dev(x, dev), wp, 0.5, want_acc=True))
    q_ref, g_ref = oracle.quant_act(x)
    np.testing.assert_array_equal(q, q_ref)
    np.testing.assert_array_equal(g, g_ref)
    y_ref, acc_ref = oracle.forward(q_ref, g_ref, w, 0.5)
    np.testing.assert_array_equal(acc, acc_ref)
    assert_y_close(y, y_ref)


def test_quant_forward_empty(dev):
    wp = torch.zeros((5, 4), dtype=torch.int32, device=dev)
    y, q, g = bl.quant_forward(torch.zeros((0, 64), device=dev), wp, 1.0)
    assert y.shape == (0, 5) and q.shape == (0, 64)
    y, q, g = bl.quant_forward(torch.ones((1, 64), device=dev), wp[:0], 1.0)
    assert y.shape == (1, 0) and host(g)[0] == 1.0


# ------------------------------------------------------------------ HIP graph replay

def test_graph_replays_match_eager(dev):
    """The calls of a decode step, a GEMM-sized call and the stacked GLU glue
    captured in one HIP graph: each of three replays (with eager work and
    synchronisation in between) reproduces the eager outputs bit for bit."""
    K, N, F = 4096, 3000, 1024
    rng = workloads.rng_for(1300)
    w = workloads.ternary(rng, N, K, workloads.TERNARY_UNIFORM)
    wp = gpu_pack(w, dev)
    wgu = gpu_pack(workloads.ternary(rng, 2 * F, K, workloads.TERNARY_HALF_ZERO), dev)
    beta = 0.03
    xs = [to_dev(rng.standard_normal((M, K)).astype(np.float32), dev) for M in (1, 4, 16, 300)]

    def run(bufs):
        for x, b in zip(xs, bufs):
            bl.quant_forward(x, wp, beta, out=(b["y"], b["q"], b["g"]))
        b = bufs[-1]
        bl.forward(b["q"], b["g"], wgu, 1.0, acc_only=True, acc_out=b["acc_gu"])
        h_q, g_h = b["hq"], b["gh"]
        st = bl.lib.bitlinear_silu_mul_quant_acc(b["acc_gu"].data_ptr(), b["g"].data_ptr(), 300, F,
                                                 ctypes.c_float(0.02), ctypes.c_float(0.04), None,
                                                 h_q.data_ptr(), g_h.data_ptr(),
                                                 torch.cuda.current_stream().cuda_stream)
        assert st == 0, bl.last_error()

    def bufs_for():
        out = []
        for x in xs:
            M = x.shape[0]
            out.append(dict(y=torch.empty((M, N), device=dev), q=torch.empty((M, K), dtype=torch.int8, device=dev),
                            g=torch.empty(M, device=dev)))
        out[-1].update(acc_gu=torch.empty((300, 2 * F), dtype=torch.int32, device=dev),
                       hq=torch.empty((300, F), dtype=torch.int8, device=dev),
                       gh=torch.empty(300, device=dev))
        return out

    ref = bufs_for()
    run(ref)
    torch.cuda.synchronize()
    ref = [{k: host(v) for k, v in b.items()} for b in ref]
    got = bufs_for()
    s = torch.cuda.Stream(device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run(got)
    for _ in range(3):
        for b in got:
            for v in b.values():
                v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for b, r in zip(got, ref):
            for k, v in b.items():
                np.testing.assert_array_equal(host(v).view(np.uint8), r[k].view(np.uint8), err_msg=k)


def test_graph_replays_widened_paths(dev):
    """The widened products captured in one HIP graph -- base-3 on MFMA (16
    tokens), 1-bit on the LDS decode kernel, the grouped decode (G = 4), the
    vector GEMV with K split over two waves, the 64-row GEMM tiles with two
    steps (K = 4608) and one step (K = 768) a group per stage:
    each of three replays (outputs cleared and synchronised in between)
    reproduces the eager outputs bit for bit."""
    rng = workloads.rng_for(1310)
    K, N = 4096, 700
    w = workloads.ternary(rng, N, K, workloads.TERNARY_UNIFORM)
    p3, _ = bl.pack_weights3(to_dev(w, dev))
    p1, _ = bl.pack_weights1(to_dev(np.where(w >= 0, 1, -1).astype(np.int8), dev))
    pg = pack_grouped(w, 4, dev)
    beta_g = to_dev(np.array([0.02, 0.03, 0.04, 0.05], np.float32), dev)
    q16, g16 = bl.quant_act(to_dev(rng.standard_normal((16, K)).astype(np.float32), dev))
    qg, gg = bl.quant_act_grouped(to_dev(rng.standard_normal((16, K)).astype(np.float32), dev), 4)
    w_long = gpu_pack(workloads.ternary(rng, 2560, 6912, workloads.TERNARY_HALF_ZERO), dev)
    q1, g1 = bl.quant_act(to_dev(rng.standard_normal((1, 6912)).astype(np.float32), dev))
    w_k3 = gpu_pack(workloads.ternary(rng, 1000, 4608, workloads.TERNARY_UNIFORM), dev)
    qm, gm = bl.quant_act(to_dev(rng.standard_normal((100, 4608)).astype(np.float32), dev))
    w_p1 = gpu_pack(workloads.ternary(rng, 700, 768, workloads.TERNARY_UNIFORM), dev)
    qp, gp = bl.quant_act(to_dev(rng.standard_normal((64, 768)).astype(np.float32), dev))

    def run():
        return [bl.forward3(q16, g16, p3, 0.02, want_acc=True),
                bl.forward1(q16, g16, p1, 0.02, want_acc=True),
                bl.forward_grouped(qg, gg, pg, beta_g),
                bl.forward(q1, g1, w_long, 0.02, want_acc=True),
                bl.forward(qm, gm, w_k3, 0.02, path=bl.PATH_GEMM, want_acc=True),
                bl.forward(qp, gp, w_p1, 0.02, path=bl.PATH_GEMM, want_acc=True)]

    ref = [[host(t) for t in outs] for outs in run()]
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        got = run()
    for _ in range(3):
        for outs in got:
            for t in outs:
                t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for outs, r in zip(got, ref):
            for t, rt in zip(outs, r):
                np.testing.assert_array_equal(host(t).view(np.uint8), rt.view(np.uint8))


# The register-only MFMA floor (a measurement aid, not a step of the layer)
# runs on ragged shapes and the sweep's GEMM shape without a fault; its sink
# holds either the caller's value or the one constant it may store.
@pytest.mark.parametrize("M,K,N", [(1, 128, 1), (300, 256, 700), (512, 8192, 28672)])
def test_floor_mfma_runs(dev, M, K, N):
    rng = np.random.default_rng(M + K + N)
    q = to_dev(rng.integers(-127, 128, (M, K)).astype(np.int8), dev)
    w = gpu_pack(workloads.ternary(rng, N, K, workloads.TERNARY_HALF_ZERO), dev)
    sink = torch.full((1,), 0x1234567, dtype=torch.int32, device=dev)
    st = bl.lib.bitlinear_floor_mfma(q.data_ptr(), M, K, w.data_ptr(), N, sink.data_ptr(),
                                     torch.cuda.current_stream(dev).cuda_stream)
    assert st == bl.OK, bl.last_error()
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF in (0x1234567, 0x9E3779B9)
