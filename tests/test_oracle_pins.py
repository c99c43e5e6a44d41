"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something it does not compute itself:
hand-derived worked examples (tests/golden), exact rational arithmetic,
closed forms, symmetries, exhaustive enumeration and float64 brute force via a
library matmul.  A plausible slip in the oracle (dropped clip, wrong rounding
mode, transposed operand, wrong bit position, wrong scale) fails one of them.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- worked examples

def test_worked_example_4x4():
    g = _golden("worked_4x4.json")
    x = np.array(g["x"], dtype=np.float32)
    W = np.array(g["W"], dtype=np.int8)
    q, gamma = oracle.quant_act(x)
    np.testing.assert_array_equal(q, np.array(g["q"], dtype=np.int8))
    np.testing.assert_array_equal(gamma, np.array(g["gamma"], dtype=np.float32))
    y, acc = oracle.forward(q, gamma, W, g["beta"])
    np.testing.assert_array_equal(acc, np.array(g["acc"], dtype=np.int32))
    np.testing.assert_array_equal(y, np.array(g["y"], dtype=np.float32))
    # the tie in token B separates ties-to-even from ties-away
    assert q[1, 0] != g["ties_away_would_give"]["q_B0"]


def test_packed_word_example():
    g = _golden("packed_word.json")
    w = np.array([g["w"]], dtype=np.int8)
    p, bad = oracle.pack(w)
    assert bad == 0
    assert int(p[0, 0]) == int(g["word"], 16)
    assert int(oracle.pack(-w)[0][0, 0]) == int(g["word_of_negated_w"], 16)
    assert int(oracle.pack(np.zeros_like(w))[0][0, 0]) == int(g["word_of_zero_row"], 16)
    word = int(p[0, 0])
    for shift, fields in g["fields_by_shift"].items():
        v = (word >> int(shift)) & 0x03030303
        assert [(v >> (8 * b)) & 0xFF for b in range(4)] == fields


# ---------------------------------------------------------------- packing

def _unpack_python(packed, K):
    """Independent per-field decode of the packing contract."""
    N = packed.shape[0]
    out = np.zeros((N, K), dtype=np.int16)
    for n in range(N):
        for c in range(K // 16):
            word = int(packed[n, c])
            for e in range(16):
                j, b = divmod(e, 4)
                out[n, c * 16 + e] = ((word >> (8 * b + 2 * j)) & 3) - 1
    return out


def test_pack_roundtrip_and_independent_decode():
    rng = workloads.rng_for(1, 2, 3)
    w = workloads.ternary(rng, 7, 96)
    p, bad = oracle.pack(w)
    assert bad == 0 and p.shape == (7, 6) and p.dtype == np.uint32
    np.testing.assert_array_equal(_unpack_python(p, 96), w.astype(np.int16))
    np.testing.assert_array_equal(oracle.unpack(p, 96), w)


def test_pack_negation_is_fieldwise_two_minus_code():
    w = workloads.ternary(workloads.rng_for(5), 3, 64)
    p = oracle.pack(w)[0].astype(np.uint64)
    pn = oracle.pack(-w)[0].astype(np.uint64)
    # every 2-bit field f maps to 2 - f, i.e. 0xAAAAAAAA - word (no borrows)
    np.testing.assert_array_equal(pn, 0xAAAAAAAA - p)


def test_pack_flags_non_ternary_entries():
    w = np.zeros((2, 32), dtype=np.int8)
    w[0, 3] = 2
    w[1, 17] = -2
    w[1, 31] = 127
    p, bad = oracle.pack(w)
    assert bad == 3
    dec = _unpack_python(p, 32)
    assert dec[0, 3] == 2 and dec[1, 17] == 2 and dec[1, 31] == 2   # code 3 marker
    assert np.count_nonzero(dec) == 3


# ---------------------------------------------------------------- quantiser

def _nearest_even(z: Fraction) -> int:
    f = math.floor(z)
    d = z - f
    if d > Fraction(1, 2):
        return f + 1
    if d < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


def test_quant_against_exact_rationals():
    """Codes equal round(128*x/gamma) computed in exact rationals (clipped to
    +-127), except inside the fp32 rounding band around a half-integer, where
    they are one of the two neighbours."""
    rng = workloads.rng_for(11)
    x = rng.standard_normal((6, 512), dtype=np.float32)
    x[2] *= np.float32(1e-30)
    x[3] = rng.standard_t(3, size=512).astype(np.float32)
    q, gamma = oracle.quant_act(x)
    band = Fraction(1, 1 << 18)  # half an ulp of t for |t| < 128
    for m in range(x.shape[0]):
        gm = Fraction(float(np.abs(x[m]).max()))
        assert Fraction(float(gamma[m])) == gm
        for k in range(x.shape[1]):
            z = Fraction(float(x[m, k])) * 128 / gm
            exact = max(-127, min(127, _nearest_even(z)))
            dist = abs(z - (math.floor(z) + Fraction(1, 2)))
            if dist > band:
                assert q[m, k] == exact, (m, k, z)
            else:
                lo = max(-127, min(127, math.floor(z)))
                hi = max(-127, min(127, math.floor(z) + 1))
                assert q[m, k] in (lo, hi)


def test_quant_ties_round_to_even():
    # gamma = 128 makes t = x exactly, so x = k + 1/2 is an exact tie
    ks = np.arange(-127, 127)
    x = np.concatenate([[128.0], ks + 0.5]).astype(np.float32)[None, :]
    q, gamma = oracle.quant_act(x)
    assert gamma[0] == 128.0
    for k, c in zip(ks, q[0, 1:]):
        even = k if k % 2 == 0 else k + 1
        assert c == max(-127, min(127, even)), (k, c)


def test_quant_clip_and_absmax_maps_to_127():
    x = np.array([[3.0, -3.0, 2.98, 2.97, 0.0],
                  [-5.0, 4.99, 1.0, 0.0, 0.0]], dtype=np.float32)
    q, gamma = oracle.quant_act(x)
    np.testing.assert_array_equal(gamma, [3.0, 5.0])
    # 128*2.98/3 = 127.15 -> 127; 128*2.97/3 = 126.72 -> 127
    assert list(q[0]) == [127, -127, 127, 127, 0]
    # -128 -> -127; 128*4.99/5 = 127.744 -> clipped 127; 25.6 -> 26
    assert list(q[1]) == [-127, 127, 26, 0, 0]
    assert q.min() >= -127 and q.max() <= 127


def test_quant_zero_token_and_empty():
    q, gamma = oracle.quant_act(np.zeros((2, 16), dtype=np.float32))
    assert not q.any() and not gamma.any()
    q, gamma = oracle.quant_act(np.zeros((3, 0), dtype=np.float32))
    assert q.shape == (3, 0) and not gamma.any()


def test_quant_power_of_two_scaling_and_odd_symmetry():
    x = workloads.rng_for(12).standard_normal((4, 256), dtype=np.float32)
    q, g = oracle.quant_act(x)
    for s in (-20, -3, 1, 7, 30):
        qs, gs = oracle.quant_act(x * np.float32(2.0 ** s))
        np.testing.assert_array_equal(qs, q)
        np.testing.assert_array_equal(gs, g * np.float32(2.0 ** s))
    qn, gn = oracle.quant_act(-x)
    np.testing.assert_array_equal(qn, -q)
    np.testing.assert_array_equal(gn, g)


def test_bf16_widening():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x3E20], dtype=np.uint16)
    f = oracle.bf16_to_f32(bits)
    assert list(f[:4]) == [1.0, -2.0, 0.0, 0.0] and np.signbit(f[3])
    assert np.isinf(f[4]) and f[5] == 0.15625


# ---------------------------------------------------------------- accumulation

def test_exhaustive_ternary_rows_k8():
    K = 8
    grid = np.array(np.meshgrid(*[[-1, 0, 1]] * K, indexing="ij")).reshape(K, -1).T
    w = np.ascontiguousarray(grid, dtype=np.int8)              # all 3^8 rows
    q = workloads.rng_for(13).integers(-127, 128, size=(5, K)).astype(np.int8)
    acc = oracle.accumulate(q, w)
    ref = q.astype(np.int64) @ w.astype(np.int64).T            # library matmul
    np.testing.assert_array_equal(acc, ref)


def test_dequantised_float64_brute_force_dyadic_exact():
    rng = workloads.rng_for(14)
    for K in (16, 48, 64):
        w = workloads.ternary(rng, 9, K)
        x = rng.standard_normal((4, K), dtype=np.float32)
        x[:, 0] = np.float32(2.0) ** rng.integers(-3, 4, size=4)   # absmax = power of two
        x[:, 1:] = np.clip(x[:, 1:], -0.99 * x[:, :1], 0.99 * x[:, :1])
        q, gamma = oracle.quant_act(x)
        assert all(math.log2(float(g)).is_integer() for g in gamma)
        beta = 0.25
        y, acc = oracle.forward(q, gamma, w, beta)
        y64 = (gamma[:, None].astype(np.float64) * q.astype(np.float64) / 128.0) @ \
              (beta * w.astype(np.float64)).T
        np.testing.assert_array_equal(y.astype(np.float64), y64)
        np.testing.assert_array_equal(acc, q.astype(np.int64) @ w.astype(np.int64).T)


def test_dequantised_float64_brute_force_general():
    x, w, beta = workloads.random_case(15, 6, 33, 160)
    q, gamma = oracle.quant_act(x)
    y, acc = oracle.forward(q, gamma, w, beta)
    y64 = (gamma[:, None].astype(np.float64) * q.astype(np.float64) / 128.0) @ \
          (float(beta) * w.astype(np.float64)).T
    np.testing.assert_allclose(y.astype(np.float64), y64, rtol=2.0 ** -22, atol=0)


def test_zero_weights_give_zero():
    x, w, beta = workloads.random_case(16, 3, 8, 64)
    q, g = oracle.quant_act(x)
    y, acc = oracle.forward(q, g, np.zeros_like(w), beta)
    assert not acc.any() and not y.any()


def test_sign_flip_symmetry():
    x, w, beta = workloads.random_case(17, 4, 21, 128)
    q, g = oracle.quant_act(x)
    y, acc = oracle.forward(q, g, w, beta)
    yn, accn = oracle.forward(q, g, -w, beta)
    np.testing.assert_array_equal(accn, -acc)
    np.testing.assert_array_equal(yn, -y)
    # the whole layer on -x
    yx, accx, _, _ = oracle.bitlinear(-x, w, beta)
    np.testing.assert_array_equal(accx, -acc)
    np.testing.assert_array_equal(yx, -y)


def test_closed_forms_one_hot_and_constant_rows():
    K = 64
    q = workloads.rng_for(18).integers(-127, 128, size=(3, K)).astype(np.int8)
    eye = np.eye(K, dtype=np.int8)
    np.testing.assert_array_equal(oracle.accumulate(q, eye), q.astype(np.int32))
    ones = np.ones((2, K), dtype=np.int8)
    s = q.astype(np.int64).sum(axis=1)
    np.testing.assert_array_equal(oracle.accumulate(q, ones), np.stack([s, s], 1))
    np.testing.assert_array_equal(oracle.accumulate(q, -ones), -np.stack([s, s], 1))


def test_permutation_invariance():
    x, w, beta = workloads.random_case(19, 3, 10, 96)
    q, g = oracle.quant_act(x)
    perm = workloads.rng_for(20).permutation(96)
    np.testing.assert_array_equal(oracle.accumulate(q, w),
                                  oracle.accumulate(q[:, perm].copy(), w[:, perm].copy()))


def test_accumulator_bound_and_extreme():
    K = 1 << 17
    q = np.full((1, K), 127, dtype=np.int8)
    w = np.ones((2, K), dtype=np.int8)
    w[1] = -1
    acc = oracle.accumulate(q, w)
    assert acc.tolist() == [[127 * K, -127 * K]]
    assert 127 * K < 2 ** 24                      # fp32 holds every accumulator exactly


def test_rescale_rounding_and_scale():
    acc = np.array([[1, -3, 16777215, 0]], dtype=np.int32)
    gamma = np.array([3.0], dtype=np.float32)
    y = oracle.rescale(acc, gamma, 0.1)
    b = float(np.float32(0.1))
    for a, v in zip(acc[0], y[0]):
        exact = Fraction(int(a)) * Fraction(b) * 3 / 128
        # within half an fp32 ulp of the exact rational (plus the float64 step)
        assert abs(Fraction(float(v)) - exact) <= abs(exact) * Fraction(1, 1 << 23)
    assert y[0, 3] == 0.0 and not np.signbit(y[0, 3])


# ---------------------------------------------------------------- RMSNorm + quant

def test_rmsnorm_closed_form_constant_vector():
    c, eps, K = np.float32(-0.75), 1e-6, 64
    x = np.full((1, K), c, dtype=np.float32)
    q, gamma = oracle.rmsnorm_quant_act(x, np.ones(K, np.float32), eps)
    assert (q == -127).all()
    expect = abs(float(c)) / math.sqrt(float(c) ** 2 + float(np.float32(eps)))
    assert abs(float(gamma[0]) - expect) <= expect * 2 ** -23


def test_rmsnorm_closed_form_three_four():
    # x = [3, 4, 3, 4, ...]: mean(x^2) = 12.5, absmax 4
    K, eps = 32, 1e-6
    x = np.tile(np.array([3.0, 4.0], np.float32), K // 2)[None, :]
    q, gamma = oracle.rmsnorm_quant_act(x, np.ones(K, np.float32), eps)
    assert q[0, :2].tolist() == [96, 127]
    expect = 4.0 / math.sqrt(12.5 + float(np.float32(eps)))
    assert abs(float(gamma[0]) - expect) <= expect * 2 ** -23


def test_rmsnorm_codes_cancel_at_unit_gain():
    x = workloads.rng_for(21).standard_normal((5, 2560), dtype=np.float32)
    q0, g0 = oracle.quant_act(x)
    q1, g1 = oracle.rmsnorm_quant_act(x, np.ones(2560, np.float32), 1e-6)
    np.testing.assert_array_equal(q1, q0)
    assert (g1 != g0).all()  # the RMS factor is in gamma


def test_rmsnorm_gain_enters_codes():
    rng = workloads.rng_for(22)
    x = rng.standard_normal((3, 128), dtype=np.float32)
    gain = rng.uniform(0.5, 2.0, size=128).astype(np.float32)
    q1, _ = oracle.rmsnorm_quant_act(x, gain, 1e-6)
    q2, _ = oracle.quant_act(x * gain)
    np.testing.assert_array_equal(q1, q2)


def test_rmsnorm_literal_float64_agrees_outside_ties():
    x = workloads.rng_for(23).standard_normal((8, 2560), dtype=np.float32)
    gain = np.ones(2560, np.float32)
    q, g = oracle.rmsnorm_quant_act(x, gain, 1e-6)
    ql, gl = oracle.rmsnorm_quant_act_literal(x, gain, 1e-6)
    np.testing.assert_allclose(g.astype(np.float64), gl, rtol=2 ** -23)
    diff = q.astype(np.int32) - ql.astype(np.int32)
    assert np.abs(diff).max() <= 1 and np.count_nonzero(diff) <= 4


# ---------------------------------------------------------------- SiLU * up

def test_silu_textbook_values_and_identities():
    # sigmoid(1) = 1/(1+e^-1) = 0.7310585786300049 (textbook constant)
    z = np.array([0.0, 1.0, -1.0, 40.0, 3.5, -3.5], dtype=np.float32)
    h = oracle.silu_mul(z, np.ones_like(z))
    assert h[0] == 0.0
    assert abs(h[1] - 0.7310585786300049) < 1e-15
    assert h[3] == 40.0
    # silu(z) - silu(-z) = z
    assert abs((h[1] - h[2]) - 1.0) < 1e-15 and abs((h[4] - h[5]) - 3.5) < 1e-14
    # the second operand multiplies
    h2 = oracle.silu_mul(z, np.full_like(z, -2.0))
    np.testing.assert_array_equal(h2, -2.0 * h)


def test_glu_with_identity_down_projection_tracks_h():
    D = F = 64
    rng = workloads.rng_for(24)
    x = rng.standard_normal((3, D), dtype=np.float32)
    wg = workloads.ternary(rng, F, D)
    wu = workloads.ternary(rng, F, D)
    eye = np.eye(F, dtype=np.int8)
    st = oracle.glu(x, wg, wu, eye, (0.02, 0.03, 1.0), np.ones(D, np.float32))
    # identity down: acc_down = h_q and y = h_q * gamma_h / 128 ~ h within a step
    np.testing.assert_array_equal(st["acc_down"], st["h_q"].astype(np.int32))
    step = st["gamma_h"][:, None].astype(np.float64) / 128.0
    assert (np.abs(st["y"] - st["h"]) <= step * 1.01).all()
    # zero up-projection kills the block
    st0 = oracle.glu(x, wg, np.zeros_like(wu), eye, (0.02, 0.03, 1.0), np.ones(D, np.float32))
    assert not st0["y"].any() and not st0["h_q"].any()


# ---------------------------------------------------------------- absmean ternarisation

def test_ternarize_worked_example():
    g = _golden("ternarize_2x16.json")
    W = np.array(g["W"], dtype=np.float32)
    w, beta = oracle.ternarize(W)
    assert beta == g["beta"]
    np.testing.assert_array_equal(w, np.array(g["codes"], dtype=np.int8))


def test_ternarize_recovers_a_scaled_ternary_matrix():
    # W = a * T with T ternary: beta = a * nnz / (N K) (exact here: dyadic a,
    # N K a power of two) and every nonzero satisfies |W| = a > beta / 2
    rng = workloads.rng_for(900, 1)
    T = workloads.ternary(rng, 64, 256, workloads.TERNARY_UNIFORM)
    a = 0.375
    w, beta = oracle.ternarize(T.astype(np.float32) * np.float32(a))
    np.testing.assert_array_equal(w, T)
    assert Fraction(beta) == Fraction(3, 8) * Fraction(int(np.count_nonzero(T)), 64 * 256)


def test_ternarize_scale_and_sign_symmetries():
    rng = workloads.rng_for(900, 2)
    W = rng.standard_normal((48, 320)).astype(np.float32)
    w, beta = oracle.ternarize(W)
    w2, beta2 = oracle.ternarize(W * np.float32(8.0))
    np.testing.assert_array_equal(w2, w)
    assert beta2 == 8.0 * beta  # power-of-two scaling is exact in every partial sum
    wn, betan = oracle.ternarize(-W)
    np.testing.assert_array_equal(wn, -w)
    assert betan == beta


def test_ternarize_ties_clip_and_zero():
    # sum |W| = 8 over 8 entries: beta = 1, half = 0.5; the three entries of
    # magnitude 0.5 are ties and go to 0, 1.5 and 3.0 clip to +-1
    W = np.array([[0.5, -0.5, 0.625, -1.5, 3.0, 0.0, 1.375, -0.5]], np.float32)
    w, beta = oracle.ternarize(W)
    assert beta == 1.0
    np.testing.assert_array_equal(w[0], [0, 0, 1, -1, 1, 0, 1, 0])
    # one ulp above the tie rounds away from zero
    W2 = W.copy()
    W2[0, 0] = np.nextafter(np.float32(0.5), np.float32(1.0))
    W2[0, 2] = np.float32(0.625) - (W2[0, 0] - np.float32(0.5))  # same ulp: sum |W| stays 8
    w2, beta2 = oracle.ternarize(W2)
    assert beta2 == 1.0 and w2[0, 0] == 1
    z, bz = oracle.ternarize(np.zeros((3, 32), np.float32))
    assert bz == 0.0 and not z.any()


def test_ternarize_against_exact_rational_mean():
    # beta against the exactly rounded mean (math.fsum); the oracle's ordered
    # double sum may differ from it only by rounding, and every code must agree
    # with the exact threshold except entries within that rounding of it
    rng = workloads.rng_for(900, 3)
    W = (rng.standard_normal((37, 416)) * 0.02).astype(np.float32)
    w, beta = oracle.ternarize(W)
    exact = math.fsum(abs(float(v)) for v in W.ravel()) / W.size
    assert abs(beta - exact) <= 1e-12 * exact
    d = W.astype(np.float64)
    ref = np.where(d > exact / 2, 1, np.where(d < -exact / 2, -1, 0))
    near = np.abs(np.abs(d) - exact / 2) <= 1e-12 * exact
    np.testing.assert_array_equal(w[~near], ref[~near])
    assert 0.25 < np.count_nonzero(w) / w.size < 0.75


def test_ternarize_sum_is_pairwise():
    # |W| = [1, 2^-53 x 4, 0, 0, 0]: adding left to right every 1 + 2^-53 ties
    # back to 1 (sum 1); the pairwise tree adds the small terms first:
    # ((1 + 2^-53) + (2^-53 + 2^-53)) + ((2^-53 + 0) + 0) = (1 + 2^-52) + 2^-53,
    # a tie between 1 + 2^-52 and 1 + 2^-51 that goes to the even 1 + 2^-51,
    # which is also the exact sum
    e = 2.0 ** -53
    W = np.array([[1.0, e, -e, e, -e, 0.0, 0.0, 0.0] * 4], np.float32)  # K = 32, 4 copies
    _, beta = oracle.ternarize(W)
    block = 1.0 + 2.0 ** -51   # pairwise sum of one group of 8, exact
    assert beta == (4 * block) / 32  # the four equal group sums add exactly
    assert beta != 4.0 / 32


# ---------------------------------------------------------------- 1-bit weights

def test_binarize_worked_example():
    g = _golden("binarize_2x32.json")
    W = np.array(g["W"], dtype=np.float32)
    w, alpha = oracle.binarize(W)
    assert alpha == g["alpha"] == 0.25
    np.testing.assert_array_equal(w, np.array(g["codes"], dtype=np.int8))
    packed, bad = oracle.pack1(w)
    assert bad == 0
    np.testing.assert_array_equal(packed, np.array(g["packed"], dtype=np.uint32))
    np.testing.assert_array_equal(oracle.unpack1(packed, 32), w)


def test_pack1_bit_positions_and_round_trip():
    # entry e = 4j + b at bit 8b + j: a single +1 at e lights exactly that bit
    for e in range(32):
        w = -np.ones((1, 32), np.int8)
        w[0, e] = 1
        packed, _ = oracle.pack1(w)
        assert int(packed[0, 0]) == 1 << (8 * (e % 4) + e // 4)
    rng = workloads.rng_for(910, 1)
    w = np.where(rng.random((9, 96)) < 0.5, 1, -1).astype(np.int8)
    packed, bad = oracle.pack1(w)
    assert bad == 0
    np.testing.assert_array_equal(oracle.unpack1(packed, 96), w)
    w[3, 7] = 0
    assert oracle.pack1(w)[1] == 1


def test_binarize_shift_and_sign_symmetries():
    rng = workloads.rng_for(910, 2)
    # dyadic entries on a grid of 2^-10: every partial sum is exact
    W = (rng.integers(-4096, 4096, (32, 64)) / 1024.0).astype(np.float32)  # N K = 2^11
    w, alpha = oracle.binarize(W)
    assert Fraction(alpha) == Fraction(int((W.astype(np.float64) * 1024).sum()), 1024 * W.size)
    w2, alpha2 = oracle.binarize(W + np.float32(0.5))
    np.testing.assert_array_equal(w2, w)
    assert alpha2 == alpha + 0.5
    wn, alphan = oracle.binarize(-W)
    assert alphan == -alpha
    tie = W.astype(np.float64) == alpha
    np.testing.assert_array_equal(wn[~tie], -w[~tie])
    assert (wn[tie] == -1).all() and (w[tie] == -1).all()


def test_binary_weights_closed_form():
    # with w in {-1, +1}: acc = 2 * sum_{w = +1} q - sum q
    rng = workloads.rng_for(910, 3)
    q = rng.integers(-127, 128, (3, 64)).astype(np.int8)
    w = np.where(rng.random((5, 64)) < 0.5, 1, -1).astype(np.int8)
    acc = oracle.accumulate(q, w)
    S = q.astype(np.int64).sum(axis=1)
    for m in range(3):
        for n in range(5):
            pos = q[m].astype(np.int64)[w[n] == 1].sum()
            assert acc[m, n] == 2 * pos - S[m]


# ---------------------------------------------------------------- group quantisation

def test_grouped_worked_example():
    g = _golden("grouped_1x32.json")
    x = np.array(g["x"], dtype=np.float32)
    q, gamma = oracle.quant_act_grouped(x, g["G"])
    np.testing.assert_array_equal(q, np.array(g["q"], dtype=np.int8))
    np.testing.assert_array_equal(gamma, np.array(g["gamma"], dtype=np.float32))
    y, acc = oracle.forward_grouped(q, gamma, np.array(g["w"], np.int8), np.array(g["beta"], np.float32))
    np.testing.assert_array_equal(acc, np.array(g["acc"], dtype=np.int32))
    np.testing.assert_array_equal(y, np.array(g["y"], dtype=np.float32))
    # the stored y restated in exact rationals from the stored acc
    for n in range(2):
        exact = sum(Fraction(int(g["acc"][k][0][n])) * Fraction(g["beta"][k]) * Fraction(g["gamma"][k][0]) / 128
                    for k in range(2))
        assert exact == Fraction(g["y"][0][n])


def test_grouped_one_group_is_the_ungrouped_layer():
    rng = workloads.rng_for(920, 1)
    x = rng.standard_normal((5, 96)).astype(np.float32)
    w = workloads.ternary(rng, 7, 96, workloads.TERNARY_UNIFORM)
    qg, gg = oracle.quant_act_grouped(x, 1)
    q, gm = oracle.quant_act(x)
    np.testing.assert_array_equal(qg[0], q)
    np.testing.assert_array_equal(gg[0], gm)
    gain = (rng.random(96) + 0.5).astype(np.float32)
    qg, gg = oracle.quant_act_grouped(x, 1, gain, 1e-6)
    q, gm = oracle.rmsnorm_quant_act(x, gain, 1e-6)
    np.testing.assert_array_equal(qg[0], q)
    np.testing.assert_array_equal(gg[0], gm)
    yg, accg = oracle.forward_grouped(qg, gg, w, np.array([0.03], np.float32))
    y, acc = oracle.forward(q, gm, w, 0.03)
    np.testing.assert_array_equal(accg[0], acc)
    np.testing.assert_array_equal(yg, y)


def test_grouped_groups_are_independent():
    # changing the inputs of group 1 leaves group 0's codes, scale and product alone
    rng = workloads.rng_for(920, 2)
    G, KG = 3, 32
    x = rng.standard_normal((4, G * KG)).astype(np.float32)
    w = workloads.ternary(rng, 6, G * KG, workloads.TERNARY_UNIFORM)
    q, gamma = oracle.quant_act_grouped(x, G)
    x2 = x.copy()
    x2[:, KG:2 * KG] *= np.float32(-3.0)
    x2[1, KG + 5] = np.float32(100.0)
    q2, gamma2 = oracle.quant_act_grouped(x2, G)
    for g in (0, 2):
        np.testing.assert_array_equal(q2[g], q[g])
        np.testing.assert_array_equal(gamma2[g], gamma[g])
    w2 = w.copy()
    w2[:, KG:2 * KG] = -w2[:, KG:2 * KG]
    _, acc = oracle.forward_grouped(q, gamma, w, np.ones(G, np.float32))
    _, acc2 = oracle.forward_grouped(q, gamma, w2, np.ones(G, np.float32))
    np.testing.assert_array_equal(acc2[0], acc[0])
    np.testing.assert_array_equal(acc2[2], acc[2])
    np.testing.assert_array_equal(acc2[1], -acc[1])


def test_grouped_scale_of_one_group():
    # scaling group g's activations by 2^e scales its gamma by 2^e, keeps every
    # code, and changes y by exactly (2^e - 1) times that group's term
    rng = workloads.rng_for(920, 3)
    G, KG = 4, 16
    x = (rng.integers(-64, 65, (3, G * KG)) / 16.0).astype(np.float32)  # dyadic
    w = workloads.ternary(rng, 5, G * KG, workloads.TERNARY_UNIFORM)
    beta = np.array([0.5, 0.25, 0.125, 1.0], np.float32)
    q, gamma = oracle.quant_act_grouped(x, G)
    y, acc = oracle.forward_grouped(q, gamma, w, beta)
    x2 = x.copy()
    x2[:, 2 * KG:3 * KG] *= np.float32(4.0)
    q2, gamma2 = oracle.quant_act_grouped(x2, G)
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(gamma2[2], gamma[2] * 4)
    y2, acc2 = oracle.forward_grouped(q2, gamma2, w, beta)
    np.testing.assert_array_equal(acc2, acc)
    term = acc[2].astype(np.float64) * 0.125 * gamma[2].astype(np.float64)[:, None] / 128
    np.testing.assert_array_equal(y2.astype(np.float64) - y.astype(np.float64), 3 * term)


def test_grouped_with_a_shared_absmax_equals_the_ungrouped_product():
    # every group of a token holds the token's absmax: the group codes are the
    # ungrouped codes and the group products add up to the ungrouped product
    rng = workloads.rng_for(920, 4)
    G, KG = 4, 24
    x = rng.uniform(-1, 1, (3, G * KG)).astype(np.float32)
    for m in range(3):
        for g in range(G):
            x[m, g * KG + (m + g) % KG] = np.float32(2.0 if (m + g) % 2 else -2.0)
    w = workloads.ternary(rng, 9, G * KG, workloads.TERNARY_UNIFORM)
    q, gamma = oracle.quant_act_grouped(x, G)
    q1, g1 = oracle.quant_act(x)
    np.testing.assert_array_equal(np.concatenate(list(q), axis=1), q1)
    assert (gamma == g1[None, :]).all()
    _, acc = oracle.forward_grouped(q, gamma, w, np.ones(G, np.float32))
    np.testing.assert_array_equal(acc.astype(np.int64).sum(axis=0), oracle.accumulate(q1, w))
    # with RMSNorm the whole-row factor r is shared: each group's gamma is the
    # ungrouped RMSNorm gamma
    gain = np.ones(G * KG, np.float32)
    qr, gr = oracle.quant_act_grouped(x, G, gain, 1e-6)
    qr1, gr1 = oracle.rmsnorm_quant_act(x, gain, 1e-6)
    np.testing.assert_array_equal(np.concatenate(list(qr), axis=1), qr1)
    assert (gr == gr1[None, :]).all()


def test_ternarize_grouped_recovers_scaled_ternary_blocks():
    # W = a_g * T in group g: every code comes back and beta_g = a_g * nnz_g / (N K/G)
    rng = workloads.rng_for(920, 5)
    G, N, KG = 4, 32, 64
    T = workloads.ternary(rng, N, G * KG, workloads.TERNARY_UNIFORM)
    a = [0.5, 0.125, 2.0, 0.375]
    W = np.concatenate([T[:, g * KG:(g + 1) * KG].astype(np.float32) * np.float32(a[g]) for g in range(G)],
                       axis=1)
    w, betas = oracle.ternarize_grouped(W, G)
    np.testing.assert_array_equal(w, T)
    for g in range(G):
        nnz = int(np.count_nonzero(T[:, g * KG:(g + 1) * KG]))
        assert Fraction(betas[g]) == Fraction(a[g]) * Fraction(nnz, N * KG)
    w1, b1 = oracle.ternarize_grouped(W, 1)
    w0, b0 = oracle.ternarize(W)
    np.testing.assert_array_equal(w1, w0)
    assert b1[0] == b0


# ---------------------------------------------------------------- base-3 packing

def test_pack3_worked_example():
    g = _golden("pack3_1x96.json")
    w = np.zeros((1, g["K"]), np.int8)
    for k, v in g["nonzero"].items():
        w[0, int(k)] = v
    packed, bad = oracle.pack3(w)
    assert bad == 0
    np.testing.assert_array_equal(packed[0], np.array(g["packed"], np.uint8))
    np.testing.assert_array_equal(oracle.unpack3(packed, g["K"]), w)


def test_pack3_every_byte_value():
    # all 243 five-trit combinations in byte 0 of word 0: the stored byte is
    # ceil(256 v / 243) of the base-3 value (most significant digit first),
    # computed here from the definition, and unpacks back
    import itertools
    rows = []
    for digits in itertools.product((0, 1, 2), repeat=5):
        w = np.zeros(80, np.int8)
        for i, d in enumerate(digits):
            w[4 * i] = d - 1
        rows.append(w)
    W = np.stack(rows)
    packed, bad = oracle.pack3(W)
    assert bad == 0
    for r, digits in enumerate(itertools.product((0, 1, 2), repeat=5)):
        v = sum(d * 3 ** (4 - i) for i, d in enumerate(digits))
        assert int(packed[r, 0]) == -(-256 * v // 243)
        assert (packed[r, 1:] == 128).all()
    np.testing.assert_array_equal(oracle.unpack3(packed, 80), W)
    assert len(set(packed[:, 0].tolist())) == 243


def test_pack3_bytes_decode_by_multiplication():
    # the stored byte b = ceil(256 v / 243) gives v's base-3 digits by the
    # multiplication walk x <- 3x, digit = x // 256, x <- x mod 256 (five
    # steps), for every v: the decode the vector-ALU kernels use
    for v in range(243):
        b = -(-256 * v // 243)
        x, digits = b, []
        for _ in range(5):
            x *= 3
            digits.append(x >> 8)
            x &= 0xFF
        assert sum(d * 3 ** (4 - i) for i, d in enumerate(digits)) == v, v


def test_pack3_sizes_ranges_and_round_trip():
    rng = workloads.rng_for(930, 1)
    for K in (16, 80, 96, 4096, 2560, 6912):
        w = workloads.ternary(rng, 5, K, workloads.TERNARY_UNIFORM)
        packed, bad = oracle.pack3(w)
        assert packed.shape == (5, 16 * ((K + 79) // 80)) and bad == 0
        np.testing.assert_array_equal(oracle.unpack3(packed, K), w)
    assert oracle.pack3(np.zeros((1, 80), np.int8))[0].tolist() == [[128] * 16]
    assert oracle.pack3(np.ones((1, 80), np.int8))[0].tolist() == [[255] * 16]
    assert oracle.pack3(-np.ones((1, 80), np.int8))[0].tolist() == [[0] * 16]
    w = np.zeros((2, 32), np.int8)
    w[1, 5] = 3
    assert oracle.pack3(w)[1] == 1
