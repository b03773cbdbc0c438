"""Pins of the oracle's residual-add RMS norm (page "vllm.models.flint.ops.moe",
_add_rms_norm / flint_moe_ll) against values fixed by the mathematics: a
hand-computed row, closed forms and exact invariances."""
import numpy as np
import pytest

import oracle



def bf(v):
    return oracle.f32_to_bf16(np.asarray(v, dtype=np.float32))


def val(bits):
    return oracle.bf16_to_f32(bits).astype(np.float64)


def test_hand_computed_row():
    # s = [3, 4], mean s^2 = 12.5, xn = s / sqrt(12.5) = [0.848528.., 1.131370..];
    # to 8 significant bits (round to nearest even): 217/256 and 145/128.
    res, xn = oracle.add_rms_norm(bf([[3.0, 4.0]]), bf([[0.0, 0.0]]), bf([1.0, 1.0]), 0.0)
    assert np.array_equal(val(res), [[3.0, 4.0]])
    assert np.array_equal(val(xn), [[217 / 256, 145 / 128]])


def test_residual_is_the_rounded_fp32_sum():
    rng = np.random.default_rng(1)
    a = bf(rng.standard_normal((4, 64)) * 3)
    r = bf(rng.standard_normal((4, 64)) * 40)
    res, _ = oracle.add_rms_norm(a, r, bf(np.ones(64)), 1e-6)
    exact = val(a) + val(r)  # exact in fp64
    want = oracle.f32_to_bf16(exact.astype(np.float32))  # one fp32 rounding, then bf16
    assert np.array_equal(res, want)
    res0, _ = oracle.add_rms_norm(a, oracle.f32_to_bf16(-val(a).astype(np.float32)), bf(np.ones(64)), 1e-6)
    assert np.all(val(res0) == 0)


def test_constant_row_normalises_to_sign():
    for c in (0.375, -5.0, 1024.0):
        res, xn = oracle.add_rms_norm(bf(np.full((1, 128), c)), bf(np.zeros((1, 128))), bf(np.ones(128)), 0.0)
        assert np.all(val(xn) == np.sign(c))


def test_unit_rms_and_exact_invariances():
    rng = np.random.default_rng(2)
    H = 2048
    a = bf(rng.standard_normal((3, H)))
    r = bf(rng.standard_normal((3, H)) * 0.5)
    w1 = bf(np.ones(H))
    _, xn = oracle.add_rms_norm(a, r, w1, 0.0)
    rms = np.sqrt(np.mean(val(xn) ** 2, axis=1))
    assert np.all(np.abs(rms - 1) < 2.0 ** -8)
    # scaling both inputs by a power of two changes nothing (eps = 0)
    _, xn4 = oracle.add_rms_norm(bf(val(a) * 4), bf(val(r) * 4), w1, 0.0)
    assert np.array_equal(xn, xn4)
    # a power-of-two weight scales the output exactly; weights act per column
    _, xn2 = oracle.add_rms_norm(a, r, bf(np.full(H, 2.0)), 0.0)
    assert np.array_equal(val(xn2), 2 * val(xn))
    w = np.ones(H)
    w[5] = -1.0
    _, xnn = oracle.add_rms_norm(a, r, bf(w), 0.0)
    assert np.array_equal(val(xnn)[:, 5], -val(xn)[:, 5])
    assert np.array_equal(np.delete(xnn, 5, axis=1), np.delete(xn, 5, axis=1))


def test_eps_enters_under_the_root():
    # s = [1, 1] (mean 1): xn = 1 / sqrt(1 + eps); eps = 3 gives 0.5 exactly
    _, xn = oracle.add_rms_norm(bf([[1.0, 1.0]]), bf([[0.0, 0.0]]), bf([1.0, 1.0]), 3.0)
    assert np.array_equal(val(xn), [[0.5, 0.5]])
    _, z = oracle.add_rms_norm(bf([[0.0, 0.0]]), bf([[0.0, 0.0]]), bf([1.0, 1.0]), 1e-6)
    assert np.all(val(z) == 0)


def test_f64_to_bf16_single_rounding():
    # 1 + 2^-8 + 2^-30 lies just above the bf16 midpoint 1 + 2^-8: fp32 rounds it
    # onto the midpoint, a second rounding would go to even (1.0); one rounding
    # gives 1 + 2^-7.
    x = 1 + 2.0 ** -8 + 2.0 ** -30
    assert val(oracle.f64_to_bf16(np.array([x])))[0] == 1 + 2.0 ** -7
    assert val(oracle.f64_to_bf16(np.array([1 + 2.0 ** -8])))[0] == 1.0
    assert val(oracle.f64_to_bf16(np.array([-(1 + 2.0 ** -8 + 2.0 ** -30)])))[0] == -(1 + 2.0 ** -7)
