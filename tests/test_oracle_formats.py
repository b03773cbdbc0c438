"""Pins of the oracle's number formats and routing arithmetic (CPU only).

Each check compares the oracle with something other than itself: a library
cast (torch), a published code table (tests/golden), exact rational / 60-digit
decimal arithmetic, or a closed form.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_e2m1():
    tab = {}
    with open(os.path.join(GOLDEN, "e2m1_codes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            tab[int(c, 16)] = float(v)
    return tab


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),   # subnormals
        (rng.standard_normal(2000) * 1e38).astype(np.float32),    # near overflow
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38,
                  3.4028235e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9,
                  1.0 + 3 * 2 ** -9, 2 ** -149, -(2 ** -149)], dtype=np.float32),
    ])
    # exact ties: random bf16 values with the 16 dropped bits = 0x8000
    ties = (rng.integers(0, 2 ** 32, 4000, dtype=np.uint64).astype(np.uint32) & 0xFFFF0000) | 0x8000
    ties = ties[(ties & 0x7F800000) != 0x7F800000].view(np.float32)
    vals = np.concatenate([vals, ties])
    ours = oracle.f32_to_bf16(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # NaN stays NaN
    nan_b = oracle.f32_to_bf16(np.array([np.nan], dtype=np.float32))[0]
    assert (nan_b & 0x7F80) == 0x7F80 and (nan_b & 0x7F) != 0


def test_e4m3fn_all_bytes_match_torch():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([oracle.e4m3fn(i) for i in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ref[~nan], ours[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_e2m1_matches_ocp_table():
    tab = _golden_e2m1()
    assert len(tab) == 16
    for c, v in tab.items():
        got = oracle.e2m1(c)
        assert got == v and np.signbit(got) == np.signbit(v), (c, got, v)


def test_dequant_exhaustive_exact():
    """All 16 codes x 256 scale bytes: value * scale, exact in bf16."""
    tab = _golden_e2m1()
    e4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    K = 32
    rows = 256
    # row r uses scale byte r for both of its 16-element blocks; element k of
    # every row holds code k % 16 (byte c packs element 2c low, 2c+1 high)
    codes = np.arange(K) % 16
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    w = np.tile(packed, (rows, 1))
    s = np.repeat(np.arange(256, dtype=np.uint8)[:, None], K // 16, axis=1)
    out = oracle.nvfp4_dequant(w, s)
    got = oracle.bf16_to_f32(out).astype(np.float64)
    want = np.array([[tab[int(codes[k])] * e4[r] for k in range(K)] for r in range(rows)])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # exactness: every finite product is representable in bf16
    fin = want[~nan]
    back = torch.from_numpy(fin).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, fin)


def test_dequant_nibble_order():
    """Reading of the packing: element 2c is the low nibble of byte c."""
    w = np.array([[0x21, 0x43, 0x65, 0x07, 0xF8, 0xDC, 0xBA, 0x09]], dtype=np.uint8)
    s = np.array([[0x38]], dtype=np.uint8)  # E4M3 0x38 = 1.0
    got = oracle.bf16_to_f32(oracle.nvfp4_dequant(w, s))[0]
    want = [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 0.0,
            -0.0, -6.0, -2.0, -3.0, -1.0, -1.5, -0.5, 0.0]
    assert list(got) == want


def _score_reference(b: int) -> float:
    """s = RN32(1 / RN32(1 + RN32(exp(-l)))) with exp from 60-digit decimal."""
    l = exact.bf16_bits_value(b)
    if np.isnan(l):
        return float("nan")
    if np.isinf(l):
        return 1.0 if l > 0 else 0.0
    q = -Fraction(l)
    if q > 89:            # exp(-l) > 4.4e38: rounds to +inf in fp32
        a = float("inf")
    elif q < -104:        # exp(-l) < 2^-150: rounds to 0
        a = 0.0
    else:
        a = exact.rn32(exact.exp_decimal(q))
    d = np.float32(1.0) + np.float32(a)
    return float(np.float32(1.0) / d)


def test_router_score_exhaustive_over_bf16():
    """Every bf16 logit: oracle score == 60-digit-decimal reference."""
    bad = []
    for b in range(65536):
        got = oracle.router_score(b)
        want = _score_reference(b)
        if np.isnan(want):
            if not np.isnan(got):
                bad.append(b)
        elif exact.f32_bits(got) != exact.f32_bits(want):
            bad.append(b)
    assert not bad, [hex(b) for b in bad[:20]]


def _ulp_bf16(v: float) -> float:
    v = abs(v)
    if v == 0:
        return 2.0 ** -133
    e = max(int(np.floor(np.log2(v))), -126)
    return 2.0 ** (e - 7)


def _key_sort_ids(vals, k):
    """Brute force: indices sorted by (value descending, index ascending)."""
    order = sorted(range(len(vals)), key=lambda e: (-vals[e], e))
    return order[:k]


@pytest.mark.parametrize("E", [1, 3, 8, 32, 128, 256])
def test_topk_matches_brute_force_sort(E):
    rng = np.random.default_rng(E)
    M = 40
    # few distinct values so ties are frequent; no NaN and no signed zeros
    pool = np.unique(rng.standard_normal(7).astype(np.float32))
    pool = pool[pool != 0]
    vals = rng.choice(pool, size=(M, E))
    lg = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    fv = oracle.bf16_to_f32(lg)
    for k in sorted({1, min(E, 2), min(E, 8), E}):
        ids, tw, sc = oracle.topk(lg, k)
        for t in range(M):
            assert list(ids[t]) == _key_sort_ids(list(fv[t]), k)


def test_topk_special_values():
    # +0 ranks above -0; +NaN above +inf; -NaN below -inf; ties -> low index
    row = np.array([0x8000, 0x0000, 0xFF80, 0x7F80, 0x7FC0, 0xFFC0, 0x3F80, 0x3F80],
                   dtype=np.uint16)  # -0, +0, -inf, +inf, +nan, -nan, 1.0, 1.0
    ids, tw, sc = oracle.topk(row[None, :], 8)
    assert list(ids[0]) == [4, 3, 6, 7, 1, 0, 2, 5]
    assert np.isnan(tw[0]).all()  # a NaN score poisons the renormalisation
    ids, tw, sc = oracle.topk(row[None, [3, 6, 7, 2]], 3)
    assert list(ids[0]) == [0, 1, 2]
    assert sc[0, 0] == 1.0  # sigmoid(+inf)


def test_topk_any_bit_pattern_matches_sign_magnitude_sort():
    """Every bf16 bit pattern, NaNs and signed zeros included, against a brute
    force sort on the sign-magnitude integer of the bits (negative patterns
    below every non-negative one, ordered by decreasing magnitude; -0 just
    below +0), ties to the lower index: the total order the pages' selection
    key induces, stated without that key."""
    rng = np.random.default_rng(11)
    for E in (5, 64, 256):
        lg = rng.integers(0, 1 << 16, size=(30, E)).astype(np.uint16)
        lg[:, : E // 3] = lg[:, [0]]  # repeated patterns: ties
        for k in sorted({1, min(E, 4), E}):
            ids, tw, sc = oracle.topk(lg, k)
            for t in range(lg.shape[0]):
                def sm(b):
                    b = int(b)
                    return (b & 0x7FFF) if b < 0x8000 else -(b & 0x7FFF) - 1
                order = sorted(range(E), key=lambda e: (-sm(lg[t, e]), e))[:k]
                assert list(ids[t]) == order


def test_routing_weights_closed_forms():
    # all logits equal: s_j equal, tw = RNb(1/k) exactly representable for k=2^n
    for k in (1, 2, 4, 8):
        row = np.full((1, 16), 0x0000, dtype=np.uint16)  # +0 -> s = 0.5
        ids, tw, sc = oracle.topk(row, k)
        assert list(ids[0]) == list(range(k))
        assert np.all(sc == 0.5)
        assert np.all(tw == np.float32(1.0 / k))
    # top_k = 1: tw = s / RN32(s + 1e-20) = 1 exactly while s >> 1e-20
    rng = np.random.default_rng(5)
    lg = torch.from_numpy(rng.uniform(-20, 20, (200, 64)).astype(np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ids, tw, sc = oracle.topk(lg, 1)
    assert np.all(tw == 1.0)
    # all scores 0 (logits very negative): tw = 0
    ids, tw, sc = oracle.topk(np.full((1, 8), 0xC3C8, dtype=np.uint16), 4)  # -400
    assert np.all(sc == 0) and np.all(tw == 0)


def test_routing_weight_sums_are_one():
    rng = np.random.default_rng(7)
    lg = torch.from_numpy((rng.standard_normal((500, 128)) * 2).astype(np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for k in (2, 8, 16):
        ids, tw, sc = oracle.topk(lg, k)
        for t in range(lg.shape[0]):
            s = sum(float(v) for v in tw[t])
            bound = sum(_ulp_bf16(float(v)) / 2 for v in tw[t]) + 2 * k * 2.0 ** -24
            assert abs(s - 1.0) <= bound, (t, s)
        # scores are sigmoids of the selected logits, in descending order
        assert np.all(np.diff(sc, axis=1) <= 0)


def test_silu_special_cases():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(100.0) == np.float32(100.0)
    assert oracle.silu(-200.0) == 0.0 or abs(oracle.silu(-200.0)) < 1e-80
    # silu(x) - silu(-x) = x (sigmoid(x) + sigmoid(-x) = 1)
    for v in (0.5, 1.0, 3.0, 7.25):
        d = float(oracle.silu(v)) - float(oracle.silu(-v))
        assert abs(d - v) <= 4 * 2.0 ** -24 * v
    # exact value at 1: 1/(1+e^-1) = 0.7310585786300049
    assert oracle.silu(1.0) == np.float32(0.7310585786300049)
