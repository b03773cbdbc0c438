"""Pins of the oracle's whole block (CPU only).

* An exact-rational brute force (fractions + 60-digit decimal exp) on tiny
  shapes fixes every rounding point of the numerics rule.
* One-expert and all-experts cases reduce the block to a dense SwiGLU that is
  recomputed with numpy float64 matmuls and library casts.
* Invariants: expert relabelling, power-of-two global scales, batch
  independence.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import exact


def _e4m3_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def _dequant_f64(codes, scales):
    """Library-side dequant: golden E2M1 table x torch E4M3 decode (float64)."""
    e4 = _e4m3_table()
    lo = codes & 15
    hi = codes >> 4
    c = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.int64)
    c[..., 0::2] = lo
    c[..., 1::2] = hi
    v = np.array(E2M1)[c]
    sc = np.repeat(e4[scales], 16, axis=-1)
    return v * sc


def _bf(bits):
    return oracle.bf16_to_f32(bits).astype(np.float64)


def _to_bf16_bits(v32):
    return torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------- exact brute force

def _frac_silu(g: float) -> float:
    """RN32(g * sigmoid(g)) from a 60-digit exp."""
    G = Fraction(g)
    return exact.rn32(G / (1 + exact.exp_decimal(-G)))


def _brute_force_block(inp):
    cfg = inp["cfg"]
    M, H, E, I, k = cfg["M"], cfg["H"], cfg["E"], cfg["I"], cfg["top_k"]
    F = Fraction
    x = [[F(float(v)) for v in row] for row in _bf(inp["x"])]
    R = [[F(float(v)) for v in row] for row in _bf(inp["router"])]
    nv = "w13" in inp
    if nv:
        W13 = _dequant_f64(inp["w13"], inp["s13"])
        W2 = _dequant_f64(inp["w2"], inp["s2"])
        a13 = [F(float(a)) for a in inp["a13"]]
        a2 = [F(float(a)) for a in inp["a2"]]
    else:
        W13 = _bf(inp["bw13"])
        W2 = _bf(inp["bw2"])
    Wsgu = _bf(inp["sgu"])
    Wsd = _bf(inp["sdown"])
    SI = Wsgu.shape[0] // 2
    eps = F(float(np.float32(1e-20)))
    res = dict(logits=np.zeros((M, E), np.float64), ids=np.zeros((M, k), np.int64),
               tw=np.zeros((M, k)), act=np.zeros((M * k, I)), y=np.zeros((M * k, H)),
               sh=np.zeros((M, H)), out=np.zeros((M, H)))
    for t in range(M):
        lg = [exact.rnbf16(F(exact.rn32(sum(x[t][h] * R[e][h] for h in range(H)))))
              for e in range(E)]
        res["logits"][t] = lg
        order = sorted(range(E), key=lambda e: (-lg[e], e))[:k]
        res["ids"][t] = order
        s = []
        for e in order:
            q = -F(lg[e])
            a = exact.rn32(exact.exp_decimal(q))
            d = exact.rn32(1 + F(a))
            s.append(exact.rn32(1 / F(d)))
        S = F(0)
        for v in s:
            S = F(exact.rn32(S + F(v)))
        D = F(exact.rn32(S + eps))
        tw = [exact.rnbf16(F(exact.rn32(F(v) / D))) for v in s]
        res["tw"][t] = tw
        # shared expert (bf16 weights, no global scale)
        sact = []
        for n in range(SI):
            g = exact.rn32(sum(x[t][h] * F(Wsgu[n, h]) for h in range(H)))
            u = exact.rn32(sum(x[t][h] * F(Wsgu[SI + n, h]) for h in range(H)))
            sact.append(F(exact.rnbf16(F(exact.rn32(F(_frac_silu(g)) * F(u))))))
        sh = [exact.rnbf16(F(exact.rn32(sum(sact[i] * F(Wsd[h, i]) for i in range(SI)))))
              for h in range(H)]
        res["sh"][t] = sh
        ys = []
        for j, e in enumerate(order):
            p = t * k + j
            act = []
            for n in range(I):
                g = F(exact.rn32(sum(x[t][h] * F(W13[e, n, h]) for h in range(H))))
                u = F(exact.rn32(sum(x[t][h] * F(W13[e, I + n, h]) for h in range(H))))
                if nv:
                    g, u = F(exact.rn32(g * a13[e])), F(exact.rn32(u * a13[e]))
                act.append(F(exact.rnbf16(F(exact.rn32(F(_frac_silu(float(g))) * u)))))
            res["act"][p] = [float(v) for v in act]
            y = []
            for h in range(H):
                acc = F(exact.rn32(sum(act[i] * F(W2[e, h, i]) for i in range(I))))
                if nv:
                    acc = F(exact.rn32(acc * a2[e]))
                y.append(exact.rnbf16(acc))
            res["y"][p] = y
            ys.append(y)
        for h in range(H):
            Rr = exact.rn32(sum(F(tw[j]) * F(ys[j][h]) for j in range(k)))
            routed = exact.rnbf16(F(Rr))
            res["out"][t, h] = exact.rnbf16(F(exact.rn32(F(routed) + F(sh[h]))))
    return res


@pytest.mark.parametrize("experts", ["nvfp4", "bf16"])
def test_brute_force_exact_rationals(experts):
    inp = synth.make_small(11, M=3, H=32, E=4, I=16, SI=16, top_k=2, experts=experts,
                           router_std=0.5)
    want = _brute_force_block(inp)
    got = oracle.moe_block(inp)
    assert np.array_equal(_bf(got["logits"]), want["logits"])
    assert np.array_equal(got["ids"], want["ids"])
    assert np.array_equal(got["tw"].astype(np.float64), want["tw"])
    for name in ("act", "y", "sh", "out"):
        g = _bf(got[name])
        assert np.array_equal(g, want[name]), name


# ------------------------------------------- reductions to a dense SwiGLU

def _dense_swiglu_f64(x, W13, W2, a13, a2, I):
    """Dense SwiGLU with numpy float64 matmuls, float32 casts for RN32 and
    torch casts for RNb."""
    X = _bf(x)
    Gs = (X @ W13[:I].T).astype(np.float32)
    Us = (X @ W13[I:].T).astype(np.float32)
    if a13 is not None:
        Gs = Gs * np.float32(a13)
        Us = Us * np.float32(a13)
    g64 = Gs.astype(np.float64)
    silu = (g64 / (1.0 + np.exp(-g64))).astype(np.float32)
    act = _to_bf16_bits((silu.astype(np.float64) * Us.astype(np.float64)).astype(np.float32))
    Y = (_bf(act) @ W2.T).astype(np.float32)
    if a2 is not None:
        Y = Y * np.float32(a2)
    return act, _to_bf16_bits(Y)


@pytest.mark.parametrize("experts", ["nvfp4", "bf16"])
def test_single_expert_reduces_to_dense_swiglu(experts):
    inp = synth.make_small(21, M=5, H=256, E=1, I=64, SI=64, top_k=1, experts=experts)
    got = oracle.moe_block(inp)
    assert np.all(got["ids"] == 0) and np.all(got["tw"] == 1.0)
    if experts == "nvfp4":
        W13 = _dequant_f64(inp["w13"], inp["s13"])[0]
        W2 = _dequant_f64(inp["w2"], inp["s2"])[0]
        a13, a2 = inp["a13"][0], inp["a2"][0]
    else:
        W13, W2 = _bf(inp["bw13"])[0], _bf(inp["bw2"])[0]
        a13 = a2 = None
    act, y = _dense_swiglu_f64(inp["x"], W13, W2, a13, a2, 64)
    sact, sh = _dense_swiglu_f64(inp["x"], _bf(inp["sgu"]), _bf(inp["sdown"]), None, None, 64)
    assert np.array_equal(got["act"], act)
    assert np.array_equal(got["sh"], sh)
    out = _to_bf16_bits((_bf(y) + _bf(sh)).astype(np.float32))
    assert np.array_equal(got["out"], out)


def test_all_experts_selected_reduces_to_dense_sum():
    E = 4
    inp = synth.make_small(31, M=4, H=128, E=E, I=32, SI=32, top_k=E)
    got = oracle.moe_block(inp)
    assert all(sorted(r) == list(range(E)) for r in got["ids"])
    W13 = _dequant_f64(inp["w13"], inp["s13"])
    W2 = _dequant_f64(inp["w2"], inp["s2"])
    ys = [_dense_swiglu_f64(inp["x"], W13[e], W2[e], inp["a13"][e], inp["a2"][e], 32)[1]
          for e in range(E)]
    sh = _dense_swiglu_f64(inp["x"], _bf(inp["sgu"]), _bf(inp["sdown"]), None, None, 32)[1]
    tw = got["tw"].astype(np.float64)
    M, H = inp["x"].shape[0], 128
    routed = np.zeros((M, H))
    for t in range(M):
        for j, e in enumerate(got["ids"][t]):
            routed[t] += tw[t, j] * _bf(ys[e][t])
    routed_b = _to_bf16_bits(routed.astype(np.float32))
    out = _to_bf16_bits((_bf(routed_b) + _bf(sh)).astype(np.float32))
    assert np.array_equal(got["routed"], routed_b)
    assert np.array_equal(got["out"], out)


# ------------------------------------------------------------- invariants

def test_expert_relabelling_permutes_ids_only():
    inp = synth.make_small(41, M=6, H=128, E=16, I=32, SI=32, top_k=4, router_std=0.2)
    base = oracle.moe_block(inp)
    perm = np.random.default_rng(3).permutation(16)   # new label n holds old expert perm[n]
    inp2 = dict(inp)
    for key in ("router", "w13", "s13", "a13", "w2", "s2", "a2"):
        inp2[key] = np.ascontiguousarray(inp[key][perm])
    got = oracle.moe_block(inp2)
    inv = np.argsort(perm)
    # equal logits are ordered by expert index, which relabelling changes:
    # compare the tokens whose logits are all distinct
    distinct = [t for t in range(6) if len(set(base["logits"][t])) == 16]
    assert len(distinct) >= 3
    d = np.array(distinct)
    assert np.array_equal(got["ids"][d], inv[base["ids"][d]])
    assert np.array_equal(got["tw"][d], base["tw"][d])
    assert np.array_equal(got["out"][d], base["out"][d])


def test_power_of_two_global_scale_doubles_y():
    inp = synth.make_small(51, M=3, H=128, E=8, I=32, SI=0, top_k=2)
    base = oracle.moe_block(inp)
    inp2 = dict(inp, a2=(inp["a2"] * np.float32(2)).astype(np.float32))
    got = oracle.moe_block(inp2)
    assert np.array_equal(_bf(got["y"]), 2 * _bf(base["y"]))
    assert base["sh"] is None


def test_batch_independence():
    inp = synth.make_small(61, M=9, H=128, E=8, I=32, SI=32, top_k=3)
    full = oracle.moe_block(inp)
    sub = [7, 2, 4]
    part = oracle.moe_block(inp, tokens=sub)
    assert np.array_equal(part["out"], full["out"][sub])
    assert np.array_equal(part["ids"], full["ids"][sub])


def test_forced_routing_matches_own_routing():
    inp = synth.make_small(71, M=4, H=128, E=8, I=32, SI=32, top_k=2)
    full = oracle.moe_block(inp)
    forced = oracle.moe_block(inp, forced_ids=full["ids"], forced_tw=full["tw"])
    assert np.array_equal(forced["out"], full["out"])


def test_thread_count_does_not_change_results():
    inp = synth.make_small(81, M=6, H=256, E=8, I=64, SI=64, top_k=2)
    oracle.set_threads(1)
    a = oracle.moe_block(inp)
    oracle.set_threads(4)
    b = oracle.moe_block(inp)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["act"], b["act"])
