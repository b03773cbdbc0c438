"""CPU oracle of the Flint routed-expert MoE block (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (built from
``flint_oracle.c`` by ``oracle/build.py``) with numpy arrays of storage bits:
bf16 tensors are uint16 arrays, packed E2M1 codes and E4M3 scales are uint8,
global scales are float32.

Every stage follows the numerics rule of the page "vllm.models.flint.ops.moe"
(module docstring, "Numerics"); each C function states its step.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

FMT_NVFP4 = 0
FMT_BF16 = 1

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        lg = ctypes.c_long
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_e2m1.restype = ctypes.c_double
        L.orc_e2m1.argtypes = [ctypes.c_uint]
        L.orc_e4m3fn.restype = ctypes.c_double
        L.orc_e4m3fn.argtypes = [ctypes.c_uint]
        L.orc_router_score.restype = ctypes.c_float
        L.orc_router_score.argtypes = [ctypes.c_uint16]
        L.orc_silu.restype = ctypes.c_float
        L.orc_silu.argtypes = [ctypes.c_float]
        L.orc_nvfp4_dequant.restype = None
        L.orc_nvfp4_dequant.argtypes = [P, P, lg, lg, P]
        L.orc_logits.restype = None
        L.orc_logits.argtypes = [P, P, lg, lg, lg, P]
        L.orc_topk.restype = None
        L.orc_topk.argtypes = [P, lg, lg, lg, P, P, P]
        L.orc_gate_up.restype = None
        L.orc_gate_up.argtypes = [P, lg, lg, lg, lg, P, ctypes.c_int, P, P, P,
                                  P, lg, P, P, P, P, P]
        L.orc_down.restype = None
        L.orc_down.argtypes = [P, lg, lg, lg, P, ctypes.c_int, P, P, P, P, lg,
                               P, P, P]
        L.orc_combine.restype = None
        L.orc_combine.argtypes = [P, P, P, lg, lg, lg, P, P]
        L.orc_set_threads.restype = None
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_get_threads.restype = ctypes.c_int
        L.orc_get_threads.argtypes = []
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


# ----------------------------------------------------------------- formats

def bf16_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(vals) -> np.ndarray:
    v = np.asarray(vals, dtype=np.float32)
    f = lib().orc_f32_to_bf16
    return np.array([f(float(x)) for x in v.ravel()], dtype=np.uint16).reshape(v.shape)


def f64_to_bf16(vals) -> np.ndarray:
    """fp64 -> bf16 bits, one round to nearest even (no double rounding).

    The value goes to fp32 first; when that lands exactly halfway between
    two bf16 values without being exact, the fp32 bits are moved one step
    toward the fp64 value so the bf16 rounding goes the way the fp64 value
    lies (finite values)."""
    x = np.asarray(vals, dtype=np.float64)
    f = x.astype(np.float32)
    b = f.view(np.uint32).copy()
    tie = (b & 0xFFFF) == 0x8000
    inexact = f.astype(np.float64) != x
    away = np.abs(x) > np.abs(f.astype(np.float64))
    nudge = tie & inexact
    b = np.where(nudge & away, b + 1, np.where(nudge & ~away, b - 1, b)).astype(np.uint32)
    return f32_to_bf16(b.view(np.float32))


def e2m1(code: int) -> float:
    return lib().orc_e2m1(int(code))


def e4m3fn(byte: int) -> float:
    return lib().orc_e4m3fn(int(byte))


def router_score(logit_bits: int) -> np.float32:
    return np.float32(lib().orc_router_score(int(logit_bits)))


def silu(g: float) -> np.float32:
    return np.float32(lib().orc_silu(float(g)))


def nvfp4_dequant(w, s) -> np.ndarray:
    """[rows, K/2] codes + [rows, K/16] scales -> [rows, K] bf16 bits."""
    w = _c(w, np.uint8)
    s = _c(s, np.uint8)
    rows, K = w.shape[0], w.shape[1] * 2
    assert s.shape == (rows, K // 16)
    out = np.empty((rows, K), dtype=np.uint16)
    lib().orc_nvfp4_dequant(_p(w), _p(s), rows, K, _p(out))
    return out


# ----------------------------------------------------------------- routing

def logits(x, router) -> np.ndarray:
    x = _c(x, np.uint16)
    r = _c(router, np.uint16)
    M, H = x.shape
    E = r.shape[0]
    out = np.empty((M, E), dtype=np.uint16)
    lib().orc_logits(_p(x), _p(r), M, H, E, _p(out))
    return out


def topk(lg, k: int):
    """Returns (ids int32 [M,k], tw float32 [M,k], scores float32 [M,k])."""
    lg = _c(lg, np.uint16)
    M, E = lg.shape
    assert 1 <= k <= E <= 256
    ids = np.empty((M, k), dtype=np.int32)
    tw = np.empty((M, k), dtype=np.float32)
    sc = np.empty((M, k), dtype=np.float32)
    lib().orc_topk(_p(lg), M, E, k, _p(ids), _p(tw), _p(sc))
    return ids, tw, sc


# ------------------------------------------------------------ expert stages

def _expert_args(w: dict, which: str):
    """(fmt, codes, scales, alpha, bf16, E) for 'w13' or 'w2' of an input dict
    (NVFP4 keys w13/s13/a13, w2/s2/a2; BF16 keys bw13/bw2)."""
    if which in w and w[which] is not None and w[which].dtype == np.uint8:
        sk = "s13" if which == "w13" else "s2"
        ak = "a13" if which == "w13" else "a2"
        codes = _c(w[which], np.uint8)
        return (FMT_NVFP4, codes, _c(w[sk], np.uint8), _c(w[ak], np.float32),
                None, codes.shape[0])
    bw = _c(w["b" + which], np.uint16)
    return FMT_BF16, None, None, None, bw, bw.shape[0]


def gate_up(x, ids, k: int, w: dict, I: int, want_detail: bool = False):
    """act [M*k, I] bf16 bits for every pair p = t*k + j (expert ids[p])."""
    x = _c(x, np.uint16)
    ids = _c(ids, np.int32).reshape(-1)
    M, H = x.shape
    assert ids.size == M * k
    fmt, codes, scales, alpha, bw, E = _expert_args(w, "w13")
    act = np.empty((M * k, I), dtype=np.uint16)
    det = None
    if want_detail:
        det = dict(g=np.empty((M * k, I), np.float32), u=np.empty((M * k, I), np.float32),
                   gabs=np.empty((M * k, I), np.float64),
                   uabs=np.empty((M * k, I), np.float64))
    lib().orc_gate_up(_p(x), M, H, I, k, _p(ids), fmt, _p(codes), _p(scales),
                      _p(alpha), _p(bw), E, _p(act),
                      *(_p(det[n]) if det else None for n in ("g", "u", "gabs", "uabs")))
    return (act, det) if want_detail else act


def down(act, ids, w: dict, H: int, want_detail: bool = False):
    """y [npairs, H] bf16 bits: y[p] = RNb(RN32(RN32(act[p] . W2[ids[p]]) * a2))."""
    act = _c(act, np.uint16)
    ids = _c(ids, np.int32).reshape(-1)
    npairs, I = act.shape
    assert ids.size == npairs
    fmt, codes, scales, alpha, bw, E = _expert_args(w, "w2")
    y = np.empty((npairs, H), dtype=np.uint16)
    det = None
    if want_detail:
        det = dict(yacc=np.empty((npairs, H), np.float32),
                   yabs=np.empty((npairs, H), np.float64))
    lib().orc_down(_p(act), npairs, H, I, _p(ids), fmt, _p(codes), _p(scales),
                   _p(alpha), _p(bw), E, _p(y),
                   _p(det["yacc"]) if det else None, _p(det["yabs"]) if det else None)
    return (y, det) if want_detail else y


def combine(y, tw, sh, k: int):
    """(out, routed) [M, H] bf16 bits; sh None means no shared expert."""
    y = _c(y, np.uint16)
    tw = _c(tw, np.float32).reshape(-1)
    H = y.shape[1]
    M = y.shape[0] // k
    assert tw.size == M * k
    shc = None if sh is None else _c(sh, np.uint16)
    out = np.empty((M, H), dtype=np.uint16)
    routed = np.empty((M, H), dtype=np.uint16)
    lib().orc_combine(_p(y), _p(tw), _p(shc), M, H, k, _p(out), _p(routed))
    return out, routed


def shared_expert(x, sgu, sdown, want_detail: bool = False):
    """Ungated shared SwiGLU expert under the routed rule with bf16 weights and
    no global scale: (sact [M, SI], sh [M, H]) bf16 bits."""
    x = _c(x, np.uint16)
    M, H = x.shape
    SI = sgu.shape[0] // 2
    zeros = np.zeros(M, dtype=np.int32)
    wv = dict(bw13=np.asarray(sgu)[None], bw2=np.asarray(sdown)[None])
    r1 = gate_up(x, zeros, 1, wv, SI, want_detail)
    sact = r1[0] if want_detail else r1
    r2 = down(sact, zeros, wv, H, want_detail)
    if want_detail:
        return sact, r2[0], dict(gate_up=r1[1], down=r2[1])
    return sact, r2


def add_rms_norm(a, r, w, eps: float):
    """Residual add and RMS norm in front of the block (page
    "vllm.models.flint.ops.moe", _add_rms_norm and flint_moe_ll): for each
    row, s = a + r in fp32 (one fp32 rounding of two bf16 values);
    residual' = bf16(s); xn = bf16(s * rsqrt(mean(s^2) + eps) * w).  The
    pages reduce mean(s^2) in fp32 in an order they do not fix and leave
    their rsqrt helper unprinted; here the mean, the reciprocal square root
    and the products are exact (fp64), rounded once to bf16.

    a, r: [M, H] bf16 bits; w: [H] bf16 bits.  Returns (residual', xn) as
    bf16 bits."""
    af = bf16_to_f32(a)
    rf = bf16_to_f32(r)
    s = (af + rf).astype(np.float32)  # IEEE fp32 addition, round to nearest even
    res = f32_to_bf16(s)
    s64 = s.astype(np.float64)
    H = s64.shape[-1]
    ms = np.sum(s64 * s64, axis=-1, keepdims=True) / H
    inv = 1.0 / np.sqrt(ms + np.float64(np.float32(eps)))
    xn = f64_to_bf16(s64 * inv * bf16_to_f32(w).astype(np.float64))
    return res, xn


def moe_block(inp: dict, tokens=None, forced_ids=None, forced_tw=None,
              want_detail: bool = False) -> dict:
    """The whole block for the given tokens (default: all).

    forced_ids / forced_tw ([len(tokens), k]) replace steps 1-3 (logits,
    top-k, weights).  Returns a dict with logits, ids, tw, act, y, sact, sh,
    routed, out (each restricted to the tokens)."""
    cfg = inp["cfg"]
    k, I, H = cfg["top_k"], cfg["I"], cfg["H"]
    x = np.asarray(inp["x"])
    if tokens is not None:
        x = x[np.asarray(tokens)]
    r = dict()
    if forced_ids is None:
        r["logits"] = logits(x, inp["router"])
        r["ids"], r["tw"], r["scores"] = topk(r["logits"], k)
    else:
        r["ids"] = _c(forced_ids, np.int32)
        r["tw"] = _c(forced_tw, np.float32)
    ga = gate_up(x, r["ids"], k, inp, I, want_detail)
    r["act"], r["gate_up_detail"] = (ga if want_detail else (ga, None))
    dn = down(r["act"], r["ids"], inp, H, want_detail)
    r["y"], r["down_detail"] = (dn if want_detail else (dn, None))
    if inp.get("sgu") is not None:
        sres = shared_expert(x, inp["sgu"], inp["sdown"], want_detail)
        r["sact"], r["sh"] = sres[0], sres[1]
        if want_detail:
            r["shared_detail"] = sres[2]
    else:
        r["sact"], r["sh"] = None, None
    r["out"], r["routed"] = combine(r["y"], r["tw"], r["sh"], k)
    return r
