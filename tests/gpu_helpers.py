"""Helpers of the GPU parity tests: moving synthetic inputs to the device,
running the HIP path through the C ABI, and the tolerance rules.

Tolerances (derived from the arithmetic, see the oracle's header):
* router logits: the GPU's fp32 accumulation order differs from the exact
  sum, so a logit may differ by one bf16 ulp;
* ids / tw: bit-exact given the same logits; dequantisation bit-exact;
* act, y (and the shared expert's): |gpu - ref| <= 1 bf16 ulp of ref plus the
  propagated bound of an fp32 accumulation in any order, gamma * sum|terms|
  with gamma = 64 * 2^-24, plus the SiLU approximation (2^-20 relative);
* combine: bit-exact given the same y, tw and shared output (the GPU forms
  the k-term sum exactly before its single fp32 rounding);
* end to end: |out_gpu - out_ref| <= 2 bf16 ulp of m, m = max(|out|,
  |routed|, |shared|, max_j |tw_j y_j|) of the oracle (the operands of the
  last two roundings), for tokens routed identically; tokens whose top-k
  differs are counted as near-tie flips and must come from logits within one
  ulp of the oracle's.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

GAMMA = 64 * 2.0 ** -24


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy storage bits -> torch device tensor with the same bytes."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().contiguous().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a if dtype is None else a.view(dtype)


def ulp_bf16(v) -> np.ndarray:
    """bf16 ulp of |v| (subnormal floor 2^-133)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.maximum(e, -126)
    u = np.exp2(e - 7)
    return np.where(v > 0, u, 2.0 ** -133)


def bf(bits) -> np.ndarray:
    return oracle.bf16_to_f32(bits).astype(np.float64)


def device_inputs(inp: dict, device="cuda") -> dict:
    d = {}
    for k, v in inp.items():
        if isinstance(v, np.ndarray):
            d[k] = dev(v, device)
    return d


def experts_of(d: dict) -> dict:
    if "w13" in d:
        return {k: d[k] for k in ("w13", "s13", "a13", "w2", "s2", "a2")}
    return {"w13": d["bw13"], "w2": d["bw2"]}


def shared_of(d: dict):
    return (d["sgu"], d["sdown"]) if "sgu" in d else None


def run_block(binding, inp: dict, path: str = "decode", forced=None, want_debug=True,
              ws=None):
    """Runs the HIP path on `inp`; returns host arrays of out and intermediates."""
    cfg = inp["cfg"]
    M, H, E, I, SI, k = cfg["M"], cfg["H"], cfg["E"], cfg["I"], cfg["SI"], cfg["top_k"]
    d = device_inputs(inp)
    if ws is None:
        ws = binding.make_workspace(M, H, E, I, SI if "sgu" in inp else 0, k)
    dbg = None
    if want_debug:
        z = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
        dbg = dict(logits_out=z((M, E), torch.int16), ids_out=z((M, k), torch.int32),
                   tw_out=z((M, k), torch.float32), act_out=z((M * k, I), torch.int16),
                   y_out=z((M * k, H), torch.int16))
        if "sgu" in inp:
            dbg.update(sact_out=z((M, SI), torch.int16), sh_out=z((M, H), torch.int16))
    if forced is not None:
        dbg = dict(dbg or {})
        dbg["ids_in"] = dev(np.ascontiguousarray(forced[0], dtype=np.int32))
        dbg["tw_in"] = dev(np.ascontiguousarray(forced[1], dtype=np.float32))
    x = d["x"]
    out = torch.empty((M, H), dtype=torch.int16, device="cuda")
    fn = {"decode": binding.flint_moe_decode, "grouped": binding.flint_moe_grouped,
          "bf16_decode": binding.flint_moe_bf16_decode}[path]
    fn(x, d["router"], experts_of(d), shared_of(d), k, ws, out=out, debug=dbg)
    torch.cuda.synchronize()
    r = dict(out=host(out))
    if dbg:
        for key, v in dbg.items():
            if key.endswith("_out"):
                r[key[:-4]] = host(v)
    return r


# ------------------------------------------------------------ tolerance

def check_act(gpu_act, ref_act, det, label=""):
    """act within 1 ulp + propagated fp32 accumulation bound."""
    g = det["g"].astype(np.float64)
    u = det["u"].astype(np.float64)
    eg = GAMMA * det["gabs"] + np.abs(g) * 2.0 ** -23
    eu = GAMMA * det["uabs"] + np.abs(u) * 2.0 ** -23
    silu = g / (1.0 + np.exp(-np.clip(g, -700, 700)))
    tol = (ulp_bf16(bf(ref_act)) + 1.1 * np.abs(u) * eg + np.abs(silu) * eu
           + 2.0 ** -20 * np.abs(silu * u) + 2.0 ** -126)
    err = np.abs(bf(gpu_act) - bf(ref_act))
    bad = err > tol
    assert not bad.any(), (f"{label} act: {bad.sum()} elements beyond tolerance; worst "
                           f"err/tol {np.max(err / tol):.3g}")
    return float(np.mean(err > 0))


def check_y(gpu_y, ref_y, det, label=""):
    tol = ulp_bf16(bf(ref_y)) + GAMMA * det["yabs"] + 2.0 ** -126
    err = np.abs(bf(gpu_y) - bf(ref_y))
    bad = err > tol
    assert not bad.any(), (f"{label} y: {bad.sum()} elements beyond tolerance; worst "
                           f"err/tol {np.max(err / tol):.3g}")
    return float(np.mean(err > 0))


def end_to_end_ulps(out_gpu, ref: dict, k: int, rows=None):
    """|out_gpu - out_ref| in units of ulp_bf16(m) per element, over `rows`
    (a boolean token mask; default all tokens)."""
    M = ref["out"].shape[0]
    rows = np.ones(M, bool) if rows is None else np.asarray(rows, bool)
    out_r = bf(ref["out"])[rows]
    routed = bf(ref["routed"])[rows]
    sh = bf(ref["sh"])[rows] if ref.get("sh") is not None else np.zeros_like(out_r)
    y = bf(ref["y"]).reshape(M, k, -1)[rows]
    tw = ref["tw"].astype(np.float64)[rows][:, :, None]
    m = np.maximum.reduce([np.abs(out_r), np.abs(routed), np.abs(sh),
                           np.max(np.abs(tw * y), axis=1)])
    return np.abs(bf(np.asarray(out_gpu)[rows]) - out_r) / ulp_bf16(m)
