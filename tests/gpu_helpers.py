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

import ctypes

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


def hip_events(n):
    """n hipEvent_t handles (a ctypes array) from the HIP runtime."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    arr = (ctypes.c_void_p * n)()
    for i in range(n):
        ev = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(ev)) == 0
        arr[i] = ev
    return arr


def hip_record(ev, stream=None):
    """hipEventRecord(ev, stream) (default: torch's current stream)."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    st = (stream or torch.cuda.current_stream()).cuda_stream
    assert hip.hipEventRecord(ev, ctypes.c_void_p(st)) == 0


def run_block(binding, inp: dict, path: str = "decode", forced=None, want_debug=True,
              ws=None, stage_events=None):
    """Runs the HIP path on `inp`; returns host arrays of out and intermediates.
    stage_events: optional hipEvent_t array recorded around every stage."""
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
    if stage_events is not None:
        dbg = dict(dbg or {})
        dbg["stage_events"] = stage_events
    x = d["x"]
    out = torch.empty((M, H), dtype=torch.int16, device="cuda")
    fn = {"decode": binding.flint_moe_decode, "grouped": binding.flint_moe_grouped,
          "bf16_decode": binding.flint_moe_bf16_decode,
          "bf16_grouped": binding.flint_moe_bf16_grouped}[path]
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


def check_logits(gpu_lg, ref_lg, x, router, label=""):
    """Router logits within one bf16 ulp plus the bound of an fp32 sum in any
    order (GAMMA * sum |x_h R_eh|)."""
    mag = np.abs(bf(x)) @ np.abs(bf(router)).T
    tol = ulp_bf16(bf(ref_lg)) + GAMMA * mag
    err = np.abs(bf(gpu_lg) - bf(ref_lg))
    bad = err > tol
    assert not bad.any(), (f"{label} logits: {bad.sum()} beyond tolerance; worst err/tol "
                           f"{np.max(err / tol):.3g}")


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


def same_f32(a, b) -> bool:
    """Bitwise equality of float32 arrays (NaN == NaN)."""
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(
        a[~np.isnan(a)].view(np.uint32), b[~np.isnan(b)].view(np.uint32))


def error_report(out_gpu, ref: dict, k: int, rows=None) -> dict:
    """Plain error figures of out against the oracle's out over `rows`
    (tokens routed identically): max absolute error, max relative error
    (|err| / |ref| over nonzero ref), and the histogram of |err| in units of
    ulp_bf16(out_ref) (0, 1, 2, >2)."""
    M = ref["out"].shape[0]
    rows = np.ones(M, bool) if rows is None else np.asarray(rows, bool)
    r = bf(ref["out"])[rows]
    g = bf(np.asarray(out_gpu))[rows]
    err = np.abs(g - r)
    nz = r != 0
    u = err / ulp_bf16(r)
    hist = {"0": int(np.sum(u == 0)), "1": int(np.sum((u > 0) & (u <= 1))),
            "2": int(np.sum((u > 1) & (u <= 2))), ">2": int(np.sum(u > 2))}
    return dict(max_abs=float(err.max()) if err.size else 0.0,
                max_rel=float(np.max(err[nz] / np.abs(r[nz]))) if np.any(nz) else 0.0,
                ulp_out_hist=hist, elements=int(err.size))


def record(entry: dict) -> None:
    """Appends one JSON line to the file named by $FLINT_PARITY_REPORT (if set)."""
    import json
    import os
    path = os.environ.get("FLINT_PARITY_REPORT")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps(entry) + "\n")


def stagewise_routing(inp, r):
    """Logits within tolerance; ids / tw bit-exact given the GPU's logits."""
    cfg = inp["cfg"]
    ref_lg = oracle.logits(inp["x"], inp["router"])
    check_logits(r["logits"], ref_lg, inp["x"], inp["router"], cfg["name"])
    rids, rtw, _ = oracle.topk(r["logits"], cfg["top_k"])
    assert np.array_equal(r["ids"], rids), "ids differ from the oracle's top-k of the GPU's logits"
    assert same_f32(r["tw"], rtw), "tw differ from the oracle's top-k of the GPU's logits"


def stagewise_routed(inp, r):
    """Routed act on the GPU's routing and y on the GPU's act."""
    cfg = inp["cfg"]
    k, I, H, label = cfg["top_k"], cfg["I"], cfg["H"], cfg["name"]
    act, det = oracle.gate_up(inp["x"], r["ids"], k, inp, I, want_detail=True)
    check_act(r["act"], act, det, label)
    y, ydet = oracle.down(r["act"], r["ids"], inp, H, want_detail=True)
    check_y(r["y"], y, ydet, label)


def end_to_end(inp, r, say=print, sh_in=None, extra=None):
    """The GPU's out against the oracle's own routing (tokens routed
    identically), within 2 ulp of m; prints and records the error figures.
    sh_in: a precomputed shared output that replaces the oracle's shared
    expert."""
    cfg = inp["cfg"]
    k, label = cfg["top_k"], cfg["name"]
    full = oracle.moe_block(inp)
    if sh_in is not None:
        full = dict(full)
        full["sh"] = sh_in
        full["out"], full["routed"] = oracle.combine(full["y"], full["tw"], sh_in, k)
    same = np.all(full["ids"] == r["ids"], axis=1)
    ulps = end_to_end_ulps(r["out"], full, k, rows=same)
    rep = error_report(r["out"], full, k, rows=same)
    say(f"{label}: tokens {cfg['M']}, near-tie flips {int((~same).sum())}, "
        f"max ulp(m) {ulps.max() if ulps.size else 0:.3f}, "
        f"mean nonzero {np.mean(ulps > 0) if ulps.size else 0:.4f}, "
        f"max abs {rep['max_abs']:.3g}, max rel {rep['max_rel']:.3g}, "
        f"ulp(out_ref) histogram {rep['ulp_out_hist']}")
    entry = dict(workload=label, M=cfg["M"], E=cfg["E"], top_k=k, H=cfg["H"], I=cfg["I"],
                 near_tie_flips=int((~same).sum()),
                 max_ulp_m=float(ulps.max()) if ulps.size else 0.0, **rep)
    entry.update(extra or {})
    record(entry)
    assert ulps.size == 0 or ulps.max() <= 2.0
    return full


def stagewise(inp, r, say=print, extra=None):
    """Checks every stage of a GPU run against the oracle fed with the GPU's
    own upstream values; returns the oracle's end-to-end result."""
    cfg = inp["cfg"]
    k, H = cfg["top_k"], cfg["H"]
    label = cfg["name"]
    stagewise_routing(inp, r)
    stagewise_routed(inp, r)
    sh = None
    if "sgu" in inp:
        sact, sh_ref, sdet = oracle.shared_expert(inp["x"], inp["sgu"], inp["sdown"], True)
        check_act(r["sact"], sact, sdet["gate_up"], label + " shared")
        zeros = np.zeros(cfg["M"], np.int32)
        sh2, shdet = oracle.down(r["sact"], zeros, dict(bw2=inp["sdown"][None]), H, True)
        check_y(r["sh"], sh2, shdet, label + " shared")
        sh = r["sh"]
    # combine: bit-exact on the GPU's y, tw and shared output
    out_c, _ = oracle.combine(r["y"], r["tw"], sh, k)
    assert np.array_equal(r["out"], out_c), "combine differs"
    return end_to_end(inp, r, say, extra=extra)
