"""Benchmark of the Flint routed-expert MoE block on one MI355X.

A step is one call of the whole block (router, top-k, routing plan, routed
gate/up + SwiGLU, routed down, shared expert, combine) on one batch of
seeded synthetic tokens, with every input already resident in HBM.  The
headline workload is decode of M=8 tokens against E=128 NVFP4 experts
(H=2048, I=768, top_k=8, shared SwiGLU expert of width 768).  Weights are
rotated over L layer copies so the working set exceeds twice the 256 MB
Infinity Cache and weight bytes really come from HBM.

Prints one JSON line: tokens/s, the achieved HBM bandwidth over the step's
algorithmic bytes, the roofline of the dominant kernel (its duration timed
with HIP events on the stream it runs on), the CPU oracle's throughput on a
bounded sample of the same workload and, unless --no-grouped, the prefill
workload (M=4096) on the grouped MFMA path with its own roofline.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
METRIC = "MoE-layer tokens/sec at M=8 decode; achieved HBM GB/s vs peak"


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1, help="decode workload index (0-3)")
    ap.add_argument("--layers", type=int, default=0, help="weight copies rotated (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-grouped", action="store_true", help="skip the M=4096 grouped line")
    ap.add_argument("--no-ll", action="store_true", help="skip the flint_moe_ll line")
    ap.add_argument("--grouped-steps", type=int, default=30)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain fp32 copy of MIB MiB 5 times (HBM counter scale)")
    return ap.parse_args()


# Kernel sources whose digest stamps a measured-traffic file: a file taken
# with other sources no longer describes the kernel and is ignored.
KERNEL_SOURCES = {
    "decode_kernel": ["decode.hip", "rowdot.hpp", "common.hpp", "internal.hpp"],
    "routed_gemm_kernel": ["grouped.hip", "common.hpp", "internal.hpp"],
}


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "nvfp4_w4a16_routed_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(profile: str, kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from a committed counter summary
    (profiles/<profile>.txt, "key: value" lines), or None when there is none
    or it was taken on other sources or another workload."""
    path = os.path.join(ROOT, "profiles", profile + ".txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "#", "|")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_digest(kernel) or kv.get("workload") != workload:
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch, mib: int):
    """A plain device copy of known size (fp32 negation: reads and writes
    exactly n bytes each), run 5 times, for scaling the HBM byte counters."""
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": "torch.neg fp32", "bytes_read_per_launch": n,
                      "bytes_written_per_launch": n, "launches": 5}), flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime (timing on our stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
            arr[i] = ev
        return arr

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        assert rc == 0, rc
        return float(ms.value)

    def destroy(self, arr):
        for ev in arr:
            self.hip.hipEventDestroy(ev)


def algorithmic_bytes(cfg: dict, U: int) -> dict:
    """Bytes the method must move per step: router, touched experts' weights,
    scales and global scales, shared expert, x in, out out."""
    M, H, E, I, SI = cfg["M"], cfg["H"], cfg["E"], cfg["I"], cfg["SI"]
    if cfg["experts"] == "nvfp4":
        gate_up = 2 * I * H // 2 + 2 * I * H // 16 + 4
        down = H * I // 2 + H * I // 16 + 4
    else:
        gate_up = 2 * I * H * 2
        down = H * I * 2
    router = E * H * 2
    shared = (2 * SI * H + H * SI) * 2
    x = M * H * 2
    out = M * H * 2
    return dict(per_expert_gate_up=gate_up, per_expert_down=down, router=router, shared=shared,
                x=x, out=out, total=router + U * (gate_up + down) + shared + x + out)


def flops(cfg: dict) -> dict:
    """Multiply-add work of one step (2 flops each)."""
    M, H, E, I, SI, k = cfg["M"], cfg["H"], cfg["E"], cfg["I"], cfg["SI"], cfg["top_k"]
    P = M * k
    f = dict(router=2 * M * E * H, gate_up=2 * P * 2 * I * H, down=2 * P * H * I,
             shared_gate_up=2 * M * 2 * SI * H, shared_down=2 * M * H * SI)
    f["total"] = sum(f.values())
    return f


def cpu_baseline(inp: dict, seconds: float) -> dict:
    import oracle
    cfg = inp["cfg"]
    threads = oracle.get_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.moe_block(inp)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    return {"value": cfg["M"] * reps / el, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{reps} full steps of this workload ({cfg['M']} tokens each, own "
                      f"routing, all stages) on the host CPU, {el:.1f} s"}


def run(fm, synth, torch, cfg_idx: int, path: str, steps: int, warmup: int, layers: int):
    """Times `steps` calls of `path` on workload cfg_idx.  Returns a dict with
    the step time, per-stage event times and the workload's sizes."""
    inp = synth.make_inputs(cfg_idx)
    cfg = inp["cfg"]
    M, H, E, I, SI, k = cfg["M"], cfg["H"], cfg["E"], cfg["I"], cfg["SI"], cfg["top_k"]
    nvfp4 = cfg["experts"] == "nvfp4"
    dev = torch.device("cuda", 0)

    def up(x):
        x = np.ascontiguousarray(x)
        t = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x)
        return t.to(dev)

    keys = ["w13", "s13", "a13", "w2", "s2", "a2"] if nvfp4 else ["bw13", "bw2"]
    base = {kk: up(inp[kk]) for kk in keys + ["router", "sgu", "sdown"]}
    per_layer = sum(v.numel() * v.element_size() for v in base.values())
    L = layers or max(2, int(np.ceil(2 * 256e6 / per_layer)) + 1)
    lays = [base] + [{kk: v.clone() for kk, v in base.items()} for _ in range(L - 1)]
    x = up(inp["x"])
    del inp
    if path == "sh_in":  # a precomputed shared output in place of the shared expert
        sh_buf = torch.zeros((M, H), dtype=torch.int16, device=dev)
    if path == "nv_shared":  # an NVFP4 shared expert of the same shape
        nvs = {kk: up(v) for kk, v in synth.nvfp4_experts(7, 1, H, SI).items()}
    if path == "ll":  # the residual-add RMS norm inputs in front of the block
        lli = synth.make_ll_inputs(1, M, H)
        la, lr, lw = up(lli["attn_out"]), up(lli["residual"]), up(lli["ln_weight"])
        lres = torch.empty((M, H), dtype=torch.int16, device=dev)
        lxn = torch.empty((M, H), dtype=torch.int16, device=dev)
    out = torch.empty((M, H), dtype=torch.int16, device=dev)
    ws = fm.make_workspace(M, H, E, I, SI, k)
    ids = torch.empty((M, k), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    lib = fm.lib()
    fn = {"decode": lib.flint_moe_decode, "grouped": lib.flint_moe_grouped,
          "bf16_decode": lib.flint_moe_bf16_decode, "ll": lib.flint_moe_ll,
          "sh_in": lib.flint_moe_decode, "nv_shared": lib.flint_moe_grouped}[path]
    keep = []

    def c_args(lay, dbg=None):
        if nvfp4:
            w = fm.nvfp4_experts_struct(*(lay[kk] for kk in keys))
        else:
            w = fm.Bf16Experts(fm._ptr(lay["bw13"]), fm._ptr(lay["bw2"]))
        sh = fm.SharedExpert(fm._ptr(lay["sgu"]), fm._ptr(lay["sdown"]), SI)
        if path == "sh_in":
            sh = fm.SharedExpert(None, None, 0, fm._ptr(sh_buf), None)
        if path == "nv_shared":
            sh = fm.SharedExpert(fm._ptr(nvs["w13"]), fm._ptr(nvs["w2"]), SI, None, None, fm._ptr(nvs["s13"]),
                                 fm._ptr(nvs["s2"]), fm._ptr(nvs["a13"]), fm._ptr(nvs["a2"]))
        keep.extend([w, sh, dbg])
        if path == "ll":
            return (fm._ptr(la), fm._ptr(lr), fm._ptr(lw), ctypes.c_float(lli["eps"]),
                    fm._ptr(lay["router"]), ctypes.byref(w), ctypes.byref(sh), M, H, E, I, k,
                    fm._ptr(out), fm._ptr(lres), fm._ptr(lxn),
                    ctypes.byref(dbg) if dbg is not None else None, fm._ptr(ws), ws.numel(), sp)
        return (fm._ptr(x), fm._ptr(lay["router"]), ctypes.byref(w), ctypes.byref(sh), M, H, E,
                I, k, fm._ptr(out), ctypes.byref(dbg) if dbg is not None else None, fm._ptr(ws),
                ws.numel(), sp)

    plain = [c_args(lay) for lay in lays]
    # touched experts of the workload, from one call
    dbg = fm.MoeDebug(None, None, None, fm._ptr(ids), None, None, None, None, None, None)
    assert fn(*c_args(lays[0], dbg)) == 0
    torch.cuda.synchronize()
    U = int(np.unique(ids.cpu().numpy()).size)

    # Pass A: back-to-back steps (the step throughput)
    for i in range(warmup):
        assert fn(*plain[i % L]) == 0
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        fn(*plain[i % L])
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps

    # Pass B: the same steps with HIP events around every stage (kernel)
    hev = HipEvents()
    nev = fm.FLINT_STAGE_EVENTS
    evs = [hev.create(nev) for _ in range(steps)]
    staged = []
    for i in range(steps):
        d = fm.MoeDebug(None, None, None, None, None, None, None, None, None,
                        ctypes.cast(evs[i], ctypes.POINTER(ctypes.c_void_p)))
        staged.append(c_args(lays[i % L], d))
    torch.cuda.synchronize()
    for i in range(steps):
        fn(*staged[i])
    torch.cuda.synchronize()
    stage_ms = np.zeros(nev - 1)
    for i in range(steps):
        for s in range(nev - 1):
            stage_ms[s] += hev.elapsed_ms(evs[i][s], evs[i][s + 1])
    stage_ms /= steps
    for e in evs:
        hev.destroy(e)
    del lays, plain, staged, keep
    torch.cuda.empty_cache()
    return dict(cfg=cfg, U=U, L=L, per_layer=per_layer, ms_step=ms_step, stage_ms=stage_ms)


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {a.gpus} requested): the Flint MoE "
              "block here runs on a single MI355X; sharding across GPUs is a design note, not a "
              "measured path.", file=sys.stderr)
        sys.exit(2)

    import torch

    if a.copy_calibration:
        copy_calibration(torch, a.copy_calibration)
        return

    import nvfp4_w4a16_routed_amd as fm
    import synth

    fm.lib()
    cfg_idx = a.config
    path = "bf16_decode" if synth.CONFIGS[cfg_idx]["experts"] == "bf16" else "decode"
    if cfg_idx == 4:
        path = "grouped"
    r = run(fm, synth, torch, cfg_idx, path, a.steps, a.warmup, a.layers)
    cfg = r["cfg"]
    M = cfg["M"]
    nbytes = algorithmic_bytes(cfg, r["U"])
    gbps = nbytes["total"] / (r["ms_step"] * 1e-3) / 1e9
    # The decode path is one kernel (stage 0): its bytes are the step's
    # algorithmic bytes and its duration the stage-0 event time.
    kern_ms = float(r["stage_ms"][0]) if path != "grouped" else float(r["stage_ms"][3])
    if path == "grouped":
        fl = flops(cfg)
        tfl = fl["gate_up"] / (kern_ms * 1e-3) / 1e12
        roof = {"kernel": "routed_gemm_kernel<gate/up>", "bound": "mfma",
                "achieved": round(tfl, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tfl / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic("routed_gemm_kernel_gate_up_m4096_hbm_traffic",
                                            "routed_gemm_kernel", cfg["name"]),
                "flops_per_launch": fl["gate_up"], "avg_launch_us": round(kern_ms * 1e3, 3)}
    else:
        dom_gbps = nbytes["total"] / (kern_ms * 1e-3) / 1e9
        roof = {"kernel": "decode_kernel", "bound": "hbm", "achieved": round(dom_gbps, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(f"decode_kernel_{cfg['name']}_hbm_traffic",
                                            "decode_kernel", cfg["name"]),
                "bytes_per_launch": nbytes["total"],
                "avg_launch_us": round(kern_ms * 1e3, 3)}
    res = {
        "metric": METRIC,
        "value": round(M / (r["ms_step"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(r["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 x nvfp4 (fp32 accumulate)" if cfg["experts"] == "nvfp4" else "bf16",
        "data": "synthetic (seeded; random weights of the Flint MoE shapes)",
        "config": {"workload": cfg["name"], "M": M, "H": cfg["H"], "E": cfg["E"], "I": cfg["I"],
                   "SI": cfg["SI"], "top_k": cfg["top_k"], "experts": cfg["experts"],
                   "touched_experts": r["U"], "layers_rotated": r["L"],
                   "weights_bytes_per_layer": r["per_layer"]},
        "hbm_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": nbytes["total"],
        "roofline": roof,
    }
    if path == "grouped":
        res["stage_us"] = {n: round(float(t) * 1e3, 2) for n, t in zip(fm.STAGES, r["stage_ms"])}
    if not a.no_cpu_baseline:
        inp = synth.make_inputs(cfg_idx)
        res["cpu_baseline"] = cpu_baseline(inp, a.cpu_seconds)
        del inp
    if path == "decode" and not a.no_ll:
        # flint_moe_ll on the same workload: the residual-add RMS norm in
        # front of the same decode block, same protocol and weight rotation
        ll = run(fm, synth, torch, cfg_idx, "ll", a.steps, a.warmup, a.layers)
        res["ll"] = {"entry": "flint_moe_ll", "workload": ll["cfg"]["name"],
                     "us_per_call": round(ll["ms_step"] * 1e3, 3),
                     "decode_us_per_call": round(r["ms_step"] * 1e3, 3),
                     "tokens_per_s": round(M / (ll["ms_step"] * 1e-3), 1)}
    if path == "decode" and not a.no_ll:
        # the same call with a precomputed shared output (no shared expert
        # computed; the output is added after the kernel)
        so = run(fm, synth, torch, cfg_idx, "sh_in", a.steps, a.warmup, a.layers)
        res["shared_output"] = {"entry": "flint_moe_decode + sh_in", "workload": so["cfg"]["name"],
                                "us_per_call": round(so["ms_step"] * 1e3, 3)}
    if not a.no_grouped and path != "grouped":
        g = run(fm, synth, torch, 4, "grouped", a.grouped_steps, 3, 1)
        gc = g["cfg"]
        fl = flops(gc)
        st = g["stage_ms"]
        gemm_ms = {"gate_up": st[3], "down": st[4], "shared_gate_up": st[2],
                   "shared_down": st[5]}
        res["grouped"] = {
            "workload": gc["name"], "M": gc["M"], "steps": a.grouped_steps,
            "ms_per_step": round(g["ms_step"], 4),
            "tokens_per_s": round(gc["M"] / (g["ms_step"] * 1e-3), 1),
            "tflops_per_s": round(fl["total"] / (g["ms_step"] * 1e-3) / 1e12, 1),
            "mfma_frac": round(fl["total"] / (g["ms_step"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "stage_us": {n: round(float(t) * 1e3, 2) for n, t in zip(fm.STAGES, st)},
            "gemm_tflops": {n: round(fl[n] / (gemm_ms[n] * 1e-3) / 1e12, 1) for n in gemm_ms},
            "roofline": {"kernel": "routed_gemm_kernel<gate/up>", "bound": "mfma",
                         "achieved": round(fl["gate_up"] / (st[3] * 1e-3) / 1e12, 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(fl["gate_up"] / (st[3] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("routed_gemm_kernel_gate_up_m4096_hbm_traffic",
                                                     "routed_gemm_kernel", gc["name"]),
                         "flops_per_launch": fl["gate_up"], "avg_launch_us": round(st[3] * 1e3, 2)},
        }
        # the same workload with an NVFP4 shared expert (routed kernels, E = 1)
        nv = run(fm, synth, torch, 4, "nv_shared", a.grouped_steps, 3, 1)
        res["grouped"]["nvfp4_shared_ms_per_step"] = round(nv["ms_step"], 4)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
