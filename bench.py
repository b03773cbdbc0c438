"""Benchmark of the Flint routed-expert MoE block on one MI355X.

A step is one call of the whole block (router, top-k, routing plan, routed
gate/up + SwiGLU, routed down, shared expert, combine) on one batch of
seeded synthetic tokens, with every input already resident in HBM.  The
headline workload is decode of M=8 tokens against E=128 NVFP4 experts
(H=2048, I=768, top_k=8, shared SwiGLU expert of width 768).  Weights are
rotated over L layer copies, L sized from the bytes one call touches, so the
same weights are reused only after more than twice the 256 MB Infinity Cache
has streamed: weight bytes really come from HBM.  Every timing runs the
workload untimed for --settle seconds (0.3 by default) and then the warm-up
calls before its timed calls, so the GPU's clocks are at their loaded level.

Prints one JSON line: tokens/s of the headline workload, the achieved HBM
bandwidth over its algorithmic bytes, the roofline of its one kernel (the
decode kernel's average duration from HIP events on its launch stream around
the back-to-back timed launches), the CPU oracle's throughput on a bounded
sample of the same workload, and the other workloads: decode M=1 (E=32),
M=64 with Zipf routing, BF16 experts, the fused residual-add + RMS norm
entry, the precomputed shared output, an NVFP4 shared expert, and the
prefill workload M=4096 on the grouped MFMA path (NVFP4 and BF16 experts)
with the roofline of its dominant kernel.
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
FP32_VALU_TFLOPS = 157.3    # MI355X fp32 vector (the dot2 bf16 rate counts 4 flop per lane)
MALL_BYTES = 256e6          # Infinity Cache
SETTLE_S = 0.3              # untimed seconds before each timing (set from --settle)
METRIC = "MoE-layer tokens/sec at M=8 decode; achieved HBM GB/s vs peak"


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle", type=float, default=0.3, metavar="S",
                    help="seconds of untimed calls before each timing's warm-up steps, so the "
                         "GPU's clocks are at their loaded level (0 = none)")
    ap.add_argument("--config", type=int, default=1, help="headline decode workload index (0-3)")
    ap.add_argument("--layers", type=int, default=0, help="weight copies rotated (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline workload (for profiling its kernel)")
    ap.add_argument("--no-grouped", action="store_true", help="skip the M=4096 grouped lines")
    ap.add_argument("--grouped-only", action="store_true",
                    help="time only the M=4096 NVFP4 grouped line (for profiling its kernels)")
    ap.add_argument("--grouped-steps", type=int, default=30)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain fp32 copy of MIB MiB 5 times (HBM counter scale)")
    ap.add_argument("--mfma-calibration", type=int, default=0, metavar="N",
                    help="only time a dense bf16 N x N x N product through torch on random data "
                         "(the vendor GEMM's rate, and the MFMA counters' scale)")
    return ap.parse_args()


# Kernel sources whose digest stamps a measured-traffic file: a file taken
# with other sources no longer describes the kernel and is ignored.
KERNEL_SOURCES = {
    "decode_kernel": ["decode.hip", "rowdot.hpp", "common.hpp", "internal.hpp", "topk.hpp"],
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


def mfma_calibration(torch, n: int):
    """A dense bf16 product C = A B (N x N x N, A and B ~ N(0, 1), seeded)
    through torch (the vendor GEMM library), 10 untimed and 20 timed
    launches: the rate a tuned library reaches on this part with random data,
    and a known FLOP count for reading the MFMA busy counters."""
    g = torch.Generator(device="cuda").manual_seed(1234)
    a = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
    c = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    for _ in range(10):
        torch.matmul(a, b, out=c)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(20):
        torch.matmul(a, b, out=c)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / 20
    flops = 2.0 * n * n * n
    print(json.dumps({"mfma_calibration": "torch.matmul bf16 random N(0,1)", "n": n, "flops_per_launch": flops,
                      "avg_launch_us": round(us, 2), "tflops_per_s": round(flops / us / 1e6, 1),
                      "of_2500_tflops": round(flops / us / 1e6 / 2500.0, 4)}), flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime (timing on our stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
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

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ev, stream) == 0

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        assert rc == 0, rc
        return float(ms.value)

    def destroy(self, arr):
        for ev in arr:
            self.hip.hipEventDestroy(ev)


def expert_bytes(cfg: dict) -> tuple:
    """(gate/up, down) bytes of one routed expert: codes, block scales and
    the fp32 global scale (NVFP4) or the bf16 matrices."""
    H, I = cfg["H"], cfg["I"]
    if cfg["experts"] == "nvfp4":
        return 2 * I * H // 2 + 2 * I * H // 16 + 4, H * I // 2 + H * I // 16 + 4
    return 2 * I * H * 2, H * I * 2


def shared_bytes(cfg: dict, nvfp4: bool = False) -> int:
    H, SI = cfg["H"], cfg["SI"]
    if nvfp4:
        return (2 * SI * H + H * SI) // 2 + (2 * SI * H + H * SI) // 16 + 8
    return (2 * SI * H + H * SI) * 2


def algorithmic_bytes(cfg: dict, U: int, shared: str = "bf16") -> dict:
    """Bytes the method must move per step: router, the touched experts'
    weights (codes, scales, global scales), shared expert, x in, out out.
    shared: "bf16", "nvfp4" or "none" (a precomputed shared output: its
    [M, H] bf16 read instead)."""
    M, H, E = cfg["M"], cfg["H"], cfg["E"]
    gu, dn = expert_bytes(cfg)
    router = E * H * 2
    sh = {"bf16": shared_bytes(cfg), "nvfp4": shared_bytes(cfg, True), "none": M * H * 2}[shared]
    x = M * H * 2
    out = M * H * 2
    return dict(per_expert_gate_up=gu, per_expert_down=dn, router=router, shared=sh, x=x, out=out,
                total=router + U * (gu + dn) + sh + x + out)


def flops(cfg: dict) -> dict:
    """Multiply-add work of one step (2 flops each)."""
    M, H, E, I, SI, k = cfg["M"], cfg["H"], cfg["E"], cfg["I"], cfg["SI"], cfg["top_k"]
    P = M * k
    f = dict(router=2 * M * E * H, gate_up=2 * P * 2 * I * H, down=2 * P * H * I,
             shared_gate_up=2 * M * 2 * SI * H, shared_down=2 * M * H * SI)
    f["total"] = sum(f.values())
    return f


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp: dict, seconds: float) -> dict:
    """The CPU oracle (plain C, double-accumulated, OpenMP over output
    elements) on the host cores: whole steps of the workload for about
    `seconds`, then one thread on a shorter sample."""
    import oracle
    cfg = inp["cfg"]

    def timed(limit):
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.moe_block(inp)
            reps += 1
            el = time.perf_counter() - t0
            if el >= limit or reps >= 1000:
                return reps, el

    threads = oracle.get_threads()
    reps, el = timed(seconds)
    oracle.set_threads(1)
    reps1, el1 = timed(max(1.0, seconds / 3))
    oracle.set_threads(threads)
    return {"value": cfg["M"] * reps / el, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{reps} full steps of {cfg['name']} ({cfg['M']} tokens each, own routing, "
                      f"all stages) on {threads} host threads, {el:.1f} s",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "ms_per_step": round(1e3 * el / reps, 3),
            "single_thread": {"value": cfg["M"] * reps1 / el1, "unit": "tokens/s",
                              "ms_per_step": round(1e3 * el1 / reps1, 3),
                              "sample": f"{reps1} full steps on 1 thread, {el1:.1f} s"}}


class Workload:
    """Device copies of one workload's inputs, rotated over L layer copies,
    and the C-ABI argument tuples of one call per layer."""

    def __init__(self, fm, synth, torch, cfg_idx, path, layers, M=None):
        self.fm, self.torch, self.path = fm, torch, path
        inp = synth.make_inputs(cfg_idx, M=M)
        cfg = self.cfg = dict(inp["cfg"])
        self.M, self.H, self.E = cfg["M"], cfg["H"], cfg["E"]
        self.I, self.SI, self.k = cfg["I"], cfg["SI"], cfg["top_k"]
        self.nvfp4 = cfg["experts"] == "nvfp4"
        dev = self.dev = torch.device("cuda", 0)
        self.keys = ["w13", "s13", "a13", "w2", "s2", "a2"] if self.nvfp4 else ["bw13", "bw2"]
        base = {kk: self.up(inp[kk]) for kk in self.keys + ["router", "sgu", "sdown"]}
        if path in ("nv_shared", "nv_shared_grouped"):  # an NVFP4 shared expert of the same shape
            for kk, v in synth.nvfp4_experts(7, 1, self.H, self.SI).items():
                base["sh_" + kk] = self.up(v)
        self.per_layer = sum(v.numel() * v.element_size() for v in base.values())
        self.x = self.up(inp["x"])
        self.inp = inp
        if path == "sh_in":
            self.sh_buf = self.up(synth.bf16_normal(5, 1, (self.M, self.H), 0.5))
        if path == "ll":
            lli = synth.make_ll_inputs(1, self.M, self.H)
            self.la, self.lr, self.lw = (self.up(lli["attn_out"]), self.up(lli["residual"]),
                                         self.up(lli["ln_weight"]))
            self.eps = lli["eps"]
            self.lres = torch.empty((self.M, self.H), dtype=torch.int16, device=dev)
            self.lxn = torch.empty((self.M, self.H), dtype=torch.int16, device=dev)
        self.out = torch.empty((self.M, self.H), dtype=torch.int16, device=dev)
        self.ws = fm.make_workspace(self.M, self.H, self.E, self.I, self.SI, self.k)
        self.stream = torch.cuda.current_stream()
        self.sp = ctypes.c_void_p(self.stream.cuda_stream)
        lib = fm.lib()
        self.fn = {"decode": lib.flint_moe_decode, "grouped": lib.flint_moe_grouped,
                   "bf16_decode": lib.flint_moe_bf16_decode, "ll": lib.flint_moe_ll,
                   "sh_in": lib.flint_moe_decode, "nv_shared": lib.flint_moe_decode,
                   "nv_shared_grouped": lib.flint_moe_grouped,
                   "bf16_grouped": lib.flint_moe_bf16_grouped}[path]
        self.keep = []
        # touched experts of the workload, from one call
        ids = torch.empty((self.M, self.k), dtype=torch.int32, device=dev)
        dbg = fm.MoeDebug(None, None, None, fm._ptr(ids), None, None, None, None, None, None, 0, 0)
        assert self.fn(*self.args(base, dbg)) == 0
        torch.cuda.synchronize()
        self.U = int(np.unique(ids.cpu().numpy()).size)
        gu, dn = expert_bytes(cfg)
        touched = self.U * (gu + dn) + self.E * self.H * 2 + shared_bytes(cfg)
        # reuse distance of a layer's weights above twice the Infinity Cache
        self.L = layers or int(min(24, max(2, int(np.ceil(2 * MALL_BYTES / touched)) + 1)))
        self.lays = [base] + [{kk: v.clone() for kk, v in base.items()} for _ in range(self.L - 1)]
        self.plain = [self.args(lay) for lay in self.lays]

    def up(self, x):
        x = np.ascontiguousarray(x)
        t = self.torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x)
        return t.to(self.dev)

    def args(self, lay, dbg=None):
        fm = self.fm
        if self.nvfp4:
            w = fm.nvfp4_experts_struct(*(lay[kk] for kk in self.keys))
        else:
            w = fm.Bf16Experts(fm._ptr(lay["bw13"]), fm._ptr(lay["bw2"]))
        sh = fm.SharedExpert(fm._ptr(lay["sgu"]), fm._ptr(lay["sdown"]), self.SI)
        if self.path == "sh_in":
            sh = fm.SharedExpert(None, None, 0, fm._ptr(self.sh_buf), None)
        if self.path in ("nv_shared", "nv_shared_grouped"):
            sh = fm.SharedExpert(fm._ptr(lay["sh_w13"]), fm._ptr(lay["sh_w2"]), self.SI, None, None,
                                 fm._ptr(lay["sh_s13"]), fm._ptr(lay["sh_s2"]),
                                 fm._ptr(lay["sh_a13"]), fm._ptr(lay["sh_a2"]))
        self.keep.extend([w, sh, dbg])
        d = ctypes.byref(dbg) if dbg is not None else None
        if self.path == "ll":
            return (fm._ptr(self.la), fm._ptr(self.lr), fm._ptr(self.lw), ctypes.c_float(self.eps),
                    fm._ptr(lay["router"]), ctypes.byref(w), ctypes.byref(sh), self.M, self.H, self.E,
                    self.I, self.k, fm._ptr(self.out), fm._ptr(self.lres), fm._ptr(self.lxn), d,
                    fm._ptr(self.ws), self.ws.numel(), self.sp)
        return (fm._ptr(self.x), fm._ptr(lay["router"]), ctypes.byref(w), ctypes.byref(sh), self.M,
                self.H, self.E, self.I, self.k, fm._ptr(self.out), d, fm._ptr(self.ws), self.ws.numel(),
                self.sp)

    def time_steps(self, steps, warmup) -> float:
        """ms per step: HIP events on the launch stream around `steps`
        back-to-back calls (nothing else queued between them), after
        SETTLE_S seconds of untimed calls (bursts of 32, each synchronised)
        and then `warmup` untimed calls.  An idle GPU runs its first
        milliseconds of work at lower clocks: the headline call measured
        43.8-46.1 us in the first 20 steps after set-up against 41.7-41.9 us
        once settled, and 43.9 us again after 0.5 s idle."""
        torch = self.torch
        t_end = time.perf_counter() + SETTLE_S
        j = 0
        while time.perf_counter() < t_end:
            for _ in range(32):
                assert self.fn(*self.plain[j % self.L]) == 0
                j += 1
            torch.cuda.synchronize()
        for i in range(warmup):
            assert self.fn(*self.plain[i % self.L]) == 0
        torch.cuda.synchronize()
        hev = HipEvents()
        ev = hev.create(2)
        hev.record(ev[0], self.sp)
        for i in range(steps):
            self.fn(*self.plain[i % self.L])
        hev.record(ev[1], self.sp)
        torch.cuda.synchronize()
        ms = hev.elapsed_ms(ev[0], ev[1]) / steps
        hev.destroy(ev)
        return ms

    def time_stages(self, steps) -> np.ndarray:
        """Per-stage ms: the same calls with HIP events before every stage
        (the grouped path's kernels; the decode path is one kernel)."""
        torch, fm = self.torch, self.fm
        hev = HipEvents()
        nev = fm.FLINT_STAGE_EVENTS
        evs = [hev.create(nev) for _ in range(steps)]
        staged = []
        for i in range(steps):
            d = fm.MoeDebug(None, None, None, None, None, None, None, None, None,
                            ctypes.cast(evs[i], ctypes.POINTER(ctypes.c_void_p)), 0, 0)
            staged.append(self.args(self.lays[i % self.L], d))
        torch.cuda.synchronize()
        for i in range(steps):
            self.fn(*staged[i])
        torch.cuda.synchronize()
        st = np.zeros(nev - 1)
        for i in range(steps):
            for s in range(nev - 1):
                st[s] += hev.elapsed_ms(evs[i][s], evs[i][s + 1])
        for e in evs:
            hev.destroy(e)
        return st / steps

    def free(self):
        del self.lays, self.plain, self.keep
        self.torch.cuda.empty_cache()


# The decode entry points run the one-kernel decode path up to this many
# tokens and the grouped chain on the skinny GEMMs past it.
DECODE_KERNEL_MAX_M = 16


def decode_entry(w: Workload, ms: float, shared: str = "bf16") -> dict:
    cfg = w.cfg
    skinny_path = cfg["M"] > DECODE_KERNEL_MAX_M
    nb = algorithmic_bytes(cfg, w.U, shared)
    gbps = nb["total"] / (ms * 1e-3) / 1e9
    e = {"workload": cfg["name"], "M": cfg["M"], "E": cfg["E"], "experts": cfg["experts"],
         "touched_experts": w.U, "layers_rotated": w.L, "us_per_call": round(ms * 1e3, 3),
         "tokens_per_s": round(cfg["M"] / (ms * 1e-3), 1),
         "roofline": {"kernel": "decode_kernel" if skinny_path is False else "skinny chain",
                      "bound": "hbm", "achieved": round(gbps, 1),
                      "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                      "bytes_per_launch": nb["total"], "avg_launch_us": round(ms * 1e3, 3)}}
    if skinny_path:
        # past 16 tokens the decode entry points run the grouped chain with
        # the skinny MFMA GEMMs: whole-call bytes over the call's time above,
        # and the products against the bf16 matrix-core peak here
        fl = flops(cfg)["total"]
        tf = fl / (ms * 1e-3) / 1e12
        e["path"] = "router + top-k + skinny gate/up + skinny down + combine"
        e["mfma_roofline"] = {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 5),
                              "flops_per_launch": fl}
    return e


def grouped_entry(w: Workload, ms: float, st: np.ndarray, fm) -> dict:
    cfg = w.cfg
    fl = flops(cfg)
    gemm_ms = {"gate_up": st[3], "down": st[4], "shared_gate_up": st[2], "shared_down": st[5]}
    kern = "routed_gemm_kernel<gate/up>" if w.nvfp4 else "gemm_kernel<bf16 routed gate/up>"
    tfl = fl["gate_up"] / (st[3] * 1e-3) / 1e12
    return {
        "workload": cfg["name"] if w.nvfp4 else "bf16_grouped_m4096_e128", "M": cfg["M"],
        "experts": cfg["experts"], "ms_per_step": round(ms, 4),
        "tokens_per_s": round(cfg["M"] / (ms * 1e-3), 1),
        "tflops_per_s": round(fl["total"] / (ms * 1e-3) / 1e12, 1),
        "mfma_frac": round(fl["total"] / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "stage_us": {n: round(float(t) * 1e3, 2) for n, t in zip(fm.STAGES, st)},
        "gemm_tflops": {n: round(fl[n] / (gemm_ms[n] * 1e-3) / 1e12, 1) for n in gemm_ms},
        "roofline": {"kernel": kern, "bound": "mfma", "achieved": round(tfl, 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tfl / BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("routed_gemm_kernel_gate_up_m4096_hbm_traffic",
                                                 "routed_gemm_kernel", cfg["name"]) if w.nvfp4 else None,
                     "flops_per_launch": fl["gate_up"], "avg_launch_us": round(st[3] * 1e3, 2),
                     "timing": "HIP events before and after the stage on the launch stream"},
    }


def main():
    global SETTLE_S
    a = _args()
    SETTLE_S = max(0.0, a.settle)
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {a.gpus} requested): the Flint MoE "
              "block here runs on a single MI355X; sharding across GPUs is a design note, not a "
              "measured path.", file=sys.stderr)
        sys.exit(2)

    import torch

    if a.mfma_calibration:
        mfma_calibration(torch, a.mfma_calibration)
        return
    if a.copy_calibration:
        copy_calibration(torch, a.copy_calibration)
        return

    import nvfp4_w4a16_routed_amd as fm
    import synth

    fm.lib()
    if a.grouped_only:
        wg = Workload(fm, synth, torch, 4, "grouped", 2)
        msg = wg.time_steps(a.grouped_steps, 3)
        print(json.dumps({"grouped": grouped_entry(wg, msg, wg.time_stages(a.grouped_steps), fm)}),
              flush=True)
        return
    cfg_idx = a.config
    path = "bf16_decode" if synth.CONFIGS[cfg_idx]["experts"] == "bf16" else "decode"
    w = Workload(fm, synth, torch, cfg_idx, path, a.layers)
    ms = w.time_steps(a.steps, a.warmup)
    cfg = w.cfg
    M = cfg["M"]
    head = decode_entry(w, ms)
    roof = dict(head["roofline"])
    roof["traffic"] = measured_traffic(f"decode_kernel_{cfg['name']}_hbm_traffic", "decode_kernel",
                                       cfg["name"])
    roof["timing"] = ("HIP events on the launch stream around the timed back-to-back launches "
                      f"(one kernel per call), after {SETTLE_S:g} s of untimed calls and the "
                      "warm-up steps")
    res = {
        "metric": METRIC,
        "value": round(M / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 x nvfp4 (fp32 accumulate)" if cfg["experts"] == "nvfp4" else "bf16",
        "data": "synthetic (seeded; random weights of the Flint MoE shapes)",
        "config": {"workload": cfg["name"], "M": M, "H": cfg["H"], "E": cfg["E"], "I": cfg["I"],
                   "SI": cfg["SI"], "top_k": cfg["top_k"], "experts": cfg["experts"],
                   "touched_experts": w.U, "layers_rotated": w.L,
                   "weights_bytes_per_layer": w.per_layer},
        "hbm_gbps": roof["achieved"],
        "hbm_frac": roof["frac"],
        "algorithmic_bytes_per_step": roof["bytes_per_launch"],
        "roofline": roof,
    }
    w.free()
    if not a.no_cpu_baseline:
        inp = synth.make_inputs(cfg_idx)
        res["cpu_baseline"] = cpu_baseline(inp, a.cpu_seconds)
        del inp
    if not a.headline_only:
        # the other decode workloads
        res["configs"] = {}
        for ci in (0, 1, 2, 3):
            if ci == cfg_idx:
                continue
            p = "bf16_decode" if synth.CONFIGS[ci]["experts"] == "bf16" else "decode"
            wc = Workload(fm, synth, torch, ci, p, a.layers)
            res["configs"][wc.cfg["name"]] = decode_entry(wc, wc.time_steps(a.steps, a.warmup))
            wc.free()
        if path == "decode":
            # flint_moe_ll: the residual add + RMS norm formed inside the
            # decode kernel, same workload and protocol
            wl = Workload(fm, synth, torch, cfg_idx, "ll", a.layers)
            e = decode_entry(wl, wl.time_steps(a.steps, a.warmup))
            e.update(entry="flint_moe_ll", decode_us_per_call=round(ms * 1e3, 3))
            res["ll"] = e
            wl.free()
            # a precomputed shared output read by the kernel's combine
            wsh = Workload(fm, synth, torch, cfg_idx, "sh_in", a.layers)
            e = decode_entry(wsh, wsh.time_steps(a.steps, a.warmup), shared="none")
            e.update(entry="flint_moe_decode + sh_in")
            res["shared_output"] = e
            wsh.free()
            # an NVFP4 shared expert in the decode kernel
            wnv = Workload(fm, synth, torch, cfg_idx, "nv_shared", a.layers)
            e = decode_entry(wnv, wnv.time_steps(a.steps, a.warmup), shared="nvfp4")
            e.update(entry="flint_moe_decode + NVFP4 shared expert")
            res["nvfp4_shared"] = e
            wnv.free()
    if not a.no_grouped and not a.headline_only:
        gs = a.grouped_steps
        wg = Workload(fm, synth, torch, 4, "grouped", 2)
        msg = wg.time_steps(gs, 3)
        res["grouped"] = grouped_entry(wg, msg, wg.time_stages(gs), fm)
        wg.free()
        wn = Workload(fm, synth, torch, 4, "nv_shared_grouped", 2)
        res["grouped"]["nvfp4_shared_ms_per_step"] = round(wn.time_steps(gs, 3), 4)
        wn.free()
        wb = Workload(fm, synth, torch, 3, "bf16_grouped", 2, M=4096)
        msb = wb.time_steps(gs, 3)
        res["bf16_grouped"] = grouped_entry(wb, msb, wb.time_stages(gs), fm)
        wb.free()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
