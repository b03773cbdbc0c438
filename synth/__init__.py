"""Seeded synthetic inputs for the Flint routed-expert MoE block.

This module only draws random tensors; it contains none of the block's
arithmetic.  Both the CPU oracle's tests and the HIP path's tests and
benchmark take their inputs from here, so the two sides see the same bytes.

Random numbers come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) used as a counter-based stream:
draw i of stream (seed, tensor_id) is mix64(key + (i + 1) * GOLDEN), with
key = mix64(seed * 2**32 + tensor_id).  Normals use the Box-Muller transform
in float64.  The generator is written here instead of using numpy's or
torch's so the byte stream never changes with a library version.

Rounding of the drawn reals into storage formats (bfloat16, float8_e4m3fn) is
done by torch's CPU casts (round to nearest even); those casts are library
routines, not part of the method.

Workload recipes (shapes fixed by the Flint MoE configuration: hidden size
H = 2048, expert width I = 768, shared-expert width SI = 768, top_k = 8):

* x ~ N(0, 1) rounded to bf16; router ~ N(0, 0.02) bf16.
* NVFP4 experts: every E2M1 code uniform over all 16 codes (so packed bytes
  are uniform over 0..255), one E4M3 scale per 16 consecutive K elements drawn
  uniform on [0.25, 2] and rounded to float8_e4m3fn, per-expert fp32 global
  scales uniform on [0.005, 0.01].
* Shared expert: bf16 N(0, 0.02) weights, [gate; up] of shape [2*SI, H] and
  down of shape [H, SI].
* BF16 experts: w13 [E, 2I, H] and w2 [E, H, I] bf16 N(0, 0.02).
* Zipf routing (decode M=64): expert popularity p_e proportional to
  (e+1)^-1.1; each token's target logits are ln p_e + Gumbel(0, 1), so its
  top-k is a Plackett-Luce draw without replacement; the router is the
  minimum-norm exact solution R^T = X^T (X X^T)^-1 T, rounded to bf16, so the
  router GEMV really produces (nearly) those logits.
"""
from __future__ import annotations

import numpy as np
import torch

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Tensor ids of the streams (stable: never renumber).
T_X, T_ROUTER, T_W13, T_S13, T_A13, T_W2, T_S2, T_A2 = 1, 2, 3, 4, 5, 6, 7, 8
T_SGU, T_SDOWN, T_BW13, T_BW2, T_ZIPF_GUMBEL = 9, 10, 11, 12, 13

H, I, SI, TOP_K = 2048, 768, 768, 8

# The five workloads of the Flint MoE block measured here.
CONFIGS = {
    0: dict(name="decode_m1_e32", M=1, H=H, E=32, I=I, SI=SI, top_k=TOP_K,
            experts="nvfp4", routing="normal"),
    1: dict(name="decode_m8_e128", M=8, H=H, E=128, I=I, SI=SI, top_k=TOP_K,
            experts="nvfp4", routing="normal"),
    2: dict(name="decode_m64_e128_zipf", M=64, H=H, E=128, I=I, SI=SI,
            top_k=TOP_K, experts="nvfp4", routing="zipf"),
    3: dict(name="bf16_decode_m8_e128", M=8, H=H, E=128, I=I, SI=SI,
            top_k=TOP_K, experts="bf16", routing="normal"),
    4: dict(name="grouped_m4096_e128", M=4096, H=H, E=128, I=I, SI=SI,
            top_k=TOP_K, experts="nvfp4", routing="normal"),
}


def _mix64(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def u64_stream(seed: int, tensor_id: int, n: int, start: int = 0) -> np.ndarray:
    """Draws start .. start+n-1 of stream (seed, tensor_id) as uint64."""
    key = _mix64(np.array([(seed << 32) + tensor_id], dtype=np.uint64))[0]
    idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(key + idx * GOLDEN)


def uniform(seed: int, tensor_id: int, n: int, start: int = 0) -> np.ndarray:
    """Doubles in [0, 1) from the top 53 bits of each draw."""
    z = u64_stream(seed, tensor_id, n, start)
    return (z >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def normal(seed: int, tensor_id: int, n: int, std: float = 1.0) -> np.ndarray:
    """Box-Muller normals: pair (2i, 2i+1) of uniforms gives draw i."""
    u = uniform(seed, tensor_id, 2 * n)
    u1 = 1.0 - u[0::2]  # (0, 1]
    u2 = u[1::2]
    return std * np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3_bits(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def random_bytes(seed: int, tensor_id: int, n: int) -> np.ndarray:
    z = u64_stream(seed, tensor_id, (n + 7) // 8)
    return z.view(np.uint8)[:n].copy()


def bf16_normal(seed: int, tensor_id: int, shape, std: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    chunk = 1 << 22
    # Chunked so large expert tensors do not need a float64 copy of the whole
    # tensor; chunk c uses draws [2*c*chunk, 2*(c+1)*chunk) of the stream.
    for c0 in range(0, n, chunk):
        m = min(chunk, n - c0)
        u = uniform(seed, tensor_id, 2 * m, start=2 * c0)
        v = std * np.sqrt(-2.0 * np.log(1.0 - u[0::2])) * np.cos(2.0 * np.pi * u[1::2])
        out[c0:c0 + m] = to_bf16_bits(v)
    return out.reshape(shape)


def nvfp4_experts(seed: int, E: int, H: int, I: int) -> dict:
    """ModelOpt-layout NVFP4 experts: codes, E4M3 block scales, fp32 alphas."""
    w13 = random_bytes(seed, T_W13, E * 2 * I * H // 2).reshape(E, 2 * I, H // 2)
    w2 = random_bytes(seed, T_W2, E * H * I // 2).reshape(E, H, I // 2)
    s13 = to_e4m3_bits(0.25 + 1.75 * uniform(seed, T_S13, E * 2 * I * H // 16))
    s2 = to_e4m3_bits(0.25 + 1.75 * uniform(seed, T_S2, E * H * I // 16))
    a13 = (0.005 + 0.005 * uniform(seed, T_A13, E)).astype(np.float32)
    a2 = (0.005 + 0.005 * uniform(seed, T_A2, E)).astype(np.float32)
    return dict(w13=w13, s13=s13.reshape(E, 2 * I, H // 16), a13=a13,
                w2=w2, s2=s2.reshape(E, H, I // 16), a2=a2)


def zipf_router(seed: int, x_bits: np.ndarray, E: int, s: float = 1.1) -> np.ndarray:
    """Router whose logits on x are ln p_e + Gumbel noise (p_e ~ Zipf(s))."""
    M, Hh = x_bits.shape
    X = bf16_bits_to_f32(x_bits).astype(np.float64)
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    p /= p.sum()
    u = uniform(seed, T_ZIPF_GUMBEL, M * E).reshape(M, E)
    gumbel = -np.log(-np.log(np.clip(u, 1e-300, None)))
    T = np.log(p)[None, :] + gumbel
    # Minimum-norm exact fit: X @ R^T = T with R^T = X^T (X X^T)^-1 T.
    Rt = X.T @ np.linalg.solve(X @ X.T, T)
    return to_bf16_bits(Rt.T.copy())


_MEMO: dict = {}


def _experts_memo(seed: int, kind: str, E: int, Hh: int, Ii: int) -> dict:
    """The routed experts of a workload (NVFP4 or BF16), kept for the last two
    keys so workloads that differ only in M share one draw (callers must not
    write into the arrays)."""
    key = (seed, kind, E, Hh, Ii)
    if key not in _MEMO:
        if kind == "nvfp4":
            w = nvfp4_experts(seed, E, Hh, Ii)
        else:
            w = dict(bw13=bf16_normal(seed, T_BW13, (E, 2 * Ii, Hh), 0.02),
                     bw2=bf16_normal(seed, T_BW2, (E, Hh, Ii), 0.02))
        while len(_MEMO) >= 2:
            _MEMO.pop(next(iter(_MEMO)))
        _MEMO[key] = w
    return dict(_MEMO[key])


def make_inputs(cfg: dict | int, seed: int | None = None, M: int | None = None,
                with_shared: bool = True) -> dict:
    """All inputs of one workload as numpy arrays of storage bits.

    bf16 tensors are uint16 bit patterns, E4M3 scales and packed E2M1 codes are
    uint8, global scales are float32.  `M` overrides the token count (same
    streams, so the first rows of x are shared between M values).
    """
    if isinstance(cfg, int):
        idx = cfg
        cfg = CONFIGS[cfg]
        if seed is None:
            seed = 0xF117 + idx
    assert seed is not None
    M = cfg["M"] if M is None else M
    Hh, E, Ii, SIi = cfg["H"], cfg["E"], cfg["I"], cfg["SI"]
    x = bf16_normal(seed, T_X, (M, Hh), 1.0)
    if cfg.get("routing") == "zipf":
        router = zipf_router(seed, x, E)
    else:
        router = bf16_normal(seed, T_ROUTER, (E, Hh), 0.02)
    d = dict(cfg=dict(cfg, M=M), seed=seed, x=x, router=router)
    d.update(_experts_memo(seed, cfg["experts"], E, Hh, Ii))
    if with_shared and SIi > 0:
        d["sgu"] = bf16_normal(seed, T_SGU, (2 * SIi, Hh), 0.02)
        d["sdown"] = bf16_normal(seed, T_SDOWN, (Hh, SIi), 0.02)
    return d


def make_small(seed: int, M: int, H: int, E: int, I: int, SI: int, top_k: int,
               experts: str = "nvfp4", routing: str = "normal",
               router_std: float = 0.02) -> dict:
    """Same recipe at arbitrary (small) shapes, for parity and oracle tests."""
    cfg = dict(name=f"small_m{M}_h{H}_e{E}_i{I}", M=M, H=H, E=E, I=I, SI=SI,
               top_k=top_k, experts=experts, routing=routing)
    x = bf16_normal(seed, T_X, (M, H), 1.0)
    if routing == "zipf":
        router = zipf_router(seed, x, E)
    else:
        router = bf16_normal(seed, T_ROUTER, (E, H), router_std)
    d = dict(cfg=cfg, seed=seed, x=x, router=router)
    if experts == "nvfp4":
        d.update(nvfp4_experts(seed, E, H, I))
    else:
        d["bw13"] = bf16_normal(seed, T_BW13, (E, 2 * I, H), 0.02)
        d["bw2"] = bf16_normal(seed, T_BW2, (E, H, I), 0.02)
    if SI > 0:
        d["sgu"] = bf16_normal(seed, T_SGU, (2 * SI, H), 0.02)
        d["sdown"] = bf16_normal(seed, T_SDOWN, (H, SI), 0.02)
    return d


def make_ll_inputs(seed: int, M: int, H: int) -> dict:
    """Inputs of the residual-add RMS norm in front of the block: attn_out
    ~ N(0, 1) and residual ~ N(0, 4) as [M, H] bf16 bits, ln_weight = 1 +
    N(0, 0.1) as [H] bf16 bits, eps = 1e-6."""
    attn = bf16_normal(seed, 101, (M, H), 1.0)
    res = bf16_normal(seed, 102, (M, H), 4.0)
    lw = to_bf16_bits(1.0 + bf16_bits_to_f32(bf16_normal(seed, 103, (H,), 0.1)).astype(np.float64))
    return dict(attn_out=attn, residual=res, ln_weight=lw, eps=1e-6)
