"""Python binding of libflint_moe (the MI355X Flint routed-expert MoE block).

Argument marshalling only: every step runs in the HIP kernels of
``libflint_moe.so``; this module passes device pointers, sizes and the
current HIP stream through the C ABI declared in ``include/flint_moe.h`` and
raises ``FlintError`` on a non-zero status.  There is no fallback: if the
library is missing, importing the binding's functions raises.

Tensors are torch tensors on the GPU holding storage bits: bf16 data may be
``torch.bfloat16`` or 16-bit integer tensors of the same bits; packed E2M1
codes and E4M3 scales are ``torch.uint8``; global scales ``torch.float32``;
ids ``torch.int32``; routing weights ``torch.float32``.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libflint_moe.so")

FLINT_OK = 0
STATUS = {0: "FLINT_OK", -1: "FLINT_ERR_NULL", -2: "FLINT_ERR_SHAPE", -3: "FLINT_ERR_ALIGN",
          -4: "FLINT_ERR_WORKSPACE", -5: "FLINT_ERR_HIP"}

# Every symbol include/flint_moe.h declares.
EXPORTS = ("flint_status_str", "flint_last_hip_error", "flint_moe_workspace_bytes",
           "flint_moe_workspace_init", "flint_nvfp4_dequant", "flint_moe_topk",
           "flint_moe_route", "flint_moe_decode", "flint_moe_grouped",
           "flint_moe_bf16_decode", "flint_moe_ll", "flint_moe_wait_errors",
           "flint_moe_decode_noalloc", "flint_moe_bf16_grouped")


class FlintError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = STATUS.get(status, str(status))
        if status == -5:
            msg += f" (hipError {lib().flint_last_hip_error()})"
        super().__init__(f"{fn}: {msg}: {lib().flint_status_str(status).decode()}")


P = ctypes.c_void_p
I32 = ctypes.c_int


class NvFp4Experts(ctypes.Structure):
    _fields_ = [("w13", P), ("s13", P), ("a13", P), ("w2", P), ("s2", P), ("a2", P)]


class Bf16Experts(ctypes.Structure):
    _fields_ = [("w13", P), ("w2", P)]


class SharedExpert(ctypes.Structure):
    _fields_ = [("w_gu", P), ("w_down", P), ("SI", I32), ("sh_in", P), ("sh_ready", P),
                ("s_gu", P), ("s_down", P), ("a_gu", P), ("a_down", P)]


FLINT_STAGE_EVENTS = 8
STAGES = ("route", "pair_lists", "shared_gate_up", "gate_up", "down", "shared_down", "combine")


class MoeDebug(ctypes.Structure):
    _fields_ = [("ids_in", P), ("tw_in", P), ("logits_out", P), ("ids_out", P),
                ("tw_out", P), ("act_out", P), ("y_out", P), ("sact_out", P),
                ("sh_out", P), ("stage_events", ctypes.POINTER(P)), ("wait_polls", I32),
                ("wait_probe", I32)]


# Bits of the word flint_moe_wait_errors returns (include/flint_moe.h).
WAIT_KINDS = {1: "logits", 2: "shared_gate_up", 4: "gate_up", 8: "combine_shared",
              16: "combine_down", 32: "lds", 64: "probe"}


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libflint_moe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m "
                "nvfp4_w4a16_routed_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.flint_status_str.restype = ctypes.c_char_p
        L.flint_status_str.argtypes = [I32]
        L.flint_last_hip_error.restype = I32
        L.flint_last_hip_error.argtypes = []
        L.flint_moe_workspace_bytes.restype = I32
        L.flint_moe_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32,
                                                ctypes.POINTER(ctypes.c_size_t)]
        L.flint_moe_workspace_init.restype = I32
        L.flint_moe_workspace_init.argtypes = [P, ctypes.c_size_t, P]
        L.flint_nvfp4_dequant.restype = I32
        L.flint_nvfp4_dequant.argtypes = [P, P, I32, I32, P, P]
        L.flint_moe_topk.restype = I32
        L.flint_moe_topk.argtypes = [P, I32, I32, I32, P, P, P, P]
        L.flint_moe_route.restype = I32
        L.flint_moe_route.argtypes = [P, P, I32, I32, I32, I32, P, P, P, P, ctypes.c_size_t, P]
        moe_args = [P, P, P, P, I32, I32, I32, I32, I32, P, P, P, ctypes.c_size_t, P]
        for name in ("flint_moe_decode", "flint_moe_grouped", "flint_moe_bf16_decode",
                     "flint_moe_bf16_grouped"):
            fn = getattr(L, name)
            fn.restype = I32
            fn.argtypes = moe_args
        L.flint_moe_decode_noalloc.restype = I32
        L.flint_moe_decode_noalloc.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, P, P, P]
        L.flint_moe_wait_errors.restype = I32
        L.flint_moe_wait_errors.argtypes = [P, ctypes.c_size_t, P, P]
        L.flint_moe_ll.restype = I32
        L.flint_moe_ll.argtypes = [P, P, P, ctypes.c_float, P, P, P, I32, I32, I32, I32, I32, P, P, P,
                                   P, P, ctypes.c_size_t, P]
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, status: int) -> None:
    if status != FLINT_OK:
        raise FlintError(fn, status)


def _new(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


# ------------------------------------------------------------------ ABI

def flint_moe_workspace_bytes(max_M: int, H: int, E: int, I: int, SI: int, top_k: int) -> int:
    n = ctypes.c_size_t(0)
    _check("flint_moe_workspace_bytes",
           lib().flint_moe_workspace_bytes(max_M, H, E, I, SI, top_k, ctypes.byref(n)))
    return int(n.value)


def flint_moe_workspace_init(ws: torch.Tensor, stream=None) -> None:
    _check("flint_moe_workspace_init",
           lib().flint_moe_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def make_workspace(max_M: int, H: int, E: int, I: int, SI: int, top_k: int,
                   device="cuda") -> torch.Tensor:
    """Allocates (with torch) and zero-initialises a workspace."""
    n = flint_moe_workspace_bytes(max_M, H, E, I, SI, top_k)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    flint_moe_workspace_init(ws)
    return ws


def flint_moe_wait_errors(ws, errors=None, stream=None) -> torch.Tensor:
    """Queues a copy of the workspace's wait-error word into `errors` (a
    device int32 tensor of one element, allocated when None) and clears the
    word; returns `errors` (read it after synchronising).  ws=None reads the
    library's own scratch (flint_moe_decode_noalloc) on the current device."""
    if errors is None:
        errors = torch.zeros(1, dtype=torch.int32,
                             device=ws.device if ws is not None else "cuda")
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check("flint_moe_wait_errors",
           lib().flint_moe_wait_errors(_ptr(ws), nbytes, _ptr(errors), _stream(stream)))
    return errors


def flint_nvfp4_dequant(w: torch.Tensor, s: torch.Tensor, out: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    rows, K = w.shape[0], w.shape[1] * 2
    if out is None:
        out = _new((rows, K), torch.int16, w)
    _check("flint_nvfp4_dequant",
           lib().flint_nvfp4_dequant(_ptr(w), _ptr(s), rows, K, _ptr(out), _stream(stream)))
    return out


def flint_moe_topk(logits: torch.Tensor, top_k: int, ids=None, tw=None, scores=None,
                   want_scores: bool = False, stream=None):
    M, E = logits.shape
    ids = _new((M, top_k), torch.int32, logits) if ids is None else ids
    tw = _new((M, top_k), torch.float32, logits) if tw is None else tw
    if want_scores and scores is None:
        scores = _new((M, top_k), torch.float32, logits)
    _check("flint_moe_topk", lib().flint_moe_topk(_ptr(logits), M, E, top_k, _ptr(ids),
                                                  _ptr(tw), _ptr(scores), _stream(stream)))
    return ids, tw, scores


def flint_moe_route(x, router, top_k: int, ws, logits=None, ids=None, tw=None, stream=None):
    M, H = x.shape
    E = router.shape[0]
    ids = _new((M, top_k), torch.int32, x) if ids is None else ids
    tw = _new((M, top_k), torch.float32, x) if tw is None else tw
    _check("flint_moe_route",
           lib().flint_moe_route(_ptr(x), _ptr(router), M, H, E, top_k, _ptr(logits), _ptr(ids),
                                 _ptr(tw), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)))
    return ids, tw


def _shared_struct(shared):
    """shared: (w_gu, w_down), or dict(sh_in=[M, H] tensor, sh_ready=hipEvent_t
    handle or None) for a precomputed shared output, or None."""
    if shared is None:
        return None
    if isinstance(shared, dict) and "sh_in" in shared:
        return SharedExpert(None, None, 0, _ptr(shared["sh_in"]), shared.get("sh_ready"))
    if isinstance(shared, dict):  # NVFP4 shared expert (grouped path)
        return SharedExpert(_ptr(shared["w13"]), _ptr(shared["w2"]), int(shared["w13"].shape[-2]) // 2, None,
                            None, _ptr(shared["s13"]), _ptr(shared["s2"]), _ptr(shared["a13"]),
                            _ptr(shared["a2"]))
    gu, down = shared
    return SharedExpert(_ptr(gu), _ptr(down), int(gu.shape[0]) // 2)


def _debug_struct(debug):
    """debug: dict of tensors named after MoeDebug's pointer fields;
    "stage_events" may hold a ctypes array of FLINT_STAGE_EVENTS hipEvent_t
    handles; "wait_polls" and "wait_probe" are ints (test hooks)."""
    if not debug:
        return None
    vals = [_ptr(debug.get(f)) for f, _ in MoeDebug._fields_[:9]]
    ev = debug.get("stage_events")
    return MoeDebug(*vals, ctypes.cast(ev, ctypes.POINTER(P)) if ev is not None else None,
                    int(debug.get("wait_polls", 0)), int(debug.get("wait_probe", 0)))


def _moe_call(name, wstruct, x, router, shared, I, E, top_k, ws, out, debug, stream):
    M, H = x.shape
    out = _new((M, H), x.dtype, x) if out is None else out
    sh = _shared_struct(shared)
    dbg = _debug_struct(debug)
    fn = getattr(lib(), name)
    st = fn(_ptr(x), _ptr(router), ctypes.byref(wstruct), ctypes.byref(sh) if sh else None,
            M, H, E, I, top_k, _ptr(out), ctypes.byref(dbg) if dbg else None, _ptr(ws),
            ws.numel() * ws.element_size(), _stream(stream))
    _check(name, st)
    return out


def nvfp4_experts_struct(w13, s13, a13, w2, s2, a2) -> NvFp4Experts:
    return NvFp4Experts(*(_ptr(t) for t in (w13, s13, a13, w2, s2, a2)))


def flint_moe_decode(x, router, experts: dict, shared, top_k: int, ws, out=None, debug=None,
                     stream=None):
    """experts: dict w13 [E,2I,H/2] u8, s13 [E,2I,H/16] u8, a13 [E] f32, w2 [E,H,I/2],
    s2 [E,H,I/16], a2 [E]; shared: (w_gu [2SI,H], w_down [H,SI]) or None."""
    E, I = experts["w13"].shape[0], experts["w2"].shape[2] * 2
    st = nvfp4_experts_struct(*(experts[k] for k in ("w13", "s13", "a13", "w2", "s2", "a2")))
    return _moe_call("flint_moe_decode", st, x, router, shared, I, E, top_k, ws, out, debug, stream)


def flint_moe_decode_noalloc(x, router, experts: dict, shared, top_k: int, out=None, debug=None,
                             stream=None):
    """flint_moe_decode on the library's own scratch (no workspace; the
    library allocates nothing).  `out` must be given by callers that cannot
    allocate (when None it is allocated here with torch)."""
    E, I = experts["w13"].shape[0], experts["w2"].shape[2] * 2
    M, H = x.shape
    out = _new((M, H), x.dtype, x) if out is None else out
    st = nvfp4_experts_struct(*(experts[k] for k in ("w13", "s13", "a13", "w2", "s2", "a2")))
    sh = _shared_struct(shared)
    dbg = _debug_struct(debug)
    rc = lib().flint_moe_decode_noalloc(_ptr(x), _ptr(router), ctypes.byref(st),
                                        ctypes.byref(sh) if sh else None, M, H, E, I, top_k, _ptr(out),
                                        ctypes.byref(dbg) if dbg else None, _stream(stream))
    _check("flint_moe_decode_noalloc", rc)
    return out


def flint_moe_ll(attn_out, residual, ln_weight, eps: float, router, experts: dict, shared, top_k: int,
                 ws, out=None, residual_out=None, xn_out=None, debug=None, stream=None):
    """Residual add + RMS norm, then the decode block on the normed rows.
    Returns (out, residual_out, xn_out); outputs are allocated when None."""
    M, H = attn_out.shape
    E, I = experts["w13"].shape[0], experts["w2"].shape[2] * 2
    st = nvfp4_experts_struct(*(experts[k] for k in ("w13", "s13", "a13", "w2", "s2", "a2")))
    out = _new((M, H), attn_out.dtype, attn_out) if out is None else out
    residual_out = _new((M, H), attn_out.dtype, attn_out) if residual_out is None else residual_out
    xn_out = _new((M, H), attn_out.dtype, attn_out) if xn_out is None else xn_out
    sh = _shared_struct(shared)
    dbg = _debug_struct(debug)
    rc = lib().flint_moe_ll(_ptr(attn_out), _ptr(residual), _ptr(ln_weight), float(eps), _ptr(router),
                            ctypes.byref(st), ctypes.byref(sh) if sh else None, M, H, E, I, top_k,
                            _ptr(out), _ptr(residual_out), _ptr(xn_out),
                            ctypes.byref(dbg) if dbg else None, _ptr(ws), ws.numel() * ws.element_size(),
                            _stream(stream))
    _check("flint_moe_ll", rc)
    return out, residual_out, xn_out


def flint_moe_grouped(x, router, experts: dict, shared, top_k: int, ws, out=None, debug=None,
                      stream=None):
    E, I = experts["w13"].shape[0], experts["w2"].shape[2] * 2
    st = nvfp4_experts_struct(*(experts[k] for k in ("w13", "s13", "a13", "w2", "s2", "a2")))
    return _moe_call("flint_moe_grouped", st, x, router, shared, I, E, top_k, ws, out, debug, stream)


def flint_moe_bf16_grouped(x, router, experts: dict, shared, top_k: int, ws, out=None, debug=None,
                           stream=None):
    """experts: dict w13 [E,2I,H] bf16, w2 [E,H,I] bf16; any M."""
    E, I = experts["w13"].shape[0], experts["w2"].shape[2]
    st = Bf16Experts(_ptr(experts["w13"]), _ptr(experts["w2"]))
    return _moe_call("flint_moe_bf16_grouped", st, x, router, shared, I, E, top_k, ws, out, debug,
                     stream)


def flint_moe_bf16_decode(x, router, experts: dict, shared, top_k: int, ws, out=None, debug=None,
                          stream=None):
    """experts: dict w13 [E,2I,H] bf16, w2 [E,H,I] bf16."""
    E, I = experts["w13"].shape[0], experts["w2"].shape[2]
    st = Bf16Experts(_ptr(experts["w13"]), _ptr(experts["w2"]))
    return _moe_call("flint_moe_bf16_decode", st, x, router, shared, I, E, top_k, ws, out, debug,
                     stream)
