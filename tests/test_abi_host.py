"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/flint_moe.h declares, and rejects bad arguments with
the documented status codes before queueing any GPU work."""
import ctypes
import os
import re

import pytest

import nvfp4_w4a16_routed_amd as fm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flint_moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(flint_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(fm.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = fm.lib()
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings():
    L = fm.lib()
    for st in (0, -1, -2, -3, -4, -5):
        assert L.flint_status_str(st).decode()
    assert L.flint_status_str(123).decode() == "unknown status"


def test_workspace_bytes():
    n = fm.flint_moe_workspace_bytes(64, 2048, 128, 768, 768, 8)
    assert n > 0 and n % 256 == 0
    assert fm.flint_moe_workspace_bytes(64, 2048, 128, 768, 768, 8) >= \
        fm.flint_moe_workspace_bytes(8, 2048, 128, 768, 768, 8)
    with pytest.raises(fm.FlintError):
        fm.flint_moe_workspace_bytes(8, 2048, 300, 768, 768, 8)  # E > 256
    with pytest.raises(fm.FlintError):
        fm.flint_moe_workspace_bytes(8, 2048, 8, 768, 768, 9)    # top_k > E


def test_decode_workspaces_fit_the_noalloc_scratch():
    # flint_moe_decode_noalloc's scratch (5 MiB, include/flint_moe.h) holds
    # the workspace of every size the decode entry points accept; the
    # largest are at M * top_k = 512 with E = 256.
    for M, k in ((64, 8), (32, 16), (16, 32), (8, 64)):
        assert fm.flint_moe_workspace_bytes(M, 2048, 256, 768, 768, k) <= 5 << 20, (M, k)


# Fake, never-dereferenced device addresses: every case below must be
# rejected by host validation before anything is queued.
A = ctypes.c_void_p(0x10000)
MIS = ctypes.c_void_p(0x10008)


def _experts(ptr=A):
    return fm.NvFp4Experts(ptr, ptr, ptr, ptr, ptr, ptr)


def _decode(x=A, router=A, w=None, shared=None, M=8, H=2048, E=128, I=768, k=8, out=A,
            dbg=None, ws=A, ws_bytes=1 << 30):
    w = _experts() if w is None else w
    return fm.lib().flint_moe_decode(x, router, ctypes.byref(w),
                                     ctypes.byref(shared) if shared else None, M, H, E, I, k,
                                     out, ctypes.byref(dbg) if dbg else None, ws, ws_bytes, None)


def test_decode_rejects_bad_arguments():
    assert _decode(x=None) == -1
    assert _decode(out=None) == -1
    assert _decode(w=fm.NvFp4Experts(A, None, A, A, A, A)) == -1
    assert _decode(ws=None) == -4
    assert _decode(ws_bytes=1024) == -4
    assert _decode(M=65) == -2             # decode is for M <= 64
    assert _decode(k=0) == -2
    assert _decode(E=257) == -2
    assert _decode(k=200, E=256) == -2     # M * top_k beyond the decode plan
    assert _decode(H=1000) == -2
    assert _decode(I=700) == -2
    assert _decode(x=MIS) == -3
    assert _decode(w=_experts(MIS)) == -3
    sh = fm.SharedExpert(A, None, 768)
    assert _decode(shared=sh) == -1
    sh = fm.SharedExpert(A, A, 700)
    assert _decode(shared=sh) == -2
    sh = fm.SharedExpert(None, None, 0, MIS, None)
    assert _decode(shared=sh) == -3        # precomputed shared output, misaligned
    sh = fm.SharedExpert(A, A, 768, None, None, A, None, A, A)
    assert _decode(shared=sh) == -1        # an NVFP4 shared expert without its down scales
    sh = fm.SharedExpert(A, A, 768, None, None, MIS, A, A, A)
    assert _decode(shared=sh) == -3
    sh = fm.SharedExpert(A, A, 512, None, None, A, A, A, A)
    assert _decode(shared=sh) == -2        # the decode kernel's shared expert is I wide
    sh = fm.SharedExpert(A, A, 768, None, None, A, A, A, A)
    assert _decode(shared=sh, ws_bytes=1024) == -4  # accepted up to the workspace check
    dbg = fm.MoeDebug(A, None, None, None, None, None, None, None, None)
    assert _decode(dbg=dbg) == -1          # forced ids without weights
    assert _decode(M=0, x=None) == 0       # empty batch: valid no-op


def _ll(a=A, r=A, lw=A, eps=1e-6, M=8, H=2048, res=A, xn=A, ws_bytes=1 << 30):
    w = _experts()
    return fm.lib().flint_moe_ll(a, r, lw, eps, A, ctypes.byref(w), None, M, H, 128, 768, 8, A, res,
                                 xn, None, A, ws_bytes, None)


def test_ll_rejects_bad_arguments():
    for kw in (dict(a=None), dict(r=None), dict(lw=None), dict(res=None), dict(xn=None)):
        assert _ll(**kw) == -1, kw
    assert _ll(eps=-1.0) == -2
    assert _ll(eps=float("nan")) == -2
    assert _ll(M=65) == -2                 # the decode block's limit
    assert _ll(H=1000) == -2
    assert _ll(a=MIS) == -3
    assert _ll(xn=MIS) == -3
    assert _ll(ws_bytes=1024) == -4        # rejected before the norm is queued
    assert _ll(M=0, a=None) == 0           # empty batch: valid no-op


def test_bf16_decode_and_grouped_reject_bad_arguments():
    L = fm.lib()
    w = fm.Bf16Experts(A, None)
    assert L.flint_moe_bf16_decode(A, A, ctypes.byref(w), None, 8, 2048, 128, 768, 8, A, None, A,
                                   1 << 30, None) == -1
    w = fm.Bf16Experts(MIS, A)
    assert L.flint_moe_bf16_decode(A, A, ctypes.byref(w), None, 8, 2048, 128, 768, 8, A, None, A,
                                   1 << 30, None) == -3
    w = fm.Bf16Experts(A, A)
    sh = fm.SharedExpert(A, A, 768, None, None, A, A, A, A)  # NVFP4 shared: NVFP4 experts only
    assert L.flint_moe_bf16_decode(A, A, ctypes.byref(w), ctypes.byref(sh), 8, 2048, 128, 768, 8, A,
                                   None, A, 1 << 30, None) == -2


def _grouped(M=8, H=2048, E=128, I=768, k=8, shared=None, ws_bytes=1 << 62):
    w = _experts()
    return fm.lib().flint_moe_grouped(A, A, ctypes.byref(w), ctypes.byref(shared) if shared else None,
                                      M, H, E, I, k, A, None, A, ws_bytes, None)


def test_grouped_rejects_sizes_past_its_addressing():
    # x, act and sact are read through 32-bit buffer offsets: each must stay
    # below 2^31 bytes (act = M * top_k * I * 2 bytes reaches it first)
    assert _grouped(M=174762, k=8, I=768, ws_bytes=10) == -4   # act just below 2^31 bytes: accepted
    assert _grouped(M=174763, k=8, I=768) == -2                # act past 2^31 bytes
    assert _grouped(M=(1 << 30) // 2048, H=2048, k=1, I=64) == -2  # x = 2^31 bytes
    assert _grouped(M=(1 << 30) // 2048 - 1, H=2048, k=1, I=64, ws_bytes=10) == -4
    sh = fm.SharedExpert(A, A, 8192)
    assert _grouped(M=(1 << 30) // 8192, H=128, k=1, I=64, shared=sh) == -2  # sact = 2^31 bytes


def test_grouped_rejects_bad_shared_widths():
    assert _grouped(shared=fm.SharedExpert(A, A, 0)) == -2     # a shared expert of width 0
    assert _grouped(shared=fm.SharedExpert(A, A, -64)) == -2
    assert _grouped(shared=fm.SharedExpert(A, A, 96)) == -2    # not a multiple of 64
    assert _grouped(shared=fm.SharedExpert(A, A, 8256)) == -2
    assert _grouped(shared=fm.SharedExpert(A, None, 768)) == -1
    assert _grouped(shared=fm.SharedExpert(A, A, 768), ws_bytes=10) == -4  # the sizes pass
    assert _grouped(M=0) == 0


def test_wait_errors_rejects_bad_arguments():
    L = fm.lib()
    assert L.flint_moe_wait_errors(A, 1 << 20, None, None) == -1
    assert L.flint_moe_wait_errors(A, 16, A, None) == -4
    assert L.flint_moe_wait_errors(MIS, 1 << 20, A, None) == -3


def test_topk_route_dequant_reject_bad_arguments():
    L = fm.lib()
    assert L.flint_moe_topk(A, 4, 300, 8, A, A, None, None) == -2
    assert L.flint_moe_topk(A, 4, 16, 17, A, A, None, None) == -2
    assert L.flint_moe_topk(None, 4, 16, 8, A, A, None, None) == -1
    assert L.flint_moe_topk(MIS, 4, 16, 8, A, A, None, None) == -3
    assert L.flint_moe_topk(None, 0, 16, 8, None, None, None, None) == 0
    assert L.flint_moe_route(A, A, 4, 1000, 16, 8, None, A, A, A, 1 << 30, None) == -2
    assert L.flint_moe_route(A, A, 4, 2048, 16, 8, None, A, A, None, 1 << 30, None) == -4
    assert L.flint_moe_route(A, A, 4, 2048, 16, 8, None, A, A, A, 64, None) == -4
    assert L.flint_nvfp4_dequant(A, A, 4, 33, A, None) == -2
    assert L.flint_nvfp4_dequant(None, A, 4, 32, A, None) == -1
    assert L.flint_nvfp4_dequant(A, MIS, 4, 32, A, None) == -3
    assert L.flint_moe_workspace_init(None, 1 << 20, None) == -1
    assert L.flint_moe_workspace_init(A, 16, None) == -4


def _noalloc(x=A, router=A, w=None, shared=None, M=8, H=2048, E=128, I=768, k=8, out=A, dbg=None):
    w = _experts() if w is None else w
    return fm.lib().flint_moe_decode_noalloc(x, router, ctypes.byref(w),
                                             ctypes.byref(shared) if shared else None, M, H, E, I, k,
                                             out, ctypes.byref(dbg) if dbg else None, None)


def test_decode_noalloc_rejects_bad_arguments():
    assert _noalloc(x=None) == -1
    assert _noalloc(out=None) == -1
    assert _noalloc(w=fm.NvFp4Experts(A, None, A, A, A, A)) == -1
    assert _noalloc(M=65) == -2
    assert _noalloc(k=200, E=256) == -2
    assert _noalloc(H=1000) == -2
    assert _noalloc(x=MIS) == -3
    assert _noalloc(shared=fm.SharedExpert(A, A, 700)) == -2
    assert _noalloc(M=0, x=None) == 0


def test_bf16_grouped_rejects_bad_arguments():
    L = fm.lib()

    def call(w, M=8, H=2048, I=768, k=8, shared=None, ws_bytes=1 << 62):
        return L.flint_moe_bf16_grouped(A, A, ctypes.byref(w), ctypes.byref(shared) if shared else None,
                                        M, H, 128, I, k, A, None, A, ws_bytes, None)

    assert call(fm.Bf16Experts(A, None)) == -1
    assert call(fm.Bf16Experts(MIS, A)) == -3
    assert call(fm.Bf16Experts(A, A), H=1000) == -2
    assert call(fm.Bf16Experts(A, A), M=174763) == -2         # act past 2^31 bytes
    assert call(fm.Bf16Experts(A, A), shared=fm.SharedExpert(A, A, 0)) == -2
    assert call(fm.Bf16Experts(A, A), ws_bytes=10) == -4
    assert call(fm.Bf16Experts(None, None), M=0) == 0
