"""The decode kernel's bounded waits report when they give up, through the C
ABI: a test hook makes one wait target a word that nothing sets, with a
small poll limit, so that wait gives up while every kernel still ends
normally; flint_moe_wait_errors must then return its bit, and the next
ordinary call on the same workspace must be correct with no error.  Also:
decode calls on two streams (each with its own workspace) are ordered by the
library and both match the oracle."""
import numpy as np
import pytest
import torch

import synth
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

fm = None


@pytest.fixture(scope="module", autouse=True)
def _binding():
    global fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_w4a16_routed_amd as m
    m.lib()
    fm = m
    yield


def _errors(ws):
    e = fm.flint_moe_wait_errors(ws)
    torch.cuda.synchronize()
    return int(e.item())


def test_wait_probe_is_reported_and_cleared():
    print("wait errors: probe, then an ordinary call", flush=True)
    inp = synth.make_small(901, M=5, H=256, E=16, I=128, SI=128, top_k=4, router_std=0.3)
    cfg = inp["cfg"]
    M, H, E, I, SI, k = cfg["M"], cfg["H"], cfg["E"], cfg["I"], cfg["SI"], cfg["top_k"]
    ws = fm.make_workspace(M, H, E, I, SI, k)
    d = G.device_inputs(inp)
    G.run_block(fm, inp, "decode", ws=ws)
    assert _errors(ws) == 0
    # the probe's wait gives up after 64 polls; the call still completes
    out = fm.flint_moe_decode(d["x"], d["router"], G.experts_of(d), G.shared_of(d), k, ws,
                              debug=dict(wait_polls=64, wait_probe=1))
    torch.cuda.synchronize()
    assert out.shape == (M, H)
    err = _errors(ws)
    print(f"  error word after the probe: {err:#x}", flush=True)
    assert err & 64, err
    assert _errors(ws) == 0  # the query cleared it
    # an ordinary call on the same workspace is correct and reports nothing
    r = G.run_block(fm, inp, "decode", ws=ws)
    G.stagewise(inp, r, lambda *a: print(*a, flush=True))
    assert _errors(ws) == 0


def test_decode_on_two_streams():
    print("decode on two streams", flush=True)
    inp = synth.make_small(902, M=8, H=512, E=32, I=256, SI=256, top_k=8, router_std=0.3)
    cfg = inp["cfg"]
    M, H, E, I, SI, k = cfg["M"], cfg["H"], cfg["E"], cfg["I"], cfg["SI"], cfg["top_k"]
    d = G.device_inputs(inp)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [fm.make_workspace(M, H, E, I, SI, k) for _ in streams]
    torch.cuda.synchronize()
    outs = []
    for it in range(6):
        i = it % 2
        with torch.cuda.stream(streams[i]):
            outs.append(fm.flint_moe_decode(d["x"], d["router"], G.experts_of(d), G.shared_of(d),
                                            k, wss[i], stream=streams[i]))
    torch.cuda.synchronize()
    ref = G.run_block(fm, inp, "decode")
    G.stagewise(inp, ref, lambda *a: print(*a, flush=True))
    for o in outs:
        assert np.array_equal(G.host(o), ref["out"])
    for ws in wss:
        assert _errors(ws) == 0
