"""A precomputed shared-expert output (page "vllm.models.flint.ops.moe",
flint_moe's shared_output / shared_ready), through the C ABI: with the
shared output the block computed itself passed back in, with or without a
ready event recorded on another stream, the block's output is bit-identical
to the call that computed the shared expert (decode and grouped paths)."""
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


@pytest.mark.parametrize("path,M", [("decode", 7), ("decode", 64), ("grouped", 300)])
def test_precomputed_shared_output(path, M):
    print(f"shared_output path={path} M={M}", flush=True)
    inp = synth.make_small(801 + M, M=M, H=512, E=16, I=256, SI=256, top_k=4, router_std=0.3)
    cfg = inp["cfg"]
    H, E, I, SI, k = cfg["H"], cfg["E"], cfg["I"], cfg["SI"], cfg["top_k"]
    ref = G.run_block(fm, inp, path)
    d = G.device_inputs(inp)
    fn = {"decode": fm.flint_moe_decode, "grouped": fm.flint_moe_grouped}[path]
    ws = fm.make_workspace(M, H, E, I, SI, k)
    # the shared output produced on a side stream, signalled by an event
    side = torch.cuda.Stream()
    ev = G.hip_events(1)
    with torch.cuda.stream(side):
        sh = G.dev(ref["sh"])
        G.hip_record(ev[0], side)
    out1 = fn(d["x"], d["router"], G.experts_of(d), dict(sh_in=sh, sh_ready=ev[0]), k, ws)
    torch.cuda.synchronize()
    assert np.array_equal(G.host(out1), ref["out"])
    # and with no event (the output is already complete)
    out2 = fn(d["x"], d["router"], G.experts_of(d), dict(sh_in=sh, sh_ready=None), k, ws)
    torch.cuda.synchronize()
    assert np.array_equal(G.host(out2), ref["out"])
