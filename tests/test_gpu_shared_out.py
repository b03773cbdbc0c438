"""A precomputed shared-expert output (page "vllm.models.flint.ops.moe",
flint_moe's shared_output / shared_ready), through the C ABI, against the
oracle.

The shared output is an independent seeded bf16 tensor produced on a side
stream by device work that is still running when the call is queued; the
call's stream waits on the event recorded after it.  The output must equal
the oracle's combine of the call's own y and tw with that shared output,
bit for bit, and every routed stage is checked against the oracle as in the
other parity tests."""
import numpy as np
import pytest
import torch

import oracle
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
    oracle.set_threads(16)
    yield


def _busy(stream, tensor):
    """Queues about a millisecond of device work on `stream` that ends by
    writing `tensor` (so a reader that does not wait for it sees old data)."""
    with torch.cuda.stream(stream):
        a = torch.randn((1024, 1024), device="cuda", dtype=torch.float32)
        for _ in range(40):
            a = torch.mm(a, a) * 1e-3
        tensor.add_(a[:1, :1].to(tensor.dtype) * 0)  # depends on the chain


@pytest.mark.parametrize("path,M,E,k,H,I", [("decode", 7, 16, 4, 512, 256),
                                            ("decode", 64, 16, 4, 512, 256),
                                            ("decode", 8, 128, 8, 2048, 768),
                                            ("grouped", 300, 16, 4, 512, 256)])
def test_precomputed_shared_output(path, M, E, k, H, I):
    print(f"shared_output path={path} M={M} E={E} k={k} H={H} I={I}", flush=True)
    inp = synth.make_small(801 + M, M=M, H=H, E=E, I=I, SI=I, top_k=k, router_std=0.3)
    # the block with its own shared expert, every stage against the oracle
    ref = G.run_block(fm, inp, path)
    G.stagewise(inp, ref, lambda *a: print(*a, flush=True))
    # an independent shared output
    sh_bits = synth.bf16_normal(802 + M, 1, (M, H), 0.5)
    d = G.device_inputs(inp)
    fn = {"decode": fm.flint_moe_decode, "grouped": fm.flint_moe_grouped}[path]
    ws = fm.make_workspace(M, H, E, I, 0, k)
    z = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
    for use_event in (True, False):
        dbg = dict(logits_out=z((M, E), torch.int16), ids_out=z((M, k), torch.int32),
                   tw_out=z((M, k), torch.float32), act_out=z((M * k, I), torch.int16),
                   y_out=z((M * k, H), torch.int16))
        sh = torch.zeros((M, H), dtype=torch.int16, device="cuda")
        side = torch.cuda.Stream()
        src = G.dev(sh_bits)
        torch.cuda.synchronize()
        ev = G.hip_events(1)
        if use_event:
            # the producer: a long chain on the side stream, then sh's bits
            _busy(side, sh)
            with torch.cuda.stream(side):
                sh.copy_(src)
            G.hip_record(ev[0], side)
        else:
            sh.copy_(src)
            torch.cuda.synchronize()
        out = fn(d["x"], d["router"], G.experts_of(d),
                 dict(sh_in=sh, sh_ready=ev[0] if use_event else None), k, ws, debug=dbg)
        torch.cuda.synchronize()
        r = {kk[:-4]: G.host(v) for kk, v in dbg.items()}
        r["out"] = G.host(out)
        # routing and routed stages as in the other tests
        G.stagewise_routing(inp, r)
        G.stagewise_routed(inp, r)
        # the rule's last step with the given shared output, bit for bit
        want, _ = oracle.combine(r["y"], r["tw"], sh_bits, k)
        assert np.array_equal(r["out"], want), f"combine with sh_in differs (event={use_event})"
        G.end_to_end(inp, r, lambda *a: print(*a, flush=True), sh_in=sh_bits,
                     extra=dict(path=path + "+sh_in", event=use_event))
