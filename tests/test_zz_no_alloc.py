"""flint_moe_decode_noalloc (the decode block on the library's own scratch,
no workspace and no allocation) through the C ABI: its output and every
exported intermediate are bit-identical to flint_moe_decode's on the same
inputs, over two calls in a row (the second with fewer tokens and a smaller
expert set), and its stages match the oracle as in the other parity tests."""
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


def _debug(M, E, k, I, H, SI):
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device="cuda")
    d = dict(logits_out=z((M, E), torch.int16), ids_out=z((M, k), torch.int32),
             tw_out=z((M, k), torch.float32), act_out=z((M * k, I), torch.int16),
             y_out=z((M * k, H), torch.int16))
    if SI:
        d.update(sact_out=z((M, SI), torch.int16), sh_out=z((M, H), torch.int16))
    return d


def test_noalloc_matches_decode_on_two_calls():
    cases = [# the largest decode workspace (M * top_k = 512, E = 256: 4.28 MiB of the 5 MiB)
             synth.make_small(991, M=64, H=2048, E=256, I=768, SI=768, top_k=8, router_std=0.3),
             synth.make_small(989, M=40, H=512, E=16, I=256, SI=256, top_k=4, router_std=0.3),
             # (M > 16: the grouped chain on the skinny GEMMs, shared expert inline)
             synth.make_inputs(1),  # M = 8, E = 128, H = 2048, I = 768, k = 8
             synth.make_small(990, M=3, H=2048, E=32, I=768, SI=768, top_k=4, router_std=0.3)]
    for inp in cases:
        cfg = inp["cfg"]
        M, H, E, I, SI, k = cfg["M"], cfg["H"], cfg["E"], cfg["I"], cfg["SI"], cfg["top_k"]
        print(f"noalloc vs decode: {cfg['name']} M={M} E={E} k={k}", flush=True)
        d = G.device_inputs(inp)
        ws = fm.make_workspace(M, H, E, I, SI, k)
        out_a = torch.zeros((M, H), dtype=torch.int16, device="cuda")
        out_b = torch.zeros((M, H), dtype=torch.int16, device="cuda")
        dbg_a, dbg_b = _debug(M, E, k, I, H, SI), _debug(M, E, k, I, H, SI)
        fm.flint_moe_decode(d["x"], d["router"], G.experts_of(d), G.shared_of(d), k, ws, out=out_a,
                            debug=dbg_a)
        fm.flint_moe_decode_noalloc(d["x"], d["router"], G.experts_of(d), G.shared_of(d), k,
                                    out=out_b, debug=dbg_b)
        err = fm.flint_moe_wait_errors(None)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert np.array_equal(G.host(out_a), G.host(out_b))
        for key in dbg_a:
            assert np.array_equal(G.host(dbg_a[key]), G.host(dbg_b[key])), key
        r = {kk[:-4]: G.host(v) for kk, v in dbg_b.items()}
        r["out"] = G.host(out_b)
        G.stagewise(inp, r, lambda *a: print(*a, flush=True), extra=dict(path="decode_noalloc"))
