"""GPU parity of flint_moe_ll: the residual add and RMS norm in front of the
decode block (page "vllm.models.flint.ops.moe", flint_moe_ll and
_add_rms_norm), through the C ABI, against the CPU oracle.

residual' is bit-exact; xn is within one bf16 ulp of the oracle's exactly
rounded value (the kernel reduces mean(s^2) in fp32); the block's output is
checked end to end on the GPU's own xn, as the decode tests do.
"""
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


@pytest.mark.parametrize("seed,M", [(11, 8), (12, 1), (13, 37), (14, 64)])
def test_ll_matches_oracle(seed, M):
    print(f"flint_moe_ll seed={seed} M={M}", flush=True)
    inp = synth.make_inputs(1, M=M)
    cfg = inp["cfg"]
    H, E, I, SI, k = cfg["H"], cfg["E"], cfg["I"], cfg["SI"], cfg["top_k"]
    ll = synth.make_ll_inputs(seed, M, H)
    d = G.device_inputs(inp)
    ws = fm.make_workspace(M, H, E, I, SI, k)
    dbg = dict(ids_out=torch.empty((M, k), dtype=torch.int32, device="cuda"))
    out, res, xn = fm.flint_moe_ll(G.dev(ll["attn_out"]), G.dev(ll["residual"]), G.dev(ll["ln_weight"]),
                                   ll["eps"], d["router"], G.experts_of(d), G.shared_of(d), k, ws,
                                   debug=dbg)
    torch.cuda.synchronize()
    res_ref, xn_ref = oracle.add_rms_norm(ll["attn_out"], ll["residual"], ll["ln_weight"], ll["eps"])
    assert np.array_equal(G.host(res).view(np.uint16), res_ref)
    xg = G.host(xn).view(np.uint16)
    err = np.abs(G.bf(xg) - G.bf(xn_ref))
    assert np.all(err <= G.ulp_bf16(G.bf(xn_ref))), "xn beyond one bf16 ulp"
    print(f"  xn bit-exact {np.mean(xg == xn_ref):.4f}", flush=True)
    # the block on the GPU's xn
    inp2 = dict(inp)
    inp2["x"] = xg
    full = oracle.moe_block(inp2)
    ids = G.host(dbg["ids_out"])
    same = np.all(full["ids"] == ids, axis=1)
    ulps = G.end_to_end_ulps(G.host(out), full, k, rows=same)
    assert ulps.size == 0 or ulps.max() <= 2.0
    print(f"  tokens {M}, near-tie flips {int((~same).sum())}, max ulp(m) {ulps.max() if ulps.size else 0:.3f}",
          flush=True)
