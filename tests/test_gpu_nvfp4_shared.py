"""An NVFP4 shared expert on the grouped path (page "vllm.models.flint.ops.moe":
E4M3 block scales and one fp32 global scale per matrix, computed as a routed
expert with E = 1), through the C ABI, against the oracle's routed steps with
one expert that every token selects."""
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


@pytest.mark.parametrize("M,H,SI", [(300, 512, 256), (37, 256, 128), (20, 512, 256)])
def test_grouped_nvfp4_shared_expert(M, H, SI):
    print(f"grouped NVFP4 shared expert M={M} H={H} SI={SI}", flush=True)
    inp = synth.make_small(950 + M, M=M, H=H, E=16, I=SI, SI=0, top_k=4, router_std=0.3)
    cfg = inp["cfg"]
    E, I, k = cfg["E"], cfg["I"], cfg["top_k"]
    shw = synth.nvfp4_experts(951 + M, 1, H, SI)
    d = G.device_inputs(inp)
    shd = {kk: G.dev(v) for kk, v in shw.items()}
    ws = fm.make_workspace(M, H, E, I, SI, k)
    z = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
    dbg = dict(logits_out=z((M, E), torch.int16), ids_out=z((M, k), torch.int32),
               tw_out=z((M, k), torch.float32), act_out=z((M * k, I), torch.int16),
               y_out=z((M * k, H), torch.int16), sact_out=z((M, SI), torch.int16),
               sh_out=z((M, H), torch.int16))
    out = fm.flint_moe_grouped(d["x"], d["router"], G.experts_of(d), shd, k, ws, debug=dbg)
    torch.cuda.synchronize()
    r = {kk[:-4]: G.host(v) for kk, v in dbg.items()}
    r["out"] = G.host(out)
    # the routed experts at these shapes, as in the other parity tests
    G.stagewise_routing(inp, r)
    G.stagewise_routed(inp, r)
    one = np.zeros((M, 1), dtype=np.int32)
    sact = G.host(dbg["sact_out"]).view(np.uint16)
    ref_sact, det = oracle.gate_up(inp["x"], one, 1, shw, SI, want_detail=True)
    G.check_act(sact, ref_sact, det, "nvfp4 shared gate/up")
    sh = G.host(dbg["sh_out"]).view(np.uint16)
    ref_sh, det2 = oracle.down(sact, one, shw, H, want_detail=True)
    G.check_y(sh, ref_sh, det2, "nvfp4 shared down")
    out_c, _ = oracle.combine(G.host(dbg["y_out"]).view(np.uint16), G.host(dbg["tw_out"]), sh, k)
    assert np.array_equal(G.host(out).view(np.uint16), out_c)
    # end to end: the oracle's block with the NVFP4 shared expert's output
    # (its own gate/up and down with one expert every token selects)
    full = oracle.moe_block(inp)
    ref_sact_own = oracle.gate_up(inp["x"], one, 1, shw, SI)
    ref_sh_own = oracle.down(ref_sact_own, one, shw, H)
    full["sh"] = ref_sh_own
    full["out"], full["routed"] = oracle.combine(full["y"], full["tw"], ref_sh_own, k)
    same = np.all(full["ids"] == r["ids"], axis=1)
    ulps = G.end_to_end_ulps(r["out"], full, k, rows=same)
    assert ulps.size == 0 or ulps.max() <= 2.0
    print(f"  near-tie flips {int((~same).sum())}, max ulp(m) {ulps.max() if ulps.size else 0:.3f}",
          flush=True)


def _oracle_nv_shared(x, shw, H, SI):
    """The NVFP4 shared expert under the routed rule, one expert that every
    token selects: (sact, sh) bf16 bits."""
    one = np.zeros((x.shape[0], 1), dtype=np.int32)
    sact = oracle.gate_up(x, one, 1, shw, SI)
    return sact, oracle.down(sact, one, shw, H)


def _check_nv_shared_run(inp, shw, r, label):
    """Stages of a decode run with an NVFP4 shared expert against the oracle."""
    cfg = inp["cfg"]
    M, H, SI, k = cfg["M"], cfg["H"], cfg["I"], cfg["top_k"]
    G.stagewise_routing(inp, r)
    G.stagewise_routed(inp, r)
    one = np.zeros((M, 1), dtype=np.int32)
    ref_sact, det = oracle.gate_up(inp["x"], one, 1, shw, SI, want_detail=True)
    G.check_act(r["sact"], ref_sact, det, label + " nvfp4 shared gate/up")
    ref_sh, det2 = oracle.down(r["sact"], one, shw, H, want_detail=True)
    G.check_y(r["sh"], ref_sh, det2, label + " nvfp4 shared down")
    out_c, _ = oracle.combine(r["y"], r["tw"], r["sh"], k)
    assert np.array_equal(r["out"], out_c), "combine differs"
    _, own_sh = _oracle_nv_shared(inp["x"], shw, H, SI)
    G.end_to_end(inp, r, lambda *a: print(*a, flush=True), sh_in=own_sh,
                 extra=dict(path=label + " nvfp4 shared"))


@pytest.mark.parametrize("path,M,H,I,E,k", [("decode", 8, 2048, 768, 128, 8),
                                            ("decode", 5, 256, 128, 16, 4),
                                            ("noalloc", 3, 512, 256, 32, 8),
                                            ("decode", 24, 512, 256, 16, 4),    # skinny GEMMs, side stream
                                            ("noalloc", 20, 512, 256, 32, 8)])  # skinny GEMMs, inline
def test_decode_nvfp4_shared_expert(path, M, H, I, E, k):
    print(f"decode NVFP4 shared expert path={path} M={M} H={H} I={I} E={E} k={k}", flush=True)
    inp = synth.make_small(960 + M, M=M, H=H, E=E, I=I, SI=0, top_k=k, router_std=0.3)
    shw = synth.nvfp4_experts(961 + M, 1, H, I)
    d = G.device_inputs(inp)
    shd = {kk: G.dev(v) for kk, v in shw.items()}
    z = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
    dbg = dict(logits_out=z((M, E), torch.int16), ids_out=z((M, k), torch.int32),
               tw_out=z((M, k), torch.float32), act_out=z((M * k, I), torch.int16),
               y_out=z((M * k, H), torch.int16), sact_out=z((M, I), torch.int16),
               sh_out=z((M, H), torch.int16))
    if path == "noalloc":
        out = fm.flint_moe_decode_noalloc(d["x"], d["router"], G.experts_of(d), shd, k, debug=dbg)
    else:
        ws = fm.make_workspace(M, H, E, I, I, k)
        out = fm.flint_moe_decode(d["x"], d["router"], G.experts_of(d), shd, k, ws, debug=dbg)
    torch.cuda.synchronize()
    r = {kk[:-4]: G.host(v) for kk, v in dbg.items()}
    r["out"] = G.host(out)
    _check_nv_shared_run(inp, shw, r, path)


def test_ll_nvfp4_shared_expert():
    """flint_moe_ll (residual add + RMS norm, then the decode block) with an
    NVFP4 shared expert, as the pages' fused decode block holds it."""
    print("flint_moe_ll with an NVFP4 shared expert, M=8 E=128", flush=True)
    M, E, k = 8, 128, 8
    inp = synth.make_inputs(1, M=M)
    cfg = inp["cfg"]
    H, I = cfg["H"], cfg["I"]
    shw = synth.nvfp4_experts(977, 1, H, I)
    ll = synth.make_ll_inputs(978, M, H)
    d = G.device_inputs(inp)
    shd = {kk: G.dev(v) for kk, v in shw.items()}
    ws = fm.make_workspace(M, H, E, I, I, k)
    z = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
    dbg = dict(logits_out=z((M, E), torch.int16), ids_out=z((M, k), torch.int32),
               tw_out=z((M, k), torch.float32), act_out=z((M * k, I), torch.int16),
               y_out=z((M * k, H), torch.int16), sact_out=z((M, I), torch.int16),
               sh_out=z((M, H), torch.int16))
    out, res, xn = fm.flint_moe_ll(G.dev(ll["attn_out"]), G.dev(ll["residual"]), G.dev(ll["ln_weight"]),
                                   ll["eps"], d["router"], G.experts_of(d), shd, k, ws, debug=dbg)
    torch.cuda.synchronize()
    res_ref, xn_ref = oracle.add_rms_norm(ll["attn_out"], ll["residual"], ll["ln_weight"], ll["eps"])
    assert np.array_equal(G.host(res), res_ref)
    xg = G.host(xn)
    assert np.all(np.abs(G.bf(xg) - G.bf(xn_ref)) <= G.ulp_bf16(G.bf(xn_ref))), "xn beyond one bf16 ulp"
    inp2 = dict(inp)
    inp2["x"] = xg
    inp2.pop("sgu", None)
    inp2.pop("sdown", None)
    r = {kk[:-4]: G.host(v) for kk, v in dbg.items()}
    r["out"] = G.host(out)
    _check_nv_shared_run(inp2, shw, r, "ll")
