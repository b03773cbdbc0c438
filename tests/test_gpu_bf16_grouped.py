"""GPU parity of the BF16-expert grouped path (flint_moe_bf16_grouped: the
BF16 experts' rule on grouped MFMA GEMMs, for prefill-size batches) against
the CPU oracle, through the C ABI.  Sizes span several 256-row and
128-column tiles with ragged tails, E up to 256; the M=4096 prefill shape
is checked on every token's routing and on a sample of tokens end to end."""
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


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("M,E,k,H,I,SI", [
    (1, 8, 2, 256, 128, 128),        # one token, every tile ragged
    (300, 16, 4, 512, 256, 192),     # experts with > 64 rows, 3 shared column tiles
    (700, 4, 4, 256, 128, 64),       # every expert > 256 rows: several row tiles each
    (129, 32, 8, 2048, 768, 768),    # the real H and I
    (300, 256, 8, 256, 128, 0),      # E = 256, no shared expert
])
def test_bf16_grouped_stagewise(M, E, k, H, I, SI):
    _say(f"bf16 grouped M={M} E={E} k={k} H={H} I={I} SI={SI}")
    inp = synth.make_small(1600 + M + E, M=M, H=H, E=E, I=I, SI=SI, top_k=k, experts="bf16",
                           router_std=0.3)
    r = G.run_block(fm, inp, "bf16_grouped")
    G.stagewise(inp, r, _say, extra=dict(path="bf16_grouped"))


def test_bf16_grouped_agrees_with_bf16_decode():
    _say("bf16 grouped vs bf16 decode, M=8 E=128")
    inp = synth.make_inputs(3)
    rd = G.run_block(fm, inp, "bf16_decode")
    rg = G.run_block(fm, inp, "bf16_grouped")
    same_lg = np.all(rd["logits"] == rg["logits"], axis=1)
    assert np.array_equal(rd["ids"][same_lg], rg["ids"][same_lg])
    G.stagewise(inp, rg, _say, extra=dict(path="bf16_grouped"))


def test_bf16_grouped_full_prefill_sampled():
    """M=4096, E=128, k=8 BF16 experts: every token's routing checked, 32
    tokens end to end."""
    _say("bf16 grouped full-size prefill (M=4096, E=128)")
    inp = synth.make_inputs(3, M=4096)
    cfg = inp["cfg"]
    M, H, E, I, SI, k = cfg["M"], cfg["H"], cfg["E"], cfg["I"], cfg["SI"], cfg["top_k"]
    d = G.device_inputs(inp)
    ws = fm.make_workspace(M, H, E, I, SI, k)
    z = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
    dbg = dict(logits_out=z((M, E), torch.int16), ids_out=z((M, k), torch.int32),
               tw_out=z((M, k), torch.float32))
    out = z((M, H), torch.int16)
    fm.flint_moe_bf16_grouped(d["x"], d["router"], G.experts_of(d), G.shared_of(d), k, ws, out=out,
                              debug=dbg)
    torch.cuda.synchronize()
    lg, ids, tw = G.host(dbg["logits_out"]), G.host(dbg["ids_out"]), G.host(dbg["tw_out"])
    rids, rtw, _ = oracle.topk(lg, k)
    assert np.array_equal(ids, rids) and G.same_f32(tw, rtw)
    rng = np.random.default_rng(3)
    sample = np.sort(rng.choice(M, 32, replace=False))
    ref = oracle.moe_block(inp, tokens=sample)
    G.check_logits(lg[sample], ref["logits"], inp["x"][sample], inp["router"], "bf16 prefill")
    same = np.all(ref["ids"] == ids[sample], axis=1)
    ulps = G.end_to_end_ulps(G.host(out)[sample], ref, k, rows=same)
    rep = G.error_report(G.host(out)[sample], ref, k, rows=same)
    _say(f"  sampled tokens {len(sample)}, near-tie flips {int((~same).sum())}, "
         f"max ulp(m) {ulps.max():.3f}, max abs {rep['max_abs']:.3g}, max rel {rep['max_rel']:.3g}, "
         f"ulp(out_ref) histogram {rep['ulp_out_hist']}")
    G.record(dict(workload="bf16_grouped_m4096_e128", M=M, E=E, top_k=k, H=H, I=I, path="bf16_grouped",
                  sampled_tokens=len(sample), near_tie_flips=int((~same).sum()),
                  max_ulp_m=float(ulps.max()), **rep))
    assert ulps.max() <= 2.0
    assert (~same).sum() <= 2
