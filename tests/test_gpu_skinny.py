"""GPU parity of the skinny expert GEMMs through the C ABI.  Decode-size
batches (M <= 64 tokens, H and I multiples of 256) run every expert GEMM of
the grouped chain on the skinny MFMA kernel: flint_moe_grouped and
flint_moe_bf16_grouped at any such M, and flint_moe_decode /
flint_moe_bf16_decode for M > 16.  The cases span one token, exactly one
and just over one group of 16 rows per expert, experts holding every token
(four groups), E = 256 (the per-block expert prefix over four waves), odd
and even counts of 256-wide K chunks (down projection K = 768: three), no
shared expert, and BF16 experts; each is checked against the CPU oracle
stage by stage (routing bit-exact, act / y / out within the tolerance)."""
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
    (1, 8, 2, 256, 256, 256),        # one token
    (5, 16, 4, 512, 256, 256),
    (16, 32, 8, 256, 512, 256),      # at most one full group per expert
    (17, 4, 2, 256, 256, 0),         # groups of 16 and 1 rows, no shared expert
    (40, 2, 2, 512, 256, 256),       # every expert 40 rows: three groups
    (64, 3, 3, 256, 768, 256),       # top_k = E: every expert 64 rows (four groups), down K = 768
    (64, 256, 8, 256, 256, 256),     # E = 256
    (33, 128, 8, 2048, 768, 768),    # the real H and I
])
def test_skinny_grouped_stagewise(M, E, k, H, I, SI):
    _say(f"skinny grouped M={M} E={E} k={k} H={H} I={I} SI={SI}")
    inp = synth.make_small(1100 + M + E, M=M, H=H, E=E, I=I, SI=SI, top_k=k, router_std=0.3)
    r = G.run_block(fm, inp, "grouped")
    G.stagewise(inp, r, _say, extra=dict(path="grouped_skinny"))


@pytest.mark.parametrize("M,E,k,H,I,SI", [
    (24, 16, 4, 512, 256, 256),
    (64, 16, 8, 256, 256, 256),      # (H, I) among the decode entry's shapes
])
def test_skinny_decode_entry_stagewise(M, E, k, H, I, SI):
    """flint_moe_decode past 16 tokens: the grouped chain on the skinny GEMMs."""
    _say(f"skinny via decode M={M} E={E} k={k} H={H} I={I} SI={SI}")
    inp = synth.make_small(1200 + M + E, M=M, H=H, E=E, I=I, SI=SI, top_k=k, router_std=0.3)
    r = G.run_block(fm, inp, "decode")
    G.stagewise(inp, r, _say, extra=dict(path="decode_skinny"))


@pytest.mark.parametrize("path,M,E,k,H,I,SI", [
    ("bf16_grouped", 9, 16, 4, 256, 256, 256),
    ("bf16_grouped", 50, 8, 4, 512, 256, 256),   # experts with several groups
    ("bf16_decode", 20, 16, 4, 256, 256, 256),   # the BF16 decode entry past 16 tokens
])
def test_skinny_bf16_experts_stagewise(path, M, E, k, H, I, SI):
    _say(f"skinny {path} M={M} E={E} k={k} H={H} I={I} SI={SI}")
    inp = synth.make_small(1300 + M + E, M=M, H=H, E=E, I=I, SI=SI, top_k=k, router_std=0.3,
                           experts="bf16")
    r = G.run_block(fm, inp, path)
    G.stagewise(inp, r, _say, extra=dict(path=path + "_skinny"))
