"""moe_forward captured in a HIP graph: every replay, with other eager work and
synchronisations between replays, gives bitwise the eager result (the forward
is deterministic and enqueues no memset or allocation, so it can be
captured)."""
import pytest
import torch

from mixture_experts_layer_align_amd import _binding as B
from workloads import LAYERS, LayerShape, make_layer, make_tokens

pytestmark = pytest.mark.gpu

CASES = [
    # (shape, T): decode stream path with split-K, fused routing; tiled path
    (LAYERS[1], 4),
    (LayerShape(301, "graph-tiled", E=4, k=2, d=256, d_ff=256, act="bf16", wdt="bf16", seed=7),
     300),
    (LayerShape(302, "graph-mx", E=16, k=4, d=512, d_ff=256, act="bf16", wdt="mxfp4", seed=8),
     24),
    # two tokens, long K: gate|up splits K and the down GEMM forms h from
    # the partials
    (LayerShape(303, "graph-fold", E=16, k=4, d=1024, d_ff=256, act="bf16", wdt="bf16", seed=9),
     2),
    (LayerShape(304, "graph-fold-fp8", E=16, k=4, d=1024, d_ff=256, act="bf16", wdt="fp8",
                seed=10), 2),
    # fp8 with >= 4 entries per expert: the gate|up GEMM's block pairs
    (LayerShape(305, "graph-pairs-fp8", E=16, k=4, d=512, d_ff=256, act="bf16", wdt="fp8",
                seed=11), 200),
]


@pytest.mark.parametrize("sh,T", CASES,
                         ids=["decode-bf16", "tiled-bf16", "mxfp4", "fold-bf16", "fold-fp8",
                              "pairs-fp8"])
def test_graph_replays_match_eager(sh, T):
    print(f"graph replay {sh.name} T={T}", flush=True)
    layer = make_layer(sh, T, "cuda")
    x = make_tokens(sh, T, "cuda")
    fwd = B.Forward(layer.w_router, layer.bias, layer.w_gate_up, layer.w_down, sh.k,
                    layer.scale_gate_up, layer.scale_down)
    eager = fwd(x)[0].clone()
    out = torch.empty_like(x)
    fwd(x, out)  # workspace allocated before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(x, out)
    for i in range(4):
        out.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager forward"
        del junk
