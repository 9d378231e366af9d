"""The forward's routing equals the standalone entry points' bit for bit.

moe_forward routes few tokens (T <= 16) with its one-launch top-k +
alignment kernel and more tokens with the top-k and alignment kernels that
moe_route / moe_align use; both must give the same logits, ids, weights and
alignment (same router plan, same plane-sum order, same selection and weight
arithmetic)."""
import pytest
import torch

from mixture_experts_layer_align_amd import _binding as B
from workloads import LayerShape, make_layer, make_tokens

pytestmark = pytest.mark.gpu

CASES = [
    # E, k, d, T, zipf
    (8, 2, 4096, 1, None),
    (8, 2, 4096, 16, None),      # largest batch of the one-launch path
    (8, 2, 4096, 17, None),      # smallest batch of the separate path
    (128, 8, 2048, 3, None),
    (128, 8, 2048, 64, 1.0),
    (256, 8, 7168, 16, 1.2),
    (6, 6, 256, 9, None),        # k = E
    (128, 8, 2048, 4, 1.0),
    (6, 6, 256, 3, None),        # router rows not 16-byte aligned
    (64, 64, 256, 4, 0.5),       # 256 entries: the workgroup aligns them
    (256, 8, 7168, 4, 1.2),      # more than 128 experts, at most 8 tokens
    (200, 8, 1024, 1, None),
    (256, 8, 2048, 8, 1.0),
]


@pytest.mark.parametrize("E,k,d,T,zipf", CASES)
def test_forward_routing_equals_route_and_align(E, k, d, T, zipf):
    print(f"route paths E={E} k={k} d={d} T={T}", flush=True)
    sh = LayerShape(400 + E, "route-paths", E=E, k=k, d=d, d_ff=256, act="bf16", wdt="bf16",
                    seed=900 + T)
    layer = make_layer(sh, T, "cuda", zipf=zipf)
    x = make_tokens(sh, T, "cuda")
    fwd = B.Forward(layer.w_router, layer.bias, layer.w_gate_up, layer.w_down, k)
    rb = fwd.routing_buffers(T)
    _, bm, _ = fwd(x, routing=rb)
    logits, ids, w = B.route(x, layer.w_router, layer.bias, k)
    al = B.align(ids, E, bm)
    torch.cuda.synchronize()
    cap = B.align_capacity(T, E, k, bm)
    assert torch.equal(rb["logits"], logits)
    assert torch.equal(rb["topk_ids"], ids)
    assert torch.equal(rb["topk_w"], w)
    assert torch.equal(rb["counts"], al["counts"])
    assert torch.equal(rb["offsets"], al["offsets"])
    assert torch.equal(rb["sorted_ids"][:cap], al["sorted_ids"][:cap])
    assert torch.equal(rb["inv_pos"], al["inv_pos"])
