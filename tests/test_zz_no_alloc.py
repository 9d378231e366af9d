"""moe_forward_noalloc (the forward on the library's static scratch, for
callers that cannot allocate) gives the same output and routing as
moe_forward with a caller workspace, bit for bit: the same kernels run on the
same inputs.  Two calls in a row share the scratch, the second on a smaller
batch.  (A batch too large for the scratch is refused before any launch:
tests/test_abi.py.)"""
import pytest
import torch

from mixture_experts_layer_align_amd import _binding as B
from workloads import LayerShape, make_layer, make_tokens

pytestmark = pytest.mark.gpu

CASES = [
    # layer, then the two batch sizes of consecutive calls (second smaller)
    (LayerShape(700, "noalloc-bf16", E=8, k=2, d=4096, d_ff=14336, act="bf16", wdt="bf16",
                seed=41), 64, 3),
    (LayerShape(701, "noalloc-fine", E=128, k=8, d=2048, d_ff=768, act="bf16", wdt="bf16",
                seed=42), 256, 17),
    (LayerShape(702, "noalloc-fp8", E=256, k=8, d=7168, d_ff=2048, act="bf16", wdt="fp8",
                seed=43), 16, 1),
    (LayerShape(703, "noalloc-tiled", E=8, k=2, d=512, d_ff=512, act="bf16", wdt="bf16",
                seed=44), 1200, 300),
    (LayerShape(704, "noalloc-f32", E=8, k=2, d=128, d_ff=256, act="f32", wdt="f32",
                seed=45), 16, 5),
    # fp8 gate|up block pairs (>= 4 entries per expert in both calls)
    (LayerShape(705, "noalloc-pairs-fp8", E=16, k=4, d=512, d_ff=512, act="bf16", wdt="fp8",
                seed=46), 200, 20),
]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _both(fwd, x):
    T = x.shape[0]
    ra, rb = fwd.routing_buffers(T), fwd.routing_buffers(T)
    want, bm_a, _ = fwd(x, routing=ra)
    got = torch.full_like(x, float("nan"))
    _, bm_b = fwd.noalloc(x, got, routing=rb)
    torch.cuda.synchronize()
    return want, got, ra, rb, bm_a, bm_b


@pytest.mark.parametrize("sh,T1,T2", CASES, ids=[c[0].name for c in CASES])
def test_noalloc_matches_forward(sh, T1, T2):
    print(f"noalloc {sh.name} T={T1} then T={T2}", flush=True)
    layer = make_layer(sh, None, "cuda", zipf=None)
    fwd = B.Forward(layer.w_router, layer.bias, layer.w_gate_up, layer.w_down, sh.k,
                    layer.scale_gate_up, layer.scale_down)
    for T in (T1, T2):
        x = make_tokens(sh, T, "cuda")
        want, got, ra, rb, bm_a, bm_b = _both(fwd, x)
        assert bm_a == bm_b
        assert torch.equal(_bits(want), _bits(got)), f"T={T}: outputs differ"
        n = T * sh.k
        cap = B.align_capacity(T, sh.E, sh.k, bm_a)
        for key in ("logits", "topk_ids", "topk_w", "counts", "offsets"):
            assert torch.equal(ra[key], rb[key]), f"T={T}: {key}"
        assert torch.equal(ra["sorted_ids"][:cap], rb["sorted_ids"][:cap])
        assert torch.equal(ra["inv_pos"][:n], rb["inv_pos"][:n])
