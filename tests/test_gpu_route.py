"""moe_route (router logits, softmax, top-k, renormalisation) against the
oracle: the oracle's top-k of the GPU's own fp32 logits equals the GPU's ids
bit for bit (boundary-fed), logits and weights within 1e-4*(1+|ref|) of the
float64 oracle, and where the oracle's own fp32 decision differs (a near tie)
the GPU's choice is a valid top-k within that logit tolerance (reported)."""
import numpy as np
import pytest
import torch

import parity as P
from mixture_experts_layer_align_amd import _binding as B
from oracle import moe_oracle as O
from workloads import LayerShape, make_bias, make_router, make_tokens

pytestmark = pytest.mark.gpu

CASES = [
    # T, d, E, k, act, zipf
    (1, 128, 8, 2, "bf16", None),
    (5, 256, 6, 6, "bf16", 1.0),       # E not a multiple of 8: masked weight loads
    (37, 512, 128, 8, "bf16", 1.0),
    (130, 2048, 256, 8, "bf16", 1.2),
    (64, 128, 1024, 16, "bf16", 0.5),
    (16, 128, 8, 2, "f32", None),
    (300, 4096, 8, 2, "bf16", None),   # several 32-row blocks
    (3, 7168, 256, 8, "bf16", 1.2),    # deep split over d
    (1, 64, 1, 1, "f32", None),        # a single expert
    (9, 192, 33, 3, "f32", 1.0),
    (0, 128, 8, 2, "bf16", None),      # empty batch
    # more than 1024 tokens: one wave per token
    (1500, 256, 64, 8, "bf16", 1.0),
    # k > 64: the selections go through LDS
    (1200, 128, 128, 72, "bf16", None),
    (40, 128, 200, 100, "f32", None),
    (1100, 128, 1024, 70, "bf16", 0.5),
    # a few tokens
    (4, 2048, 128, 8, "bf16", 1.0),
    (3, 1024, 256, 8, "bf16", 1.2),
    (2, 4096, 8, 2, "f32", None),
    (4, 512, 6, 6, "bf16", None),      # router rows not 16-byte aligned
    (4, 256, 64, 64, "bf16", 0.5),     # k = E = 64
    # E within one router slab: the workgroup's two waves split the k-steps,
    # here odd counts per split (5, 3 + 2) and a short last split
    (5, 320, 16, 4, "bf16", None),
    (3, 704, 100, 5, "bf16", 1.0),
    # many token blocks and E not a multiple of 4 (partial planes stored one
    # float at a time): a shared one-slab tile, and two-slab tiles
    (600, 256, 37, 5, "bf16", 1.0),
    (700, 128, 150, 6, "f32", 0.5),
]


@pytest.mark.parametrize("T,d,E,k,act,zipf", CASES)
def test_route_matches_oracle(T, d, E, k, act, zipf):
    sh = LayerShape(100 + E, "route", E=E, k=k, d=d, d_ff=64, act=act, wdt=act,
                    seed=1000 + T * 7 + E)
    wr = make_router(sh, "cuda")
    x = make_tokens(sh, T, "cuda")
    bias = make_bias(sh, zipf, "cuda")
    print(f"route T={T} d={d} E={E} k={k} act={act} zipf={zipf}", flush=True)
    logits, ids, w = B.route(x, wr, bias, k)
    torch.cuda.synchronize()
    if T == 0:
        return
    b64 = None if bias is None else bias.cpu().numpy().astype(np.float64)
    L64, oids, ow = O.route(P.decode(x), P.decode(wr), b64, k)
    gids = ids.cpu().numpy()
    P.assert_boundary_fed(logits.cpu().numpy(), gids, w.cpu().numpy(), k, what="route")
    P.assert_close_f32(logits.cpu().numpy(), L64, "logits")
    ties = P.classify_ids(L64, gids, oids)
    if ties.size:
        print(f"{ties.size} near ties (GPU selection valid within the logit tolerance)")
    P.assert_close_f32(w.cpu().numpy(), O.topk_weights(L64, gids), "topk_w")
    assert np.allclose(w.cpu().numpy().sum(axis=1), 1.0, atol=1e-6)


def test_route_exact_ties_go_to_lower_index():
    # duplicated router columns give bit-identical logits on the GPU too
    sh = LayerShape(150, "route", E=16, k=4, d=256, d_ff=64, act="bf16", wdt="bf16", seed=77)
    wr = make_router(sh, "cuda")
    wr[:, 9] = wr[:, 2]
    wr[:, 5] = wr[:, 12]
    x = make_tokens(sh, 40, "cuda")
    logits, ids, _ = B.route(x, wr, None, 16)
    g = ids.cpu().numpy()
    pos = {e: np.argmax(g == e, axis=1) for e in (2, 9, 5, 12)}
    assert (pos[2] < pos[9]).all() and (pos[5] < pos[12]).all()
    lg = logits.cpu().numpy()
    assert (lg[:, 2] == lg[:, 9]).all()


def test_route_exact_ties_go_to_lower_index_few_tokens():
    # the same for a few tokens
    sh = LayerShape(152, "route", E=16, k=4, d=256, d_ff=64, act="bf16", wdt="bf16", seed=79)
    wr = make_router(sh, "cuda")
    wr[:, 9] = wr[:, 2]
    wr[:, 5] = wr[:, 12]
    x = make_tokens(sh, 3, "cuda")
    logits, ids, _ = B.route(x, wr, None, 16)
    g = ids.cpu().numpy()
    pos = {e: np.argmax(g == e, axis=1) for e in (2, 9, 5, 12)}
    assert (pos[2] < pos[9]).all() and (pos[5] < pos[12]).all()
    lg = logits.cpu().numpy()
    assert (lg[:, 2] == lg[:, 9]).all() and (lg[:, 5] == lg[:, 12]).all()


def test_route_is_deterministic():
    sh = LayerShape(151, "route", E=256, k=8, d=7168, d_ff=64, act="bf16", wdt="bf16", seed=78)
    wr = make_router(sh, "cuda")
    x = make_tokens(sh, 77, "cuda")
    a = B.route(x, wr, None, 8)
    b = B.route(x, wr, None, 8)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


MASKED = [
    # T, E, k, finite experts: a -inf logit bias leaves fewer than k finite
    # logits, so the last selections fall among the -inf experts (lowest ids
    # first, each once) with weight 0
    (3, 128, 8, 5),      # few tokens: the one-launch top-k + alignment
    (40, 128, 8, 3),     # a workgroup per token
    (1500, 64, 8, 6),    # a wave per token
    (40, 200, 100, 30),  # k > 64: selections through LDS
    (5, 256, 8, 1),      # E > 128 in the few-token path
]


@pytest.mark.parametrize("T,E,k,n_finite", MASKED)
def test_route_masking_bias_fewer_finite_than_k(T, E, k, n_finite):
    sh = LayerShape(160 + E, "route", E=E, k=k, d=256, d_ff=64, act="bf16", wdt="bf16",
                    seed=3000 + T + n_finite)
    wr = make_router(sh, "cuda")
    x = make_tokens(sh, T, "cuda")
    g = torch.Generator().manual_seed(T * 31 + E)
    finite = torch.randperm(E, generator=g)[:n_finite]
    bias = torch.full((E,), float("-inf"))
    bias[finite] = torch.randn(n_finite, generator=g)
    bias = bias.to("cuda")
    print(f"masked route T={T} E={E} k={k} finite={n_finite}", flush=True)
    logits, ids, w = B.route(x, wr, bias, k)
    fwd = B.Forward(wr, bias, *_tiny_experts(E, 256), k)
    rb = fwd.routing_buffers(T)
    fwd(x, routing=rb)
    torch.cuda.synchronize()
    gl, gids, gw = logits.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()
    assert np.isneginf(gl[:, np.setdiff1d(np.arange(E), finite.numpy())]).all()
    P.assert_boundary_fed(gl, gids, gw, k, what="masked route")
    for row in gids:
        assert len(set(row.tolist())) == k, f"repeated expert {row}"
    want = O.select_topk(gl, k)
    assert (gids == want).all()
    assert (gw[:, n_finite:] == 0).all() and np.allclose(gw.sum(axis=1), 1.0, atol=1e-6)
    # the forward's own routing (few-token path for T <= 16) selects the same
    assert (rb["topk_ids"].cpu().numpy() == gids).all()


def _tiny_experts(E, d):
    dff = 128
    wgu = torch.zeros((E, d, 2 * dff), dtype=torch.bfloat16, device="cuda")
    wdn = torch.zeros((E, dff, d), dtype=torch.bfloat16, device="cuda")
    return wgu, wdn
