"""moe_forward (the whole layer) against the oracle.

Routing is checked both ways (tests/parity.py): the oracle's top-k, weights
and alignment on the GPU's own fp32 logits must match the GPU bit for bit on
every token, and the GPU's logits must match the oracle's float64 logits.
Float outputs are compared on every token of every layer, the
full-size benchmark layers (up to 16,384 tokens of the E=256 top-8
d=7168 layer) included, against the oracle's experts on the GPU's selection,
with no token exempt.  The five benchmark layers run at full size in the
launch configuration the benchmark uses."""
import dataclasses
import functools

import numpy as np
import pytest
import torch

import parity as P
from mixture_experts_layer_align_amd import _binding as B
from oracle import moe_oracle as O
from workloads import LAYERS, LayerShape, make_bias, make_layer, make_tokens

pytestmark = pytest.mark.gpu

def run_and_check(layer, x, what=""):
    sh = layer.shape
    T = x.shape[0]
    fwd = B.Forward(layer.w_router, layer.bias, layer.w_gate_up, layer.w_down, sh.k,
                    layer.scale_gate_up, layer.scale_down)
    rb = fwd.routing_buffers(T)
    out, bm, _ = fwd(x, routing=rb)
    torch.cuda.synchronize()
    if T == 0:
        return out, rb, bm
    wr64, b64, efn = P.oracle_layer(layer)
    x64 = P.decode(x)
    glog = rb["logits"].cpu().numpy()
    gids = rb["topk_ids"].cpu().numpy()
    gw = rb["topk_w"].cpu().numpy()
    cap = O.capacity(T, sh.E, sh.k, bm)
    got = {k_: rb[k_].cpu().numpy() for k_ in ("counts", "offsets", "sorted_ids", "inv_pos")}
    got["sorted_ids"] = got["sorted_ids"][:cap]
    got["inv_pos"] = got["inv_pos"][:T * sh.k]
    # (i) boundary-fed: O2-O5 on the GPU's logits, bit-exact for every token
    P.assert_boundary_fed(glog, gids, gw, sh.k, sh.E, bm, got, what)
    # (ii) logits against O1; the oracle's own fp32 decision differs only at
    # near ties within the logit tolerance (reported)
    L64 = O.router_logits(x64, wr64, b64)
    P.assert_close_f32(glog, L64, f"{what} logits")
    ties = P.classify_ids(L64, gids, O.select_topk(L64.astype(np.float32), sh.k))
    if ties.size:
        print(f"{what}: {ties.size} near ties (GPU selection valid within the logit tolerance)")
    w64 = O.topk_weights(L64, gids)
    P.assert_close_f32(gw, w64, f"{what} topk_w (ii)")
    # output of every token, on the GPU's selection
    ref_out = O.outputs_for_tokens(x64, np.arange(T), gids, w64, efn)
    P.assert_out_close(P.decode(out), ref_out, sh.act, f"{what} T={T}")
    return out, rb, bm


SMALL = [
    # E, k, d, d_ff, act, wdt, T, zipf
    (8, 2, 128, 256, "f32", "f32", 16, None),
    (8, 2, 128, 128, "bf16", "bf16", 1, None),
    (8, 2, 256, 384, "bf16", "bf16", 33, None),
    (16, 4, 384, 256, "bf16", "bf16", 100, 1.0),     # d a multiple of 128, not of 256
    (1, 1, 128, 128, "bf16", "bf16", 70, None),      # a single expert: dense SwiGLU
    (6, 6, 256, 128, "bf16", "bf16", 9, None),       # k = E: every token on every expert
    (32, 8, 512, 256, "bf16", "fp8", 40, 1.2),
    (128, 8, 256, 128, "bf16", "bf16", 3, None),     # most experts empty
    (8, 2, 256, 256, "bf16", "fp8", 257, 1.2),
    (4, 2, 128, 128, "f32", "f32", 300, 0.5),
    (8, 2, 128, 128, "bf16", "bf16", 0, None),       # empty batch
    # few rows, long K: gate|up splits K and the down GEMM forms h from the
    # fp32 partials (fp32 h; bf16-pair h)
    (8, 2, 512, 256, "f32", "f32", 2, None),
    (16, 4, 1024, 256, "bf16", "bf16", 2, None),
    # >= 64 routed rows per expert and d % 256 == 0: the MFMA-tiled GEMM
    (4, 2, 256, 256, "bf16", "bf16", 300, None),
    (8, 2, 512, 384, "bf16", "bf16", 700, 1.2),      # skewed, ragged blocks
    (1, 1, 256, 256, "bf16", "bf16", 200, None),     # one expert, 2 blocks
    (1, 1, 256, 128, "bf16", "bf16", 200, None),     # d_ff too shallow to tile: streamed
    (16, 4, 768, 640, "bf16", "bf16", 1111, 0.8),
    # ... with fp8 weights (scales applied to the fp32 sums)
    (4, 2, 256, 512, "bf16", "fp8", 400, None),
    (16, 4, 512, 256, "bf16", "fp8", 700, 1.0),      # skewed, ragged blocks
    (2, 1, 768, 256, "bf16", "fp8", 600, None),      # 24 k-steps of gate|up
    # fp8 on the stream GEMM with >= 4 entries per expert: the gate|up GEMM
    # applies one weight stream to pairs of an expert's 32-row blocks
    # (skewed: heavy experts fill pairs, light ones leave the second empty;
    # odd block counts end in a single)
    (16, 4, 512, 256, "bf16", "fp8", 100, 1.2),
    (8, 2, 1024, 512, "bf16", "fp8", 150, None),
    (64, 8, 512, 512, "bf16", "fp8", 300, 1.0),
    (4, 2, 2048, 256, "bf16", "fp8", 16, None),      # k-split gate|up (folded) and down
    # either side of the regime switches: 4 entries per expert (pairs from
    # T*k = 64 at E=16) and 64 per expert (the tiled GEMM from T*k = 256 at E=4)
    (16, 4, 512, 256, "bf16", "fp8", 15, 1.2),
    (16, 4, 512, 256, "bf16", "fp8", 16, 1.2),
    (4, 2, 256, 256, "bf16", "fp8", 127, None),
    (4, 2, 256, 256, "bf16", "fp8", 128, None),
    # MXFP4 experts (E2M1 codes, an E8M0 scale per 32 k): always the stream GEMM
    (8, 2, 256, 256, "bf16", "mxfp4", 5, None),
    (32, 8, 512, 256, "bf16", "mxfp4", 40, 1.2),
    (4, 2, 256, 512, "bf16", "mxfp4", 300, None),    # many rows per expert
    (16, 4, 768, 256, "bf16", "mxfp4", 257, 1.0),    # 24 scale blocks along d
    (16, 4, 512, 512, "bf16", "mxfp4", 100, 1.2),    # heavy experts, many blocks
    (4, 2, 2048, 256, "bf16", "mxfp4", 16, None),    # k-split gate|up
    (1024, 4, 256, 256, "bf16", "bf16", 300, None),  # MOE_MAX_EXPERTS experts
    # MXFP8 experts (e4m3fn codes, an E8M0 scale per 32 k): the stream GEMM
    (8, 2, 256, 256, "bf16", "mxfp8", 5, None),
    (32, 8, 512, 256, "bf16", "mxfp8", 40, 1.2),
    (4, 2, 256, 512, "bf16", "mxfp8", 300, None),    # many rows per expert
    (16, 4, 768, 256, "bf16", "mxfp8", 257, 1.0),    # 24 scale blocks along d
    (16, 4, 512, 512, "bf16", "mxfp8", 100, 1.2),    # heavy experts, many blocks
    (4, 2, 2048, 256, "bf16", "mxfp8", 16, None),    # k-split gate|up
]


@pytest.mark.parametrize("E,k,d,d_ff,act,wdt,T,zipf", SMALL)
def test_forward_small_layers(E, k, d, d_ff, act, wdt, T, zipf):
    sh = LayerShape(200 + E, "small", E=E, k=k, d=d, d_ff=d_ff, act=act, wdt=wdt,
                    seed=500 + E * 3 + d + T)
    print(f"forward small E={E} k={k} d={d} d_ff={d_ff} {act}/{wdt} T={T}", flush=True)
    layer = make_layer(sh, T, "cuda", zipf=zipf)
    x = make_tokens(sh, T, "cuda")
    run_and_check(layer, x, what="small")


@pytest.mark.parametrize("T", [64, 1024])
def test_forward_all_tokens_on_one_expert_in_full_blocks(T):
    # a one-hot bias sends every token's slot 0 to expert 3; the tokens fill
    # whole blocks (two 32-row blocks of the streaming GEMM at T=64, four
    # 256-row blocks of the tiled GEMM at T=1024)
    sh = LayerShape(250, "onehot", E=8, k=1, d=256, d_ff=256, act="bf16", wdt="bf16", seed=9)
    layer = make_layer(sh, T, "cuda", zipf=None)
    bias = torch.zeros(8, dtype=torch.float32, device="cuda")
    bias[3] = 1e4
    layer = dataclasses.replace(layer, bias=bias)
    x = make_tokens(sh, T, "cuda")
    _, rb, bm = run_and_check(layer, x, what="one-hot")
    c = rb["counts"].cpu().numpy()
    assert c[3] == T and c.sum() == T and T % bm == 0
    assert bm == (256 if T == 1024 else 32)


HALF_ROWS = [
    # E, k, d, d_ff, wdt, T, zipf: both GEMMs have an even number of 256-column
    # tiles, so experts are padded to 128 rows and an expert's last 128 rows
    # run as a half tile (128 rows x 512 columns)
    (8, 2, 512, 256, "bf16", 700, 1.2),
    (16, 4, 1024, 512, "bf16", 1500, 1.0),
    (8, 2, 512, 512, "fp8", 900, 1.2),
    (32, 4, 512, 256, "fp8", 1600, 0.6),
]


@pytest.mark.parametrize("E,k,d,d_ff,wdt,T,zipf", HALF_ROWS)
def test_forward_tiled_half_rows(E, k, d, d_ff, wdt, T, zipf):
    sh = LayerShape(260 + E, "half-rows", E=E, k=k, d=d, d_ff=d_ff, act="bf16", wdt=wdt,
                    seed=40 + E + T)
    print(f"forward half rows E={E} k={k} d={d} d_ff={d_ff} {wdt} T={T}", flush=True)
    layer = make_layer(sh, T, "cuda", zipf=zipf)
    x = make_tokens(sh, T, "cuda")
    _, rb, bm = run_and_check(layer, x, what="half rows")
    assert bm == 128
    rem = rb["counts"].cpu().numpy() % 256
    assert ((rem > 0) & (rem <= 128)).any(), "no expert ends in a half row"
    assert (rem > 128).any(), "no expert ends in a partly filled full row"


def test_forward_tiled_at_max_experts():
    # 1024 experts with 64 routed rows each on average: the tiled GEMM, rows of
    # every kind (empty experts, half rows, full rows)
    sh = LayerShape(270, "max-experts", E=1024, k=4, d=512, d_ff=256, act="bf16", wdt="bf16",
                    seed=71)
    T = 16384
    print(f"forward E=1024 k=4 d=512 d_ff=256 T={T}", flush=True)
    layer = make_layer(sh, T, "cuda", zipf=0.8)
    x = make_tokens(sh, T, "cuda")
    _, _, bm = run_and_check(layer, x, what="max experts")
    assert bm == 128


def test_forward_is_deterministic():
    sh = LAYERS[3]
    layer = make_layer(sh, 256, "cuda")
    x = make_tokens(sh, 256, "cuda")
    fwd = B.Forward(layer.w_router, layer.bias, layer.w_gate_up, layer.w_down, sh.k)
    a = fwd(x)[0].clone()
    b = fwd(x)[0].clone()
    assert torch.equal(a, b)


@functools.lru_cache(maxsize=1)
def _config_layer(cfg):
    torch.cuda.empty_cache()
    return make_layer(LAYERS[cfg], None, "cuda", zipf=None)


FULL = [(c, T) for c in sorted(LAYERS) for T in LAYERS[c].tokens]


@pytest.mark.parametrize("cfg,T", FULL)
def test_forward_benchmark_layers_full_size(cfg, T):
    sh = LAYERS[cfg]
    print(f"forward config {cfg} ({sh.name}) T={T}", flush=True)
    base = _config_layer(cfg)
    layer = dataclasses.replace(base, bias=make_bias(sh, sh.zipf_for(T), "cuda"))
    x = make_tokens(sh, T, "cuda")
    run_and_check(layer, x, what=f"config {cfg}")
