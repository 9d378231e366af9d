"""moe_forward at the largest routed-entry count it accepts: T*k = 2^24 - 8,
just below MOE_MAX_ENTRIES.  The token rows, h and the per-slot outputs then
span several GiB each, so every kernel's row and slot offsets run past 2^31
elements.  One layer per expert GEMM: d = 256 takes the LDS-tiled GEMM
(about 2M rows per expert), d = 128 the weight-streaming GEMM.

Routing and alignment are checked bit for bit on every token: the oracle's
top-k and weights on the GPU's own fp32 logits, and the alignment by its
defining properties (which fix it uniquely).  Logits and
outputs are checked on 4096 sampled tokens spread over the whole batch (the
first and last included) against the oracle, to the usual bounds."""
import numpy as np
import pytest
import torch

import parity as P
from mixture_experts_layer_align_amd import _binding as B
from oracle import moe_oracle as O
from workloads import LayerShape, make_layer, make_tokens

pytestmark = pytest.mark.gpu

MAX_ENTRIES = 1 << 24


@pytest.mark.parametrize("d,d_ff", [(256, 256), (128, 128)])
def test_forward_at_the_maximum_entry_count(d, d_ff):
    E, k = 8, 2
    T = (MAX_ENTRIES - 8) // k
    sh = LayerShape(260 + d, "max", E=E, k=k, d=d, d_ff=d_ff, act="bf16", wdt="bf16", seed=77)
    print(f"forward max entries T={T} k={k} d={d} d_ff={d_ff}", flush=True)
    layer = make_layer(sh, T, "cuda", zipf=None)
    x = make_tokens(sh, T, "cuda")
    fwd = B.Forward(layer.w_router, layer.bias, layer.w_gate_up, layer.w_down, k)
    rb = fwd.routing_buffers(T)
    out, bm, _ = fwd(x, routing=rb)
    torch.cuda.synchronize()
    print(f"  block_m {bm}", flush=True)
    assert bm in (32, 128, 256)

    glog = rb["logits"].cpu().numpy()
    gids = rb["topk_ids"].cpu().numpy()
    gw = rb["topk_w"].cpu().numpy()
    # the oracle's top-k and weights on the GPU's logits, every token; the
    # alignment by its defining properties (which fix it uniquely: the
    # oracle's explicit loops over 2^24 entries would take minutes)
    P.assert_boundary_fed(glog, gids, gw, k, what=f"max d={d}")
    g = {key: rb[key].cpu().numpy() for key in ("counts", "offsets", "sorted_ids", "inv_pos")}
    P.check_alignment_properties(gids, E, bm, g["counts"], g["offsets"], g["sorted_ids"],
                                 g["inv_pos"])

    rng = np.random.default_rng(d)
    rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 4094, replace=False)]))
    idx = torch.from_numpy(rows).cuda()
    wr64, b64, efn = P.oracle_layer(layer)
    x64 = P.decode(x[idx])
    L64 = O.router_logits(x64, wr64, b64)
    P.assert_close_f32(glog[rows], L64, f"max d={d} logits (sampled)")
    w64 = O.topk_weights(L64, gids[rows])
    ref = O.outputs_for_tokens(x64, np.arange(rows.size), gids[rows], w64, efn)
    P.assert_out_close(P.decode(out[idx]), ref, "bf16", f"max d={d} T={T} (sampled)")
