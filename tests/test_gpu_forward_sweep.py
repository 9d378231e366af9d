"""moe_forward on a seeded sweep of random layers, every token against the
oracle (tests/test_gpu_forward.py's checks: routing bit-exact on the GPU's
own logits, logits and outputs to their bounds).

The draw spans the regimes the forward picks between — the weight-streaming
GEMM (single 32-row blocks, and for fp8 pairs of an expert's blocks), split K
with the down GEMM's fold, and the LDS-tiled GEMM with full and half rows —
over every weight format, with and without router skew."""
import random

import pytest

from test_gpu_forward import run_and_check
from workloads import LayerShape, make_layer, make_tokens

pytestmark = pytest.mark.gpu


def _cases(n=32, seed=20240):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        wdt = rng.choice(["bf16", "bf16", "fp8", "fp8", "mxfp4", "mxfp8", "f32"])
        act = "f32" if wdt == "f32" else "bf16"
        E = rng.choice([2, 4, 8, 16, 32, 64])
        k = rng.choice([c for c in (1, 2, 4, 8) if c <= E])
        scaled = wdt in ("fp8", "mxfp4", "mxfp8")
        d = rng.choice([256, 512, 768, 1024] if scaled else [128, 256, 384, 512, 768])
        dff = rng.choice([256, 512, 768] if scaled else [128, 256, 384, 512])
        # entries per expert on average: decode, around the pair switch, or prefill
        per = rng.choice([0.25, 1, 3, 4, 6, 20, 40, 70, 120])
        T = max(1, int(per * E / k))
        z = rng.choice([None, None, 0.8, 1.2])
        out.append((i, E, k, d, dff, act, wdt, T, z))
    return out


@pytest.mark.parametrize("i,E,k,d,dff,act,wdt,T,z", _cases(),
                         ids=lambda v: str(v) if not isinstance(v, (float, type(None))) else "")
def test_forward_random_layer(i, E, k, d, dff, act, wdt, T, z):
    sh = LayerShape(800 + i, "sweep", E=E, k=k, d=d, d_ff=dff, act=act, wdt=wdt, seed=3000 + i)
    print(f"sweep {i}: E={E} k={k} d={d} d_ff={dff} {act}/{wdt} T={T} zipf={z}", flush=True)
    layer = make_layer(sh, T, "cuda", zipf=z)
    x = make_tokens(sh, T, "cuda")
    run_and_check(layer, x, what=f"sweep {i}")
