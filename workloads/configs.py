"""The five synthetic MoE layers the benchmark and the parity tests run.

Shapes and value laws follow the workload statement (router softmax over E,
top-k with ties to the lower index, renormalised; SwiGLU experts; fp8 expert
weights with one fp32 scale per output column).  The hidden size `d`, the
per-expert FFN width `d_ff`, the expert count `E` and the top-`k` mirror public
MoE model families: E=128/top-8/d=2048/d_ff=768 is the Qwen3-30B class named in
"CuTeDSL at Perplexity", section on local (TP=1) MoE dispatch.
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional


@dataclass(frozen=True)
class LayerShape:
    cfg: int
    name: str
    E: int
    k: int
    d: int
    d_ff: int
    act: str            # "f32" | "bf16"   (x, out, router weight)
    wdt: str            # "f32" | "bf16" | "fp8" | "mxfp4" | "mxfp8"  (expert weights)
    tokens: List[int] = field(default_factory=list)
    # Zipf exponent of the router-logit bias per token count (None: no bias)
    zipf: Dict[int, Optional[float]] = field(default_factory=dict)
    seed: int = 0

    def zipf_for(self, T: int) -> Optional[float]:
        return self.zipf.get(T)


def _z(ts, s):
    return {t: s for t in ts}


LAYERS = {
    0: LayerShape(0, "tiny-fp32", E=8, k=2, d=128, d_ff=256, act="f32", wdt="f32",
                  tokens=[16], zipf=_z([16], None), seed=0),
    1: LayerShape(1, "decode-bf16", E=8, k=2, d=4096, d_ff=14336, act="bf16", wdt="bf16",
                  tokens=[1, 4, 16, 64], zipf=_z([1, 4, 16, 64], None), seed=1),
    2: LayerShape(2, "prefill-bf16-zipf1.2", E=8, k=2, d=4096, d_ff=14336, act="bf16",
                  wdt="bf16", tokens=[512, 4096], zipf=_z([512, 4096], 1.2), seed=2),
    3: LayerShape(3, "fine-grained-bf16", E=128, k=8, d=2048, d_ff=768, act="bf16",
                  wdt="bf16", tokens=[1, 32, 256, 8192],
                  zipf={1: None, 32: None, 256: None, 8192: 1.0}, seed=3),
    4: LayerShape(4, "large-fp8-zipf1.2", E=256, k=8, d=7168, d_ff=2048, act="bf16",
                  wdt="fp8", tokens=[1, 16, 128, 16384], zipf=_z([1, 16, 128, 16384], 1.2),
                  seed=4),
    # not one of the five benchmark layers: the E=256 top-8 fp8 layer with MXFP4
    # experts (the microscaling variant), decode batches only
    5: LayerShape(5, "large-mxfp4-zipf1.2", E=256, k=8, d=7168, d_ff=2048, act="bf16",
                  wdt="mxfp4", tokens=[1, 16, 128], zipf=_z([1, 16, 128], 1.2), seed=5),
    # ... and with MXFP8 experts (e4m3fn codes, E8M0 block scales)
    6: LayerShape(6, "large-mxfp8-zipf1.2", E=256, k=8, d=7168, d_ff=2048, act="bf16",
                  wdt="mxfp8", tokens=[1, 16, 128], zipf=_z([1, 16, 128], 1.2), seed=6),
}


def layer_shape(cfg: int) -> LayerShape:
    return LAYERS[cfg]
