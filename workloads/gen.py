"""Seeded generators of MoE layer inputs (weights, router bias, tokens).

Every tensor is drawn from its own torch.Generator whose seed comes from
numpy's SeedSequence([cfg_seed, tensor_id, index]); expert weights are drawn
expert by expert so any single expert can be regenerated without the rest.

Value laws (the workload statement's, with the readings documented alongside
the oracle):
  * x ~ N(0, 1), stored in the activation dtype (fp32, or bf16 by RNE).
  * W_router[d, E], W_gate/W_up[E, d, d_ff] ~ N(0, 1/d); W_down[E, d_ff, d] ~
    N(0, 1/d_ff)  (variance 1/fan_in), drawn in fp32 then stored in the weight
    dtype.
  * fp8 experts: per expert and per output column, scale = max_k |w[k, n]| / 448
    (the OCP e4m3fn maximum), code = e4m3fn(w / scale) by torch's RNE cast; gate
    and up columns are scaled separately.
  * MXFP4 experts: per block of 32 consecutive k of one output column, an
    E8M0 exponent floor(log2(max|w|)) - 2 and E2M1 codes (quantize_mxfp4).
  * Zipf router skew: bias[e] = -s * ln(rank[e]) with rank a seeded permutation
    of 1..E, which multiplies each expert's softmax mass by rank^-s.

Generation may run on any torch device; values depend on that device's RNG, so
a test feeds the oracle host copies of exactly the tensors the GPU consumed.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import LayerShape

FP8_MAX = 448.0

TENSOR_X, TENSOR_WR, TENSOR_WG, TENSOR_WU, TENSOR_WD, TENSOR_PERM, TENSOR_IDS = range(7)

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _seed(*parts: int) -> int:
    ss = np.random.SeedSequence([int(p) & 0xFFFFFFFF for p in parts])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)


def _gen(device, *parts: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _normal(shape, std, device, *parts):
    g = _gen(device, *parts)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def quantize_e4m3fn_per_column(w: torch.Tensor):
    """w: [K, N] fp32 -> (codes [K, N] float8_e4m3fn, scale [N] fp32)."""
    amax = w.abs().amax(dim=0)
    scale = amax / FP8_MAX
    scale = torch.where(amax > 0, scale, torch.ones_like(scale))
    q = (w / scale).clamp_(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q, scale.to(torch.float32)


MX_BLOCK = 32
# E2M1 magnitudes of codes 0..7
_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def quantize_mxfp4(w: torch.Tensor):
    """w: [K, N] fp32 (K a multiple of 32) -> (packed [K/2, N] uint8, scales
    [K/32, N] uint8).  Per block of 32 consecutive k of one column: shared
    exponent floor(log2(max|w|)) - 2 (E2M1's largest magnitude is 1.5 * 2^2),
    stored biased by 127 (E8M0); each element divided by 2^exponent and rounded
    to the nearest E2M1 magnitude (ties to the even code, beyond 6 clamped to
    6); codes two per byte along K, even k in the low nibble.  An all-zero
    block gets exponent 0 and zero codes."""
    K, N = w.shape
    blk = w.reshape(K // MX_BLOCK, MX_BLOCK, N)
    amax = blk.abs().amax(dim=1)
    ex = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax, 1.0))) - 2.0,
                     torch.zeros_like(amax)).clamp_(-127.0, 127.0)
    x = (blk / torch.exp2(ex)[:, None, :]).reshape(K, N)
    grid = torch.tensor(_E2M1_GRID, dtype=torch.float32, device=w.device)
    mag = x.abs().clamp(max=6.0)
    dist = (mag[..., None] - grid).abs()
    # exact ties go to the even code (mantissa bit 0)
    dist = dist + (torch.arange(8, device=w.device) & 1).to(torch.float32) * 1e-12
    code = dist.argmin(dim=-1).to(torch.uint8)
    code = torch.where((x < 0) & (code > 0), code | 8, code)
    packed = (code[0::2] | (code[1::2] << 4)).to(torch.uint8)
    return packed.contiguous(), (ex + 127.0).to(torch.uint8).contiguous()


def quantize_mxfp8(w: torch.Tensor):
    """w: [K, N] fp32 (K a multiple of 32) -> (codes [K, N] float8_e4m3fn,
    scales [K/32, N] uint8).  Per block of 32 consecutive k of one column:
    shared exponent floor(log2(max|w|)) - 8 (e4m3's largest binade is 2^8),
    stored biased by 127 (E8M0); each element divided by 2^exponent, clamped
    to +-448 (the largest e4m3fn magnitude) and rounded to the nearest e4m3fn
    value (ties to even).  An all-zero block gets exponent 0 and zero codes."""
    K, N = w.shape
    blk = w.reshape(K // MX_BLOCK, MX_BLOCK, N)
    amax = blk.abs().amax(dim=1)
    ex = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax, 1.0))) - 8.0,
                     torch.zeros_like(amax)).clamp_(-127.0, 127.0)
    x = (blk / torch.exp2(ex)[:, None, :]).reshape(K, N).clamp(-448.0, 448.0)
    return x.to(torch.float8_e4m3fn).contiguous(), (ex + 127.0).to(torch.uint8).contiguous()


@dataclass
class Layer:
    shape: LayerShape
    w_router: torch.Tensor            # [d, E] act dtype
    w_gate_up: torch.Tensor           # [E, d, 2*d_ff] weight dtype (gate cols first)
    w_down: torch.Tensor              # [E, d_ff, d]
    scale_gate_up: Optional[torch.Tensor]  # fp8: [E, 2*d_ff] fp32; MX: [E, d/32, 2*d_ff] uint8
    scale_down: Optional[torch.Tensor]     # fp8: [E, d] fp32; MX: [E, d_ff/32, d] uint8
    bias: Optional[torch.Tensor]      # [E] fp32 router-logit bias or None

    @property
    def device(self):
        return self.w_gate_up.device


def make_bias(shape: LayerShape, s: Optional[float], device="cpu") -> Optional[torch.Tensor]:
    if s is None:
        return None
    g = _gen("cpu", shape.seed, TENSOR_PERM, 0)
    rank = torch.randperm(shape.E, generator=g).to(torch.float64) + 1.0
    return (-float(s) * torch.log(rank)).to(torch.float32).to(device)


def make_router(shape: LayerShape, device="cpu") -> torch.Tensor:
    """W_router[d, E] ~ N(0, 1/d) in the activation dtype (the same draw
    make_layer uses)."""
    return _normal((shape.d, shape.E), shape.d ** -0.5, device, shape.seed, TENSOR_WR, 0).to(
        _TORCH_DT[shape.act])


def make_layer(shape: LayerShape, T: Optional[int] = None, device="cpu",
               zipf: Optional[float] = "auto") -> Layer:
    """Draw the layer of `shape` on `device`.

    The router bias follows the shape's Zipf law for token count T unless
    `zipf` is given explicitly (None for no bias)."""
    E, d, dff = shape.E, shape.d, shape.d_ff
    s = shape.seed
    w_router = make_router(shape, device)
    if shape.wdt == "mxfp4":
        wgu = torch.empty((E, d // 2, 2 * dff), dtype=torch.uint8, device=device)
        wdn = torch.empty((E, dff // 2, d), dtype=torch.uint8, device=device)
        sgu = torch.empty((E, d // MX_BLOCK, 2 * dff), dtype=torch.uint8, device=device)
        sdn = torch.empty((E, dff // MX_BLOCK, d), dtype=torch.uint8, device=device)
    elif shape.wdt == "mxfp8":
        wgu = torch.empty((E, d, 2 * dff), dtype=torch.float8_e4m3fn, device=device)
        wdn = torch.empty((E, dff, d), dtype=torch.float8_e4m3fn, device=device)
        sgu = torch.empty((E, d // MX_BLOCK, 2 * dff), dtype=torch.uint8, device=device)
        sdn = torch.empty((E, dff // MX_BLOCK, d), dtype=torch.uint8, device=device)
    elif shape.wdt == "fp8":
        wgu = torch.empty((E, d, 2 * dff), dtype=torch.float8_e4m3fn, device=device)
        wdn = torch.empty((E, dff, d), dtype=torch.float8_e4m3fn, device=device)
        sgu = torch.empty((E, 2 * dff), dtype=torch.float32, device=device)
        sdn = torch.empty((E, d), dtype=torch.float32, device=device)
    else:
        wdt = _TORCH_DT[shape.wdt]
        wgu = torch.empty((E, d, 2 * dff), dtype=wdt, device=device)
        wdn = torch.empty((E, dff, d), dtype=wdt, device=device)
        sgu = sdn = None
    for e in range(E):
        wg = _normal((d, dff), d ** -0.5, device, s, TENSOR_WG, e)
        wu = _normal((d, dff), d ** -0.5, device, s, TENSOR_WU, e)
        wd = _normal((dff, d), dff ** -0.5, device, s, TENSOR_WD, e)
        if shape.wdt == "mxfp4":
            wgu[e], sgu[e] = quantize_mxfp4(torch.cat([wg, wu], dim=1))
            wdn[e], sdn[e] = quantize_mxfp4(wd)
        elif shape.wdt == "mxfp8":
            wgu[e], sgu[e] = quantize_mxfp8(torch.cat([wg, wu], dim=1))
            wdn[e], sdn[e] = quantize_mxfp8(wd)
        elif shape.wdt == "fp8":
            qg, sg = quantize_e4m3fn_per_column(wg)
            qu, su = quantize_e4m3fn_per_column(wu)
            qd, sd = quantize_e4m3fn_per_column(wd)
            wgu[e, :, :dff] = qg
            wgu[e, :, dff:] = qu
            sgu[e, :dff] = sg
            sgu[e, dff:] = su
            wdn[e] = qd
            sdn[e] = sd
        else:
            wgu[e, :, :dff] = wg.to(wgu.dtype)
            wgu[e, :, dff:] = wu.to(wgu.dtype)
            wdn[e] = wd.to(wdn.dtype)
        del wg, wu, wd
    if zipf == "auto":
        zipf = shape.zipf_for(T) if T is not None else None
    bias = make_bias(shape, zipf, device)
    return Layer(shape, w_router, wgu, wdn, sgu, sdn, bias)


def make_tokens(shape: LayerShape, T: int, device="cpu") -> torch.Tensor:
    """x[T, d] ~ N(0, 1) in the activation dtype."""
    x = _normal((T, shape.d), 1.0, device, shape.seed, TENSOR_X, T)
    return x.to(_TORCH_DT[shape.act])


def make_topk_ids(T: int, E: int, k: int, seed: int, skew: Optional[float] = None,
                  device="cpu") -> torch.Tensor:
    """Seeded routing tables for exercising alignment on its own: each row holds
    k distinct expert ids.  With `skew`, experts are drawn with probability
    proportional to rank^-skew (rank = 1 + expert id), otherwise uniformly."""
    g = _gen("cpu", seed, TENSOR_IDS, T * 1315423911 + E * 2654435761 + k)
    if skew is None:
        keys = torch.rand((T, E), generator=g, dtype=torch.float64)
    else:
        w = torch.arange(1, E + 1, dtype=torch.float64).pow(-float(skew))
        # Gumbel-top-k draws k distinct ids with the given sampling weights
        u = torch.rand((T, E), generator=g, dtype=torch.float64).clamp_(1e-300, 1.0)
        keys = torch.log(w)[None, :] - torch.log(-torch.log(u))
    ids = torch.topk(keys, k, dim=1).indices.to(torch.int32)
    return ids.to(device)
