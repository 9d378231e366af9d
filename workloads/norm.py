"""Seeded row-RMSNorm inputs: hidden-state rows x [T, d] and a gain [d].

Each row's values are N(0, s^2) with s drawn per row log-uniformly in
[1/8, 8] (rows of very different magnitudes meet one kernel); the gain is
N(1, 0.1^2).  Values are drawn in fp32 and stored in the requested dtype (RNE
for bf16).  Nothing here computes any part of the norm."""
import torch

from .gen import _gen

TENSOR_ROWS, TENSOR_ROW_SCALE, TENSOR_GAIN = range(310, 313)
_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def make_rows(T: int, d: int, dtype: str = "bf16", seed: int = 0, device="cpu"):
    dt = _DT[dtype]
    x = torch.randn((T, d), generator=_gen(device, seed, TENSOR_ROWS, T), device=device)
    u = torch.rand((T, 1), generator=_gen(device, seed, TENSOR_ROW_SCALE, T), device=device)
    x = (x * torch.exp2(u * 6.0 - 3.0)).to(dt).contiguous()
    g = (1.0 + 0.1 * torch.randn(d, generator=_gen(device, seed, TENSOR_GAIN, d),
                                 device=device)).to(dt)
    return x, g
