"""Seeded activation rows for the MXFP8 quantiser: x [rows, n].

Values are N(0, 1) scaled per row by 2^u, u uniform in [-3, 3], and in about
1 % of the columns (the same columns in every row, as outlier channels of
hidden states) by a further 2^v, v uniform in [3, 8], so that blocks of one
row take scales spread over a dozen binades.  Drawn in fp32, stored in the
requested dtype (RNE for bf16).  Nothing here computes any part of the
quantisation."""
import torch

from .gen import _gen

TENSOR_VALUES, TENSOR_ROW_SCALE, TENSOR_OUTLIER_COLS, TENSOR_OUTLIER_SCALE = range(320, 324)
_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def make_mx_rows(rows: int, n: int, dtype: str = "bf16", seed: int = 0, device="cpu"):
    x = torch.randn((rows, n), generator=_gen(device, seed, TENSOR_VALUES, rows), device=device)
    u = torch.rand((rows, 1), generator=_gen(device, seed, TENSOR_ROW_SCALE, rows), device=device)
    cols = torch.rand(n, generator=_gen(device, seed, TENSOR_OUTLIER_COLS, n), device=device) < 0.01
    v = torch.rand(n, generator=_gen(device, seed, TENSOR_OUTLIER_SCALE, n), device=device)
    col_scale = torch.where(cols, torch.exp2(3.0 + 5.0 * v), torch.ones_like(v))
    x = x * torch.exp2(u * 6.0 - 3.0) * col_scale
    return x.to(_DT[dtype]).contiguous()
