"""Seeded QK-norm inputs: q [T, nq, hd], k [T, nk, hd] and their weights [hd].

Each head's values are N(0, s^2) with s drawn per (token, head) log-uniformly
in [1/8, 8], so heads of very different magnitudes meet one kernel; weights are
N(1, 0.1^2).  Values are drawn in fp32 and stored in the requested dtype (RNE
for bf16).  Nothing here computes any part of the norm."""
import torch

from .gen import _gen

TENSOR_Q, TENSOR_K, TENSOR_WQ, TENSOR_WK, TENSOR_SQ, TENSOR_SK = range(300, 306)
_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _heads(T, n, hd, seed, tv, ts, device):
    x = torch.randn((T, n, hd), generator=_gen(device, seed, tv, T), device=device)
    u = torch.rand((T, n, 1), generator=_gen(device, seed, ts, T), device=device)
    return x * torch.exp2(u * 6.0 - 3.0)


def make_qk(T: int, nq: int, nk: int, hd: int, dtype: str = "bf16", seed: int = 0,
            device="cpu"):
    dt = _DT[dtype]
    q = _heads(T, nq, hd, seed, TENSOR_Q, TENSOR_SQ, device).to(dt).contiguous()
    k = _heads(T, nk, hd, seed, TENSOR_K, TENSOR_SK, device).to(dt).contiguous()
    wq = (1.0 + 0.1 * torch.randn(hd, generator=_gen(device, seed, TENSOR_WQ), device=device)).to(dt)
    wk = (1.0 + 0.1 * torch.randn(hd, generator=_gen(device, seed, TENSOR_WK), device=device)).to(dt)
    return q, k, wq, wk
