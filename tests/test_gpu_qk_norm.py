"""moe_qk_norm (per-head RMS normalisation of q and k, in place) against the
fp64 oracle, element by element.

Tolerances, derived from the arithmetic: the kernel sums squares and scales in
fp32 (relative error a few 1e-7, the reciprocal square root within ~2 ulp) and
rounds once to the element type.
  * bf16: one round-to-nearest-even to bf16 is within 2^-9 relative of the
    fp32 value, which is itself within ~1e-6 of the exact one, so
    |got - ref| <= 2^-8 * |ref| (a zero head stays exactly zero).
  * fp32: |got - ref| <= 1e-5 * (|ref| + RMS(ref head)).
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_align_amd import _binding as B
from oracle import qk_norm_oracle as Q
from workloads.qk import make_qk

pytestmark = pytest.mark.gpu


def _np64(t):
    return t.detach().to("cpu", torch.float64).numpy() if t is not None else None


def _check(got, ref, dtype, what):
    got = got.astype(np.float64)
    if dtype == "bf16":
        bad = np.abs(got - ref) > 2.0 ** -8 * np.abs(ref)
    else:
        rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
        bad = np.abs(got - ref) > 1e-5 * (np.abs(ref) + rms)
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance; worst "
                           f"{np.max(np.abs(got - ref)[bad]):.3e}")


CASES = [
    # T, nq, nk, head_dim, dtype, weight_bias, eps
    (1, 32, 4, 128, "bf16", 0.0, 1e-6),
    (7, 1, 0, 64, "bf16", 1.0, 1e-5),       # q only, biased weight
    (33, 0, 3, 256, "bf16", 0.0, 1e-6),     # k only
    (64, 32, 4, 128, "bf16", 0.0, 1e-6),
    (100, 16, 2, 64, "f32", 0.5, 1e-6),
    (5, 2, 2, 256, "f32", 0.0, 0.0),        # eps = 0
    (513, 3, 5, 64, "bf16", 0.0, 1e-6),     # ragged: heads do not fill the last wave
    (257, 7, 1, 256, "f32", 0.0, 1e-6),
    (0, 4, 1, 128, "bf16", 0.0, 1e-6),      # empty batch
]


@pytest.mark.parametrize("T,nq,nk,hd,dtype,bias,eps", CASES)
def test_qk_norm_matches_oracle(T, nq, nk, hd, dtype, bias, eps):
    print(f"qk_norm T={T} nq={nq} nk={nk} hd={hd} {dtype} bias={bias} eps={eps}", flush=True)
    q, k, wq, wk = make_qk(T, nq, nk, hd, dtype, seed=T + 31 * hd, device="cuda")
    q0, k0, wq0, wk0 = _np64(q), _np64(k), _np64(wq), _np64(wk)
    B.qk_norm(q if nq else None, k if nk else None, wq if nq else None, wk if nk else None,
              weight_bias=bias, eps=eps)
    torch.cuda.synchronize()
    rq, rk = Q.qk_norm_pair(q0, k0, wq0, wk0, bias, eps)
    if nq:
        _check(_np64(q), rq, dtype, "q")
    if nk:
        _check(_np64(k), rk, dtype, "k")
    np.testing.assert_array_equal(_np64(wq), wq0)  # weights untouched
    np.testing.assert_array_equal(_np64(wk), wk0)


def test_qk_norm_zero_head_stays_zero_and_is_deterministic():
    q, k, wq, wk = make_qk(40, 8, 2, 128, "bf16", seed=5, device="cuda")
    q[3, 2].zero_()
    q2, k2 = q.clone(), k.clone()
    B.qk_norm(q, k, wq, wk, eps=1e-6)
    B.qk_norm(q2, k2, wq, wk, eps=1e-6)
    torch.cuda.synchronize()
    assert torch.count_nonzero(q[3, 2]) == 0
    assert torch.equal(q, q2) and torch.equal(k, k2)


def test_qk_norm_large_batch_full_check():
    # the benchmarked shape (32 query heads, 4 key heads of 128, 8192 tokens)
    q, k, wq, wk = make_qk(8192, 32, 4, 128, "bf16", seed=11, device="cuda")
    q0, k0, wq0, wk0 = _np64(q), _np64(k), _np64(wq), _np64(wk)
    B.qk_norm(q, k, wq, wk, eps=1e-6)
    torch.cuda.synchronize()
    rq, rk = Q.qk_norm_pair(q0, k0, wq0, wk0, 0.0, 1e-6)
    _check(_np64(q), rq, "bf16", "q")
    _check(_np64(k), rk, "bf16", "k")
