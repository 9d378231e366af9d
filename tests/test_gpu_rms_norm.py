"""moe_rms_norm (one-pass row RMSNorm) against the fp64 oracle, element by
element, on every row.

Tolerances, derived from the arithmetic: the kernel sums the squares of a row
in fp32 (for rows of up to 16384 values the relative error of the sum, and so
of the common scale, stays well below 2^-13), takes a reciprocal square root
within ~2 ulp, and rounds each value once to the element type.
  * bf16: one round-to-nearest-even to bf16 is within 2^-8 relative, so
    |got - ref| <= (2^-8 + 2^-13) * |ref| (a zero row stays exactly zero);
  * fp32: |got - ref| <= 1e-5 * (|ref| + RMS(ref row)).
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_align_amd import _binding as B
from oracle import rms_norm_oracle as N
from workloads.norm import make_rows

pytestmark = pytest.mark.gpu


def _np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _check(got, ref, dtype, what):
    if dtype == "bf16":
        bad = np.abs(got - ref) > (2.0 ** -8 + 2.0 ** -13) * np.abs(ref)
    else:
        rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
        bad = np.abs(got - ref) > 1e-5 * (np.abs(ref) + rms)
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance; worst "
                           f"{np.max(np.abs(got - ref)[bad]):.3e}")


CASES = [
    # T, d, dtype, weight_bias, eps
    (1, 7168, "bf16", 0.0, 1e-6),     # a decode token of the E=256 layer's hidden size
    (16, 4096, "bf16", 0.0, 1e-6),
    (8192, 2048, "bf16", 0.0, 1e-6),  # the E=128 layer's hidden size, a prefill batch
    (4096, 7168, "bf16", 1.0, 1e-5),  # biased gain
    (300, 5120, "bf16", 0.0, 1e-6),   # pieces per lane not a multiple of the bucket
    (77, 96, "bf16", 0.0, 1e-6),      # 12 pieces: fewer than a wave, not a power of two
    (33, 64, "bf16", 0.5, 0.0),       # 8 pieces: eight rows per wave, eps = 0
    (9, 16384, "bf16", 0.0, 1e-6),    # the largest bf16 row
    (100, 2048, "f32", 0.0, 1e-6),
    (5, 8192, "f32", 0.25, 1e-5),     # the largest fp32 row
    (65, 4, "f32", 0.0, 1e-6),        # one piece per row
    (0, 2048, "bf16", 0.0, 1e-6),     # empty batch
]


@pytest.mark.parametrize("T,d,dtype,bias,eps", CASES)
def test_rms_norm_matches_oracle(T, d, dtype, bias, eps):
    print(f"rms_norm T={T} d={d} {dtype} bias={bias} eps={eps}", flush=True)
    x, g = make_rows(T, d, dtype, seed=T + 7 * d, device="cuda")
    x0, g0 = _np64(x), _np64(g)
    y = B.rms_norm(x, g, weight_bias=bias, eps=eps)
    torch.cuda.synchronize()
    if T == 0:
        return
    _check(_np64(y), N.rms_norm(x0, g0, eps, bias), dtype, "out")
    np.testing.assert_array_equal(_np64(x), x0)  # input untouched out of place
    # in place gives the same bits
    B.rms_norm(x, g, out=x, weight_bias=bias, eps=eps)
    torch.cuda.synchronize()
    assert torch.equal(x, y)


def test_rms_norm_zero_row_stays_zero_and_is_deterministic():
    x, g = make_rows(50, 4096, "bf16", seed=9, device="cuda")
    x[17].zero_()
    a = B.rms_norm(x, g, eps=1e-6)
    b = B.rms_norm(x, g, eps=1e-6)
    torch.cuda.synchronize()
    assert torch.count_nonzero(a[17]) == 0
    assert torch.equal(a, b)
