"""moe_quantize_mxfp8 against the oracle's quantiser, bit for bit.

Codes and scale bytes are integer results, so the bar is exact equality.
Both sides decide from the same values: the oracle from the exact float64
input, the kernel from fp32, in which every bf16 and fp32 input, its absmax
and x * 2^-s are exact, so the rounding decisions coincide.

Cases: every finite bf16 value (in ascending order, so that blocks of one
binade meet every scale byte, and shuffled), ragged shapes (block counts not
a multiple of four: the scale words at the end), zero, negative-zero, tiny
(subnormal) and saturating blocks, fp32 inputs, and the benchmarked shape
(16384 x 7168 bf16) on sampled rows.  Guard bytes after both outputs must
stay untouched."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_align_amd import _binding as B
from oracle import mx_quant_oracle as Q
from workloads.mxq import make_mx_rows

pytestmark = pytest.mark.gpu

GUARD = 256


def _np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _quantize_guarded(x):
    """Run the kernel into buffers with GUARD sentinel bytes after each output."""
    rows, n = x.shape
    cbuf = torch.full((rows * n + GUARD,), 0xA5, dtype=torch.uint8, device=x.device)
    sbuf = torch.full((rows * n // 32 + GUARD,), 0x5A, dtype=torch.uint8, device=x.device)
    codes = cbuf[: rows * n].view(rows, n)
    scales = sbuf[: rows * n // 32].view(rows, n // 32)
    B.quantize_mxfp8(x, codes, scales)
    torch.cuda.synchronize()
    assert bool((cbuf[rows * n:] == 0xA5).all()), "codes written past the end"
    assert bool((sbuf[rows * n // 32:] == 0x5A).all()), "scales written past the end"
    return codes.cpu().numpy(), scales.cpu().numpy()


def _check(x, what):
    got_c, got_s = _quantize_guarded(x)
    want_c, want_s = Q.quantize_mxfp8(_np64(x))
    bad_s = np.argwhere(got_s != want_s)
    assert bad_s.size == 0, f"{what}: {len(bad_s)} scale bytes differ, first {bad_s[:4].tolist()}"
    bad = np.argwhere(got_c != want_c)
    if bad.size:
        r, i = bad[0]
        raise AssertionError(f"{what}: {len(bad)} codes differ; first at {r},{i}: x="
                             f"{_np64(x)[r, i]!r} got {got_c[r, i]:#04x} want {want_c[r, i]:#04x}")


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]          # drop infinities and NaNs
    vals = (bits << 16).view(np.float32)
    return vals


def test_every_finite_bf16_value_in_order():
    vals = np.sort(_all_finite_bf16())
    pad = (-len(vals)) % 256
    vals = np.concatenate([vals, np.zeros(pad, np.float32)])
    x = torch.from_numpy(vals.reshape(-1, 256)).to(torch.bfloat16).cuda()
    print(f"mx_quant exhaustive bf16 ordered rows={x.shape[0]}", flush=True)
    _check(x, "every bf16, ascending")


def test_every_finite_bf16_value_shuffled():
    vals = _all_finite_bf16()
    vals = vals[np.random.default_rng(5).permutation(len(vals))]
    pad = (-len(vals)) % 96
    vals = np.concatenate([vals, np.zeros(pad, np.float32)])
    x = torch.from_numpy(vals.reshape(-1, 96)).to(torch.bfloat16).cuda()
    print(f"mx_quant exhaustive bf16 shuffled rows={x.shape[0]}", flush=True)
    _check(x, "every bf16, shuffled")


SHAPES = [
    # rows, n, dtype
    (1, 32, "bf16"), (3, 32, "bf16"), (5, 96, "bf16"), (7, 224, "f32"), (1, 32, "f32"),
    (64, 7168, "bf16"), (33, 2048, "bf16"), (129, 4096, "f32"), (1000, 160, "bf16"),
]


@pytest.mark.parametrize("rows,n,dtype", SHAPES)
def test_random_rows(rows, n, dtype):
    print(f"mx_quant rows={rows} n={n} {dtype}", flush=True)
    x = make_mx_rows(rows, n, dtype, seed=rows + n, device="cuda")
    _check(x, f"{rows}x{n} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_special_blocks(dtype):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    n = 32 * 8
    x = torch.zeros((4, n), dtype=torch.float64)
    x[0, 32:64] = -0.0                                   # negative zeros
    x[0, 64:96] = 2.0 ** -130 * torch.arange(1, 33)      # subnormal bf16 / fp32 values
    x[0, 96:128] = -2.0 ** -140                          # tiny, one value
    x[1, 0:32] = 1.9375                                  # q = 496: saturates to 448
    x[1, 32] = 1.9375
    x[1, 33:64] = 2.0 ** -10                             # beside a saturating max
    x[1, 64:96] = torch.linspace(-3.0, 3.0, 32)
    x[2, :] = 2.0 ** 100 * torch.randn(n, generator=torch.Generator().manual_seed(1))
    x[3, :] = 2.0 ** -100 * torch.randn(n, generator=torch.Generator().manual_seed(2))
    x[3, 0:32] = torch.tensor([0.53125, 0.515625] * 16)  # ties and near-ties at 2^8
    x[3, 5] = 1.0
    _check(x.to(dt).cuda(), f"special blocks {dtype}")


def test_zero_rows_is_a_no_op():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    c, s = B.quantize_mxfp8(x)
    torch.cuda.synchronize()
    assert c.shape == (0, 64) and s.shape == (0, 2)


def test_benchmarked_shape_sampled_rows_and_determinism():
    rows, n = 16384, 7168
    x = make_mx_rows(rows, n, "bf16", seed=3, device="cuda")
    print(f"mx_quant rows={rows} n={n} bf16 (sampled rows)", flush=True)
    c1, s1 = B.quantize_mxfp8(x)
    c2, s2 = B.quantize_mxfp8(x)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
    pick = np.sort(np.random.default_rng(9).choice(rows, 256, replace=False))
    pick = np.concatenate([[0], pick, [rows - 1]])
    idx = torch.from_numpy(pick).cuda()
    want_c, want_s = Q.quantize_mxfp8(_np64(x[idx]))
    np.testing.assert_array_equal(s1[idx].cpu().numpy(), want_s)
    np.testing.assert_array_equal(c1[idx].cpu().numpy(), want_c)
