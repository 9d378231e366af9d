"""Pins of the oracle's microscaling (MXFP4, MXFP8) decoding and of the
harness's MX quantizers.

E2M1 is pinned by its defining properties (eight magnitudes 0, 0.5, 1, 1.5,
2, 3, 4, 6 in code order, a sign bit), E8M0 against torch's own
float8_e8m0fnu, the storage layout by hand-worked bytes, and the block scales
by the factoring identity a GEMM over MXFP4 weights relies on."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from workloads.gen import quantize_mxfp4, quantize_mxfp8


def test_e2m1_magnitudes_and_sign():
    v = O.decode_e2m1(np.arange(16))
    np.testing.assert_array_equal(v[:8], [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    np.testing.assert_array_equal(v[8:], -v[:8])
    assert np.signbit(v[8])  # code 8 is negative zero
    # the high nibble of a byte is ignored by the per-code decoder
    np.testing.assert_array_equal(O.decode_e2m1(np.arange(16) | 0xF0), v)


def test_e8m0_matches_torch():
    codes = np.arange(255, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.decode_e8m0(codes), want)
    assert np.isnan(O.decode_e8m0(np.array([255])))[0]
    assert O.decode_e8m0(np.array([127]))[0] == 1.0


def test_mxfp4_layout_hand_worked():
    # one 32-row block, two columns: byte 0x21 holds k=0 -> code 1 (0.5),
    # k=1 -> code 2 (1.0); 0xF7 holds +6 (code 7) and -6 (code 15)
    packed = np.zeros((16, 2), np.uint8)
    packed[0, 0] = 0x21
    packed[0, 1] = 0xF7
    packed[5, 1] = 0x40          # k=10 -> 0, k=11 -> code 4 (2.0)
    scales = np.array([[127, 128]], np.uint8)  # 1.0 and 2.0
    w = O.decode_mxfp4(packed, scales)
    assert w.shape == (32, 2)
    assert (w[0, 0], w[1, 0]) == (0.5, 1.0)
    assert (w[0, 1], w[1, 1]) == (12.0, -12.0)
    assert (w[10, 1], w[11, 1]) == (0.0, 4.0)
    assert np.count_nonzero(w) == 5


def test_mxfp4_scale_applies_to_its_32_rows_only():
    K, N = 96, 3
    packed = np.full((K // 2, N), 0x22, np.uint8)   # every code 2 = 1.0
    scales = np.array([[120, 127, 130], [127, 127, 127], [140, 100, 127]], np.uint8)
    w = O.decode_mxfp4(packed, scales)
    for b in range(3):
        for n in range(N):
            np.testing.assert_array_equal(w[32 * b:32 * (b + 1), n],
                                          2.0 ** (int(scales[b, n]) - 127))


def test_block_factoring_identity():
    # sum_k a_k W[k,n] = sum_b 2^(e_b-127) * sum_{k in b} a_k e2m1(q_kn), exactly
    rng = np.random.default_rng(0)
    K, N = 128, 5
    codes = rng.integers(0, 16, (K, N)).astype(np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    scales = rng.integers(110, 140, (K // 32, N)).astype(np.uint8)
    a = rng.integers(-8, 9, K).astype(np.float64)  # small integers: every sum exact
    lhs = a @ O.decode_mxfp4(packed, scales)
    q = O.decode_e2m1(codes)
    rhs = np.zeros(N)
    for b in range(K // 32):
        rhs += O.decode_e8m0(scales[b]) * (a[32 * b:32 * (b + 1)] @ q[32 * b:32 * (b + 1)])
    np.testing.assert_array_equal(lhs, rhs)


def test_quantizer_reproduces_representable_weights():
    # weights already on the E2M1 grid times a block scale whose block maximum
    # is 6 * 2^s come back exactly
    rng = np.random.default_rng(1)
    K, N = 64, 4
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    mags = grid[rng.integers(0, 8, (K, N))]
    mags[0::32] = 6.0                        # block maximum 6
    sign = np.where(rng.random((K, N)) < 0.5, -1.0, 1.0)
    ex = rng.integers(-6, 3, (K // 32, N))
    w = sign * mags * np.exp2(np.repeat(ex, 32, axis=0))
    packed, scales = quantize_mxfp4(torch.tensor(w, dtype=torch.float32))
    np.testing.assert_array_equal(O.decode_mxfp4(packed.numpy(), scales.numpy()), w)
    np.testing.assert_array_equal(scales.numpy().astype(np.int64) - 127, ex)


@pytest.mark.parametrize("seed", [2, 3])
def test_quantizer_error_within_half_a_grid_step(seed):
    rng = np.random.default_rng(seed)
    w = rng.normal(0, 0.05, (128, 16)).astype(np.float32)
    packed, scales = quantize_mxfp4(torch.from_numpy(w))
    d = O.decode_mxfp4(packed.numpy(), scales.numpy())
    X = np.repeat(O.decode_e8m0(scales.numpy()), 32, axis=0)
    # widest E2M1 gap is 2 (between 4 and 6); values beyond 6 clamp to 6 but
    # stay below 8 by the exponent choice
    assert np.all(np.abs(d - w) <= 2.0 * X)
    assert np.all(np.abs(w) < 8.0 * X)


# ---------------------------------------------------------------- MXFP8

def test_mxfp8_layout_hand_worked():
    # one 32-row block, two columns: e4m3fn 0x38 = 1.0, 0xB8 = -1.0, 0x7E = 448,
    # 0x01 = 2^-9 (smallest subnormal); scales 2^0 and 2^1
    codes = np.zeros((32, 2), np.uint8)
    codes[0, 0], codes[5, 0], codes[31, 0] = 0x38, 0xB8, 0x01
    codes[0, 1], codes[1, 1] = 0x7E, 0x40          # 448 and 2.0
    scales = np.array([[127, 128]], np.uint8)
    w = O.decode_mxfp8(codes, scales)
    assert (w[0, 0], w[5, 0], w[31, 0]) == (1.0, -1.0, 2.0 ** -9)
    assert (w[0, 1], w[1, 1]) == (896.0, 4.0)
    assert np.count_nonzero(w) == 5


def test_mxfp8_scale_applies_to_its_32_rows_only():
    K, N = 96, 3
    codes = np.full((K, N), 0x38, np.uint8)             # every code 1.0
    scales = np.array([[120, 127, 130], [127, 127, 127], [140, 100, 127]], np.uint8)
    w = O.decode_mxfp8(codes, scales)
    for b in range(3):
        for n in range(N):
            np.testing.assert_array_equal(w[32 * b:32 * (b + 1), n],
                                          2.0 ** (int(scales[b, n]) - 127))


def test_mxfp8_codes_match_torch_e4m3fn():
    codes = np.arange(256, dtype=np.uint8).reshape(256, 1)   # 8 blocks of 32
    scales = np.full((8, 1), 127, np.uint8)                     # scale 1
    want = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_mxfp8(codes, scales)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])


def test_mxfp8_quantizer_reproduces_representable_weights():
    # e4m3fn values times a block scale whose block maximum is 1.75 * 2^8 * 2^s
    rng = np.random.default_rng(4)
    K, N = 64, 5
    grid = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mags = grid[rng.integers(0, grid.size, (K, N))]
    mags[0::32] = 448.0
    sign = np.where(rng.random((K, N)) < 0.5, -1.0, 1.0)
    ex = rng.integers(-20, 5, (K // 32, N))
    w = sign * mags * np.exp2(np.repeat(ex, 32, axis=0))
    codes, scales = quantize_mxfp8(torch.tensor(w, dtype=torch.float32))
    d = O.decode_mxfp8(codes.view(torch.uint8).numpy(), scales.numpy())
    np.testing.assert_array_equal(d, w)
    np.testing.assert_array_equal(scales.numpy().astype(np.int64) - 127, ex)


@pytest.mark.parametrize("seed", [5, 6])
def test_mxfp8_quantizer_error_within_half_a_step(seed):
    rng = np.random.default_rng(seed)
    w = rng.normal(0, 0.05, (128, 16)).astype(np.float32)
    w[0, 0] = 0.0
    codes, scales = quantize_mxfp8(torch.from_numpy(w))
    d = O.decode_mxfp8(codes.view(torch.uint8).numpy(), scales.numpy())
    X = np.repeat(O.decode_e8m0(scales.numpy()), 32, axis=0)
    wa = np.abs(w.astype(np.float64))
    # normal range: half of the 3-bit mantissa step; subnormals: half of 2^-9;
    # above 448*X (at most 512*X by the exponent choice) saturation to 448*X
    bound = np.maximum(wa * 2.0 ** -4, X * 2.0 ** -10)
    sat = wa > 448.0 * X
    assert np.all(np.abs(d - w)[~sat] <= bound[~sat])
    assert np.all(np.abs(d[sat]) == 448.0 * X[sat]) and np.all(wa < 512.0 * X)
    assert d[0, 0] == 0.0


def test_mxfp8_zero_block():
    w = torch.zeros((32, 3))
    codes, scales = quantize_mxfp8(w)
    assert (scales.numpy() == 127).all()
    assert (O.decode_mxfp8(codes.view(torch.uint8).numpy(), scales.numpy()) == 0).all()
