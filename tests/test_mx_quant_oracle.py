"""Pins of the oracle's MXFP8 quantiser (reading R14, OCP MX rule for MXFP8).

Each pin is something other than the oracle's own code: the rounding step
against torch's float8_e4m3fn cast (round to nearest even) wherever no
saturation applies; saturation, the block exponent and a worked block by hand
from the formats' definitions; a brute-force nearest-code search over all 254
finite codes on small blocks; and error and range invariants on random
blocks.  A dropped clamp, an off-by-one exponent, a wrong tie rule or a lost
sign bit each fail at least one of them."""
import numpy as np
import torch

from oracle import moe_oracle as O
from oracle import mx_quant_oracle as Q


def _torch_e4m3(q):
    t = torch.from_numpy(np.asarray(q, np.float64)).to(torch.float32).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_rounding_matches_torch_cast_including_ties():
    grid = O.decode_e4m3fn(np.arange(0x7F))
    grid = np.sort(grid)
    mids = (grid[:-1] + grid[1:]) / 2          # exact ties between neighbours
    rng = np.random.default_rng(1)
    rand = rng.uniform(-448, 448, 20000)
    tiny = rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000)   # the subnormal range
    q = np.concatenate([grid, -grid, mids, -mids, rand, tiny, [0.0, -0.0]])
    np.testing.assert_array_equal(Q.round_to_e4m3(q), _torch_e4m3(q))


def test_saturation_and_signed_zero():
    q = np.array([448.0, 449.0, 464.0, 480.0, 511.99, -500.0, -448.0])
    np.testing.assert_array_equal(Q.round_to_e4m3(q),
                                  [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE])
    # below half the smallest subnormal (2^-9): zero, keeping the sign
    np.testing.assert_array_equal(Q.round_to_e4m3(np.array([2.0 ** -11, -2.0 ** -11, -0.0])),
                                  [0x00, 0x80, 0x80])


def test_block_exponent_closed_forms():
    e = np.arange(-119, 120)
    np.testing.assert_array_equal(Q.block_exponent(np.exp2(e.astype(float))), e - 8)
    np.testing.assert_array_equal(Q.block_exponent(np.exp2(e.astype(float)) * 1.999), e - 8)
    assert Q.block_exponent(np.array([0.0]))[0] == -127
    assert Q.block_exponent(np.array([2.0 ** -130]))[0] == -127   # clamped
    assert Q.block_exponent(np.array([2.0 ** -119]))[0] == -127
    assert Q.block_exponent(np.array([2.0 ** -118]))[0] == -126
    assert Q.block_exponent(np.array([float(np.finfo(np.float32).max)]))[0] == 119


def test_worked_block():
    # absmax 1.0 -> s = 0 - 8, every element is multiplied by 2^8
    x = np.zeros(32)
    x[0] = 1.0          # 256 = 2^8          -> E=15, M=0 -> 0x78
    x[1] = 0.3          # 76.8 -> 80 = 2^6*1.25 -> E=13, M=2 -> 0x6A
    x[2] = -0.0         # -> 0x80
    x[3] = -2.0 ** -12  # -2^-4 -> E=3, M=0, negative -> 0x98
    x[4] = 1e-30        # far below the smallest subnormal -> 0x00
    x[5] = 0.5 + 1 / 64  # 132 lies between 128 and 144: nearer 128 -> 0x70
    x[6] = 0.53125      # 136: a tie between 128 (M=0) and 144 (M=1) -> even, 128
    codes, scales = Q.quantize_mxfp8(x[None, :])
    assert scales.tolist() == [[119]]
    assert codes[0, :7].tolist() == [0x78, 0x6A, 0x80, 0x98, 0x00, 0x70, 0x70]
    assert not codes[0, 7:].any()


def test_all_zero_and_tiny_blocks():
    x = np.zeros((2, 64))
    x[1, 32:] = 2.0 ** -125 * np.arange(1, 33) / 32   # absmax 2^-125: clamped scale
    codes, scales = Q.quantize_mxfp8(x)
    assert scales.tolist() == [[0, 0], [0, 0]]
    assert not codes[0].any() and not codes[1, :32].any()
    # with the scale clamped at 2^-127 the values are x * 2^127 <= 4
    np.testing.assert_array_equal(O.decode_e4m3fn(codes[1, 32:]),
                                  O.decode_e4m3fn(Q.round_to_e4m3(x[1, 32:] * 2.0 ** 127)))


def test_bruteforce_nearest_code():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 64)) * np.exp2(rng.integers(-20, 20, (3, 1)))
    x[0, 5] = 0.0
    codes, scales = Q.quantize_mxfp8(x)
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    vals = {c: float(O.decode_e4m3fn(np.array([c]))[0]) for c in finite}
    for r in range(3):
        for i in range(64):
            sc = 2.0 ** (int(scales[r, i // 32]) - 127)
            best = None
            for c in finite:
                err = abs(vals[c] * sc - x[r, i])
                key = (err, c & 1, np.signbit(vals[c]) != np.signbit(x[r, i]))
                if best is None or key < best[0]:
                    best = (key, c)
            got = int(codes[r, i])
            assert vals[got] * sc == vals[best[1]] * sc, (r, i, got, best)
            assert np.signbit(vals[got]) == np.signbit(x[r, i])


def test_error_and_range_invariants():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-30, 30, (64, 1)))).astype(np.float32)
    x = x.astype(np.float64)
    codes, scales = Q.quantize_mxfp8(x)
    assert not np.isin(codes, [0x7F, 0xFF]).any()
    back = Q.dequantize_mxfp8(codes, scales)
    s = np.repeat(scales.astype(np.int64) - 127, 32, axis=-1).astype(float)
    sat = np.abs(x) >= 448 * np.exp2(s)
    assert sat.any()
    # saturated elements decode to +-448 * 2^s; the others lie within half
    # a step of E4M3 (2^-4 relative for normals, 2^-10 * 2^s for subnormals)
    np.testing.assert_array_equal(back[sat], np.sign(x[sat]) * 448 * np.exp2(s[sat]))
    bound = np.maximum(2.0 ** -4 * np.abs(x), np.exp2(s - 10))
    assert np.all(np.abs(back - x)[~sat] <= bound[~sat])
    # each block's largest element lands in the top binade [256, 448] * 2^s
    blk = np.abs(back).reshape(64, 8, 32).max(axis=-1)
    sc = np.exp2(scales.astype(float) - 127)
    assert np.all(blk >= 256 * sc) and np.all(blk <= 448 * sc)


def test_agrees_with_the_weight_generator_on_nonzero_blocks():
    # the harness's weight quantiser states the same rule and rounds with
    # torch's cast; it differs only on all-zero blocks (it stores exponent 0)
    from workloads.gen import quantize_mxfp8 as harness_q
    rng = np.random.default_rng(11)
    w = rng.standard_normal((128, 48)).astype(np.float32)
    c_h, s_h = harness_q(torch.from_numpy(w))
    codes, scales = Q.quantize_mxfp8(w.astype(np.float64).T)  # blocks along K
    np.testing.assert_array_equal(codes.T, c_h.view(torch.uint8).numpy())
    np.testing.assert_array_equal(scales.T, s_h.numpy())
