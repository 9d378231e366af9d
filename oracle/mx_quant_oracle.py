"""CPU oracle of the MXFP8 activation quantiser.

TEST INFRASTRUCTURE.  Plain, slow, obviously-correct definition that the GPU
quantiser is checked against; only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import it, and it imports nothing from
the library (the E4M3 and E8M0 decoders come from the oracle's own
`moe_oracle`, pinned there).

Source: "CuTeDSL at Perplexity", section on Blackwell support: the
block-scaled formats (MXFP8, MXFP4) quantise a tensor in blocks of 32
consecutive elements that share one scale, found from the block's largest
magnitude (an absmax over 32 elements, taken with sub-warp reductions).

Reading R14 (the pages name the formats and the absmax but not how the scale
follows from it): the OCP Microscaling (MX) v1.0 rule for MXFP8 — E4M3 ("fn")
elements, an E8M0 power-of-two scale per block:
  s     = floor(log2(absmax)) - 8        (8: the exponent of E4M3's top binade,
                                          whose largest value is 1.75 * 2^8 = 448)
          clamped to E8M0's range, at least -127; an all-zero block takes -127;
  code  = E4M3(x / 2^s), rounded to nearest with ties to the even code,
          magnitudes above 448 saturated to 448 (x / 2^s < 512 always), the
          sign bit that of x (a negative value that rounds to zero gives -0);
  scale byte = s + 127.
Blocks run along the last axis; its length must be a multiple of 32.  Inputs
are finite; everything is computed in float64 from their exact values.
"""
import numpy as np

from oracle.moe_oracle import MX_BLOCK, decode_e4m3fn, decode_e8m0

E4M3_MAX = 448.0
E4M3_EMAX = 8  # exponent of the top binade [256, 448]


def _e4m3_magnitudes():
    """The finite non-negative E4M3 values in ascending order with their codes
    (0x00..0x7E; 0x7F is NaN), from the format's decoder."""
    codes = np.arange(0x7F)
    vals = decode_e4m3fn(codes)
    order = np.argsort(vals, kind="stable")
    return vals[order], codes[order]


def round_to_e4m3(q: np.ndarray) -> np.ndarray:
    """E4M3 code of each float64 value q: the nearest representable magnitude
    (ties to the code whose last bit is 0), at most 448, with q's sign bit."""
    q = np.asarray(q, dtype=np.float64)
    mag = np.minimum(np.abs(q), E4M3_MAX)
    grid, codes = _e4m3_magnitudes()
    hi_i = np.clip(np.searchsorted(grid, mag, side="left"), 0, len(grid) - 1)
    lo_i = np.clip(hi_i - 1, 0, len(grid) - 1)
    lo, hi = grid[lo_i], grid[hi_i]
    d_lo, d_hi = mag - lo, hi - mag
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi_i] & 1) == 0))
    take_hi |= mag == hi  # exact hit (also when lo == hi at the ends)
    code = np.where(take_hi, codes[hi_i], codes[lo_i]).astype(np.uint8)
    return np.where(np.signbit(q), code | 0x80, code).astype(np.uint8)


def block_exponent(absmax: np.ndarray) -> np.ndarray:
    """s = floor(log2(absmax)) - 8, at least -127; -127 for absmax == 0."""
    absmax = np.asarray(absmax, dtype=np.float64)
    _, e = np.frexp(absmax)  # absmax = m * 2^e, m in [0.5, 1)
    s = (e.astype(np.int64) - 1) - E4M3_EMAX
    s = np.where(absmax == 0.0, -127, s)
    return np.clip(s, -127, 127)


def quantize_mxfp8(x: np.ndarray):
    """(codes uint8 [..., n], scales uint8 [..., n/32]) of x [..., n] by R14."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    if n % MX_BLOCK != 0:
        raise ValueError("the last axis must be a multiple of 32")
    blocks = x.reshape(x.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    s = block_exponent(np.max(np.abs(blocks), axis=-1))
    q = blocks / np.exp2(s.astype(np.float64))[..., None]
    codes = round_to_e4m3(q).reshape(x.shape)
    scales = (s + 127).astype(np.uint8)
    return codes, scales


def dequantize_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """x'[..., i] = e4m3(code[..., i]) * 2^(scale[..., i/32] - 127)."""
    vals = decode_e4m3fn(codes)
    sc = decode_e8m0(scales)
    return vals * np.repeat(sc, MX_BLOCK, axis=-1)
