"""CPU oracle of the row RMS normalisation (RMSNorm) over the hidden size.

TEST INFRASTRUCTURE.  The plain, slow, obviously-correct definition that the
GPU row RMSNorm is checked against.  Only the test suite, the package smoke
check and the benchmark may import it; the library never does, and this
module imports nothing from the library.  Computed in NumPy float64 from the
exact input values (bf16 decoded bit-exactly, fp32 widened).

Source: "La fusion de noyaux", section 4.2, reduction + elementwise fusion:
for a row x of d values and a gain g of d values,
    y_i = x_i / sqrt((1/d) * sum_j x_j^2 + eps) * g_i,
accumulated in fp32 by the fused kernel (one load of x, one store of y).
"CuTeDSL at Perplexity" (the library overview and its RMS-norm section)
notes that some models add a constant bias to the weight; that variant is
the gain g + weight_bias, with weight_bias = 0 giving the formula above.
"""
import numpy as np


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float, weight_bias: float = 0.0) -> np.ndarray:
    """x [..., d] float64, g [d] float64: every row divided by the square root
    of its mean square plus eps, then multiplied by the (biased) gain."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    mean_sq = np.sum(x * x, axis=-1, keepdims=True) / x.shape[-1]
    return x / np.sqrt(mean_sq + eps) * (g + weight_bias)


def rms_norm_bruteforce(x, g, eps: float, weight_bias: float = 0.0) -> np.ndarray:
    """The same definition with explicit Python loops (tiny inputs only)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    flat = x.reshape(-1, d)
    out = np.empty_like(flat)
    for r in range(flat.shape[0]):
        s = 0.0
        for j in range(d):
            s += float(flat[r, j]) ** 2
        den = (s / d + eps) ** 0.5
        for i in range(d):
            out[r, i] = float(flat[r, i]) / den * (float(g[i]) + weight_bias)
    return out.reshape(x.shape)
