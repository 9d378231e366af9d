"""CPU oracle of the per-head RMS normalisation of query and key heads (QK-norm).

TEST INFRASTRUCTURE.  The plain, slow, obviously-correct definition that the
GPU QK-norm is checked against.  Only the test suite, the package smoke check
and the benchmark may import it; the library never does, and this module
imports nothing from the library.  Computed in NumPy float64 from the exact
input values (bf16 decoded bit-exactly, fp32 widened).

Source: "CuTeDSL at Perplexity", section on the RMS-norm kernel specialised for
small dimensions (QK-norm of recent Qwen models): the norm is applied per
attention head over 64, 128 or 256 elements; for every token and every head of
q and of k, with x the head's values and w the weight of its tensor (one value
per position in the head, shared by all heads of that tensor),
    r = (w + WEIGHT_BIAS) * x * rsqrt(sum(x * x) / head_dim + EPS),
written back in the element type.  The section's one-line formula omits the
reciprocal square root that its kernel listing applies; the listing's form is
the one taken here.
"""
import numpy as np


def qk_norm(x: np.ndarray, w: np.ndarray, weight_bias: float, eps: float) -> np.ndarray:
    """x [..., head_dim] float64, w [head_dim] float64 -> normalised heads
    (float64): the mean of squares over the last axis, its reciprocal square
    root, then the biased weight."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return (w + weight_bias) * (x * (1.0 / np.sqrt(ms + eps)))


def qk_norm_pair(q: np.ndarray, k: np.ndarray, wq: np.ndarray, wk: np.ndarray,
                 weight_bias: float, eps: float):
    """q [T, nq, hd], k [T, nk, hd]: each tensor with its own weight."""
    return qk_norm(q, wq, weight_bias, eps), qk_norm(k, wk, weight_bias, eps)


def qk_norm_bruteforce(x, w, weight_bias: float, eps: float) -> np.ndarray:
    """The same definition with explicit Python loops (tiny inputs only)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    hd = x.shape[-1]
    flat = x.reshape(-1, hd)
    of = out.reshape(-1, hd)
    for r in range(flat.shape[0]):
        s = 0.0
        for i in range(hd):
            s += float(flat[r, i]) * float(flat[r, i])
        inv = 1.0 / (s / hd + eps) ** 0.5
        for i in range(hd):
            of[r, i] = (float(w[i]) + weight_bias) * (float(flat[r, i]) * inv)
    return out
