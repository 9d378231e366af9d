"""CPU oracle of the fused Mixture-of-Experts layer forward.

TEST INFRASTRUCTURE.  This module is the plain, slow, obviously-correct
definition that the GPU library is checked against.  Only the test suite, the
package smoke check and the benchmark's CPU-baseline leg may import it; the
library itself never does, and this module imports nothing from the library.

Everything is computed in NumPy float64 from the exact input values: bf16 and
OCP e4m3fn inputs are decoded bit-exactly by the decoders below, fp32 inputs
are widened.  No step is blocked, fused or reordered beyond what its
definition states.

Sources (the pages describe the computation, never a reference implementation):
  * "CuTeDSL at Perplexity", MoE dispatch and combine, local (TP=1) kernel: the
    router produces a routing table; dispatch counts the tokens routed to each
    expert and gives every token a unique index in its expert's list; tokens go
    to optionally padded per-expert buffers for the MoE GEMM; combine
    accumulates each token's expert outputs, weighted, from those positions.
  * vLLM fused-MoE post (spke.com), section "Swap-AB": expert compute is
    A[M,K] x B[K,N] -> C[M,N] with M token rows, K the hidden size, N the expert
    output width.
  * "La fusion de noyaux", section 4.2, GEMM + GEMM: the gated MLP is
    SwiGLU(x) = (SiLU(x W_gate) * (x W_up)) W_down, and W_gate, W_up are
    concatenated into one d x 2*d_ff GEMM.
  * The router rule (softmax over E, top-k with ties to the lower index,
    renormalise to sum 1) and the output formula sum_k w_k * SwiGLU_k(x) come
    from the workload statement, not from the pages.

Readings where the sources are silent:
  R1 the logit bias is added before selection and before the softmax;
  R2 slot j holds the j-th largest logit, ties to the lower expert index;
  R3 the top-k decision is taken on logits rounded to the kernel's precision
     (fp32), the weights from the float64 logits;
  R4 padded block size bm is an argument; padding slots hold -1;
  R5 within an expert, entries are in ascending (token, slot) order;
  R6 gate columns come first in the concatenated weight, then up columns;
  R7 SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z));
  R8 fp8 expert weight = decode(code) * scale[e, n] per output column;
  R13 MXFP4 expert weight = e2m1(code) * e8m0(scale) of its 32-element block
     along K, codes packed two per byte along K (low nibble = even k).

The microscaling formats follow the CuTeDSL post's quantisation remark
(MXFP8/MXFP4 reduce an absolute maximum over 32 elements) with the element
and scale encodings of the OCP MX formats (E2M1 elements, E8M0 scales).
"""
import math
from typing import Callable, Dict, Optional, Tuple

import numpy as np

# ----------------------------------------------------------------------------
# exact decoders of the storage formats
# ----------------------------------------------------------------------------


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32: widen the 16 stored bits
    into the high half of a 32-bit word and read it as float32 (exact)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def decode_fp32(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _e4m3fn_value(b: np.ndarray) -> np.ndarray:
    """OCP 8-bit float E4M3 ("fn": finite, no infinities): 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
    m/8 * 2^-6; the all-ones pattern S.1111.111 is NaN; the largest finite
    magnitude is 1.75 * 2^8 = 448."""
    b = np.asarray(b).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & ((b & 0x7) == 7), np.nan, v)


def decode_e4m3fn(bits: np.ndarray) -> np.ndarray:
    """Decode OCP e4m3fn codes: the value of each of the 256 codes from the
    format definition above, looked up per element."""
    table = _e4m3fn_value(np.arange(256))
    return table[np.asarray(bits).astype(np.uint8)]


def _e2m1_value(c: np.ndarray) -> np.ndarray:
    """OCP MX 4-bit float E2M1: 1 sign bit, 2 exponent bits with bias 1, 1
    mantissa bit, no infinities or NaN; exponent field 0 encodes subnormals
    m * 0.5; normals are (1 + m/2) * 2^(e-1), so the magnitudes of codes 0..7
    are 0, 0.5, 1, 1.5, 2, 3, 4, 6."""
    c = np.asarray(c).astype(np.int64)
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    normal = (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0)
    return sign * np.where(e == 0, m * 0.5, normal)


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """Decode E2M1 codes (one per element, values 0..15) by the table of the
    16 values the definition above gives."""
    table = _e2m1_value(np.arange(16))
    return table[np.asarray(codes).astype(np.uint8) & 0xF]


def decode_e8m0(bits: np.ndarray) -> np.ndarray:
    """OCP MX shared scale E8M0: an unsigned biased exponent, value 2^(e-127);
    e = 255 is NaN."""
    e = np.asarray(bits).astype(np.int64)
    return np.where(e == 255, np.nan, np.exp2(e.astype(np.float64) - 127.0))


MX_BLOCK = 32


def decode_mxfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """An MXFP4 matrix W[K, N] from its storage (reading R13): E2M1 codes two per
    byte along K, packed[k/2, n] holding code(k) in the low nibble for even k
    and code(k+1) in the high nibble; scales[k/32, n] the E8M0 scale shared by
    the block of 32 consecutive k of column n.  W[k, n] = e2m1(code) * scale."""
    packed = np.asarray(packed).astype(np.uint8)
    K2, N = packed.shape
    codes = np.empty((2 * K2, N), np.uint8)
    codes[0::2] = packed & 0xF
    codes[1::2] = packed >> 4
    vals = decode_e2m1(codes)
    sc = decode_e8m0(scales)
    return vals * np.repeat(sc, MX_BLOCK, axis=0)[: 2 * K2]


def decode_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """An MXFP8 matrix W[K, N] from its storage (reading R13): one e4m3fn code
    per element, codes[k, n]; scales[k/32, n] the E8M0 scale shared by the
    block of 32 consecutive k of column n.  W[k, n] = e4m3fn(code) * scale."""
    codes = np.asarray(codes).astype(np.uint8)
    K = codes.shape[0]
    return decode_e4m3fn(codes) * np.repeat(decode_e8m0(scales), MX_BLOCK, axis=0)[:K]


def decode(raw: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "bf16":
        return decode_bf16(raw)
    if fmt == "fp8":
        return decode_e4m3fn(raw)
    if fmt == "f32":
        return decode_fp32(raw)
    raise ValueError(fmt)


# ----------------------------------------------------------------------------
# O1-O3: router
# ----------------------------------------------------------------------------


def router_logits(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray]) -> np.ndarray:
    """L[t, e] = sum_i x[t, i] * W_r[i, e] + bias[e]   (float64; reading R1)."""
    L = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64)
    if bias is not None:
        L = L + np.asarray(bias, np.float64)[None, :]
    return L


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """ids[t, j] = the expert holding the j-th largest logit of row t, ties to
    the lower expert index (readings R2).  A stable sort of -logit keeps equal
    values in ascending index order."""
    L = np.asarray(logits)
    order = np.argsort(-L, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def topk_weights(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Softmax over all E experts, keep the selected ones, renormalise so each
    row's k weights sum to 1."""
    L = np.asarray(logits, np.float64)
    z = L - L.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, np.asarray(ids, np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route(x, w_router, bias, k: int, decision_dtype=np.float32):
    """O1-O3.  The selection is taken on the logits rounded to `decision_dtype`
    (the precision the kernel decides in, reading R3); the weights use the
    float64 logits.  Returns (logits64, ids, weights64)."""
    L = router_logits(x, w_router, bias)
    Ld = L.astype(decision_dtype) if decision_dtype is not None else L
    ids = select_topk(Ld, k)
    return L, ids, topk_weights(L, ids)


# ----------------------------------------------------------------------------
# O4-O5: alignment (histogram, padded offsets, stable permutation)
# ----------------------------------------------------------------------------


def capacity(T: int, E: int, k: int, bm: int) -> int:
    """Rows of the padded, expert-sorted buffer a caller must provide: every
    active expert pads its count up to a multiple of bm, and at most min(E, T*k)
    experts are active, so the padded total never exceeds
    floor((T*k + min(E, T*k) * (bm - 1)) / bm) blocks of bm rows."""
    n = T * k
    if n == 0:
        return 0
    return bm * ((n + min(E, n) * (bm - 1)) // bm)


def align(ids: np.ndarray, E: int, bm: int) -> Dict[str, np.ndarray]:
    """counts[e]  = number of (t, j) with ids[t, j] == e;
    offsets[0] = 0, offsets[e+1] = offsets[e] + bm * ceil(counts[e] / bm);
    sorted_ids[offsets[e] + r] = t*k + j for the r-th entry routed to e, entries
    taken in ascending t*k + j (reading R5); unused slots hold -1 (R4);
    inv_pos[t*k + j] = its slot; block_expert[b] = e for every bm-row block of
    expert e's padded range and -1 for the blocks past offsets[E]."""
    ids = np.asarray(ids, np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    counts = np.zeros(E, np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + bm * ((counts[e] + bm - 1) // bm)
    cap = capacity(T, E, k, bm)
    assert offsets[E] <= cap
    sorted_ids = np.full(cap, -1, np.int64)
    inv_pos = np.full(T * k, -1, np.int64)
    fill = offsets[:E].copy()
    for i, e in enumerate(flat):
        sorted_ids[fill[e]] = i
        inv_pos[i] = fill[e]
        fill[e] += 1
    block_expert = np.full(cap // bm, -1, np.int64)
    for e in range(E):
        block_expert[offsets[e] // bm: offsets[e + 1] // bm] = e
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "sorted_ids": sorted_ids.astype(np.int32),
        "inv_pos": inv_pos.astype(np.int32),
        "block_expert": block_expert.astype(np.int32),
    }


# ----------------------------------------------------------------------------
# O6-O7: experts and combine
# ----------------------------------------------------------------------------


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))   (reading R7)."""
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(x_rows: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
                  w_down: np.ndarray) -> np.ndarray:
    """(SiLU(X W_gate) * (X W_up)) W_down for the rows X routed to one expert."""
    G = x_rows @ w_gate
    U = x_rows @ w_up
    return (silu(G) * U) @ w_down


ExpertFn = Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]


def expert_weights_from_raw(w_gate_up, w_down, fmt: str, scale_gate_up=None,
                            scale_down=None) -> ExpertFn:
    """Expert e's float64 (W_gate[d, d_ff], W_up[d, d_ff], W_down[d_ff, d]) from
    the stored arrays.  `w_gate_up[e]` is [d, 2*d_ff], gate columns first
    (reading R6); fp8 weights are decode(code) * scale per output column (R8);
    MXFP4 and MXFP8 weights are E2M1 / e4m3fn codes times the E8M0 scale of
    their 32-element block along K (R13).
    The arrays only need `[e]` indexing returning NumPy arrays, so experts can be
    fetched one at a time."""
    def fn(e: int):
        if fmt in ("mxfp4", "mxfp8"):
            dec = decode_mxfp4 if fmt == "mxfp4" else decode_mxfp8
            gu = dec(np.asarray(w_gate_up[e]), np.asarray(scale_gate_up[e]))
            dn = dec(np.asarray(w_down[e]), np.asarray(scale_down[e]))
            dff = gu.shape[1] // 2
            return gu[:, :dff], gu[:, dff:], dn
        gu = decode(np.asarray(w_gate_up[e]), fmt)
        dn = decode(np.asarray(w_down[e]), fmt)
        if fmt == "fp8":
            gu = gu * np.asarray(scale_gate_up[e], np.float64)[None, :]
            dn = dn * np.asarray(scale_down[e], np.float64)[None, :]
        dff = gu.shape[1] // 2
        return gu[:, :dff], gu[:, dff:], dn
    return fn


def moe_forward(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray],
                expert_fn: ExpertFn, E: int, k: int, block_m: int,
                decision_dtype=np.float32) -> Dict[str, np.ndarray]:
    """O1-O7, grouped per expert.  x is float64 [T, d]."""
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    logits, ids, w = route(x, w_router, bias, k, decision_dtype)
    al = align(ids, E, block_m)
    out = np.zeros_like(x)
    for e in range(E):
        rows_t, rows_j = np.nonzero(ids == e)        # a token holds e at most once
        if rows_t.size == 0:
            continue
        wg, wu, wd = expert_fn(e)
        Y = swiglu_expert(x[rows_t], wg, wu, wd)
        out[rows_t] += w[rows_t, rows_j][:, None] * Y
    res = {"logits": logits, "topk_ids": ids, "topk_w": w, "out": out}
    res.update(al)
    return res


def outputs_for_tokens(x: np.ndarray, rows, ids: np.ndarray, w: np.ndarray,
                       expert_fn: ExpertFn) -> np.ndarray:
    """O6-O7 for the token rows `rows` only, given the routing (ids, w) of all
    tokens: out[t] = sum_j w[t, j] * SwiGLU_{ids[t, j]}(x[t]).  Each needed expert
    is fetched once (sampled checks of layers too large to run in full)."""
    x = np.asarray(x, np.float64)
    rows = np.asarray(rows, np.int64)
    out = np.zeros((rows.size, x.shape[1]))
    need: Dict[int, list] = {}
    for r, t in enumerate(rows):
        for j, e in enumerate(np.asarray(ids)[t]):
            need.setdefault(int(e), []).append((r, int(t), j))
    for e in sorted(need):
        wg, wu, wd = expert_fn(e)
        items = need[e]
        Y = swiglu_expert(x[[t for _, t, _ in items]], wg, wu, wd)
        for (r, t, j), yrow in zip(items, Y):
            out[r] += w[t, j] * yrow
    return out


# ----------------------------------------------------------------------------
# O8: brute force, explicit loops (tiny inputs only)
# ----------------------------------------------------------------------------


def moe_forward_bruteforce(x, w_router, bias, w_gate, w_up, w_down, k: int):
    """Per-token, per-slot, per-element Python loops over lists of floats; no
    array library.  w_gate/w_up: [E][d][d_ff], w_down: [E][d_ff][d].  Returns
    (ids, weights, out) as nested lists."""
    x = [[float(v) for v in row] for row in np.asarray(x)]
    T, d = len(x), len(x[0])
    wr = np.asarray(w_router).tolist()
    E = len(wr[0])
    b = [0.0] * E if bias is None else [float(v) for v in np.asarray(bias)]
    wg, wu, wd = (np.asarray(a).tolist() for a in (w_gate, w_up, w_down))
    dff = len(wg[0][0])
    all_ids, all_w, out = [], [], []
    for t in range(T):
        logit = []
        for e in range(E):
            s = 0.0
            for i in range(d):
                s += x[t][i] * wr[i][e]
            logit.append(s + b[e])
        taken, ids = set(), []
        for _ in range(k):
            best = None
            for e in range(E):
                if e in taken:
                    continue
                if best is None or logit[e] > logit[best]:
                    best = e
            taken.add(best)
            ids.append(best)
        top = max(logit)
        mass = [math.exp(v - top) for v in logit]
        z = sum(mass)
        p = [m / z for m in mass]
        psel = [p[e] for e in ids]
        wsum = sum(psel)
        wts = [v / wsum for v in psel]
        o = [0.0] * d
        for j, e in enumerate(ids):
            h = []
            for n in range(dff):
                g = u = 0.0
                for i in range(d):
                    g += x[t][i] * wg[e][i][n]
                    u += x[t][i] * wu[e][i][n]
                h.append(g / (1.0 + math.exp(-g)) * u)
            for m in range(d):
                y = 0.0
                for n in range(dff):
                    y += h[n] * wd[e][n][m]
                o[m] += wts[j] * y
        all_ids.append(ids)
        all_w.append(wts)
        out.append(o)
    return all_ids, all_w, out
