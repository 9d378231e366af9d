"""Helpers for comparing the GPU library with the CPU oracle.

Rules (the workload statement's tolerances):
  * integers (ids, counts, offsets, slots, positions): bit-exact;
  * fp32 outputs, logits and routing weights: |err| <= 1e-4 * (1 + |ref|);
  * bf16 / fp8-weight outputs: per token row, max |err| <= 2e-2 * RMS(ref row).
The top-k decision depends on floating point, so routing is checked in two
parts:
  (i)  boundary-fed: the oracle's selection, weights and alignment run on the
       fp32 logits the GPU emitted; ids, counts, offsets, slots and positions
       must then equal the GPU's bit for bit, for every token;
  (ii) the GPU's logits match the oracle's float64 logits within the fp32
       rule, and where the oracle's own fp32 decision differs from the GPU's
       (a near tie), the GPU's choice must be a valid top-k of the oracle's
       logits within that tolerance; such tokens are reported, not failed.
Float outputs are then compared for every checked token against the oracle's
expert compute on the GPU's selection, with weights from the oracle's float64
logits, so no token is exempt.
"""
import numpy as np
import torch

from oracle import moe_oracle as O

LOGIT_RTOL = 1e-4


def np_bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a tensor as an unsigned-int NumPy array (host copy)."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    if t.dtype == torch.uint8:  # MXFP4 codes / E8M0 scales
        return t.cpu().numpy()
    raise TypeError(t.dtype)


FMT = {torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8", torch.float32: "f32",
       torch.uint8: "mxfp4"}


def decode(t: torch.Tensor) -> np.ndarray:
    return O.decode(np_bits(t), FMT[t.dtype])


class _PerExpert:
    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        return np_bits(self.t[e])


def oracle_layer(layer):
    """(w_router64, bias64 or None, expert_fn) for a workloads.Layer on any device."""
    wr = decode(layer.w_router)
    bias = None if layer.bias is None else layer.bias.detach().cpu().numpy().astype(np.float64)
    fmt = FMT[layer.w_gate_up.dtype]
    if fmt == "fp8" and layer.scale_gate_up.dtype == torch.uint8:
        fmt = "mxfp8"  # e4m3fn codes with E8M0 block scales
    sgu = sdn = None
    if fmt in ("mxfp4", "mxfp8"):
        sgu, sdn = _PerExpert(layer.scale_gate_up), _PerExpert(layer.scale_down)
    elif fmt == "fp8":
        sgu, sdn = layer.scale_gate_up.cpu().numpy(), layer.scale_down.cpu().numpy()
    fn = O.expert_weights_from_raw(_PerExpert(layer.w_gate_up), _PerExpert(layer.w_down), fmt,
                                   sgu, sdn)
    return wr, bias, fn


def logit_tol(ref: np.ndarray) -> np.ndarray:
    return LOGIT_RTOL * (1.0 + np.abs(ref))


def assert_close_f32(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    tol = logit_tol(ref)
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} beyond 1e-4*(1+|ref|); "
                           f"max err {err.max():.3e}, worst at {np.unravel_index(np.argmax(err - tol), err.shape)}")


def row_rule_violations(got, ref, rel=2e-2):
    """Rows t with max_n |got - ref| > rel * RMS(ref[t])."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=1))
    err = np.max(np.abs(got - ref), axis=1)
    return np.nonzero(err > rel * rms)[0], err, rms


def assert_out_close(got, ref, act: str, what=""):
    if act == "f32":
        assert_close_f32(got, ref, what)
        return
    bad, err, rms = row_rule_violations(got, ref)
    ratio = err / np.maximum(rms, 1e-300)
    print(f"{what}: {got.shape[0]} rows compared, worst max|err|/RMS {np.max(ratio):.3e} "
          f"(bound 2e-2)", flush=True)
    assert bad.size == 0, (f"{what}: {bad.size} rows beyond 2e-2*RMS; worst ratio "
                           f"{np.max(ratio):.3e} at row {int(np.argmax(ratio))}")


def assert_boundary_fed(logits32, ids, weights, k: int, E: int = None, bm: int = None,
                        alignment=None, what=""):
    """Check (i): the oracle's top-k (O2) and weights (O3) on the GPU's own
    fp32 logits, and its alignment (O4-O5) of the GPU's ids."""
    L = np.asarray(logits32, np.float32)
    ids = np.asarray(ids)
    want = O.select_topk(L, k)
    diff = np.nonzero((want != ids).any(axis=1))[0]
    assert diff.size == 0, (f"{what}: GPU ids differ from the oracle's top-k of the GPU logits "
                            f"on {diff.size} tokens (first {diff[:5]})")
    assert_close_f32(weights, O.topk_weights(L.astype(np.float64), ids), f"{what} topk_w (i)")
    if alignment is not None:
        ref = O.align(ids, E, bm)
        for key, got in alignment.items():
            assert (np.asarray(got) == ref[key][:np.asarray(got).size]).all() and \
                np.asarray(got).size == ref[key].size, f"{what}: {key} differs from O.align"


def classify_ids(L64: np.ndarray, gpu_ids: np.ndarray, ora_ids: np.ndarray):
    """Returns the tokens whose GPU top-k differs from the oracle's, after
    checking that each such choice is a valid top-k of L64 within the logit
    tolerance (raises otherwise)."""
    diff = np.nonzero((gpu_ids != ora_ids).any(axis=1))[0]
    for t in diff:
        L = L64[t]
        g = gpu_ids[t].astype(np.int64)
        tol = logit_tol(L)
        assert len(set(g.tolist())) == len(g), f"token {t}: repeated expert {g}"
        for j in range(len(g) - 1):
            assert L[g[j]] >= L[g[j + 1]] - (tol[g[j]] + tol[g[j + 1]]), \
                f"token {t}: slots out of order beyond tolerance {g} {L[g]}"
        rest = np.setdiff1d(np.arange(L.size), g)
        if rest.size:
            worst_in = g[np.argmin(L[g])]
            best_out = rest[np.argmax(L[rest])]
            assert L[worst_in] >= L[best_out] - (tol[worst_in] + tol[best_out]), \
                f"token {t}: selected {g} misses {best_out} beyond tolerance"
    return diff


def check_alignment_properties(ids: np.ndarray, E: int, bm: int, counts, offsets, sorted_ids,
                               inv_pos, block_expert=None):
    """The defining properties of the alignment of `ids`; together they fix it
    uniquely (counts by bincount, offsets by the padded scan, slots by the
    stable order), so this is an exact check that does not use the oracle."""
    T, k = ids.shape
    n = T * k
    flat = ids.reshape(-1).astype(np.int64)
    cnt = np.bincount(flat, minlength=E)
    assert (np.asarray(counts) == cnt).all(), "counts"
    off = np.zeros(E + 1, np.int64)
    off[1:] = np.cumsum((cnt + bm - 1) // bm * bm)
    assert (np.asarray(offsets)[:E + 1] == off).all(), "offsets"
    s = np.asarray(sorted_ids)
    cap = O.capacity(T, E, k, bm)
    s = s[:cap]
    for e in range(E):
        seg = s[off[e]:off[e + 1]]
        want = np.nonzero(flat == e)[0]
        assert (seg[:cnt[e]] == want).all(), f"expert {e} slots"
        assert (seg[cnt[e]:] == -1).all(), f"expert {e} padding"
    assert (s[off[E]:] == -1).all(), "tail padding"
    assert (s[np.asarray(inv_pos)[:n]] == np.arange(n)).all(), "inv_pos"
    if block_expert is not None:
        be = np.asarray(block_expert)
        for b in range(cap // bm):
            want = -1
            if b * bm < off[E]:
                want = int(np.searchsorted(off, b * bm, side="right") - 1)
            assert be[b] == want, f"block {b}"
