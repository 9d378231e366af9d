"""Algorithmic work of the MoE layer forward and MI355X peak rates.

"Algorithmic" means what the method itself must move or compute: each active
expert's weights once, the tokens once, the output once, and the GEMM flops of
the rows actually routed.  Padding rows and the layer's own intermediates are
excluded, so a kernel's achieved rate against these figures is an honest
fraction of the hardware roofline.

The GEMM accounting follows the statement of expert compute in the vLLM
fused-MoE post, section "Swap-AB" (A[M,K] x B[K,N] -> C[M,N]: 2*M*N*K flops,
M*N output elements) and is pinned to the worked 4096^3 BF16 example of
"La fusion de noyaux", section 4.2.
"""
from dataclasses import dataclass

# MI355X (gfx950) published peaks.  Dense MFMA figures exclude 2:4 sparsity.
HBM_BYTES_PER_S = 8.0e12
MFMA_BF16_FLOPS = 2.5e15
MFMA_FP8_FLOPS = 5.0e15
VALU_FP32_FLOPS = 157.3e12
VALU_FP64_FLOPS = 78.6e12
NUM_CUS = 256
CLOCK_HZ = 2.4e9

ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}


def gemm_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def matrix_bytes(rows: int, cols: int, elem_bytes: int) -> int:
    return rows * cols * elem_bytes


@dataclass
class LayerWork:
    """Per-forward algorithmic bytes and flops, split by kernel."""
    bytes_total: int
    flops_total: int
    bytes_gate_up: int
    bytes_down: int
    flops_gate_up: int
    flops_down: int
    bytes_router: int
    flops_router: int
    bytes_combine: int


def layer_work(T: int, d: int, d_ff: int, E: int, k: int, act: str, wdt: str,
               active: int) -> LayerWork:
    """`active` is the number of distinct experts the routing selected."""
    bx = ELEM_BYTES[act]
    rows = T * k
    if wdt in ("mxfp4", "mxfp8"):
        # half a byte (MXFP4) or one byte (MXFP8) per weight, one E8M0 byte
        # per 32 k of a column
        num, den = (1, 2) if wdt == "mxfp4" else (1, 1)
        w_gu = active * (d * 2 * d_ff * num // den + (d // 32) * 2 * d_ff)
        w_dn = active * (d_ff * d * num // den + (d_ff // 32) * d)
    else:
        bw = ELEM_BYTES[wdt]
        scales_gu = active * 2 * d_ff * 4 if wdt == "fp8" else 0
        scales_dn = active * d * 4 if wdt == "fp8" else 0
        w_gu = active * matrix_bytes(d, 2 * d_ff, bw) + scales_gu
        w_dn = active * matrix_bytes(d_ff, d, bw) + scales_dn
    # gate|up reads its weights and the tokens once and writes h once;
    # down reads its weights and h once and writes the per-slot outputs once;
    # combine reads those outputs once and writes the layer output once.
    b_gu = w_gu + matrix_bytes(T, d, bx) + matrix_bytes(rows, d_ff, bx)
    b_dn = w_dn + matrix_bytes(rows, d_ff, bx) + matrix_bytes(rows, d, bx)
    b_router = matrix_bytes(d, E, bx) + matrix_bytes(T, d, bx) + matrix_bytes(T, E, 4)
    b_comb = matrix_bytes(rows, d, bx) + matrix_bytes(T, d, bx)
    f_gu = gemm_flops(rows, 2 * d_ff, d)
    f_dn = gemm_flops(rows, d, d_ff)
    f_router = gemm_flops(T, E, d)
    # whole layer: weights once, tokens in once, output once
    b_total = w_gu + w_dn + matrix_bytes(d, E, bx) + 2 * matrix_bytes(T, d, bx)
    return LayerWork(b_total, f_gu + f_dn + f_router, b_gu, b_dn, f_gu, f_dn,
                     b_router, f_router, b_comb)
