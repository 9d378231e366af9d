"""The C-ABI library loads and exports every entry point include/libmoe.h
declares; host-side logic (capacity, validation, workspace queries) behaves as
documented.  Nothing here launches a kernel: every call either fails
validation or is a workspace query, both of which return before any HIP call.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from mixture_experts_layer_align_amd import _binding as B
from oracle import moe_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "libmoe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = B.load()
    declared = _declared()
    assert set(declared) >= {"moe_route", "moe_align", "moe_forward"}
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(declared) == sorted(B.EXPORTED)


def test_abi_version_and_status_strings():
    lib = B.load()
    assert lib.moe_abi_version() == 2
    for s in (B.MOE_OK, B.MOE_ERR_INVALID, B.MOE_ERR_UNSUPPORTED, B.MOE_ERR_WORKSPACE,
              B.MOE_ERR_DEVICE, B.MOE_ERR_SCRATCH):
        assert len(B.status_string(s)) > 0


@pytest.mark.parametrize("T,E,k,bm", [(0, 8, 2, 32), (1, 8, 2, 32), (5, 4, 2, 4), (64, 8, 2, 32),
                                      (256, 128, 8, 16), (16384, 256, 8, 128), (3, 1024, 7, 256)])
def test_capacity_matches_oracle(T, E, k, bm):
    assert B.align_capacity(T, E, k, bm) == O.capacity(T, E, k, bm)


def test_capacity_rejects_bad_block():
    assert B.align_capacity(4, 8, 2, 24) == -1
    assert B.align_capacity(-1, 8, 2, 32) == -1


def _route(T=4, d=128, E=8, k=2, act=B.MOE_BF16, x=1, w=1, ids=1, tw=1, ws=None):
    lib = B.load()
    n = ctypes.c_size_t(0)
    vp = ctypes.c_void_p
    return lib.moe_route(vp(x) if x else None, vp(w) if w else None, None, T, d, E, k, act, None,
                         vp(ids) if ids else None, vp(tw) if tw else None, ws, ctypes.byref(n),
                         None), n.value


def test_route_validation_errors_before_any_launch():
    assert _route(k=9, E=8)[0] == B.MOE_ERR_INVALID
    assert _route(k=0)[0] == B.MOE_ERR_INVALID
    assert _route(E=2000, k=2)[0] == B.MOE_ERR_INVALID
    assert _route(T=-1)[0] == B.MOE_ERR_INVALID
    assert _route(d=100)[0] == B.MOE_ERR_UNSUPPORTED
    assert _route(act=B.MOE_FP8_E4M3)[0] == B.MOE_ERR_UNSUPPORTED
    assert _route(x=0, ws=ctypes.c_void_p(4096))[0] in (B.MOE_ERR_INVALID, B.MOE_ERR_WORKSPACE)
    rc, need = _route(x=0, w=0, ids=0, tw=0)          # a query needs no data pointers
    assert rc == B.MOE_OK and need > 0          # workspace query
    assert _route(T=0, x=0, w=0, ids=0, tw=0)[0] == B.MOE_OK
    # T*k at MOE_MAX_ENTRIES = 2^24 is rejected
    assert _route(T=1 << 21, E=16, k=8)[0] == B.MOE_ERR_INVALID


def test_align_validation_errors():
    lib = B.load()
    n = ctypes.c_size_t(0)
    vp = ctypes.c_void_p
    p = vp(1)
    args = lambda T, E, k, bm: (p, T, E, k, bm, p, p, p, p, p, None, ctypes.byref(n), None)
    assert lib.moe_align(*args(4, 8, 2, 24)) == B.MOE_ERR_INVALID   # not a power of two
    assert lib.moe_align(*args(4, 8, 2, 8)) == B.MOE_ERR_INVALID    # below 16
    assert lib.moe_align(*args(4, 8, 2, 512)) == B.MOE_ERR_INVALID  # above 256
    assert lib.moe_align(*args(4, 2, 3, 32)) == B.MOE_ERR_INVALID   # k > E
    assert lib.moe_align(*args(4, 8, 2, 32)) == B.MOE_OK            # query
    assert n.value == 0                                             # one workgroup, no scratch
    assert lib.moe_align(*args(3000, 8, 2, 32)) == B.MOE_OK
    assert n.value > 0                                              # multi-tile scratch
    n.value = 0
    assert lib.moe_align(None, 4, 8, 2, 32, p, p, p, p, p, vp(4096), ctypes.byref(n), None) \
        == B.MOE_ERR_INVALID                                        # data pointer missing
    # routed entries T*k must stay below MOE_MAX_ENTRIES = 2^24
    assert lib.moe_align(*args((1 << 21) - 1, 16, 8, 128)) == B.MOE_OK
    assert lib.moe_align(*args(1 << 21, 16, 8, 128)) == B.MOE_ERR_INVALID
    assert lib.moe_align(*args(1 << 24, 8, 1, 32)) == B.MOE_ERR_INVALID


def _layer(**kw):
    L = B.MoeLayer()
    L.d, L.d_ff, L.E, L.k = kw.get("d", 256), kw.get("d_ff", 256), kw.get("E", 8), kw.get("k", 2)
    L.act_dtype, L.w_dtype = kw.get("act", B.MOE_BF16), kw.get("wdt", B.MOE_BF16)
    L.w_router, L.w_gate_up, L.w_down = 1, 1, 1
    L.scale_gate_up = kw.get("sgu", None)
    L.scale_down = kw.get("sdn", None)
    return L


def _fwd(L, T=4, ws=None, nbytes=0, x=8, out=16):
    lib = B.load()
    n = ctypes.c_size_t(nbytes)
    vp = ctypes.c_void_p
    rc = lib.moe_forward(ctypes.byref(L), vp(x) if x else None, T, vp(out) if out else None,
                         ws, ctypes.byref(n), None, None)
    return rc, n.value


def test_forward_validation_and_workspace_query():
    assert _fwd(_layer())[0] == B.MOE_OK
    assert _fwd(_layer(d=192))[0] == B.MOE_ERR_UNSUPPORTED
    assert _fwd(_layer(d_ff=200))[0] == B.MOE_ERR_UNSUPPORTED
    assert _fwd(_layer(act=B.MOE_F32, wdt=B.MOE_BF16))[0] == B.MOE_ERR_UNSUPPORTED
    assert _fwd(_layer(act=B.MOE_F32, wdt=B.MOE_FP8_E4M3, sgu=1, sdn=1))[0] == B.MOE_ERR_UNSUPPORTED
    assert _fwd(_layer(wdt=B.MOE_FP8_E4M3))[0] == B.MOE_ERR_INVALID     # scales missing
    assert _fwd(_layer(wdt=B.MOE_FP8_E4M3, sgu=1, sdn=1))[0] == B.MOE_OK
    assert _fwd(_layer(k=9))[0] == B.MOE_ERR_INVALID
    assert _fwd(_layer(), x=0, out=0)[0] == B.MOE_OK                    # query: no data
    # a given workspace smaller than the requirement is refused before any launch
    _, need = _fwd(_layer(), T=64)
    assert need > 0
    assert _fwd(_layer(), T=64, ws=ctypes.c_void_p(4096), nbytes=need - 1)[0] == B.MOE_ERR_WORKSPACE
    assert _fwd(_layer(), T=64, ws=ctypes.c_void_p(4096 + 8), nbytes=need)[0] == B.MOE_ERR_WORKSPACE
    # workspace grows with T
    assert _fwd(_layer(), T=4096)[1] > need


def _qk(q=1, k=1, wq=1, wk=1, T=4, nq=2, nk=1, hd=128, dt=B.MOE_BF16, bias=0.0, eps=1e-6):
    vp = ctypes.c_void_p
    return B.load().moe_qk_norm(vp(q) if q else None, vp(k) if k else None,
                                vp(wq) if wq else None, vp(wk) if wk else None, T, nq, nk, hd,
                                dt, bias, eps, None)


def test_qk_norm_validation_before_any_launch():
    assert _qk(hd=96) == B.MOE_ERR_UNSUPPORTED
    assert _qk(hd=512) == B.MOE_ERR_UNSUPPORTED
    assert _qk(dt=B.MOE_FP8_E4M3) == B.MOE_ERR_UNSUPPORTED
    assert _qk(T=-1) == B.MOE_ERR_INVALID
    assert _qk(nq=-1) == B.MOE_ERR_INVALID
    assert _qk(eps=-1e-6) == B.MOE_ERR_INVALID
    assert _qk(eps=float("nan")) == B.MOE_ERR_INVALID
    assert _qk(eps=float("inf")) == B.MOE_ERR_INVALID
    assert _qk(bias=float("inf")) == B.MOE_ERR_INVALID
    assert _qk(q=0) == B.MOE_ERR_INVALID
    assert _qk(wk=0) == B.MOE_ERR_INVALID
    assert _qk(T=1 << 30, nq=2, nk=1) == B.MOE_ERR_INVALID


def test_qk_norm_empty_work_enqueues_nothing():
    # no heads or no tokens: OK without touching the (absent) tensors or a GPU
    assert _qk(q=0, k=0, wq=0, wk=0, T=0) == B.MOE_OK
    assert _qk(q=0, k=0, wq=0, wk=0, nq=0, nk=0) == B.MOE_OK


@pytest.mark.parametrize("wdt", [B.MOE_MXFP4, B.MOE_MXFP8])
def test_mx_layer_validation(wdt):
    # MX experts need bf16 activations, 256-wide d and d_ff, and both scales
    Bd = B
    layer = Bd.MoeLayer()
    layer.d, layer.d_ff, layer.E, layer.k = 256, 256, 8, 2
    layer.act_dtype, layer.w_dtype = Bd.MOE_BF16, wdt
    layer.w_router = layer.w_gate_up = layer.w_down = 1
    lib = Bd.load()
    n = ctypes.c_size_t(0)
    q = lambda L: lib.moe_forward(ctypes.byref(L), None, 4, None, None, ctypes.byref(n), None, None)
    assert q(layer) == Bd.MOE_ERR_INVALID          # scales missing
    layer.scale_gate_up = layer.scale_down = 1
    assert q(layer) == Bd.MOE_OK and n.value > 0    # workspace query
    layer.d_ff = 384
    assert q(layer) == Bd.MOE_ERR_UNSUPPORTED       # not a multiple of 256
    layer.d_ff, layer.act_dtype = 256, Bd.MOE_F32
    assert q(layer) == Bd.MOE_ERR_UNSUPPORTED       # fp32 activations


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    # the E=256 top-8 d=7168 fp8 layer at 128 tokens needs ~319 MiB of
    # workspace, more than the static scratch: refused on the host, before
    # any pointer is used or anything is enqueued
    L = B.MoeLayer()
    L.d, L.d_ff, L.E, L.k = 7168, 2048, 256, 8
    L.act_dtype, L.w_dtype = B.MOE_BF16, B.MOE_FP8_E4M3
    L.w_router = L.w_gate_up = L.w_down = L.scale_gate_up = L.scale_down = 256
    lib = B.load()
    n = ctypes.c_size_t(0)
    assert lib.moe_forward(ctypes.byref(L), None, 128, None, None, ctypes.byref(n), None,
                           None) == B.MOE_OK
    assert n.value > B.MOE_NOALLOC_SCRATCH_BYTES
    rc = lib.moe_forward_noalloc(ctypes.byref(L), ctypes.c_void_p(256), 128,
                                 ctypes.c_void_p(512), None, None)
    assert rc == B.MOE_ERR_SCRATCH
    assert "scratch" in B.status_string(rc)
    # invalid shapes fail validation first, as for moe_forward
    L.k = 0
    assert lib.moe_forward_noalloc(ctypes.byref(L), ctypes.c_void_p(256), 128,
                                   ctypes.c_void_p(512), None, None) == B.MOE_ERR_INVALID


def test_noalloc_scratch_size_matches_header():
    src = open(os.path.join(ROOT, "include", "libmoe.h")).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == B.MOE_NOALLOC_SCRATCH_BYTES


def test_rms_norm_validation_on_host():
    lib = B.load()
    vp = ctypes.c_void_p
    # row bytes not a multiple of 16, or above 32 KiB: unsupported
    assert lib.moe_rms_norm(vp(256), vp(256), vp(1 << 20), 4, 100, B.MOE_BF16, 0.0, 1e-6,
                            None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_rms_norm(vp(256), vp(256), vp(1 << 30), 4, 16392, B.MOE_BF16, 0.0, 1e-6,
                            None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_rms_norm(vp(256), vp(256), vp(1 << 30), 4, 8196, B.MOE_F32, 0.0, 1e-6,
                            None) == B.MOE_ERR_UNSUPPORTED
    # negative eps, missing pointers, partial overlap of out and x
    assert lib.moe_rms_norm(vp(256), vp(256), vp(1 << 20), 4, 2048, B.MOE_BF16, 0.0, -1.0,
                            None) == B.MOE_ERR_INVALID
    assert lib.moe_rms_norm(None, vp(256), vp(1 << 20), 4, 2048, B.MOE_BF16, 0.0, 1e-6,
                            None) == B.MOE_ERR_INVALID
    assert lib.moe_rms_norm(vp(4096), vp(256), vp(4096 + 4096), 4, 2048, B.MOE_BF16, 0.0, 1e-6,
                            None) == B.MOE_ERR_INVALID
    # an empty batch is valid and launches nothing
    assert lib.moe_rms_norm(None, None, None, 0, 2048, B.MOE_BF16, 0.0, 1e-6, None) == B.MOE_OK


def test_quantize_mxfp8_validation_on_host():
    lib = B.load()
    vp = ctypes.c_void_p
    X, C, S = vp(1 << 20), vp(1 << 24), vp(1 << 28)
    # n not a multiple of 32, or a dtype other than bf16/fp32: unsupported
    assert lib.moe_quantize_mxfp8(X, 4, 48, B.MOE_BF16, C, S, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_quantize_mxfp8(X, 4, 64, B.MOE_FP8_E4M3, C, S, None) == B.MOE_ERR_UNSUPPORTED
    # negative rows, n <= 0, missing pointers
    assert lib.moe_quantize_mxfp8(X, -1, 64, B.MOE_BF16, C, S, None) == B.MOE_ERR_INVALID
    assert lib.moe_quantize_mxfp8(X, 4, 0, B.MOE_BF16, C, S, None) == B.MOE_ERR_INVALID
    assert lib.moe_quantize_mxfp8(None, 4, 64, B.MOE_BF16, C, S, None) == B.MOE_ERR_INVALID
    assert lib.moe_quantize_mxfp8(X, 4, 64, B.MOE_BF16, C, None, None) == B.MOE_ERR_INVALID
    # overlapping regions: codes inside x, scales inside codes
    assert lib.moe_quantize_mxfp8(X, 4, 64, B.MOE_BF16, vp((1 << 20) + 100), S,
                                  None) == B.MOE_ERR_INVALID
    assert lib.moe_quantize_mxfp8(X, 4, 64, B.MOE_F32, C, vp((1 << 24) + 255),
                                  None) == B.MOE_ERR_INVALID
    # no rows: valid, nothing enqueued
    assert lib.moe_quantize_mxfp8(None, 0, 64, B.MOE_BF16, None, None, None) == B.MOE_OK


def test_misaligned_pointers_are_refused_on_host():
    """Each entry point refuses, before any launch, an array whose address is
    not a multiple of its kernels' widest access (16 bytes for activations and
    weights, 4 for the int32/fp32 routing arrays, 8 for MXFP8 codes)."""
    lib = B.load()
    vp = ctypes.c_void_p
    A = 1 << 20                                            # an aligned fake address
    # rms norm: x, weight and out need 16 bytes
    for args in ((A + 8, A, 4 * A), (A, A + 4, 4 * A), (A, A, 4 * A + 2)):
        assert lib.moe_rms_norm(vp(args[0]), vp(args[1]), vp(args[2]), 4, 2048, B.MOE_BF16, 0.0,
                                1e-6, None) == B.MOE_ERR_INVALID
    # qk norm: q, k and their weights
    assert _qk(q=A + 8, k=2 * A, wq=3 * A, wk=4 * A) == B.MOE_ERR_INVALID
    assert _qk(q=A, k=2 * A + 4, wq=3 * A, wk=4 * A) == B.MOE_ERR_INVALID
    assert _qk(q=A, k=2 * A, wq=3 * A + 2, wk=4 * A) == B.MOE_ERR_INVALID
    # quantiser: x 16, codes 8, scales 4
    X, C, S = 1 << 20, 1 << 24, 1 << 28
    for x, c, s in ((X + 8, C, S), (X, C + 4, S), (X, C, S + 2)):
        assert lib.moe_quantize_mxfp8(vp(x), 4, 64, B.MOE_BF16, vp(c), vp(s),
                                      None) == B.MOE_ERR_INVALID
    # route: x and the router weights 16, the fp32/int32 outputs 4
    ws = vp(1 << 30)
    n = ctypes.c_size_t(1 << 20)
    for x, w, ids, tw in ((A + 8, 2 * A, 3 * A, 4 * A), (A, 2 * A + 8, 3 * A, 4 * A),
                          (A, 2 * A, 3 * A + 2, 4 * A), (A, 2 * A, 3 * A, 4 * A + 1)):
        assert lib.moe_route(vp(x), vp(w), None, 4, 128, 8, 2, B.MOE_BF16, None, vp(ids), vp(tw),
                             ws, ctypes.byref(n), None) == B.MOE_ERR_INVALID
    # align: every int32 array 4
    for bad in range(6):
        ptrs = [vp(A * (i + 1) + (2 if i == bad else 0)) for i in range(6)]
        n = ctypes.c_size_t(1 << 20)
        assert lib.moe_align(ptrs[0], 4, 8, 2, 32, *ptrs[1:], ws, ctypes.byref(n),
                             None) == B.MOE_ERR_INVALID
    # forward: x, out, the three weight arrays and the fp8 scales 16
    _, need = _fwd(_layer(), T=64)
    for kw, x, out in (({}, A + 8, 2 * A), ({}, A, 2 * A + 4)):
        L = _layer(**kw)
        assert _fwd(L, T=64, ws=vp(1 << 30), nbytes=need, x=x, out=out)[0] == B.MOE_ERR_INVALID
    for field in ("w_router", "w_gate_up", "w_down"):
        L = _layer()
        L.w_router, L.w_gate_up, L.w_down = 3 * A, 4 * A, 5 * A
        setattr(L, field, getattr(L, field) + 8)
        assert _fwd(L, T=64, ws=vp(1 << 30), nbytes=need, x=A, out=2 * A)[0] == B.MOE_ERR_INVALID
    L = _layer(wdt=B.MOE_FP8_E4M3, sgu=6 * A + 4, sdn=7 * A)
    L.w_router, L.w_gate_up, L.w_down = 3 * A, 4 * A, 5 * A
    _, need8 = _fwd(L, T=64)
    assert _fwd(L, T=64, ws=vp(1 << 30), nbytes=need8, x=A, out=2 * A)[0] == B.MOE_ERR_INVALID
