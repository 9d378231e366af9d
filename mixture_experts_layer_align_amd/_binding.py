"""ctypes binding of libmoe's C ABI (include/libmoe.h).

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch provides device memory and the current stream.  Loading fails loudly
when libmoe.so has not been built; there is no fallback implementation.
"""
import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = 0, -1, -2, -3, -4
MOE_ERR_SCRATCH = -5
MOE_NOALLOC_SCRATCH_BYTES = 256 << 20
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4, MOE_MXFP8 = 0, 1, 2, 3, 4
MOE_BLOCK_M_MAX = 256

EXPORTED = ["moe_align_capacity", "moe_route", "moe_align", "moe_forward", "moe_forward_traced",
            "moe_forward_noalloc", "moe_rms_norm", "moe_qk_norm", "moe_quantize_mxfp8",
            "moe_status_string", "moe_abi_version"]

_c = ctypes
_vp = _c.c_void_p


class MoeLayer(_c.Structure):
    _fields_ = [("d", _c.c_int), ("d_ff", _c.c_int), ("E", _c.c_int), ("k", _c.c_int),
                ("act_dtype", _c.c_int), ("w_dtype", _c.c_int),
                ("w_router", _vp), ("logit_bias", _vp), ("w_gate_up", _vp), ("w_down", _vp),
                ("scale_gate_up", _vp), ("scale_down", _vp)]


class MoeRoutingOut(_c.Structure):
    _fields_ = [("logits", _vp), ("topk_ids", _vp), ("topk_w", _vp), ("expert_counts", _vp),
                ("padded_offsets", _vp), ("sorted_ids", _vp), ("inv_pos", _vp),
                ("block_m", _c.POINTER(_c.c_int))]


class MoeTrace(_c.Structure):
    _fields_ = [("events", _c.POINTER(_vp)), ("n_events", _c.c_int), ("n_kernels", _c.c_int),
                ("names", _c.c_char_p * 16)]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: libmoe status {status} ({status_string(status)})")


_lib = None


def load():
    """Load libmoe.so (once).  Raises if it is missing: the library is the only
    implementation of the layer."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                           "`python -m mixture_experts_layer_align_amd.build`")
    lib = _c.CDLL(LIB_PATH)
    lib.moe_align_capacity.restype = _c.c_int64
    lib.moe_align_capacity.argtypes = [_c.c_int] * 4
    lib.moe_route.restype = _c.c_int
    lib.moe_route.argtypes = [_vp, _vp, _vp, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                              _vp, _vp, _vp, _vp, _c.POINTER(_c.c_size_t), _vp]
    lib.moe_align.restype = _c.c_int
    lib.moe_align.argtypes = [_vp, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                              _vp, _vp, _vp, _vp, _vp, _vp, _c.POINTER(_c.c_size_t), _vp]
    lib.moe_forward.restype = _c.c_int
    lib.moe_forward.argtypes = [_c.POINTER(MoeLayer), _vp, _c.c_int, _vp, _vp,
                                _c.POINTER(_c.c_size_t), _c.POINTER(MoeRoutingOut), _vp]
    lib.moe_forward_traced.restype = _c.c_int
    lib.moe_forward_traced.argtypes = [_c.POINTER(MoeLayer), _vp, _c.c_int, _vp, _vp,
                                       _c.POINTER(_c.c_size_t), _c.POINTER(MoeRoutingOut),
                                       _c.POINTER(MoeTrace), _vp]
    lib.moe_forward_noalloc.restype = _c.c_int
    lib.moe_forward_noalloc.argtypes = [_c.POINTER(MoeLayer), _vp, _c.c_int, _vp,
                                        _c.POINTER(MoeRoutingOut), _vp]
    lib.moe_rms_norm.restype = _c.c_int
    lib.moe_rms_norm.argtypes = [_vp, _vp, _vp, _c.c_int, _c.c_int, _c.c_int, _c.c_float,
                                 _c.c_float, _vp]
    lib.moe_qk_norm.restype = _c.c_int
    lib.moe_qk_norm.argtypes = [_vp, _vp, _vp, _vp, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                _c.c_int, _c.c_float, _c.c_float, _vp]
    lib.moe_status_string.restype = _c.c_char_p
    lib.moe_quantize_mxfp8.restype = _c.c_int
    lib.moe_quantize_mxfp8.argtypes = [_vp, _c.c_int, _c.c_int, _c.c_int, _vp, _vp, _vp]
    lib.moe_status_string.argtypes = [_c.c_int]
    lib.moe_abi_version.restype = _c.c_int
    lib.moe_abi_version.argtypes = []
    _lib = lib
    return lib


def status_string(s: int) -> str:
    return load().moe_status_string(s).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else _vp(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return _vp(s.cuda_stream)


def _check(rc: int, what: str):
    if rc != MOE_OK:
        raise MoeError(rc, what)


_ACT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}
_WDT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.float8_e4m3fn: MOE_FP8_E4M3,
        torch.uint8: MOE_MXFP4}  # uint8 expert weights: packed MXFP4 codes


def act_code(dt: torch.dtype) -> int:
    return _ACT[dt]


def align_capacity(T: int, E: int, k: int, block_m: int) -> int:
    return int(load().moe_align_capacity(T, E, k, block_m))


def _workspace(query, device) -> torch.Tensor:
    n = _c.c_size_t(0)
    _check(query(None, _c.byref(n)), "workspace query")
    # 256-byte aligned by the caching allocator
    return torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=device), n


def route(x: torch.Tensor, w_router: torch.Tensor, bias: Optional[torch.Tensor], k: int,
          want_logits: bool = True, stream=None):
    """Returns (logits [T,E] fp32 or None, topk_ids [T,k] int32, topk_w [T,k] fp32)."""
    lib = load()
    T, d = x.shape
    E = w_router.shape[1]
    dev = x.device
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    act = act_code(x.dtype)

    def call(ws, nb):
        return lib.moe_route(_ptr(x), _ptr(w_router), _ptr(bias), T, d, E, k, act,
                             _ptr(logits), _ptr(ids), _ptr(w), ws, nb, _stream(stream))
    ws, nb = _workspace(call, dev)
    _check(call(_ptr(ws), _c.byref(nb)), "moe_route")
    return logits, ids, w


def align(topk_ids: torch.Tensor, E: int, block_m: int, stream=None):
    """Returns dict(counts, offsets, sorted_ids, inv_pos, block_expert)."""
    lib = load()
    T, k = topk_ids.shape
    dev = topk_ids.device
    cap = align_capacity(T, E, k, block_m)
    out = {
        "counts": torch.empty(E, dtype=torch.int32, device=dev),
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "sorted_ids": torch.empty(max(cap, 0), dtype=torch.int32, device=dev),
        "inv_pos": torch.empty(T * k, dtype=torch.int32, device=dev),
        "block_expert": torch.empty(max(cap // block_m, 0), dtype=torch.int32, device=dev),
    }

    def call(ws, nb):
        return lib.moe_align(_ptr(topk_ids), T, E, k, block_m, _ptr(out["counts"]),
                             _ptr(out["offsets"]), _ptr(out["sorted_ids"]), _ptr(out["inv_pos"]),
                             _ptr(out["block_expert"]), ws, nb, _stream(stream))
    ws, nb = _workspace(call, dev)
    _check(call(_ptr(ws), _c.byref(nb)), "moe_align")
    return out


def quantize_mxfp8(x: torch.Tensor, codes: Optional[torch.Tensor] = None,
                   scales: Optional[torch.Tensor] = None, stream=None):
    """MXFP8 codes (uint8 [rows, n]) and E8M0 scale bytes (uint8 [rows, n/32])
    of x [rows, n] (bf16 or fp32, blocks of 32 along the row).  Returns
    (codes, scales)."""
    rows, n = x.shape
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if codes is None:
        codes = torch.empty((rows, n), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, n // 32), dtype=torch.uint8, device=x.device)
    for t in (codes, scales):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("codes and scales: contiguous uint8")
    if codes.shape != (rows, n) or scales.shape != (rows, n // 32):
        raise ValueError("codes [rows, n] and scales [rows, n/32]")
    _check(load().moe_quantize_mxfp8(_ptr(x), rows, n, act_code(x.dtype), _ptr(codes),
                                     _ptr(scales), _stream(stream)), "moe_quantize_mxfp8")
    return codes, scales


def rms_norm(x: torch.Tensor, weight: torch.Tensor, out: Optional[torch.Tensor] = None,
             weight_bias: float = 0.0, eps: float = 1e-6, stream=None):
    """Row RMSNorm of x [T, d] with gain weight [d] into out (a new tensor, or
    x itself for in place).  Returns out."""
    T, d = x.shape
    if out is None:
        out = torch.empty_like(x)
    for t in (x, weight, out):
        if t.dtype != x.dtype or not t.is_contiguous():
            raise ValueError("x, weight and out: one dtype, contiguous")
    _check(load().moe_rms_norm(_ptr(x), _ptr(weight), _ptr(out), T, d, act_code(x.dtype),
                               float(weight_bias), float(eps), _stream(stream)), "moe_rms_norm")
    return out


def qk_norm(q: Optional[torch.Tensor], k: Optional[torch.Tensor],
            q_weight: Optional[torch.Tensor], k_weight: Optional[torch.Tensor],
            weight_bias: float = 0.0, eps: float = 1e-6, stream=None):
    """In-place QK-norm of q [T, nq, hd] and k [T, nk, hd] (either may be
    None); weights [hd] in the same dtype.  Returns (q, k)."""
    ref = q if q is not None else k
    T, _, hd = ref.shape
    nq = 0 if q is None else q.shape[1]
    nk = 0 if k is None else k.shape[1]
    for t in (q, k, q_weight, k_weight):
        if t is not None and (t.dtype != ref.dtype or not t.is_contiguous()):
            raise ValueError("q, k and the weights: one dtype, contiguous")
    if k is not None and k.shape[0] != T:
        raise ValueError("q and k: same token count")
    _check(load().moe_qk_norm(_ptr(q), _ptr(k), _ptr(q_weight), _ptr(k_weight), T, nq, nk, hd,
                              act_code(ref.dtype), float(weight_bias), float(eps),
                              _stream(stream)), "moe_qk_norm")
    return q, k


def make_layer_struct(w_router, bias, w_gate_up, w_down, k, scale_gate_up=None, scale_down=None):
    E, d, two_dff = w_gate_up.shape
    if w_gate_up.dtype == torch.uint8:
        d *= 2  # MXFP4: two codes per byte along K
    L = MoeLayer()
    L.d, L.d_ff, L.E, L.k = d, two_dff // 2, E, k
    L.act_dtype = _ACT[w_router.dtype]
    L.w_dtype = _WDT[w_gate_up.dtype]
    if L.w_dtype == MOE_FP8_E4M3 and scale_gate_up is not None and \
            scale_gate_up.dtype == torch.uint8:
        L.w_dtype = MOE_MXFP8  # e4m3fn codes with E8M0 block scales
    L.w_router, L.logit_bias = w_router.data_ptr(), (bias.data_ptr() if bias is not None else None)
    L.w_gate_up, L.w_down = w_gate_up.data_ptr(), w_down.data_ptr()
    L.scale_gate_up = scale_gate_up.data_ptr() if scale_gate_up is not None else None
    L.scale_down = scale_down.data_ptr() if scale_down is not None else None
    return L


class Forward:
    """Holds the layer description and a reusable workspace for moe_forward."""

    def __init__(self, w_router, bias, w_gate_up, w_down, k, scale_gate_up=None,
                 scale_down=None):
        self.lib = load()
        self.tensors = (w_router, bias, w_gate_up, w_down, scale_gate_up, scale_down)
        self.L = make_layer_struct(w_router, bias, w_gate_up, w_down, k, scale_gate_up,
                                   scale_down)
        self.device = w_gate_up.device
        self.ws = None
        self.ws_T = -1

    def workspace_bytes(self, T: int) -> int:
        n = _c.c_size_t(0)
        _check(self.lib.moe_forward(_c.byref(self.L), None, T, None, None, _c.byref(n), None,
                                    None), "moe_forward workspace query")
        return int(n.value)

    def _ensure_ws(self, T: int):
        need = self.workspace_bytes(T)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=self.device)
        return need

    def routing_buffers(self, T: int):
        E, k, dev = self.L.E, self.L.k, self.device
        cap = align_capacity(T, E, k, MOE_BLOCK_M_MAX)
        return {
            "logits": torch.empty((T, E), dtype=torch.float32, device=dev),
            "topk_ids": torch.empty((T, k), dtype=torch.int32, device=dev),
            "topk_w": torch.empty((T, k), dtype=torch.float32, device=dev),
            "counts": torch.empty(E, dtype=torch.int32, device=dev),
            "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "sorted_ids": torch.empty(max(cap, 1), dtype=torch.int32, device=dev),
            "inv_pos": torch.empty(max(T * k, 1), dtype=torch.int32, device=dev),
        }

    @staticmethod
    def _routing_struct(routing, bm):
        if routing is None:
            return None
        r = MoeRoutingOut()
        r.logits = routing["logits"].data_ptr()
        r.topk_ids = routing["topk_ids"].data_ptr()
        r.topk_w = routing["topk_w"].data_ptr()
        r.expert_counts = routing["counts"].data_ptr()
        r.padded_offsets = routing["offsets"].data_ptr()
        r.sorted_ids = routing["sorted_ids"].data_ptr()
        r.inv_pos = routing["inv_pos"].data_ptr()
        r.block_m = _c.pointer(bm)
        return r

    def noalloc(self, x: torch.Tensor, out: torch.Tensor, routing=None, stream=None):
        """moe_forward_noalloc: the layer on x [T, d] into the caller's `out`,
        with the library's static scratch instead of a workspace (raises
        MoeError with MOE_ERR_SCRATCH when the batch needs more).  Returns
        (out, block_m)."""
        bm = _c.c_int(0)
        r = self._routing_struct(routing, bm)
        rc = self.lib.moe_forward_noalloc(_c.byref(self.L), _ptr(x), x.shape[0], _ptr(out),
                                          _c.byref(r) if r is not None else None,
                                          _stream(stream))
        _check(rc, "moe_forward_noalloc")
        return out, bm.value

    def __call__(self, x: torch.Tensor, out: Optional[torch.Tensor] = None, routing=None,
                 events=None, stream=None):
        """Run the layer on x [T, d].  `routing`: dict from routing_buffers() to
        receive the routing; `events`: list of raw hipEvent_t handles (ints) to
        record around each kernel.  Returns (out, block_m, kernel names)."""
        T = x.shape[0]
        if out is None:
            out = torch.empty_like(x)
        need = self._ensure_ws(T)
        nb = _c.c_size_t(need)
        bm = _c.c_int(0)
        r = self._routing_struct(routing, bm)
        rp = _c.byref(r) if r is not None else None
        if events is None:
            rc = self.lib.moe_forward(_c.byref(self.L), _ptr(x), T, _ptr(out), _ptr(self.ws),
                                      _c.byref(nb), rp, _stream(stream))
            _check(rc, "moe_forward")
            return out, bm.value, None
        tr = MoeTrace()
        arr = (_vp * len(events))(*events)
        tr.events = arr
        tr.n_events = len(events)
        rc = self.lib.moe_forward_traced(_c.byref(self.L), _ptr(x), T, _ptr(out), _ptr(self.ws),
                                         _c.byref(nb), rp, _c.byref(tr), _stream(stream))
        _check(rc, "moe_forward_traced")
        names = [tr.names[i].decode() for i in range(min(tr.n_kernels, 16))]
        return out, bm.value, names


# ------------------------------------------------------------ HIP events
class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self, n: int):
        self.hip = _c.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [_c.POINTER(_vp)]
        self.hip.hipEventElapsedTime.argtypes = [_c.POINTER(_c.c_float), _vp, _vp]
        self.hip.hipEventSynchronize.argtypes = [_vp]
        self.hip.hipEventDestroy.argtypes = [_vp]
        self.handles = []
        for _ in range(n):
            h = _vp()
            rc = self.hip.hipEventCreate(_c.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            self.handles.append(h.value)

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = _c.c_float(0)
        self.hip.hipEventSynchronize(_vp(self.handles[j]))
        rc = self.hip.hipEventElapsedTime(_c.byref(ms), _vp(self.handles[i]), _vp(self.handles[j]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def __del__(self):
        try:
            for h in self.handles:
                self.hip.hipEventDestroy(_vp(h))
        except Exception:
            pass
