"""Thin ctypes binding of libmoe (include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe.so. PyTorch provides device memory and the stream. If the library is
missing this module raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libmoe.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN, MOE_ERR_DTYPE, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_VALUE, \
    MOE_ERR_DEVICE = range(9)
W_F32, W_BF16, W_Q4, W_Q3, W_NONE = 0, 1, 2, 3, -1
WTYPES = {"f32": W_F32, "bf16": W_BF16, "q4": W_Q4, "q3": W_Q3, None: W_NONE}
DECODE_MAX_TOKENS = 8

# every entry point declared in include/moe.h
EXPORTS = [
    "moe_matrix_bytes", "moe_matrix_scales", "moe_workspace_bytes", "moe_route", "moe_forward_decode",
    "moe_forward_prefill", "moe_rmsnorm", "moe_residual_add", "moe_stack_decode_layer", "moe_pack_matrix",
    "moe_pack_gate_up",
    "moe_status_string", "moe_last_error", "moe_kernel_class_count", "moe_kernel_class_name",
    "moe_timer_enable", "moe_timer_reset", "moe_timer_read", "moe_workspace_init", "moe_workspace_check",
    "moe_debug_set_wait_limit", "moe_forward_decode_noalloc",
]


class MoeLayerC(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
        ("expert_wtype", ctypes.c_int32), ("gate_up", ctypes.c_void_p), ("gate_up_scales", ctypes.c_void_p),
        ("down", ctypes.c_void_p), ("down_scales", ctypes.c_void_p), ("shared_wtype", ctypes.c_int32),
        ("shared_gate_up", ctypes.c_void_p), ("shared_down", ctypes.c_void_p),
    ]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (what, _lib_obj.moe_status_string(status).decode(),
                                          _lib_obj.moe_last_error().decode()))


_lib_obj = None


def lib():
    """Load libmoe.so (built by quantized_expert_ffn_gemv_amd/build.py)."""
    global _lib_obj
    if _lib_obj is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        P = ctypes.POINTER(MoeLayerC)
        L.moe_matrix_bytes.restype = sz; L.moe_matrix_bytes.argtypes = [i32, i32, i32]
        L.moe_matrix_scales.restype = sz; L.moe_matrix_scales.argtypes = [i32, i32, i32]
        L.moe_workspace_bytes.restype = sz; L.moe_workspace_bytes.argtypes = [P, i32, i32]
        L.moe_route.restype = i32
        L.moe_route.argtypes = [P, vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_forward_decode.restype = i32
        L.moe_forward_decode.argtypes = [P, vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_forward_decode_noalloc.restype = i32
        L.moe_forward_decode_noalloc.argtypes = [P, vp, i32, vp, vp, vp, vp]
        L.moe_forward_prefill.restype = i32
        L.moe_forward_prefill.argtypes = [P, vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_rmsnorm.restype = i32; L.moe_rmsnorm.argtypes = [vp, vp, i32, i32, ctypes.c_float, vp]
        L.moe_residual_add.restype = i32; L.moe_residual_add.argtypes = [vp, vp, i32, i32, vp]
        L.moe_stack_decode_layer.restype = i32
        L.moe_stack_decode_layer.argtypes = [P, vp, i32, ctypes.c_float, vp, vp, vp, vp, vp, sz, vp]
        L.moe_pack_matrix.restype = i32; L.moe_pack_matrix.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.moe_pack_gate_up.restype = i32
        L.moe_pack_gate_up.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.moe_status_string.restype = ctypes.c_char_p; L.moe_status_string.argtypes = [i32]
        L.moe_last_error.restype = ctypes.c_char_p; L.moe_last_error.argtypes = []
        L.moe_kernel_class_count.restype = i32; L.moe_kernel_class_count.argtypes = []
        L.moe_kernel_class_name.restype = ctypes.c_char_p; L.moe_kernel_class_name.argtypes = [i32]
        L.moe_workspace_init.restype = i32; L.moe_workspace_init.argtypes = [vp, sz, vp]
        L.moe_workspace_check.restype = i32; L.moe_workspace_check.argtypes = [vp, sz, vp]
        L.moe_debug_set_wait_limit.restype = i32; L.moe_debug_set_wait_limit.argtypes = [ctypes.c_uint64]
        L.moe_timer_enable.restype = i32; L.moe_timer_enable.argtypes = [i32]
        L.moe_timer_reset.restype = i32; L.moe_timer_reset.argtypes = []
        L.moe_timer_read.restype = i32
        L.moe_timer_read.argtypes = [i32, ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double)]
        _lib_obj = L
    return _lib_obj


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


def _np_ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _tptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------------------
# sizes and packing (host)
# ---------------------------------------------------------------------------

def moe_matrix_bytes(wt: int, rows: int, K: int) -> int:
    return lib().moe_matrix_bytes(wt, rows, K)


def moe_matrix_scales(wt: int, rows: int, K: int) -> int:
    return lib().moe_matrix_scales(wt, rows, K)


def moe_pack_matrix(wt: int, src: np.ndarray, scales: Optional[np.ndarray] = None):
    """Pack W[R][K] -> (values uint8, scales uint16 or None) in the chunk-major layout."""
    R, K = src.shape
    out = np.empty(moe_matrix_bytes(wt, R, K), np.uint8)
    ns = moe_matrix_scales(wt, R, K)
    osc = np.empty(ns, np.uint16) if ns else None
    src = np.ascontiguousarray(src)
    sc = None if scales is None else np.ascontiguousarray(scales, np.uint16)
    _check(lib().moe_pack_matrix(wt, R, K, _np_ptr(src), _np_ptr(sc), _np_ptr(out), _np_ptr(osc)), "moe_pack_matrix")
    return out, osc


def moe_pack_gate_up(wt: int, gate: np.ndarray, up: np.ndarray, gate_s=None, up_s=None, out=None, out_s=None):
    """Fuse gate [I][H] and up [I][H] into the packed GU[2I][H]."""
    I, H = gate.shape
    if out is None:
        out = np.empty(moe_matrix_bytes(wt, 2 * I, H), np.uint8)
    ns = moe_matrix_scales(wt, 2 * I, H)
    if out_s is None and ns:
        out_s = np.empty(ns, np.uint16)
    gate, up = np.ascontiguousarray(gate), np.ascontiguousarray(up)
    gs = None if gate_s is None else np.ascontiguousarray(gate_s, np.uint16)
    us = None if up_s is None else np.ascontiguousarray(up_s, np.uint16)
    _check(lib().moe_pack_gate_up(wt, I, H, _np_ptr(gate), _np_ptr(gs), _np_ptr(up), _np_ptr(us), _np_ptr(out),
                                  _np_ptr(out_s)), "moe_pack_gate_up")
    return out, out_s


def _pack_expert_into(wt, L, e, gu, gus, dn, dns):
    lb = lib()
    I, H = L.I, L.H
    if wt in (W_Q4, W_Q3):
        g, gs, u, us = L.gate_q[e], L.gate_s[e], L.up_q[e], L.up_s[e]
        d, ds = L.down_q[e], L.down_s[e]
    else:
        g, gs, u, us, d, ds = L.gate_f[e], None, L.up_f[e], None, L.down_f[e], None
    st = lb.moe_pack_gate_up(wt, I, H, g.ctypes.data, None if gs is None else gs.ctypes.data, u.ctypes.data,
                             None if us is None else us.ctypes.data, gu.ctypes.data,
                             None if gus is None else gus.ctypes.data)
    _check(st, "moe_pack_gate_up")
    st = lb.moe_pack_matrix(wt, H, I, d.ctypes.data, None if ds is None else ds.ctypes.data, dn.ctypes.data,
                            None if dns is None else dns.ctypes.data)
    _check(st, "moe_pack_matrix")


class DeviceLayer:
    """A layer's weights packed and resident on the GPU (torch tensors) plus
    the moe_layer struct pointing at them."""

    def __init__(self, host, device="cuda", threads: int = 16):
        import torch
        self.H, self.I, self.E, self.k = host.H, host.I, host.E, host.k
        wt = WTYPES[host.wtype]
        swt = WTYPES[host.shared]
        self.wt, self.swt = wt, swt
        H, I, E = self.H, self.I, self.E
        gub, gus = moe_matrix_bytes(wt, 2 * I, H), moe_matrix_scales(wt, 2 * I, H)
        dnb, dns = moe_matrix_bytes(wt, H, I), moe_matrix_scales(wt, H, I)
        gu = np.empty((E, gub), np.uint8)
        dn = np.empty((E, dnb), np.uint8)
        gus_a = np.empty((E, gus), np.uint16) if gus else None
        dns_a = np.empty((E, dns), np.uint16) if dns else None

        def one(e):
            _pack_expert_into(wt, host, e, gu[e], None if gus_a is None else gus_a[e], dn[e],
                              None if dns_a is None else dns_a[e])

        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(E)))
        dev = torch.device(device)
        up = lambda a: None if a is None else torch.from_numpy(a).to(dev)
        self.router_w = up(np.ascontiguousarray(host.router_w, np.float32))
        self.router_b = up(None if host.router_b is None else np.ascontiguousarray(host.router_b, np.float32))
        self.gate_up, self.down = up(gu), up(dn)
        self.gate_up_s, self.down_s = up(gus_a), up(dns_a)
        self.shared_gate_up = self.shared_down = None
        if swt != W_NONE:
            sg, su, sd = host.shared_gate, host.shared_up, host.shared_down
            sgu, _ = moe_pack_gate_up(swt, sg, su)
            sdn, _ = moe_pack_matrix(swt, sd)
            self.shared_gate_up, self.shared_down = up(sgu), up(sdn)
        del gu, dn
        self.c = MoeLayerC(H, I, E, self.k, _tptr(self.router_w), _tptr(self.router_b), wt, _tptr(self.gate_up),
                           _tptr(self.gate_up_s), _tptr(self.down), _tptr(self.down_s), swt,
                           _tptr(self.shared_gate_up), _tptr(self.shared_down))

    def weight_bytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.gate_up, self.down, self.gate_up_s, self.down_s,
                                                         self.shared_gate_up, self.shared_down, self.router_w)
                   if t is not None)


# ---------------------------------------------------------------------------
# compute entry points (device tensors)
# ---------------------------------------------------------------------------

def moe_workspace_bytes(layer: DeviceLayer, max_tokens: int, mode: int) -> int:
    n = lib().moe_workspace_bytes(ctypes.byref(layer.c), max_tokens, mode)
    if n == 0:
        raise MoeError(MOE_ERR_SHAPE, "moe_workspace_bytes")
    return n


def make_workspace(layer: DeviceLayer, max_tokens: int, mode: int, device="cuda", stream=None):
    """Workspace tensor; a decode workspace (mode 0) comes initialised (see moe_workspace_init)."""
    import torch
    ws = torch.empty(moe_workspace_bytes(layer, max_tokens, mode), dtype=torch.uint8, device=device)
    if mode == 0:
        moe_workspace_init(ws, stream)
    return ws


def moe_workspace_init(ws, stream=None):
    _check(lib().moe_workspace_init(_tptr(ws), ws.numel(), _stream(stream)), "moe_workspace_init")


def moe_workspace_check(ws, stream=None):
    """Raises MoeError(MOE_ERR_DEVICE) if a device-side wait of a decode call ran out."""
    _check(lib().moe_workspace_check(_tptr(ws), ws.numel(), _stream(stream)), "moe_workspace_check")


def moe_route(layer, x, topk_idx, topk_gate, ws, expert_counts=None, stream=None):
    T = x.shape[0]
    _check(lib().moe_route(ctypes.byref(layer.c), _tptr(x), T, _tptr(topk_idx), _tptr(topk_gate),
                           _tptr(expert_counts), _tptr(ws), ws.numel(), _stream(stream)), "moe_route")


def moe_forward_decode(layer, x, y, ws, topk_idx=None, topk_gate=None, stream=None):
    B = x.shape[0]
    _check(lib().moe_forward_decode(ctypes.byref(layer.c), _tptr(x), B, _tptr(y), _tptr(topk_idx), _tptr(topk_gate),
                                    _tptr(ws), ws.numel(), _stream(stream)), "moe_forward_decode")


def moe_forward_decode_noalloc(layer, x, y, topk_idx=None, topk_gate=None, stream=None):
    """moe_forward_decode with the library's static scratch array as its workspace."""
    B = x.shape[0]
    _check(lib().moe_forward_decode_noalloc(ctypes.byref(layer.c), _tptr(x), B, _tptr(y), _tptr(topk_idx),
                                            _tptr(topk_gate), _stream(stream)), "moe_forward_decode_noalloc")


def moe_forward_prefill(layer, x, y, ws, topk_idx=None, topk_gate=None, stream=None):
    T = x.shape[0]
    _check(lib().moe_forward_prefill(ctypes.byref(layer.c), _tptr(x), T, _tptr(y), _tptr(topk_idx),
                                     _tptr(topk_gate), _tptr(ws), ws.numel(), _stream(stream)),
           "moe_forward_prefill")


def moe_rmsnorm(h, z, eps: float = 1e-6, stream=None):
    T, H = h.shape
    _check(lib().moe_rmsnorm(_tptr(h), _tptr(z), T, H, eps, _stream(stream)), "moe_rmsnorm")


def moe_residual_add(h, y, stream=None):
    T, H = h.shape
    _check(lib().moe_residual_add(_tptr(h), _tptr(y), T, H, _stream(stream)), "moe_residual_add")


def moe_stack_decode_layer(layer, h, ws, eps: float = 1e-6, z_out=None, y_out=None, topk_idx=None, topk_gate=None,
                           stream=None):
    """One stacked layer at decode, in place on h (bf16 [B, H]): z = RMSNorm(h),
    y = MoE(z), h = bf16(h + y); z_out / y_out receive z and y when given."""
    B = h.shape[0]
    _check(lib().moe_stack_decode_layer(ctypes.byref(layer.c), _tptr(h), B, eps, _tptr(z_out), _tptr(y_out),
                                        _tptr(topk_idx), _tptr(topk_gate), _tptr(ws), ws.numel(), _stream(stream)),
           "moe_stack_decode_layer")


class StackBuffers:
    """Per-call tensors of a layer stack over T tokens (z, y, routing)."""

    def __init__(self, T: int, H: int, k: int, device="cuda"):
        import torch
        self.z = torch.empty((T, H), dtype=torch.int16, device=device)
        self.y = torch.empty((T, H), dtype=torch.int16, device=device)
        self.idx = torch.empty((T, k), dtype=torch.int32, device=device)
        self.gate = torch.empty((T, k), dtype=torch.float32, device=device)


def stack_forward(layers, h, ws, decode: bool, buf: "StackBuffers", eps: float = 1e-6, stream=None,
                  each_layer=None):
    """Pre-norm residual stack of MoE layers over h (bf16 [T, H], updated in
    place): per layer z = RMSNorm(h), y = MoE(z), h = bf16(h + y). Decode runs
    each layer as one moe_stack_decode_layer call (one kernel at batch 1);
    prefill as moe_rmsnorm, moe_forward_prefill and moe_residual_add. Every
    step is a library call on the same stream. each_layer(l, buf), when given,
    runs after layer l, with buf.z, buf.y and the routing of that layer filled
    in (for decode they are written only when each_layer is given)."""
    for l, layer in enumerate(layers):
        if decode:
            want = each_layer is not None
            moe_stack_decode_layer(layer, h, ws, eps, buf.z if want else None, buf.y if want else None, buf.idx,
                                   buf.gate, stream)
        else:
            moe_rmsnorm(h, buf.z, eps, stream)
            moe_forward_prefill(layer, buf.z, buf.y, ws, buf.idx, buf.gate, stream)
            moe_residual_add(h, buf.y, stream)
        if each_layer is not None:
            each_layer(l, buf)
    return h


def debug_set_wait_limit(ticks: int):
    """Bound of the batch-1 decode kernel's device-side waits (0: the default)."""
    _check(lib().moe_debug_set_wait_limit(int(ticks)), "moe_debug_set_wait_limit")


# ---------------------------------------------------------------------------
# kernel timer
# ---------------------------------------------------------------------------

def kernel_classes():
    L = lib()
    return [L.moe_kernel_class_name(i).decode() for i in range(L.moe_kernel_class_count())]


def timer_enable(on: bool):
    _check(lib().moe_timer_enable(1 if on else 0), "moe_timer_enable")


def timer_reset():
    _check(lib().moe_timer_reset(), "moe_timer_reset")


def timer_read():
    """{kernel class: (launches, total ms)} since the last reset."""
    L = lib()
    out = {}
    for i, name in enumerate(kernel_classes()):
        n = ctypes.c_int64()
        ms = ctypes.c_double()
        _check(L.moe_timer_read(i, ctypes.byref(n), ctypes.byref(ms)), "moe_timer_read")
        if n.value:
            out[name] = (n.value, ms.value)
    return out
