"""C ABI of libmoe without a GPU: every declared symbol is exported, host-side
argument validation returns its documented codes before any device work, and
the host packer writes exactly the layout include/moe.h documents (checked
with an unpacker written here from that documentation)."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from quantized_expert_ffn_gemv_amd import moe

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_declarations_match_binding_list():
    assert _declared() == sorted(moe.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings():
    L = moe.lib()
    for s in range(8):
        assert L.moe_status_string(s).decode() not in ("", "unknown status")
    assert L.moe_status_string(99).decode() == "unknown status"


def _layer_c(**kw):
    d = dict(hidden=2048, inter=512, n_experts=512, top_k=10, router_w=16, router_bias=None, expert_wtype=moe.W_Q4,
             gate_up=16, gate_up_scales=16, down=16, down_scales=16, shared_wtype=moe.W_BF16, shared_gate_up=16,
             shared_down=16)
    d.update(kw)
    return moe.MoeLayerC(**d)


def test_sizes():
    assert moe.moe_matrix_bytes(moe.W_Q4, 1024, 2048) == 1024 * 2048 // 2
    assert moe.moe_matrix_bytes(moe.W_Q3, 1024, 2048) == 1024 * 2048 * 3 // 8
    assert moe.moe_matrix_scales(moe.W_Q4, 1024, 2048) == 1024 * 64
    assert moe.moe_matrix_bytes(moe.W_BF16, 2048, 512) == 2048 * 512 * 2
    assert moe.moe_matrix_scales(moe.W_BF16, 2048, 512) == 0
    assert moe.moe_matrix_bytes(moe.W_Q4, 10, 33) == 0
    # per-expert byte counts of the 512-expert layer (3 * 2048 * 512 weights)
    per_expert = (moe.moe_matrix_bytes(moe.W_Q4, 1024, 2048) + moe.moe_matrix_bytes(moe.W_Q4, 2048, 512)
                  + 2 * (moe.moe_matrix_scales(moe.W_Q4, 1024, 2048) + moe.moe_matrix_scales(moe.W_Q4, 2048, 512)))
    assert per_expert == 1769472
    L = _layer_c()
    assert moe.lib().moe_workspace_bytes(ctypes.byref(L), 1, 0) > 0
    assert moe.lib().moe_workspace_bytes(ctypes.byref(L), 9, 0) == 0
    assert moe.lib().moe_workspace_bytes(ctypes.byref(L), 4096, 1) > 0
    bad = _layer_c(hidden=100)
    assert moe.lib().moe_workspace_bytes(ctypes.byref(bad), 1, 0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=100), moe.MOE_ERR_SHAPE),
    (dict(inter=0), moe.MOE_ERR_SHAPE),
    (dict(top_k=0), moe.MOE_ERR_SHAPE),
    (dict(top_k=17), moe.MOE_ERR_SHAPE),
    (dict(n_experts=4, top_k=5), moe.MOE_ERR_SHAPE),
    (dict(expert_wtype=9), moe.MOE_ERR_DTYPE),
    (dict(shared_wtype=moe.W_Q4), moe.MOE_ERR_DTYPE),
    (dict(router_w=None), moe.MOE_ERR_NULL),
    (dict(gate_up_scales=None), moe.MOE_ERR_NULL),
    (dict(shared_down=None), moe.MOE_ERR_NULL),
    (dict(down=24), moe.MOE_ERR_ALIGN),
])
def test_layer_validation_codes(kw, status):
    L = moe.lib()
    layer = _layer_c(**kw)
    st = L.moe_forward_decode(ctypes.byref(layer), 16, 1, 16, None, None, 16, 1 << 30, None)
    assert st == status, L.moe_last_error()
    assert L.moe_last_error().decode() != ""


def test_call_validation_codes():
    L = moe.lib()
    layer = _layer_c()
    big = 1 << 40
    assert L.moe_forward_decode(ctypes.byref(layer), None, 1, 16, None, None, 16, big, None) == moe.MOE_ERR_NULL
    assert L.moe_forward_decode(ctypes.byref(layer), 16, 0, 16, None, None, 16, big, None) == moe.MOE_ERR_SHAPE
    assert L.moe_forward_decode(ctypes.byref(layer), 16, 9, 16, None, None, 16, big, None) == moe.MOE_ERR_SHAPE
    assert L.moe_forward_decode(ctypes.byref(layer), 8, 1, 16, None, None, 16, big, None) == moe.MOE_ERR_ALIGN
    assert L.moe_forward_decode(ctypes.byref(layer), 16, 1, 16, None, None, 16, 100, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_forward_prefill(ctypes.byref(layer), 16, 0, 16, None, None, 16, big, None) == moe.MOE_ERR_SHAPE
    assert L.moe_forward_prefill(ctypes.byref(layer), 16, 4096, 16, None, None, 16, 1000, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_route(ctypes.byref(layer), 16, 8, None, 16, None, 16, big, None) == moe.MOE_ERR_NULL
    assert L.moe_rmsnorm(16, 16, 1, 12, ctypes.c_float(1e-6), None) == moe.MOE_ERR_SHAPE
    assert L.moe_rmsnorm(16, 16, 1, 2048, ctypes.c_float(-1.0), None) == moe.MOE_ERR_SHAPE
    assert L.moe_residual_add(None, 16, 1, 2048, None) == moe.MOE_ERR_NULL
    # moe_stack_decode_layer(layer, h, B, eps, z_out, y_out, idx, gate, ws, ws_bytes, stream)
    S, f, lr = L.moe_stack_decode_layer, ctypes.c_float, ctypes.byref(layer)
    assert S(lr, None, 1, f(1e-6), None, None, None, None, 16, big, None) == moe.MOE_ERR_NULL
    assert S(lr, 16, 1, f(1e-6), None, None, None, None, None, big, None) == moe.MOE_ERR_NULL
    assert S(lr, 16, 0, f(1e-6), None, None, None, None, 16, big, None) == moe.MOE_ERR_SHAPE
    assert S(lr, 16, 9, f(1e-6), None, None, None, None, 16, big, None) == moe.MOE_ERR_SHAPE
    assert S(lr, 16, 1, f(-1.0), None, None, None, None, 16, big, None) == moe.MOE_ERR_SHAPE
    assert S(lr, 8, 1, f(1e-6), None, None, None, None, 16, big, None) == moe.MOE_ERR_ALIGN
    assert S(lr, 16, 1, f(1e-6), 24, None, None, None, 16, big, None) == moe.MOE_ERR_ALIGN
    assert S(lr, 16, 1, f(1e-6), None, 40, None, None, 16, big, None) == moe.MOE_ERR_ALIGN
    assert S(lr, 16, 1, f(1e-6), None, None, None, None, 16, 100, None) == moe.MOE_ERR_WORKSPACE
    # overlapping outputs (h spans B * H * 2 = 4 KiB here)
    assert S(lr, 1 << 20, 1, f(1e-6), (1 << 20) + 16, None, None, None, 16, big, None) == moe.MOE_ERR_SHAPE
    assert S(lr, 1 << 20, 1, f(1e-6), None, (1 << 20) - 16, None, None, 16, big, None) == moe.MOE_ERR_SHAPE
    assert S(lr, 1 << 20, 1, f(1e-6), 1 << 22, (1 << 22) + 16, None, None, 16, big, None) == moe.MOE_ERR_SHAPE


# ----------------------------------------------------------------------------- packing

def _unpack_doc(wt, rows, K, packed, scales=None):
    """Decode the chunk-major layout as include/moe.h describes it."""
    if wt == moe.W_Q4:
        words = packed.view(np.uint32).reshape(K // 32, rows, 4)
        out = np.empty((rows, K), np.int64)
        for j in range(4):
            for s in range(4):
                out[:, np.arange(K // 32) * 32 + 8 * j + 2 * s] = ((words[:, :, j] >> (4 * s)) & 15).T
                out[:, np.arange(K // 32) * 32 + 8 * j + 2 * s + 1] = ((words[:, :, j] >> (16 + 4 * s)) & 15).T
        codes = out - 8
    elif wt == moe.W_Q3:
        words = packed.view(np.uint32).reshape(K // 32, rows, 3)
        out = np.empty((rows, K), np.int64)
        base = np.arange(K // 32) * 32
        for i in range(15):
            w = words[:, :, i // 5]
            out[:, base + 2 * i] = ((w >> (3 * (i % 5))) & 7).T
            out[:, base + 2 * i + 1] = ((w >> (16 + 3 * (i % 5))) & 7).T
        e30 = np.zeros_like(words[:, :, 0])
        e31 = np.zeros_like(words[:, :, 0])
        for b in range(3):
            e30 |= ((words[:, :, b] >> 15) & 1) << b
            e31 |= ((words[:, :, b] >> 31) & 1) << b
        out[:, base + 30] = e30.T
        out[:, base + 31] = e31.T
        codes = out - 4
    elif wt == moe.W_BF16:
        codes = packed.view(np.uint16).reshape(K // 8, rows, 8).transpose(1, 0, 2).reshape(rows, K)
    else:
        codes = packed.view(np.float32).reshape(K // 4, rows, 4).transpose(1, 0, 2).reshape(rows, K)
    sc = None
    if scales is not None:
        sc = scales.reshape(K // 32, rows).T
    return codes, sc


@pytest.mark.parametrize("wt,bits", [(moe.W_Q4, 4), (moe.W_Q3, 3)])
def test_pack_quant_roundtrip_all_codes(wt, bits):
    rows, K = 48, 96
    q = synth.codes(synth.key(3, 3, 3, 3, 3), (rows, K), bits)
    lo = -(1 << (bits - 1))
    q[0, :1 << bits] = np.arange(lo, -lo, dtype=np.int8)   # every code value present
    s = synth.uniform_f16(synth.key(4, 4, 4, 4, 4), (rows, K // 32), 0.005, 0.02)
    packed, ps = moe.moe_pack_matrix(wt, q, s)
    codes, sc = _unpack_doc(wt, rows, K, packed, ps)
    assert np.array_equal(codes, q.astype(np.int64))
    assert np.array_equal(sc, s)


@pytest.mark.parametrize("wt", [moe.W_BF16, moe.W_F32])
def test_pack_dense_roundtrip(wt):
    rows, K = 40, 64
    if wt == moe.W_BF16:
        a = synth.normal_bf16(synth.key(5, 5, 5, 5, 5), (rows, K), 1.0)
    else:
        a = synth.normal_f32(synth.key(5, 5, 5, 5, 5), (rows, K), 1.0)
    packed, ps = moe.moe_pack_matrix(wt, a)
    assert ps is None
    codes, _ = _unpack_doc(wt, rows, K, packed)
    assert np.array_equal(codes, a)


def test_pack_gate_up_row_groups():
    I, H = 48, 64
    g = synth.codes(synth.key(6, 0, 0, 0, 1), (I, H), 4)
    u = synth.codes(synth.key(6, 0, 0, 0, 2), (I, H), 4)
    gs = synth.uniform_f16(synth.key(6, 0, 0, 0, 3), (I, H // 32), 0.005, 0.02)
    us = synth.uniform_f16(synth.key(6, 0, 0, 0, 4), (I, H // 32), 0.005, 0.02)
    packed, ps = moe.moe_pack_gate_up(moe.W_Q4, g, u, gs, us)
    codes, sc = _unpack_doc(moe.W_Q4, 2 * I, H, packed, ps)
    for r in range(2 * I):
        q, w = divmod(r, 32)
        src, srcs = (u, us) if w >= 16 else (g, gs)
        assert np.array_equal(codes[r], src[16 * q + (w % 16)])
        assert np.array_equal(sc[r], srcs[16 * q + (w % 16)])


def test_pack_rejects_out_of_range_codes():
    q = np.zeros((4, 32), np.int8)
    q[1, 5] = 4
    s = np.zeros((4, 1), np.uint16)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_pack_matrix(moe.W_Q3, q, s)
    assert ei.value.status == moe.MOE_ERR_VALUE
    q[1, 5] = -9
    with pytest.raises(moe.MoeError):
        moe.moe_pack_matrix(moe.W_Q4, q, s)
