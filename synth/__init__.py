"""Seeded synthetic inputs for the quantized routed-expert MoE layer.

This package draws random numbers and nothing else: it holds none of the
layer's arithmetic (no routing, no dequantisation, no products). The CPU
oracle and the HIP library both consume what it returns, so both sides see
bit-identical inputs.

Values are *logical*: integer codes in int8 arrays, fp16 scales and bf16
values as raw uint16 bit patterns, fp32 as float32. Packing into the device
layout is the library's job; the oracle reads the logical arrays directly.

The workloads mirror the pages' shapes: a 512-expert layer where each token
uses 10 routed experts plus one always-on shared expert (Strata write-up,
"30-Second Overview" table; video transcript at 2:01), 48 such layers (same
write-up, section 2 "Expert Cache and CPU/GPU Split"), low-bit expert weights
(section 1 "Low-Bit Quantization"), skewed expert usage (expert-cache hit
rates in the test-data appendix), batch-1 decode and prompts read in pieces
(Strata README, "How does it work").
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import zlib
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# Tensor ids used in stream keys.
T_X, T_ROUTER_W, T_ZIPF_PERM = 1, 2, 3
T_GATE_Q, T_GATE_S, T_UP_Q, T_UP_S, T_DOWN_Q, T_DOWN_S = 10, 11, 12, 13, 14, 15
T_GATE_F, T_UP_F, T_DOWN_F = 16, 17, 18
T_SH_GATE, T_SH_UP, T_SH_DOWN = 20, 21, 22


def build_lib(force: bool = False) -> str:
    """Compile libsynth.so with gcc (host code only)."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_lib()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32, u32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_uint32, ctypes.c_double, ctypes.c_void_p)
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u32, u32, u32, u32]
        L.synth_splitmix64_at.restype = u64
        L.synth_splitmix64_at.argtypes = [u64, u64]
        L.synth_normal_f32.argtypes = [u64, i64, dbl, dbl, vp]
        L.synth_normal_bf16.argtypes = [u64, i64, dbl, vp]
        L.synth_uniform_f16.argtypes = [u64, i64, dbl, dbl, vp]
        L.synth_codes.argtypes = [u64, i64, ctypes.c_int, vp]
        L.synth_permutation.argtypes = [u64, i32, vp]
        L.synth_f32_to_bf16.argtypes = [vp, i64, vp]
        for f in ("synth_normal_f32", "synth_normal_bf16", "synth_uniform_f16", "synth_codes",
                  "synth_permutation", "synth_f32_to_bf16"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def key(seed: int, a: int, b: int, c: int, d: int) -> int:
    return lib().synth_key(seed, a, b, c, d)


def normal_f32(k: int, shape, sd: float, mean: float = 0.0) -> np.ndarray:
    out = np.empty(shape, np.float32)
    lib().synth_normal_f32(k, out.size, mean, sd, _ptr(out))
    return out


def normal_bf16(k: int, shape, sd: float) -> np.ndarray:
    out = np.empty(shape, np.uint16)
    lib().synth_normal_bf16(k, out.size, sd, _ptr(out))
    return out


def uniform_f16(k: int, shape, lo: float, hi: float) -> np.ndarray:
    out = np.empty(shape, np.uint16)
    lib().synth_uniform_f16(k, out.size, lo, hi, _ptr(out))
    return out


def codes(k: int, shape, bits: int) -> np.ndarray:
    out = np.empty(shape, np.int8)
    lib().synth_codes(k, out.size, bits, _ptr(out))
    return out


def permutation(k: int, n: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    lib().synth_permutation(k, n, _ptr(out))
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().synth_f32_to_bf16(_ptr(a), a.size, _ptr(out))
    return out


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact; a bit shift, no arithmetic)."""
    return (np.asarray(u, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# Workloads. Names describe what they are; sizes follow the pages' model
# (512 experts, 10 routed + 1 shared, 48 layers) at hidden 2048 / expert
# intermediate 512.
# ---------------------------------------------------------------------------

# Zipf skew strength for the skewed-routing workloads. The bias added to the
# logit of expert e is -ZIPF_TAU * ZIPF_S * ln(rank_e). ZIPF_TAU was found by
# bisection (tests/golden/calibrate_zipf.py, which routes with the oracle) so
# that the hottest 20% of experts take 80% of top-10 selections at logit
# standard deviation 0.905; tests/golden/zipf_tau.json records the run.
ZIPF_S = 1.1
ZIPF_TAU = 0.4405

WORKLOADS = {
    "tiny": dict(id=0, E=8, k=2, H=64, I=32, wtype="f32", shared="f32", expert_sd=0.05,
                 shared_sd=0.05, router_sd=0.1, zipf=False, tokens=16, layers=1),
    "decode_q4": dict(id=1, E=512, k=10, H=2048, I=512, wtype="q4", shared="bf16",
                      shared_sd=0.05, router_sd=0.02, zipf=False, tokens=256, layers=1,
                      batch=1),
    "decode_q3_zipf": dict(id=2, E=512, k=10, H=2048, I=512, wtype="q3", shared="bf16",
                           shared_sd=0.05, router_sd=0.02, zipf=True, tokens=256, layers=1,
                           batch=(1, 8)),
    "prefill_q4": dict(id=3, E=512, k=10, H=2048, I=512, wtype="q4", shared="bf16",
                       shared_sd=0.05, router_sd=1.0 / math.sqrt(2048.0), zipf=False,
                       tokens=4096, layers=1),
    "stack48_q4": dict(id=4, E=512, k=10, H=2048, I=512, wtype="q4", shared="bf16",
                       shared_sd=0.05, router_sd=0.02, zipf=True, tokens=512,
                       prefill_tokens=32768, layers=48),
}
SCALE_LO, SCALE_HI = 0.005, 0.02


@dataclass
class HostLayer:
    """One MoE layer's weights in logical form (host numpy arrays)."""
    H: int
    I: int
    E: int
    k: int
    wtype: str                      # "f32" | "bf16" | "q4" | "q3"
    router_w: np.ndarray            # f32 [E, H]
    router_b: Optional[np.ndarray]  # f32 [E] or None
    # quantized experts: codes int8 and fp16 scale bits, blocks of 32 along K
    gate_q: Optional[np.ndarray] = None   # [E, I, H]
    gate_s: Optional[np.ndarray] = None   # [E, I, H/32]
    up_q: Optional[np.ndarray] = None
    up_s: Optional[np.ndarray] = None
    down_q: Optional[np.ndarray] = None   # [E, H, I]
    down_s: Optional[np.ndarray] = None   # [E, H, I/32]
    # fp32 experts (float32), or bf16 experts (uint16 bit patterns)
    gate_f: Optional[np.ndarray] = None   # [E, I, H]
    up_f: Optional[np.ndarray] = None
    down_f: Optional[np.ndarray] = None   # [E, H, I]
    shared: Optional[str] = None          # "f32" | "bf16" | None
    shared_gate: Optional[np.ndarray] = None  # [I, H]  f32 or bf16 bits
    shared_up: Optional[np.ndarray] = None
    shared_down: Optional[np.ndarray] = None  # [H, I]
    meta: dict = field(default_factory=dict)

    @property
    def qbits(self) -> int:
        return {"q4": 4, "q3": 3}.get(self.wtype, 0)


def zipf_bias(seed: int, wid: int, layer: int, E: int) -> np.ndarray:
    """Per-expert logit bias -tau*s*ln(rank), rank a seeded permutation of 1..E."""
    perm = permutation(key(seed, wid, layer, T_ZIPF_PERM, 0), E)
    rank = perm.astype(np.float64) + 1.0
    return (-ZIPF_TAU * ZIPF_S * np.log(rank)).astype(np.float32)


def expert_codes(seed: int, wid: int, layer: int, e: int, H: int, I: int, bits: int):
    """Regenerate one quantized expert: (gate_q, gate_s, up_q, up_s, down_q, down_s)."""
    g = codes(key(seed, wid, layer, T_GATE_Q, e), (I, H), bits)
    gs = uniform_f16(key(seed, wid, layer, T_GATE_S, e), (I, H // 32), SCALE_LO, SCALE_HI)
    u = codes(key(seed, wid, layer, T_UP_Q, e), (I, H), bits)
    us = uniform_f16(key(seed, wid, layer, T_UP_S, e), (I, H // 32), SCALE_LO, SCALE_HI)
    d = codes(key(seed, wid, layer, T_DOWN_Q, e), (H, I), bits)
    ds = uniform_f16(key(seed, wid, layer, T_DOWN_S, e), (H, I // 32), SCALE_LO, SCALE_HI)
    return g, gs, u, us, d, ds


def make_layer(name: str, layer: int = 0, seed: int = 0, experts: bool = True, threads: int = 1) -> HostLayer:
    """Generate the weights of layer `layer` of workload `name`.

    experts=False skips the routed experts (for workloads where only a few
    experts are regenerated on demand with expert_codes). threads > 1 makes
    the experts on a thread pool (same values: each expert has its own keys)."""
    c = WORKLOADS[name]
    wid, E, k, H, I = c["id"], c["E"], c["k"], c["H"], c["I"]
    rw = normal_f32(key(seed, wid, layer, T_ROUTER_W, 0), (E, H), c["router_sd"])
    rb = zipf_bias(seed, wid, layer, E) if c["zipf"] else None
    L = HostLayer(H=H, I=I, E=E, k=k, wtype=c["wtype"], router_w=rw, router_b=rb,
                  meta=dict(workload=name, layer=layer, seed=seed))
    if experts:
        if c["wtype"] == "f32":
            sd = c["expert_sd"]
            L.gate_f = np.stack([normal_f32(key(seed, wid, layer, T_GATE_F, e), (I, H), sd) for e in range(E)])
            L.up_f = np.stack([normal_f32(key(seed, wid, layer, T_UP_F, e), (I, H), sd) for e in range(E)])
            L.down_f = np.stack([normal_f32(key(seed, wid, layer, T_DOWN_F, e), (H, I), sd) for e in range(E)])
        else:
            bits = 4 if c["wtype"] == "q4" else 3
            L.gate_q = np.empty((E, I, H), np.int8); L.up_q = np.empty((E, I, H), np.int8)
            L.down_q = np.empty((E, H, I), np.int8)
            L.gate_s = np.empty((E, I, H // 32), np.uint16); L.up_s = np.empty((E, I, H // 32), np.uint16)
            L.down_s = np.empty((E, H, I // 32), np.uint16)
            def one(e):
                (L.gate_q[e], L.gate_s[e], L.up_q[e], L.up_s[e], L.down_q[e],
                 L.down_s[e]) = expert_codes(seed, wid, layer, e, H, I, bits)
            if threads > 1:
                from concurrent.futures import ThreadPoolExecutor
                with ThreadPoolExecutor(max_workers=threads) as ex:
                    list(ex.map(one, range(E)))
            else:
                for e in range(E):
                    one(e)
    sh = c["shared"]
    if sh is not None:
        L.shared = sh
        sd = c["shared_sd"]
        if sh == "f32":
            L.shared_gate = normal_f32(key(seed, wid, layer, T_SH_GATE, 0), (I, H), sd)
            L.shared_up = normal_f32(key(seed, wid, layer, T_SH_UP, 0), (I, H), sd)
            L.shared_down = normal_f32(key(seed, wid, layer, T_SH_DOWN, 0), (H, I), sd)
        else:
            L.shared_gate = normal_bf16(key(seed, wid, layer, T_SH_GATE, 0), (I, H), sd)
            L.shared_up = normal_bf16(key(seed, wid, layer, T_SH_UP, 0), (I, H), sd)
            L.shared_down = normal_bf16(key(seed, wid, layer, T_SH_DOWN, 0), (H, I), sd)
    return L


def make_tokens(name: str, seed: int = 0, T: Optional[int] = None) -> np.ndarray:
    """Activations ~N(0,1) rounded to bf16 once: uint16 bits [T, H]."""
    c = WORKLOADS[name]
    T = c["tokens"] if T is None else T
    return normal_bf16(key(seed, c["id"], 0, T_X, 0), (T, c["H"]), 1.0)


def make_prefill_tokens(name: str, seed: int = 0, T: Optional[int] = None) -> np.ndarray:
    c = WORKLOADS[name]
    T = c.get("prefill_tokens", c["tokens"]) if T is None else T
    return normal_bf16(key(seed, c["id"], 0, T_X, 1), (T, c["H"]), 1.0)


def random_layer(E: int, k: int, H: int, I: int, wtype: str, shared: Optional[str], seed: int,
                 router_sd: float = 0.02, expert_sd: float = 0.05, zipf: bool = False) -> HostLayer:
    """A small layer of arbitrary shape (tests: ragged sizes, edge cases)."""
    wid = 100 + (zlib.crc32(repr((E, k, H, I, wtype, shared)).encode()) & 0xFFFF)
    rw = normal_f32(key(seed, wid, 0, T_ROUTER_W, 0), (E, H), router_sd)
    rb = zipf_bias(seed, wid, 0, E) if zipf else None
    L = HostLayer(H=H, I=I, E=E, k=k, wtype=wtype, router_w=rw, router_b=rb,
                  meta=dict(workload="random", seed=seed))
    if wtype in ("f32", "bf16"):
        # fp32 values, or bf16 bit patterns for bf16 experts
        mk = normal_f32 if wtype == "f32" else normal_bf16
        L.gate_f = np.stack([mk(key(seed, wid, 0, T_GATE_F, e), (I, H), expert_sd) for e in range(E)])
        L.up_f = np.stack([mk(key(seed, wid, 0, T_UP_F, e), (I, H), expert_sd) for e in range(E)])
        L.down_f = np.stack([mk(key(seed, wid, 0, T_DOWN_F, e), (H, I), expert_sd) for e in range(E)])
    else:
        bits = 4 if wtype == "q4" else 3
        parts = [expert_codes(seed, wid, 0, e, H, I, bits) for e in range(E)]
        L.gate_q, L.gate_s, L.up_q, L.up_s, L.down_q, L.down_s = [np.stack(p) for p in zip(*parts)]
    if shared is not None:
        L.shared = shared
        mk = normal_f32 if shared == "f32" else normal_bf16
        L.shared_gate = mk(key(seed, wid, 0, T_SH_GATE, 0), (I, H), 0.05)
        L.shared_up = mk(key(seed, wid, 0, T_SH_UP, 0), (I, H), 0.05)
        L.shared_down = mk(key(seed, wid, 0, T_SH_DOWN, 0), (H, I), 0.05)
    return L
