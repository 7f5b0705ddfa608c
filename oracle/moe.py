"""Plain fp64 CPU oracle of one MoE layer (test infrastructure only).

What the layer computes, per token t with activation x (bf16 at the boundary):

  1. router logits   l_e = sum_h W_r[e, h] * x[h] + b_e            (fp64)
  2. p = softmax(l) over all E experts
  3. S = the k experts ordered by (logit descending, index ascending)
  4. gates g_i = p[S_i] / sum_{j in S} p[S_j]   (renormalised top-k)
  5. for each selected expert e: w = fp16 scale * integer code, blocks of 32
     along the input dimension; a = G_e x, u = U_e x, h = SiLU(a) * u,
     y_e = D_e h                                                   (fp64)
  6. shared expert (always on, weight 1): y_s = D_s(SiLU(G_s x) * U_s x)
  7. y = sum_i g_i y_{S_i} + y_s       (slot order, then the shared expert)

Sources. The pages fix the structure: each token uses 10 of 512 routed
experts plus one always-on shared expert (Strata write-up, "The 30-Second
Overview" table; explainer video, transcript at 2:01), and the outputs of a
token's experts are added together into that token's single result (video,
transcript at 3:36). The pages give no formula for the
router, the gates, the FFN or the quantisation; steps 2-5 follow the workload
definition this build targets (softmax over router logits, then top-k with
renormalised gates; SwiGLU FFN; signed 4-/3-bit codes in 32-element blocks
with one fp16 scale per block; fp32 dequantisation and fp64 accumulation).
The readings taken where both are silent are: selection on the logits (not
on p) with ties to the lower index; no biases inside the FFN; symmetric
codes with no zero point; the shared expert has gate weight 1.

Pins (tests/test_oracle_*.py) tie every function here to something other
than itself: brute-force top-k by counting, a dense all-experts mixture,
k = E equal to the dense softmax mixture, a single expert equal to PyTorch's
SwiGLU, router independence for identical experts, closed forms (zero
router, zero input, scale doubling, expert relabelling), worked fixtures in
tests/golden/, scipy's softmax and expit.
"""
from __future__ import annotations

from typing import Callable, Optional, Tuple

import numpy as np

BLOCK = 32  # elements per quantisation block, contiguous along the input dim


# ----------------------------------------------------------------------------
# Number formats (exact widening).
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(u: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64. bf16 is the top half of an fp32."""
    u32 = np.asarray(u, np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def f16_bits_to_f64(u: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64."""
    return np.asarray(u, np.uint16).view(np.float16).astype(np.float64)


def round_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, round to nearest even.

    Rounds directly from the fp64 value: the 8 significant bits of the
    result are the nearest bf16 value, ties to even mantissa."""
    v = np.asarray(v, np.float64)
    out = np.zeros(v.shape, np.uint16)
    nz = v != 0
    m, e = np.frexp(v[nz])            # v = m * 2^e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits: scale the mantissa to an integer in [128, 256)
    q = np.rint(np.abs(m) * 256.0)    # numpy rint rounds half to even
    carry = q == 256.0
    q = np.where(carry, 128.0, q)
    e = np.where(carry, e + 1, e)
    val = np.sign(m) * q * np.ldexp(1.0, e - 8)
    out[nz] = (val.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return out


# ----------------------------------------------------------------------------
# Weights.
# ----------------------------------------------------------------------------

def dequant_blocks(q: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    """Dequantise signed codes with one fp16 scale per 32-element block.

    q: int8 [..., K]; s_bits: uint16 fp16 [..., K/32]. Returns float64 equal to
    the fp32 value s * q (exact: an 11-bit scale times a 4-bit integer)."""
    q = np.asarray(q)
    K = q.shape[-1]
    assert K % BLOCK == 0 and s_bits.shape[-1] == K // BLOCK
    s = f16_bits_to_f64(s_bits).astype(np.float32)
    w = q.astype(np.float32).reshape(q.shape[:-1] + (K // BLOCK, BLOCK)) * s[..., None]
    return w.reshape(q.shape).astype(np.float64)


def expert_weights(layer, e: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(G [I,H], U [I,H], D [H,I]) of routed expert e in float64."""
    if layer.wtype == "f32":
        return (layer.gate_f[e].astype(np.float64), layer.up_f[e].astype(np.float64),
                layer.down_f[e].astype(np.float64))
    if layer.wtype == "bf16":
        return (bf16_bits_to_f64(layer.gate_f[e]), bf16_bits_to_f64(layer.up_f[e]),
                bf16_bits_to_f64(layer.down_f[e]))
    return (dequant_blocks(layer.gate_q[e], layer.gate_s[e]),
            dequant_blocks(layer.up_q[e], layer.up_s[e]),
            dequant_blocks(layer.down_q[e], layer.down_s[e]))


def shared_weights(layer):
    """(G, U, D) of the shared expert in float64, or None."""
    if layer.shared is None:
        return None
    if layer.shared == "f32":
        conv = lambda a: np.asarray(a, np.float32).astype(np.float64)
    else:
        conv = bf16_bits_to_f64
    return conv(layer.shared_gate), conv(layer.shared_up), conv(layer.shared_down)


# ----------------------------------------------------------------------------
# Router.
# ----------------------------------------------------------------------------

def router_logits(layer, x64: np.ndarray) -> np.ndarray:
    """l[t, e] = sum_h W_r[e, h] x[t, h] + b_e, in float64."""
    W = layer.router_w.astype(np.float64)
    l = x64 @ W.T
    if layer.router_b is not None:
        l = l + layer.router_b.astype(np.float64)[None, :]
    return l


def softmax(l: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, shifted by the max for range safety."""
    m = np.max(l, axis=-1, keepdims=True)
    z = np.exp(l - m)
    return z / np.sum(z, axis=-1, keepdims=True)


def select_topk(l: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits, ordered by (logit desc, index asc).

    l: one token's logits [E], or a batch [T, E] (each row on its own)."""
    l = np.asarray(l, np.float64)
    E = l.shape[-1]
    index = np.broadcast_to(np.arange(E), l.shape)
    order = np.lexsort((index, -l), axis=-1)   # last key is the primary one
    return order[..., :k].astype(np.int32)


def route(layer, x_bits: np.ndarray):
    """Top-k routing of tokens x (bf16 bits [T, H]).

    Returns idx int32 [T, k] (ordered), gates float64 [T, k], logits [T, E]."""
    x64 = bf16_bits_to_f64(x_bits)
    l = router_logits(layer, x64)
    p = softmax(l)
    idx = select_topk(l, layer.k)
    pS = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    gates = pS / np.sum(pS, axis=1, keepdims=True)
    return idx, gates, l


# ----------------------------------------------------------------------------
# Expert FFN and the layer.
# ----------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(G: np.ndarray, U: np.ndarray, D: np.ndarray, x64: np.ndarray) -> np.ndarray:
    """y = D (SiLU(G x) * (U x)) for rows of x ([T, H] -> [T, H])."""
    a = x64 @ G.T
    u = x64 @ U.T
    h = silu(a) * u
    return h @ D.T


class DenseExperts:
    """Expert provider backed by a HostLayer (dequantises on demand)."""

    def __init__(self, layer, cache: bool = True):
        self.layer = layer
        self.cache = {} if cache else None

    def __call__(self, e: int):
        if self.cache is not None and e in self.cache:
            return self.cache[e]
        w = expert_weights(self.layer, e)
        if self.cache is not None:
            self.cache[e] = w
        return w


def moe_forward(layer, x_bits: np.ndarray,
                experts: Optional[Callable[[int], tuple]] = None,
                return_parts: bool = False):
    """MoE layer output for tokens x (bf16 bits [T, H]).

    Returns (y float64 [T, H], idx int32 [T, k], gates float64 [T, k]).
    With return_parts, also the per-slot expert outputs [T, k, H] and the
    shared expert output [T, H] (zeros when there is none)."""
    if experts is None:
        experts = DenseExperts(layer, cache=False)
    x64 = bf16_bits_to_f64(x_bits)
    T, H = x64.shape
    idx, gates, _ = route(layer, x_bits)
    k = idx.shape[1]
    parts = np.zeros((T, k, H), np.float64)
    # evaluate each used expert once on the tokens that chose it
    for e in np.unique(idx):
        rows, slots = np.nonzero(idx == e)
        G, U, D = experts(int(e))
        parts[rows, slots] = swiglu_ffn(G, U, D, x64[rows])
    ys = np.zeros((T, H), np.float64)
    sw = shared_weights(layer)
    if sw is not None:
        ys = swiglu_ffn(*sw, x64)
    y = np.zeros((T, H), np.float64)
    for i in range(k):                  # slot order, then the shared expert
        y += gates[:, i:i + 1] * parts[:, i]
    y += ys
    if return_parts:
        return y, idx, gates, parts, ys
    return y, idx, gates


def rmsnorm(h64: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """z = h / sqrt(mean(h^2) + eps) per row, unit gain."""
    ms = np.mean(h64 * h64, axis=-1, keepdims=True)
    return h64 / np.sqrt(ms + eps)
