"""Pins of the CPU oracle to things other than itself.

Each test ties an oracle function to brute force, a closed form, an invariant
of the definition, a library routine, or a hand-worked fixture, so that a
dropped term, a wrong sign or index, or a transposed operand fails here.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from synth import HostLayer

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _tiny_q(E=4, k=2, H=64, I=32, wtype="q4", shared="bf16", seed=0, **kw):
    return synth.random_layer(E, k, H, I, wtype, shared, seed, **kw)


def _tokens(T, H, seed=0, sd=1.0):
    return synth.normal_bf16(synth.key(seed, 999, T, H, 0), (T, H), sd)


# ----------------------------------------------------------------------------- formats

def test_bf16_and_f16_widening_exact():
    assert oracle.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x0000, 0x3E80], np.uint16)).tolist() == [1.0, -2.0, 0.0, 0.25]
    assert oracle.f16_bits_to_f64(np.array([0x3C00, 0x3400, 0x211F], np.uint16)).tolist() == [1.0, 0.25, 0.01000213623046875]


def test_round_to_bf16_matches_generator_rounding():
    # two independent RNE implementations (oracle: frexp/rint in fp64; generator: bit trick in C)
    v = synth.normal_f32(synth.key(5, 5, 5, 5, 5), (200000,), 3.0)
    v = np.concatenate([v, np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 65504.0, 1e-30], np.float32)])
    assert np.array_equal(oracle.round_to_bf16_bits(v.astype(np.float64)), synth.f32_to_bf16(v))


def test_dequant_worked_blocks():
    g = json.load(open(os.path.join(GOLD, "dequant_blocks.json")))
    q = np.array(g["codes"], np.int8)[None, :]
    s = np.array([int(v, 16) for v in g["scales_f16"]], np.uint16)[None, :]
    w = oracle.dequant_blocks(q, s)[0]
    assert np.array_equal(w[:32], 0.125 * np.array(g["codes"][:32], np.float64))
    for c, val in g["expect_block1"].items():
        sel = np.array(g["codes"][32:]) == int(c)
        assert np.all(w[32:][sel] == val)


def test_dequant_scale_axis_and_exactness():
    # scale j must multiply exactly the codes [32j, 32j+32) of its own row
    rng = np.random.default_rng(0)
    q = rng.integers(-8, 8, size=(3, 96)).astype(np.int8)
    s = synth.uniform_f16(synth.key(1, 2, 3, 4, 5), (3, 3), 0.005, 0.02)
    w = oracle.dequant_blocks(q, s)
    for r in range(3):
        for j in range(96):
            assert w[r, j] == float(np.float16(s.view(np.float16)[r, j // 32])) * int(q[r, j])


# ----------------------------------------------------------------------------- router

def _brute_topk(l, k):
    """e is selected iff fewer than k experts beat it (higher logit, or equal logit and lower index)."""
    E = len(l)
    sel = [e for e in range(E) if sum(1 for j in range(E) if l[j] > l[e] or (l[j] == l[e] and j < e)) < k]
    # order by the same rank count
    return sorted(sel, key=lambda e: sum(1 for j in range(E) if l[j] > l[e] or (l[j] == l[e] and j < e)))


@pytest.mark.parametrize("seed", range(6))
def test_select_topk_vs_brute_force(seed):
    rng = np.random.default_rng(seed)
    for E, k in ((8, 2), (8, 8), (13, 5), (16, 1), (32, 10)):
        l = rng.normal(size=E)
        if seed % 2:  # force ties
            l = np.round(l * 2) / 2
        assert oracle.select_topk(l, k).tolist() == _brute_topk(l, k)


def test_softmax_matches_scipy():
    rng = np.random.default_rng(1)
    l = rng.normal(size=(5, 37)) * 7
    assert np.allclose(oracle.softmax(l), scipy.special.softmax(l, axis=-1), rtol=1e-14, atol=0)


def test_gates_are_renormalised_softmax():
    L = _tiny_q(E=16, k=4, H=64, I=32, router_sd=0.3)
    x = _tokens(20, 64)
    idx, gates, logits = oracle.route(L, x)
    assert np.allclose(gates.sum(1), 1.0, atol=1e-15)
    assert np.all(np.diff(gates, axis=1) <= 0)
    # softmax restricted to the selected logits is algebraically the same thing
    for t in range(20):
        ls = logits[t, idx[t]]
        assert np.allclose(gates[t], scipy.special.softmax(ls), rtol=1e-13)
        # logits of the selected experts are the k largest
        assert ls.min() >= np.delete(logits[t], idx[t]).max()


def test_router_logits_by_loops_with_bias():
    L = _tiny_q(E=5, k=2, H=64, I=32, zipf=True, router_sd=0.1)
    x = _tokens(3, 64)
    l = oracle.router_logits(L, oracle.bf16_bits_to_f64(x))
    xf = oracle.bf16_bits_to_f64(x)
    for t in range(3):
        for e in range(5):
            acc = 0.0
            for h in range(64):
                acc += float(L.router_w[e, h]) * xf[t, h]
            acc += float(L.router_b[e])
            assert abs(acc - l[t, e]) < 1e-13


def test_zero_router_selects_first_k_with_equal_gates():
    L = _tiny_q(E=8, k=3)
    L.router_w[:] = 0
    idx, gates, _ = oracle.route(L, _tokens(4, 64))
    assert np.all(idx == np.array([0, 1, 2]))
    assert np.allclose(gates, 1 / 3, rtol=1e-15)


def test_bias_alone_decides_with_zero_router():
    L = _tiny_q(E=8, k=3)
    L.router_w[:] = 0
    L.router_b = np.array([0.1, 0.5, -1, 0.3, 0.5, 0.0, 2.0, -3], np.float32)
    idx, gates, _ = oracle.route(L, _tokens(2, 64))
    assert idx[0].tolist() == [6, 1, 4]
    b = L.router_b.astype(np.float64)[[6, 1, 4]]
    assert np.allclose(gates[0], np.exp(b) / np.exp(b).sum(), rtol=1e-14)


# ----------------------------------------------------------------------------- FFN and layer

def test_single_expert_is_torch_swiglu():
    # E = 1, k = 1, no shared expert: the layer is a plain SwiGLU FFN (PyTorch fp64 on the CPU)
    L = _tiny_q(E=1, k=1, H=96, I=64, shared=None)
    x = _tokens(7, 96)
    y, idx, gates = oracle.moe_forward(L, x)
    assert np.all(idx == 0) and np.all(gates == 1.0)
    G = torch.tensor(oracle.dequant_blocks(L.gate_q[0], L.gate_s[0]))
    U = torch.tensor(oracle.dequant_blocks(L.up_q[0], L.up_s[0]))
    D = torch.tensor(oracle.dequant_blocks(L.down_q[0], L.down_s[0]))
    xt = torch.tensor(oracle.bf16_bits_to_f64(x))
    ref = torch.nn.functional.linear(torch.nn.functional.silu(torch.nn.functional.linear(xt, G)) *
                                     torch.nn.functional.linear(xt, U), D)
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_shared_only_path_is_torch_swiglu_bf16_weights():
    L = _tiny_q(E=2, k=1, H=64, I=32, shared="bf16")
    x = _tokens(5, 64)
    _, _, _, parts, ys = oracle.moe_forward(L, x, return_parts=True)
    G, U, D = (torch.tensor(oracle.bf16_bits_to_f64(a)) for a in (L.shared_gate, L.shared_up, L.shared_down))
    xt = torch.tensor(oracle.bf16_bits_to_f64(x))
    ref = torch.nn.functional.silu(xt @ G.T) * (xt @ U.T) @ D.T
    assert np.allclose(ys, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_silu_matches_scipy_expit():
    z = np.linspace(-30, 30, 1001)
    assert np.allclose(oracle.moe.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("wtype", ["q4", "q3", "f32", "bf16"])
def test_sparse_equals_dense_masked_mixture(wtype):
    # brute force: run every expert on every token, weight by gate (0 outside S)
    L = _tiny_q(E=6, k=2, H=64, I=32, wtype=wtype, shared="bf16", router_sd=0.2)
    x = _tokens(9, 64)
    y, idx, gates = oracle.moe_forward(L, x)
    x64 = oracle.bf16_bits_to_f64(x)
    dense = np.zeros_like(y)
    for t in range(9):
        for e in range(6):
            G, U, D = oracle.expert_weights(L, e)
            g = gates[t, list(idx[t]).index(e)] if e in idx[t] else 0.0
            # second loop order for the products: explicit sums over h then j
            a = np.array([sum(G[j, h] * x64[t, h] for h in range(64)) for j in range(32)])
            u = np.array([sum(U[j, h] * x64[t, h] for h in range(64)) for j in range(32)])
            hh = a * scipy.special.expit(a) * u
            dense[t] += g * np.array([sum(D[r, j] * hh[j] for j in range(32)) for r in range(64)])
        sG, sU, sD = oracle.shared_weights(L)
        a, u = sG @ x64[t], sU @ x64[t]
        dense[t] += sD @ (a * scipy.special.expit(a) * u)
    assert np.allclose(y, dense, rtol=1e-11, atol=1e-12)


def test_k_equal_E_is_dense_softmax_mixture():
    L = _tiny_q(E=5, k=5, H=64, I=32, shared="bf16", router_sd=0.3)
    x = _tokens(6, 64)
    y, idx, gates = oracle.moe_forward(L, x)
    x64 = oracle.bf16_bits_to_f64(x)
    p = scipy.special.softmax(x64 @ L.router_w.astype(np.float64).T, axis=-1)
    ref = np.zeros_like(y)
    for e in range(5):
        G, U, D = oracle.expert_weights(L, e)
        a = x64 @ G.T
        ref += p[:, e:e + 1] * ((a * scipy.special.expit(a) * (x64 @ U.T)) @ D.T)
    sG, sU, sD = oracle.shared_weights(L)
    a = x64 @ sG.T
    ref += (a * scipy.special.expit(a) * (x64 @ sU.T)) @ sD.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_identical_experts_make_output_independent_of_router():
    L = _tiny_q(E=6, k=3, H=64, I=32, shared="bf16")
    for a in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s"):
        arr = getattr(L, a)
        arr[:] = arr[0]
    x = _tokens(8, 64)
    y1, i1, _ = oracle.moe_forward(L, x)
    L.router_w = synth.normal_f32(synth.key(42, 1, 2, 3, 4), L.router_w.shape, 0.5)
    L.router_b = np.linspace(-2, 2, 6).astype(np.float32)
    y2, i2, _ = oracle.moe_forward(L, x)
    assert not np.array_equal(i1, i2)
    assert np.allclose(y1, y2, rtol=1e-12, atol=1e-14)


def test_zero_input_gives_zero_output():
    L = _tiny_q(E=6, k=2)
    y, idx, gates = oracle.moe_forward(L, np.zeros((3, 64), np.uint16))
    assert np.all(y == 0.0)
    assert np.all(idx == np.array([0, 1]))


def test_doubling_down_scales_doubles_routed_output():
    L = _tiny_q(E=6, k=2, shared=None)
    x = _tokens(5, 64)
    y1, _, _ = oracle.moe_forward(L, x)
    s = L.down_s.view(np.float16) * np.float16(2)
    L.down_s = s.view(np.uint16)
    y2, _, _ = oracle.moe_forward(L, x)
    assert np.array_equal(y2, 2 * y1)


def test_zero_shared_down_removes_shared_contribution():
    L = _tiny_q(E=6, k=2, shared="bf16")
    x = _tokens(5, 64)
    y1, _, _, parts, ys = oracle.moe_forward(L, x, return_parts=True)
    L.shared_down = np.zeros_like(L.shared_down)
    y2, _, _ = oracle.moe_forward(L, x)
    assert np.allclose(y1 - ys, y2, rtol=1e-13, atol=1e-15)


def test_relabelling_experts_permutes_indices_only():
    L = _tiny_q(E=7, k=3, router_sd=0.2)
    x = _tokens(10, 64)
    y1, i1, g1 = oracle.moe_forward(L, x)
    perm = np.array([3, 6, 0, 5, 1, 4, 2])      # new expert n = old expert perm[n]
    L2 = HostLayer(**{**L.__dict__})
    L2.router_w = L.router_w[perm]
    for a in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s"):
        setattr(L2, a, getattr(L, a)[perm])
    y2, i2, g2 = oracle.moe_forward(L2, x)
    inv = np.argsort(perm)
    assert np.array_equal(inv[i1], i2)
    assert np.allclose(y1, y2, rtol=1e-13, atol=1e-15) and np.allclose(g1, g2, rtol=1e-14)


def test_batch_invariance():
    L = _tiny_q(E=8, k=2, router_sd=0.3)
    x = _tokens(12, 64)
    y, idx, gates = oracle.moe_forward(L, x)
    for t in range(12):
        yt, it, gt = oracle.moe_forward(L, x[t:t + 1])
        assert np.array_equal(it[0], idx[t])
        assert np.allclose(yt[0], y[t], rtol=1e-13, atol=1e-15)


def _worked_layer(g):
    E, k, H, I = g["E"], g["k"], g["H"], g["I"]
    sdef = int(g["scale_default_f16"], 16)
    L = HostLayer(H=H, I=I, E=E, k=k, wtype="q4", router_w=np.zeros((E, H), np.float32), router_b=None)
    for e, h, v in g["router_w"]:
        L.router_w[e, h] = v
    L.gate_q = np.zeros((E, I, H), np.int8); L.up_q = np.zeros((E, I, H), np.int8)
    L.down_q = np.zeros((E, H, I), np.int8)
    L.gate_s = np.full((E, I, H // 32), sdef, np.uint16); L.up_s = np.full((E, I, H // 32), sdef, np.uint16)
    L.down_s = np.full((E, H, I // 32), sdef, np.uint16)
    for name in ("gate", "up", "down"):
        q, s = getattr(L, name + "_q"), getattr(L, name + "_s")
        for e, r, c, code, sc in g["experts"][name]:
            q[e, r, c] = code
            s[e, r, c // 32] = int(sc, 16)
    L.shared = "bf16"
    bf = lambda v: int(synth.f32_to_bf16(np.array([v], np.float32))[0])
    L.shared_gate = np.zeros((I, H), np.uint16); L.shared_up = np.zeros((I, H), np.uint16)
    L.shared_down = np.zeros((H, I), np.uint16)
    for name in ("gate", "up", "down"):
        a = getattr(L, "shared_" + name)
        for r, c, v in g["shared_bf16"][name]:
            a[r, c] = bf(v)
    x = np.zeros((len(g["tokens"]), H), np.uint16)
    for t, tok in enumerate(g["tokens"]):
        for h, v in tok["x"]:
            x[t, h] = bf(v)
    return L, x


def test_worked_layer_fixture():
    g = json.load(open(os.path.join(GOLD, "worked_layer.json")))
    L, x = _worked_layer(g)
    y, idx, gates = oracle.moe_forward(L, x)
    for t, ex in enumerate(g["expect"]):
        assert idx[t].tolist() == ex["idx"]
        assert np.allclose(gates[t], ex["gates"], rtol=1e-15)
        want = np.zeros(L.H)
        for h, v in ex["y"]:
            want[h] = v
        assert np.allclose(y[t], want, rtol=1e-15, atol=1e-17)


def test_rmsnorm_closed_forms():
    c = 3.0
    z = oracle.rmsnorm(np.full((1, 16), c), eps=1e-6)
    assert np.allclose(z, c / math.sqrt(c * c + 1e-6), rtol=1e-15)
    h = np.array([[3.0, 4.0, 0.0, 0.0]])   # mean square = 25/4
    assert np.allclose(oracle.rmsnorm(h, eps=0.0), h / 2.5, rtol=1e-15)
    # scale invariance for eps = 0
    r = np.random.default_rng(3).normal(size=(4, 64))
    assert np.allclose(oracle.rmsnorm(7 * r, 0.0), oracle.rmsnorm(r, 0.0), rtol=1e-14)


@pytest.mark.parametrize("wtype", ["f32", "bf16"])
def test_single_dense_expert_is_torch_swiglu(wtype):
    # E = 1, k = 1, no shared expert, fp32 or bf16 expert weights: the layer is
    # a plain SwiGLU FFN. G, U and D come straight from the generated arrays
    # (widened by torch, not by the oracle), so a swapped gate/up or a wrong
    # widening in the oracle's dense-weight branch fails here.
    L = _tiny_q(E=1, k=1, H=96, I=64, wtype=wtype, shared=None)
    x = _tokens(7, 96)
    y, idx, gates = oracle.moe_forward(L, x)
    assert np.all(idx == 0) and np.all(gates == 1.0)
    if wtype == "f32":
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).double()
    else:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).double()
    G, U, D = conv(L.gate_f[0]), conv(L.up_f[0]), conv(L.down_f[0])
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double()
    ref = torch.nn.functional.linear(torch.nn.functional.silu(torch.nn.functional.linear(xt, G)) *
                                     torch.nn.functional.linear(xt, U), D)
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)
    # and the gate and up projections are not interchangeable
    swapped = torch.nn.functional.linear(torch.nn.functional.silu(torch.nn.functional.linear(xt, U)) *
                                         torch.nn.functional.linear(xt, G), D)
    assert not np.allclose(y, swapped.numpy(), rtol=1e-6, atol=1e-8)


def test_batched_selection_equals_per_row_selection():
    # the oracle selects all rows at once; each row must equal the brute-force count
    rng = np.random.default_rng(9)
    l = np.round(rng.normal(size=(40, 16)) * 2) / 2   # many exact ties
    got = oracle.select_topk(l, 5)
    for t in range(40):
        assert got[t].tolist() == _brute_topk(l[t], 5)
