"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Routing is compared bit-exactly (indices in order), gates and outputs within
the tolerances of tests/moe_testlib.py. Full-size workloads are checked on
every token, in the same launch configuration the benchmark times.
"""
import numpy as np
import pytest

import oracle
import synth
from moe_testlib import check_gates, check_routing, check_y, from_dev_bits, log, routing_scale, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_expert_ffn_gemv_amd import moe as m
    m.lib()
    return m


def _decode_calls(m, L, x_bits, B, ws=None):
    """Run consecutive decode calls of B tokens; returns y bits, idx, gates."""
    T, H = x_bits.shape
    xd = to_dev(x_bits)
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    idx = torch.empty((T, L.k), dtype=torch.int32, device="cuda")
    g = torch.empty((T, L.k), dtype=torch.float32, device="cuda")
    if ws is None:
        ws = m.make_workspace(L, B, 0)
    for t0 in range(0, T, B):
        t1 = min(T, t0 + B)
        m.moe_forward_decode(L, xd[t0:t1], y[t0:t1], ws, topk_idx=idx[t0:t1], topk_gate=g[t0:t1])
    torch.cuda.synchronize()
    m.moe_workspace_check(ws)  # no device-side wait ran out
    return from_dev_bits(y), idx.cpu().numpy(), g.cpu().numpy()


def _prefill(m, L, x_bits):
    T, H = x_bits.shape
    xd = to_dev(x_bits)
    ws = m.make_workspace(L, T, 1)
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    idx = torch.empty((T, L.k), dtype=torch.int32, device="cuda")
    g = torch.empty((T, L.k), dtype=torch.float32, device="cuda")
    m.moe_forward_prefill(L, xd, y, ws, topk_idx=idx, topk_gate=g)
    torch.cuda.synchronize()
    return from_dev_bits(y), idx.cpu().numpy(), g.cpu().numpy()


def _check_all(host, x, y, idx, g, what, ref=None):  # noqa: C901
    """Routing, gates and outputs of every token against the oracle (ref: a
    precomputed (y, idx, gates, logits) of the same tokens)."""
    if ref is None:
        y_ref, idx_ref, g_ref = oracle.moe_forward(host, x)
        _, _, logits = oracle.route(host, x)
    else:
        y_ref, idx_ref, g_ref, logits = ref
    n = check_routing(idx, idx_ref, logits, what, scale=routing_scale(host, x))
    if n:
        log("  %s: %d tokens ordered differently within a near-tie" % (what, n))
    check_gates(g, g_ref, what)
    check_y(y, y_ref, what)


def _oracle_ref(host, x):
    y_ref, idx_ref, g_ref = oracle.moe_forward(host, x)
    _, _, logits = oracle.route(host, x)
    return y_ref, idx_ref, g_ref, logits


# ----------------------------------------------------------------------------- tiny

def test_tiny_decode_b1_and_b8_and_prefill(moe):
    log("tiny layer: decode B=1, decode B=8, prefill T=16")
    host = synth.make_layer("tiny")
    x = synth.make_tokens("tiny")
    L = moe.DeviceLayer(host)
    for B in (1, 8):
        y, idx, g = _decode_calls(moe, L, x, B)
        _check_all(host, x, y, idx, g, "tiny decode B=%d" % B)
    y, idx, g = _prefill(moe, L, x)
    _check_all(host, x, y, idx, g, "tiny prefill")


@pytest.mark.parametrize("wtype,shared", [("q4", "bf16"), ("q3", None), ("f32", "f32"), ("bf16", "bf16")])
def test_ragged_shapes(moe, wtype, shared):
    # H/32 = 3 blocks (not a power of two), 37 experts, prefill tail of 300 tokens
    log("ragged layer E=37 k=5 H=96 I=64 %s shared=%s" % (wtype, shared))
    host = synth.random_layer(37, 5, 96, 64, wtype, shared, seed=11, router_sd=0.2)
    x = synth.normal_bf16(synth.key(11, 1, 1, 1, 1), (300, 96), 1.0)
    L = moe.DeviceLayer(host)
    y, idx, g = _prefill(moe, L, x)
    _check_all(host, x, y, idx, g, "ragged prefill %s" % wtype)
    xs = x[:24]
    for B in (1, 3, 8):
        y, idx, g = _decode_calls(moe, L, xs, B)
        _check_all(host, xs, y, idx, g, "ragged decode B=%d %s" % (B, wtype))


@pytest.mark.parametrize("wtype,H", [("q4", 8192), ("q3", 4096)])
def test_large_hidden(moe, wtype, H):
    # hidden sizes past the one-kernel decode path (H > 2048; 8192 is the
    # largest the library takes): batch-1 and batch-2 decode on the four-kernel
    # path (B * H at its 16384 limit), and a ragged prefill whose router reads
    # x in 512-element chunks
    log("large hidden: E=16 k=4 H=%d I=96 %s" % (H, wtype))
    host = synth.random_layer(16, 4, H, 96, wtype, "bf16", seed=21, router_sd=0.05)
    L = moe.DeviceLayer(host)
    x = synth.normal_bf16(synth.key(21, 2, 2, 2, 2), (100, H), 1.0)
    y, idx, g = _prefill(moe, L, x)
    _check_all(host, x, y, idx, g, "large-H prefill %s" % wtype)
    xs = x[:6]
    for B in (1, 2):
        y, idx, g = _decode_calls(moe, L, xs, B)
        _check_all(host, xs, y, idx, g, "large-H decode B=%d %s" % (B, wtype))


@pytest.mark.parametrize("E,k", [(1, 1), (4, 4), (64, 16), (1024, 16)])
def test_edge_expert_counts(moe, E, k):
    log("edge E=%d k=%d" % (E, k))
    host = synth.random_layer(E, k, 64, 32, "q4", "bf16", seed=5, router_sd=0.3)
    x = synth.normal_bf16(synth.key(5, 2, 2, 2, 2), (20, 64), 1.0)
    L = moe.DeviceLayer(host)
    y, idx, g = _prefill(moe, L, x)
    _check_all(host, x, y, idx, g, "edge prefill E=%d k=%d" % (E, k))
    y, idx, g = _decode_calls(moe, L, x[:8], 1)
    _check_all(host, x[:8], y, idx, g, "edge decode E=%d k=%d" % (E, k))


def test_decode_b1_three_kernel_shape(moe):
    # I = 2048 is beyond the one-kernel batch-1 path: batch 1 runs as three kernels
    log("decode B=1 with I=2048 (three-kernel path)")
    host = synth.random_layer(8, 2, 64, 2048, "q4", "bf16", seed=12, router_sd=0.3)
    x = synth.normal_bf16(synth.key(12, 3, 3, 3, 3), (6, 64), 1.0)
    L = moe.DeviceLayer(host)
    y, idx, g = _decode_calls(moe, L, x, 1)
    _check_all(host, x, y, idx, g, "decode B=1 I=2048")


def test_decode_graph_replay(moe):
    # the one-kernel path resets its counters itself: replays of a captured
    # sequence match the eager results bit for bit, with eager work between
    log("decode B=1 captured in a HIP graph, 3 replays against eager")
    host = synth.random_layer(64, 6, 256, 128, "q4", "bf16", seed=13, router_sd=0.3)
    x = synth.normal_bf16(synth.key(13, 4, 4, 4, 4), (12, 256), 1.0)
    L = moe.DeviceLayer(host)
    y_eager, idx_eager, _ = _decode_calls(moe, L, x, 1)
    xd = to_dev(x)
    yd = torch.zeros((12, 256), dtype=torch.int16, device="cuda")
    ws = moe.make_workspace(L, 1, 0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for t in range(12):
            moe.moe_forward_decode(L, xd[t:t + 1], yd[t:t + 1], ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for t in range(12):
            moe.moe_forward_decode(L, xd[t:t + 1], yd[t:t + 1], ws)
    for rep in range(3):
        yd.zero_()
        _decode_calls(moe, L, x[:2], 1)  # eager work between replays
        gr.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_dev_bits(yd), y_eager), "replay %d differs from eager" % rep
    moe.moe_workspace_check(ws)


def test_single_token_prefill_and_zero_input(moe):
    host = synth.random_layer(16, 4, 64, 32, "q4", "bf16", seed=6)
    L = moe.DeviceLayer(host)
    x = np.zeros((1, 64), np.uint16)
    y, idx, g = _prefill(moe, L, x)
    assert np.all(oracle.bf16_bits_to_f64(y) == 0.0)
    assert idx[0].tolist() == [0, 1, 2, 3] and np.allclose(g, 0.25)
    y, idx, g = _decode_calls(moe, L, x, 1)
    assert np.all(oracle.bf16_bits_to_f64(y) == 0.0) and idx[0].tolist() == [0, 1, 2, 3]


# ----------------------------------------------------------------------------- full-size workloads

@pytest.fixture(scope="module")
def decode_q4(moe):
    host = synth.make_layer("decode_q4", threads=16)
    return host, moe.DeviceLayer(host), synth.make_tokens("decode_q4")


@pytest.fixture(scope="module")
def decode_q4_ref(decode_q4):
    host, _, x = decode_q4
    log("oracle: 256 tokens of the Q4 decode layer")
    return _oracle_ref(host, x)


def test_decode_q4_sequence_all_tokens(moe, decode_q4, decode_q4_ref):
    # the benchmark's launch configuration: 256 consecutive batch-1 calls, every token checked
    host, L, x = decode_q4
    log("decode_q4: 256 sequential B=1 calls, all tokens checked")
    y, idx, g = _decode_calls(moe, L, x, 1)
    _check_all(host, x, y, idx, g, "decode_q4 B=1", ref=decode_q4_ref)


@pytest.mark.parametrize("B", [3, 4, 5])
def test_decode_q4_verify_batches(moe, decode_q4, B):
    # speculative-verify shapes: one call holds the current token and 2-4
    # drafts. 12 consecutive calls, every token checked; then calls whose
    # tokens repeat (drafts that route to the same experts: each expert's
    # weights serve several tokens of the call)
    host, L, x = decode_q4
    log("decode_q4: B=%d, 12 calls + 3 calls with repeated tokens" % B)
    xs = x[: 12 * B]
    y, idx, g = _decode_calls(moe, L, xs, B)
    _check_all(host, xs, y, idx, g, "decode_q4 B=%d" % B)
    rep = np.concatenate([x[[7] * B], x[[9, 9] + [11] * (B - 2)], x[[13, 14] * (B // 2) + [13] * (B % 2)]])
    y, idx, g = _decode_calls(moe, L, rep, B)
    _check_all(host, rep, y, idx, g, "decode_q4 B=%d repeated tokens" % B)
    for c in range(3):
        toks = rep[c * B:(c + 1) * B]
        for i in range(B):
            j = [jj for jj in range(B) if np.array_equal(toks[jj], toks[i])][0]
            assert np.array_equal(y[c * B + i], y[c * B + j]), "identical tokens of one call must give identical outputs"


@pytest.mark.parametrize("B", [4, 5])
def test_batched_decode_replays_bit_identical(moe, decode_q4, B):
    # the batched one-kernel path hands its per-workgroup partials over
    # through done words (the partials themselves carry no tag): the 256
    # tokens as calls of B, captured in a HIP graph and replayed with eager
    # work between the replays, give the eager results bit for bit every time
    _, L, x = decode_q4
    T = (x.shape[0] // B) * B
    x = x[:T]
    log("batched decode B=%d: %d calls captured, 3 replays against eager" % (B, T // B))
    y_eager, idx_eager, _ = _decode_calls(moe, L, x, B)
    xd = to_dev(x)
    yd = torch.zeros((T, L.H), dtype=torch.int16, device="cuda")
    ws = moe.make_workspace(L, B, 0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for t in range(0, T, B):
            moe.moe_forward_decode(L, xd[t:t + B], yd[t:t + B], ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for t in range(0, T, B):
            moe.moe_forward_decode(L, xd[t:t + B], yd[t:t + B], ws)
    for rep in range(3):
        yd.zero_()
        _decode_calls(moe, L, x[:2 * B], B)  # eager work between replays
        gr.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_dev_bits(yd), y_eager), "replay %d differs from eager" % rep
    moe.moe_workspace_check(ws)


@pytest.mark.parametrize("B", [1, 3])
def test_stack_decode_layer_matches_separate_calls(moe, decode_q4, B):
    # moe_stack_decode_layer (one kernel at batch 1: norm, MoE, residual)
    # against moe_rmsnorm -> moe_forward_decode -> moe_residual_add on the
    # same h: z, y, routing and the new h bit for bit (same sum orders); the
    # separate calls are themselves checked against the oracle elsewhere
    host, L, x = decode_q4
    log("stack decode layer, B=%d, 4 calls: fused against separate calls" % B)
    H, k = L.H, L.k
    ws = moe.make_workspace(L, B, 0)
    for c in range(4):
        h = to_dev(x[c * B:(c + 1) * B]) if c % 2 == 0 else to_dev((x[c * B:(c + 1) * B].astype(np.uint32) + 0x0080).astype(np.uint16))
        h1, h2 = h.clone(), h.clone()
        z1, y1, z2, y2 = (torch.empty((B, H), dtype=torch.int16, device="cuda") for _ in range(4))
        i1, i2 = (torch.empty((B, k), dtype=torch.int32, device="cuda") for _ in range(2))
        g1, g2 = (torch.empty((B, k), dtype=torch.float32, device="cuda") for _ in range(2))
        moe.moe_stack_decode_layer(L, h1, ws, 1e-6, z1, y1, i1, g1)
        moe.moe_rmsnorm(h2, z2, 1e-6)
        moe.moe_forward_decode(L, z2, y2, ws, i2, g2)
        moe.moe_residual_add(h2, y2)
        torch.cuda.synchronize()
        for a_, b_, n in ((z1, z2, "z"), (y1, y2, "y"), (h1, h2, "h"), (i1, i2, "idx"), (g1, g2, "gate")):
            assert torch.equal(a_, b_), "call %d: %s differs" % (c, n)
    moe.moe_workspace_check(ws)
    # without the optional outputs (the bench's form)
    h1 = to_dev(x[:B])
    h2 = h1.clone()
    moe.moe_stack_decode_layer(L, h1, ws, 1e-6)
    z2, y2 = (torch.empty((B, H), dtype=torch.int16, device="cuda") for _ in range(2))
    moe.moe_rmsnorm(h2, z2, 1e-6)
    moe.moe_forward_decode(L, z2, y2, ws)
    moe.moe_residual_add(h2, y2)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)


@pytest.fixture(scope="module")
def decode_q3(moe):
    host = synth.make_layer("decode_q3_zipf", threads=16)
    x = synth.make_tokens("decode_q3_zipf")
    log("oracle: 256 tokens of the Q3 Zipf layer")
    return host, moe.DeviceLayer(host), x, _oracle_ref(host, x)


def test_decode_q3_zipf_b1_all_tokens(moe, decode_q3):
    host, L, x, ref = decode_q3
    log("decode_q3_zipf: 256 B=1 calls, all tokens checked")
    y, idx, g = _decode_calls(moe, L, x, 1)
    _check_all(host, x, y, idx, g, "decode_q3 B=1", ref=ref)


def test_decode_q3_zipf_b8_all_tokens(moe, decode_q3):
    host, L, x, ref = decode_q3
    log("decode_q3_zipf: B=8, 32 calls, all tokens checked")
    y, idx, g = _decode_calls(moe, L, x, 8)
    _check_all(host, x, y, idx, g, "decode_q3 B=8", ref=ref)


@pytest.fixture(scope="module")
def prefill_q4(moe):
    host = synth.make_layer("prefill_q4", threads=16)
    return host, moe.DeviceLayer(host), synth.make_tokens("prefill_q4")


@pytest.mark.timeout(600)
def test_prefill_q4_all_tokens(moe, prefill_q4):
    host, L, x = prefill_q4
    log("prefill_q4: T=4096, routing, gates and outputs of every token checked")
    y, idx, g = _prefill(moe, L, x)
    _check_all(host, x, y, idx, g, "prefill_q4")


def test_route_entry_counts(moe, prefill_q4):
    host, L, x = prefill_q4
    T = x.shape[0]
    ws = moe.make_workspace(L, T, 1)
    idx = torch.empty((T, L.k), dtype=torch.int32, device="cuda")
    g = torch.empty((T, L.k), dtype=torch.float32, device="cuda")
    counts = torch.empty((L.E,), dtype=torch.int32, device="cuda")
    moe.moe_route(L, to_dev(x), idx, g, ws, expert_counts=counts)
    torch.cuda.synchronize()
    idx_ref, g_ref, logits = oracle.route(host, x)
    check_routing(idx.cpu().numpy(), idx_ref, logits, "moe_route", scale=routing_scale(host, x))
    assert np.array_equal(counts.cpu().numpy(), np.bincount(idx.cpu().numpy().ravel(), minlength=L.E))


def test_route_exact_and_near_ties(moe):
    """Prefill routing where the approximate logits cannot decide: experts
    1-3 copy expert 0's router row (exact ties, lower index first), expert 5
    is expert 4's row scaled by 1 + 2^-20 (a gap far below the approximation's
    error bound, above the tie tolerance), and some tokens are zero (every
    logit equals its bias). Routing must match the oracle's fp64 order."""
    host = synth.random_layer(64, 8, 256, 32, "q4", "bf16", seed=7, router_sd=0.3)
    w = host.router_w
    w[1:4] = w[0]
    w[5] = (w[4].astype(np.float64) * (1.0 + 2.0 ** -20)).astype(np.float32)
    if host.router_b is not None:
        host.router_b[1:4] = host.router_b[0]
        host.router_b[5] = host.router_b[4]
    L = moe.DeviceLayer(host)
    x = synth.normal_bf16(synth.key(7, 5, 5, 5, 5), (96, 256), 1.0)
    x[5] = 0
    x[40] = 0
    # pull expert 0 and 4 into the top-k for many tokens: tokens aligned with their rows
    x[10:20] = oracle.round_to_bf16_bits(np.tile(w[0].astype(np.float64), (10, 1)) * 0.5)
    x[20:30] = oracle.round_to_bf16_bits(np.tile(w[4].astype(np.float64), (10, 1)) * 0.5)
    T = x.shape[0]
    ws = moe.make_workspace(L, T, 1)
    idx = torch.empty((T, L.k), dtype=torch.int32, device="cuda")
    g = torch.empty((T, L.k), dtype=torch.float32, device="cuda")
    moe.moe_route(L, to_dev(x), idx, g, ws)
    torch.cuda.synchronize()
    idx_ref, g_ref, logits = oracle.route(host, x)
    sc = routing_scale(host, x)
    check_routing(idx.cpu().numpy(), idx_ref, logits, "ties", scale=sc)
    check_gates(g.cpu().numpy(), g_ref, "ties")
    got = idx.cpu().numpy()
    assert all(list(got[t][:4]) == [0, 1, 2, 3] for t in range(10, 20)), got[10:20, :4]
    assert all(list(got[t][:2]) == [5, 4] for t in range(20, 30)), got[20:30, :2]
    # the same tokens through the decode top-k (one-kernel batch 1; batch 4)
    for B in (1, 4):
        yd, idd, gd = _decode_calls(moe, L, x, B)
        check_routing(idd, idx_ref, logits, "ties decode B=%d" % B, scale=sc)
        check_gates(gd, g_ref, "ties decode B=%d" % B)
        assert all(list(idd[t][:4]) == [0, 1, 2, 3] for t in range(10, 20)), idd[10:20, :4]
        assert all(list(idd[t][:2]) == [5, 4] for t in range(20, 30)), idd[20:30, :2]


def test_prefill_matches_decode(moe, decode_q4):
    host, L, x = decode_q4
    xs = x[:32]
    yd, idd, _ = _decode_calls(moe, L, xs, 1)
    yp, idp, _ = _prefill(moe, L, xs)
    assert np.array_equal(idd, idp)
    check_y(yp, oracle.bf16_bits_to_f64(yd), "prefill vs decode")


# ----------------------------------------------------------------------------- between layers

def test_rmsnorm_and_residual(moe):
    T, H = 37, 2048
    h = synth.normal_bf16(synth.key(8, 8, 8, 8, 8), (T, H), 3.0)
    yv = synth.normal_bf16(synth.key(8, 8, 8, 8, 9), (T, H), 0.5)
    hd, yd = to_dev(h), to_dev(yv)
    z = torch.empty_like(hd)
    moe.moe_rmsnorm(hd, z, 1e-6)
    moe.moe_residual_add(hd, yd)
    torch.cuda.synchronize()
    z_ref = oracle.rmsnorm(oracle.bf16_bits_to_f64(h), 1e-6)
    zf = oracle.bf16_bits_to_f64(from_dev_bits(z))
    assert np.abs(zf - z_ref).max() <= 2 ** -8 * np.abs(z_ref).max()
    r_ref = oracle.bf16_bits_to_f64(h) + oracle.bf16_bits_to_f64(yv)
    rf = oracle.bf16_bits_to_f64(from_dev_bits(hd))
    assert np.all(np.abs(rf - r_ref) <= 2 ** -8 * np.abs(r_ref) + 1e-30)
