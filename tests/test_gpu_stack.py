"""GPU parity of the 48-layer stack: pre-norm RMSNorm, MoE layer, bf16
residual, 48 independent layers of the 512-expert Q4 model (own router,
Zipf bias and shared expert per layer), all resident on the GPU (44 GB).

Decode runs each layer as one moe_stack_decode_layer call (at batch 1 one
kernel: norm, MoE and residual); prefill as the three separate calls.

The check is teacher-forced, layer by layer: the oracle's MoE layer l
consumes the GPU's own bf16 z_l, so a routing decision at one layer cannot
make every later layer disagree. Routing and gates are checked for every
token at every layer (512 decode tokens, 32768 prefill tokens). On sampled
tokens, per layer, also: y_l within the usual tolerances, z_l against the
oracle's RMSNorm of the GPU's h_l within bf16 rounding, and h_{l+1} against
h_l + y_l within bf16 rounding. A free-running oracle pass
(its own z, y, h rounded to bf16 like the stack) is reported for
information only: a near-tie in routing anywhere flips it legitimately.
"""
import numpy as np
import pytest

import oracle
import synth
from moe_testlib import Y_MAX_REL, Y_MIN_COS, check_gates, check_routing, log, routing_scale, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NAME = "stack48_q4"
EPS = 1e-6


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_expert_ffn_gemv_amd import moe as m
    m.lib()
    return m


class CodesExperts:
    """Routed experts of one stack layer, regenerated from the seeded
    generator on demand and dequantised by the oracle."""

    def __init__(self, layer: int):
        c = synth.WORKLOADS[NAME]
        self.wid, self.layer, self.H, self.I = c["id"], layer, c["H"], c["I"]

    def __call__(self, e: int):
        g, gs, u, us, d, ds = synth.expert_codes(0, self.wid, self.layer, e, self.H, self.I, 4)
        return oracle.dequant_blocks(g, gs), oracle.dequant_blocks(u, us), oracle.dequant_blocks(d, ds)


@pytest.fixture(scope="module")
def stack(moe):
    nl = synth.WORKLOADS[NAME]["layers"]
    dev_layers, host_layers = [], []
    for l in range(nl):
        host = synth.make_layer(NAME, layer=l, threads=16)
        dev_layers.append(moe.DeviceLayer(host))
        del host
        host_layers.append(synth.make_layer(NAME, layer=l, experts=False))
        if l % 8 == 7:
            log("  stack: %d layers resident" % (l + 1))
    torch.cuda.synchronize()
    return dev_layers, host_layers


def _check_layers(host_layers, h_in, z, y, idx, g, h_out, what):
    """Teacher-forced checks of every layer for the tokens in the arrays
    (h_in, z, y, h_out: bf16 bits [L, n, H]; idx, g: [L, n, k])."""
    nl = len(host_layers)
    worst_err, worst_cos = 0.0, 1.0
    for l in range(nl):
        host = host_layers[l]
        hf = oracle.bf16_bits_to_f64(h_in[l])
        z_ref = oracle.rmsnorm(hf, EPS)
        zf = oracle.bf16_bits_to_f64(z[l])
        assert np.abs(zf - z_ref).max() <= 2 ** -8 * np.abs(z_ref).max(), "%s layer %d rmsnorm" % (what, l)
        y_ref, idx_ref, g_ref = oracle.moe_forward(host, z[l], experts=CodesExperts(l))
        _, _, logits = oracle.route(host, z[l])
        check_routing(idx[l], idx_ref, logits, "%s layer %d" % (what, l), scale=routing_scale(host, z[l]))
        check_gates(g[l], g_ref, "%s layer %d" % (what, l))
        yf = oracle.bf16_bits_to_f64(y[l])
        err = np.abs(yf - y_ref).max(axis=1) / np.abs(y_ref).max(axis=1)
        cos = (yf * y_ref).sum(1) / (np.linalg.norm(yf, axis=1) * np.linalg.norm(y_ref, axis=1))
        worst_err, worst_cos = max(worst_err, float(err.max())), min(worst_cos, float(cos.min()))
        assert err.max() <= Y_MAX_REL and cos.min() >= Y_MIN_COS, "%s layer %d: err %.3g cos %.7f" % (
            what, l, err.max(), cos.min())
        if l % 12 == 0:
            log("  %s layer %d: max_rel %.3e min_cos %.7f" % (what, l, err.max(), cos.min()))
        r_ref = hf + yf
        rf = oracle.bf16_bits_to_f64(h_out[l])
        assert np.all(np.abs(rf - r_ref) <= 2 ** -8 * np.abs(r_ref) + 1e-30), "%s layer %d residual" % (what, l)
    log("  %s: %d layers, worst y max_rel %.3e, min cos %.7f" % (what, nl, worst_err, worst_cos))


def _free_running(host_layers, x_bits):
    """The stack computed by the oracle alone (information only)."""
    h = x_bits.copy()
    for l, host in enumerate(host_layers):
        z = oracle.round_to_bf16_bits(oracle.rmsnorm(oracle.bf16_bits_to_f64(h), EPS))
        y, _, _ = oracle.moe_forward(host, z, experts=CodesExperts(l))
        yb = oracle.round_to_bf16_bits(y)
        h = oracle.round_to_bf16_bits(oracle.bf16_bits_to_f64(h) + oracle.bf16_bits_to_f64(yb))
    return h


def test_stack48_decode_teacher_forced(moe, stack):
    layers, hosts = stack
    x = synth.make_tokens(NAME, T=3)
    H, k = layers[0].H, layers[0].k
    log("stack48 decode: 3 tokens, batch 1, 48 layers, every layer checked")
    ws = moe.make_workspace(layers[0], 1, 0)
    buf = moe.StackBuffers(1, H, k)
    rec = {n: [] for n in ("h_in", "z", "y", "idx", "g", "h_out")}
    for t in range(x.shape[0]):
        h = to_dev(x[t:t + 1])
        h0 = h.clone()
        per = {n: [] for n in rec}

        def grab(l, b):  # after layer l (one fused kernel: norm, MoE, residual)
            per["h_out"].append(h.clone()); per["z"].append(b.z.clone()); per["y"].append(b.y.clone())
            per["idx"].append(b.idx.clone()); per["g"].append(b.gate.clone())

        moe.stack_forward(layers, h, ws, True, buf, EPS, each_layer=grab)
        torch.cuda.synchronize()
        per["h_in"] = [h0] + per["h_out"][:-1]
        for n in rec:
            rec[n].append(torch.stack(per[n]).cpu().numpy())
    moe.moe_workspace_check(ws)
    # [L, tokens, ...]
    arr = {n: np.concatenate(rec[n], axis=1) for n in rec}
    u16 = lambda a: a.view(np.uint16)
    _check_layers(hosts, u16(arr["h_in"]), u16(arr["z"]), u16(arr["y"]), arr["idx"], arr["g"],
                  u16(arr["h_out"]), "stack48 decode")
    # information only: the oracle's own stack on the first token
    h_ref = oracle.bf16_bits_to_f64(_free_running(hosts, x[:1]))
    h_gpu = oracle.bf16_bits_to_f64(u16(arr["h_out"][-1][:1]))
    cos = float((h_ref * h_gpu).sum() / (np.linalg.norm(h_ref) * np.linalg.norm(h_gpu)))
    log("  free-running 48-layer stack, token 0: cosine(GPU, oracle) = %.6f (information)" % cos)


def _check_layer_routing(host, z_bits, idx, g, what):
    """Routing and gates of every token of one layer (teacher-forced on the GPU's z)."""
    idx_ref, g_ref, logits = oracle.route(host, z_bits)
    n = check_routing(idx, idx_ref, logits, what, scale=routing_scale(host, z_bits))
    check_gates(g, g_ref, what)
    return n


@pytest.mark.timeout(900)
def test_stack48_decode_routing_all_tokens(moe, stack):
    """All 512 decode tokens, batch 1, through the 48 layers (one
    moe_stack_decode_layer call per layer and token, as the benchmark runs
    them); the routing and gates of every token at every layer against the
    oracle's routing of the GPU's own z_l."""
    layers, hosts = stack
    x = synth.make_tokens(NAME)
    T = x.shape[0]
    nl, H, k = len(layers), layers[0].H, layers[0].k
    log("stack48 decode: %d tokens x %d layers, routing of every token checked" % (T, nl))
    ws = moe.make_workspace(layers[0], 1, 0)
    Z = torch.empty((nl, T, H), dtype=torch.int16, device="cuda")
    IDX = torch.empty((nl, T, k), dtype=torch.int32, device="cuda")
    G = torch.empty((nl, T, k), dtype=torch.float32, device="cuda")
    xd = to_dev(x)
    for t in range(T):
        h = xd[t:t + 1].clone()
        for l, L in enumerate(layers):
            moe.moe_stack_decode_layer(L, h, ws, EPS, Z[l, t:t + 1], None, IDX[l, t:t + 1], G[l, t:t + 1])
    torch.cuda.synchronize()
    moe.moe_workspace_check(ws)
    Zh, Ih, Gh = Z.cpu().numpy().view(np.uint16), IDX.cpu().numpy(), G.cpu().numpy()
    near = 0
    for l in range(nl):
        near += _check_layer_routing(hosts[l], Zh[l], Ih[l], Gh[l], "stack48 decode layer %d" % l)
    log("  %d token-layers checked, %d ordered differently within a near-tie" % (T * nl, near))


@pytest.mark.timeout(900)
def test_stack48_prefill_teacher_forced(moe, stack):
    layers, hosts = stack
    T = synth.WORKLOADS[NAME]["prefill_tokens"]
    x = synth.make_prefill_tokens(NAME)
    H, k = layers[0].H, layers[0].k
    sample = torch.tensor([17, 20000, T - 1], dtype=torch.long, device="cuda")
    log("stack48 prefill: T=%d in one pass, 48 layers: routing of every token, outputs of tokens %s, at every layer"
        % (T, sample.tolist()))
    ws = moe.make_workspace(layers[0], T, 1)
    buf = moe.StackBuffers(T, H, k)
    h = to_dev(x)
    h0 = h.index_select(0, sample)
    per = {n: [] for n in ("h_out", "z", "y", "idx", "g")}

    near = [0]

    def grab(l, b):  # after layer l's residual add
        per["h_out"].append(h.index_select(0, sample)); per["z"].append(b.z.index_select(0, sample))
        per["y"].append(b.y.index_select(0, sample)); per["idx"].append(b.idx.index_select(0, sample))
        per["g"].append(b.gate.index_select(0, sample))
        # every token's routing at this layer, on the GPU's own z
        zl = b.z.cpu().numpy().view(np.uint16)
        near[0] += _check_layer_routing(hosts[l], zl, b.idx.cpu().numpy(), b.gate.cpu().numpy(),
                                        "stack48 prefill layer %d" % l)
        if l % 12 == 0:
            log("  stack48 prefill layer %d: routing of %d tokens checked" % (l, zl.shape[0]))

    moe.stack_forward(layers, h, ws, False, buf, EPS, each_layer=grab)
    torch.cuda.synchronize()
    log("  %d token-layers routed as the oracle, %d ordered differently within a near-tie" % (T * len(layers), near[0]))
    per["h_in"] = [h0] + per["h_out"][:-1]
    arr = {n: torch.stack(v).cpu().numpy() for n, v in per.items()}
    u16 = lambda a: a.view(np.uint16)
    _check_layers(hosts, u16(arr["h_in"]), u16(arr["z"]), u16(arr["y"]), arr["idx"], arr["g"],
                  u16(arr["h_out"]), "stack48 prefill")
