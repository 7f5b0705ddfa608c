#!/usr/bin/env python3
"""Benchmark of the MoE layer hot path on one MI355X.

Workload (the headline one): one 512-expert MoE layer, top-10 routed + 1
shared expert, hidden 2048, expert intermediate 512, 4-bit block-quantised
experts (32-element blocks, fp16 scales), bf16 shared expert, fp32 router;
256 sequential batch-1 decode calls on one stream. One "step" is that whole
256-token sequence; the 256 calls are captured once into a HIP graph and the
graph is replayed per step. value = decode tokens/s.

Also reported (not the headline value): the same sequence launched eagerly,
the 4096-token prefill of a layer of the same shape, the per-kernel roofline
of the dominant decode kernel (HIP events on the launch stream), and the CPU
oracle timed on a bounded sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-prefill] [--no-cpu] [--no-stack]
       (the run includes the 48-layer stack: 512 batch-1 decode tokens and a
        32768-token prefill through 48 resident layers, about 20 s more;
        --no-stack skips it)
       python bench.py --profile-sample   (short eager run for hardware-counter passes:
                                           a 2 GiB elementwise copy, then 32 decode
                                           tokens and one 4096-token prefill)
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_expert_bytes(L):
    """Algorithmic bytes of one expert's fused gate/up and down (values + scales)."""
    from quantized_expert_ffn_gemv_amd import moe
    gu = moe.moe_matrix_bytes(L.wt, 2 * L.I, L.H) + 2 * moe.moe_matrix_scales(L.wt, 2 * L.I, L.H)
    dn = moe.moe_matrix_bytes(L.wt, L.H, L.I) + 2 * moe.moe_matrix_scales(L.wt, L.H, L.I)
    sgu = moe.moe_matrix_bytes(L.swt, 2 * L.I, L.H) if L.swt != moe.W_NONE else 0
    sdn = moe.moe_matrix_bytes(L.swt, L.H, L.I) if L.swt != moe.W_NONE else 0
    return gu, dn, sgu, sdn


def run_decode(moe, torch, L, x_bits, steps, warmup, B=1):
    """Consecutive decode calls of B tokens over x; (eager s, graph s) per pass."""
    T, H = x_bits.shape
    dev = torch.device("cuda")
    xd = torch.from_numpy(x_bits.view(np.int16)).to(dev)
    y = torch.empty((T, H), dtype=torch.int16, device=dev)
    ws = moe.make_workspace(L, B, 0)

    def seq():
        for t in range(0, T, B):
            moe.moe_forward_decode(L, xd[t:t + B], y[t:t + B], ws)

    # eager
    seq()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(max(1, steps // 2)):
        seq()
    torch.cuda.synchronize()
    eager_s = (time.perf_counter() - t0) / max(1, steps // 2)
    # graph
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        seq()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    # HIP events on the stream the graph is replayed on (torch's current
    # stream) bracket the timed replays: their interval / the launches in it
    # is the kernels' average launch duration over the timed region
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    graph_s = (time.perf_counter() - t0) / steps
    run_decode.event_ms_per_replay = ev0.elapsed_time(ev1) / steps
    run_decode.launches_per_replay = (T + B - 1) // B
    # every call of the timed replays must have completed its device-side
    # waits: a wait that ran out means invalid results, and the run fails
    moe.moe_workspace_check(ws)
    return eager_s, graph_s, g


def expert_usage(idx, E):
    """Expert-usage telemetry of one layer's routing (idx [T, k]): experts
    used, and the share of all selections taken by the hottest 20% of the
    experts."""
    counts = np.bincount(np.asarray(idx).ravel(), minlength=E)
    hot = np.sort(counts)[::-1][: max(1, int(round(0.2 * E)))]
    return {"experts_used": int(np.count_nonzero(counts)),
            "hottest20_share": round(float(hot.sum()) / float(counts.sum()), 4)}


def decode_batches(moe, torch, L, x, steps, warmup, batches):
    """Decode of the tokens x as graph-replayed calls of B tokens, for each B in
    batches (x cut to a multiple of B). Bytes per call count each unique
    routed expert once (the weights of an expert chosen by several tokens of a
    call are read once), plus the shared expert and the router."""
    gu, dn, sgu, sdn = decode_expert_bytes(L)
    router_bytes = L.E * L.H * 4
    dev = torch.device("cuda")
    out = {}
    for B in batches:
        xb = x[: (x.shape[0] // B) * B]
        T = xb.shape[0]
        _, graph_s, g = run_decode(moe, torch, L, xb, steps, warmup, B=B)
        del g
        # unique routed experts per call, from the routing of the same calls
        xd = torch.from_numpy(xb.view(np.int16)).to(dev)
        idx = torch.empty((T, L.k), dtype=torch.int32, device=dev)
        yy = torch.empty_like(xd)
        ws = moe.make_workspace(L, B, 0)
        for t in range(0, T, B):
            moe.moe_forward_decode(L, xd[t:t + B], yy[t:t + B], ws, topk_idx=idx[t:t + B])
        torch.cuda.synchronize()
        moe.moe_workspace_check(ws)
        ih = idx.cpu().numpy()
        uniq = [len(np.unique(ih[t:t + B])) for t in range(0, T, B)]
        calls = len(uniq)
        bytes_total = sum(u * (gu + dn) for u in uniq) + calls * (sgu + sdn + router_bytes)
        out["b%d" % B] = {
            "tokens_per_s": round(T / graph_s, 1),
            "us_per_call": round(graph_s / calls * 1e6, 3),
            "unique_experts_per_call": round(float(np.mean(uniq)), 2),
            "weight_bytes_per_call": round(bytes_total / calls),
            "effective_GBps": round(bytes_total / graph_s / 1e9, 1),
            "frac_of_hbm": round(bytes_total / graph_s / 1e9 / HBM_PEAK_GBS, 4),
            "expert_usage": expert_usage(ih, L.E),
        }
    return out


def run_c2(moe, torch, synth, steps, warmup):
    """The Q3 / Zipf-routed layer: 256 tokens as batch-1 calls and as 32
    batch-8 calls (graph replays)."""
    name = "decode_q3_zipf"
    host = synth.make_layer(name, threads=16)
    x = synth.make_tokens(name)
    L = moe.DeviceLayer(host)
    out = {"workload": "one MoE layer, Q3 experts (32-elem blocks, fp16 scales), Zipf-skewed router bias "
                       "(hottest 20% of experts take 80% of selections), bf16 shared, fp32 router; 256 tokens"}
    out.update(decode_batches(moe, torch, L, x, steps, warmup, (1, 8)))
    return out


def run_spec_verify(moe, torch, L, x, steps, warmup):
    """Speculative-verify shapes on the batch-1 layer: one call checks the
    current token and d = 2..4 drafts (B = 1 + d). Independent tokens stand in
    for the drafts, the worst case for sharing experts within a call (drafts
    of one sequence route alike more often)."""
    out = {"workload": "the batch-1 Q4 layer at B = 3, 4, 5 tokens per call (verify of 2-4 drafts); "
                       "independent synthetic tokens as drafts"}
    out.update(decode_batches(moe, torch, L, x, steps, warmup, (3, 4, 5)))
    return out


def kernel_times(moe, torch, fn, reps=1):
    """Per-kernel-class (launches, avg ms) of fn() measured with the library timer."""
    torch.cuda.synchronize()
    moe.timer_reset()
    moe.timer_enable(True)
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    moe.timer_enable(False)
    out = {k: (n, ms / n) for k, (n, ms) in moe.timer_read().items()}
    moe.timer_reset()
    return out


# Kernel sources whose hash the committed counter summary records: the
# traffic figure is reported only while the kernel is unchanged.
TRAFFIC_SOURCES = ["quantized_expert_ffn_gemv_amd/csrc/decode1.hip", "quantized_expert_ffn_gemv_amd/csrc/dec_common.h",
                   "quantized_expert_ffn_gemv_amd/csrc/moe_device.h"]
TRAFFIC_SUMMARY = "profiles/dec_fused_decode_q4_traffic.md"


def sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def committed_traffic():
    """HBM bytes per launch of the batch-1 decode kernel from the committed
    rocprofv3 counter summary, or None if absent or taken on other sources."""
    path = os.path.join(ROOT, TRAFFIC_SUMMARY)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.strip().startswith("- "):
                k, v = line.strip()[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256") != sources_sha256():
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(host, x_bits, per_token_bytes, budget_s=24.0, max_tokens=256):
    """The fp64 oracle on the host cores, on the first tokens of the headline
    workload (one oracle call per batch-1 token): about half the budget with
    numpy's BLAS threads as configured, half with one thread."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    def timed(limit_s):
        n = 0
        t0 = time.perf_counter()
        while n < max_tokens and time.perf_counter() - t0 < limit_s:
            oracle.moe_forward(host, x_bits[n:n + 1])
            n += 1
        return n, time.perf_counter() - t0

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    n, el = timed(budget_s / 2)
    with threadpool_limits(limits=1):
        n1, el1 = timed(budget_s / 2)
    tps, tps1 = n / el, n1 / el1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    return dict(value=round(tps, 3), unit="tokens/s", cores=int(threads), kind="oracle",
                value_1thread=round(tps1, 3),
                effective_GBps=round(per_token_bytes * tps / 1e9, 4),
                effective_GBps_1thread=round(per_token_bytes * tps1 / 1e9, 4),
                cpu_model=cpu_model(), host_cpus=os.cpu_count(), cpus_in_affinity=affinity,
                sample="first %d (then %d single-thread) of the 256 batch-1 decode tokens, one call of the "
                       "fp64 numpy oracle per token; %.1f s + %.1f s; BLAS threads %d; GB/s on the same "
                       "%d expert-weight bytes per token as the GPU figure"
                       % (n, n1, el, el1, threads, per_token_bytes))


def run_tiny(moe, torch, synth, steps, warmup):
    """The tiny layer (8 experts, top-2 + shared, hidden 64, fp32 weights; 16
    tokens): batch-1 decode calls replayed as one graph, and one prefill of
    the 16 tokens. Throughput only: at this size the launch sets the time."""
    host = synth.make_layer("tiny")
    x = synth.make_tokens("tiny")
    L = moe.DeviceLayer(host)
    _, graph_s, g = run_decode(moe, torch, L, x, steps, warmup)
    del g
    dev = torch.device("cuda")
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    yd = torch.empty_like(xd)
    wsp = moe.make_workspace(L, x.shape[0], 1)
    moe.moe_forward_prefill(L, xd, yd, wsp)
    torch.cuda.synchronize()
    reps = 50
    t0 = time.perf_counter()
    for _ in range(reps):
        moe.moe_forward_prefill(L, xd, yd, wsp)
    torch.cuda.synchronize()
    pf_s = (time.perf_counter() - t0) / reps
    T = x.shape[0]
    return {"workload": "tiny MoE layer: 8 experts, top-2 + 1 shared, hidden 64, intermediate 32, fp32 weights; "
                        "16 tokens", "decode_tokens_per_s": round(T / graph_s, 1),
            "decode_us_per_token": round(graph_s / T * 1e6, 3), "prefill_tokens_per_s": round(T / pf_s, 1),
            "prefill_us": round(pf_s * 1e6, 2)}


COPY_BYTES = 2 << 30   # 8x the 256 MB last-level cache: the copy's reads come from HBM


def profile_sample(moe, torch, synth):
    """Eager launches for counter collection: a plain elementwise copy of
    known size calibrates FETCH_SIZE / WRITE_SIZE (its 2nd and 3rd dispatch
    read a source that the previous dispatch's writes pushed out of the
    last-level cache), then the decode and prefill kernels."""
    dev = torch.device("cuda")
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)          # reads COPY_BYTES, writes COPY_BYTES
    torch.cuda.synchronize()
    del a, b
    host = synth.make_layer("decode_q4")
    x = synth.make_tokens("decode_q4")
    L = moe.DeviceLayer(host)
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    yd = torch.empty_like(xd)
    ws = moe.make_workspace(L, 1, 0)
    for t in range(32):
        moe.moe_forward_decode(L, xd[t:t + 1], yd[t:t + 1], ws)
    torch.cuda.synchronize()
    log("profile sample: copy %d B x3, 32 decode tokens done" % COPY_BYTES)
    del L
    hp = synth.make_layer("prefill_q4")
    xp = synth.make_tokens("prefill_q4")
    Lp = moe.DeviceLayer(hp)
    xpd = torch.from_numpy(xp.view(np.int16)).to(dev)
    ypd = torch.empty_like(xpd)
    wsp = moe.make_workspace(Lp, xp.shape[0], 1)
    moe.moe_forward_prefill(Lp, xpd, ypd, wsp)
    torch.cuda.synchronize()
    log("profile sample: prefill %d tokens done" % xp.shape[0])


def run_stack(moe, torch, synth, steps):
    """The 48-layer stack (pre-norm RMSNorm, MoE layer, bf16 residual; 44 GB of
    weights resident): 512 batch-1 decode tokens, each one HIP-graph replay of
    the 48 layers, and the 32768-token prefill in one pass."""
    name = "stack48_q4"
    c = synth.WORKLOADS[name]
    layers = []
    t0 = time.perf_counter()
    for l in range(c["layers"]):
        layers.append(moe.DeviceLayer(synth.make_layer(name, layer=l, threads=16)))
    log("stack: %d layers resident (%.1f GB) in %.0f s" % (len(layers), sum(L.weight_bytes() for L in layers) / 1e9,
                                                          time.perf_counter() - t0))
    dev = torch.device("cuda")
    L0 = layers[0]
    H, k = L0.H, L0.k
    # decode: one graph = copy the token in, 48 layers, on a fixed buffer
    x = synth.make_tokens(name)
    T = x.shape[0]
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    out = torch.empty_like(xd)
    stage = torch.empty((1, H), dtype=torch.int16, device=dev)
    h = torch.empty((1, H), dtype=torch.int16, device=dev)
    ws = moe.make_workspace(L0, 1, 0)
    buf = moe.StackBuffers(1, H, k)

    def one():
        h.copy_(stage)
        moe.stack_forward(layers, h, ws, True, buf)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        one()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one()

    def tokens():
        for t in range(T):
            stage.copy_(xd[t:t + 1])
            g.replay()
            out[t:t + 1].copy_(h)

    tokens()
    torch.cuda.synchronize()
    reps = max(1, steps // 10)
    t0 = time.perf_counter()
    for _ in range(reps):
        tokens()
    torch.cuda.synchronize()
    dec_s = (time.perf_counter() - t0) / (reps * T)
    moe.moe_workspace_check(ws)
    gu, dn, sgu, sdn = decode_expert_bytes(L0)
    per_tok = len(layers) * (L0.k * (gu + dn) + sgu + sdn)
    del g
    # expert-usage telemetry (untimed): every token's routing at every layer
    nl, E = len(layers), L0.E
    IDX = torch.empty((nl, T, k), dtype=torch.int32, device=dev)
    for t in range(T):
        hh = xd[t:t + 1].clone()
        for l, L in enumerate(layers):
            moe.moe_stack_decode_layer(L, hh, ws, 1e-6, None, None, IDX[l, t:t + 1], None)
    torch.cuda.synchronize()
    moe.moe_workspace_check(ws)
    dec_usage = [expert_usage(a, E) for a in IDX.cpu().numpy()]
    del IDX
    # prefill: all tokens, one pass through the 48 layers
    xp = synth.make_prefill_tokens(name)
    Tp = xp.shape[0]
    xpd = torch.from_numpy(xp.view(np.int16)).to(dev)
    hp = torch.empty_like(xpd)
    wsp = moe.make_workspace(L0, Tp, 1)
    bufp = moe.StackBuffers(Tp, H, k)

    def prefill(each_layer=None):
        hp.copy_(xpd)
        moe.stack_forward(layers, hp, wsp, False, bufp, each_layer=each_layer)

    pf_counts = []
    prefill(lambda l, b: pf_counts.append(torch.bincount(b.idx.view(-1).long(), minlength=E)))
    torch.cuda.synchronize()
    pf_usage = []
    for c in pf_counts:
        c = c.cpu().numpy()
        hot = np.sort(c)[::-1][: max(1, int(round(0.2 * E)))]
        pf_usage.append({"experts_used": int(np.count_nonzero(c)),
                         "hottest20_share": round(float(hot.sum()) / float(c.sum()), 4)})
    t0 = time.perf_counter()
    prefill()
    torch.cuda.synchronize()
    pf_s = time.perf_counter() - t0
    flops = len(layers) * Tp * 2.0 * (L0.k + 1) * 3 * H * L0.I
    return {
        "workload": "48-layer stack: each layer 512 experts top-10 + shared, hidden 2048, intermediate 512, Q4 "
                    "experts, bf16 shared, fp32 router with its own Zipf bias; pre-norm RMSNorm, bf16 residual",
        "decode_tokens": T,
        "decode_us_per_token": round(dec_s * 1e6, 2),
        "decode_tokens_per_s": round(1.0 / dec_s, 1),
        "decode_expert_bytes_per_token": per_tok,
        "decode_effective_expert_GBps": round(per_tok / dec_s / 1e9, 1),
        "prefill_tokens": Tp,
        "prefill_ms": round(pf_s * 1e3, 2),
        "prefill_tokens_per_s": round(Tp / pf_s, 1),
        "prefill_expert_TFLOPs": round(flops / pf_s / 1e12, 1),
        "expert_usage_per_layer": {
            "decode": {"experts_used": [u["experts_used"] for u in dec_usage],
                       "hottest20_share": [u["hottest20_share"] for u in dec_usage]},
            "prefill": {"experts_used": [u["experts_used"] for u in pf_usage],
                        "hottest20_share": [u["hottest20_share"] for u in pf_usage]},
        },
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--profile-sample", action="store_true")
    ap.add_argument("--no-stack", action="store_true", help="skip the 48-layer stack (about 20 s with its set-up)")
    ap.add_argument("--stack", action="store_true", help=argparse.SUPPRESS)  # the stack runs by default
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from quantized_expert_ffn_gemv_amd import moe
    moe.lib()
    if args.profile_sample:
        profile_sample(moe, torch, synth)
        return

    # ---------------------------------------------------------------- headline: decode Q4 batch 1
    log("generating the 512-expert Q4 layer ...")
    host = synth.make_layer("decode_q4")
    x = synth.make_tokens("decode_q4")
    L = moe.DeviceLayer(host)
    T = x.shape[0]
    eager_s, graph_s, g = run_decode(moe, torch, L, x, args.steps, args.warmup)
    replay_launch_ms = run_decode.event_ms_per_replay / run_decode.launches_per_replay
    value = T / graph_s
    log("decode: graph %.1f us/token, eager %.1f us/token" % (graph_s / T * 1e6, eager_s / T * 1e6))

    # per-kernel times (eager pass with timer events on the launch stream)
    dev = torch.device("cuda")
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    yd = torch.empty_like(xd)
    ws = moe.make_workspace(L, 1, 0)

    def one_seq():
        for t in range(T):
            moe.moe_forward_decode(L, xd[t:t + 1], yd[t:t + 1], ws)

    kt = kernel_times(moe, torch, one_seq, reps=2)
    moe.moe_workspace_check(ws)
    gu, dn, sgu, sdn = decode_expert_bytes(L)
    router_bytes = L.E * L.H * 4
    # algorithmic bytes per launch: the expert weights the token needs (its k
    # routed experts and the shared expert); the router's 4 MiB are read in
    # the same launch and are counted in its time, not in its bytes
    kbytes = {
        "dec_fused": sgu + sdn + L.k * (gu + dn),
        "dec_router_shared": sgu + sdn,
        "dec_routed": L.k * (gu + dn),
    }
    dom = max(kbytes, key=lambda k: kt.get(k, (0, 0))[1])
    n_l, avg_ms = kt[dom]
    if dom == "dec_fused":
        # the one kernel per token: its average launch duration over the
        # timed graph replays (the replays hold nothing else)
        avg_ms = replay_launch_ms
    achieved = kbytes[dom] / (avg_ms * 1e-3) / 1e9
    per_token_bytes = L.k * (gu + dn) + sgu + sdn
    kernels = {k: dict(launches=v[0], avg_us=round(v[1] * 1e3, 3), algo_bytes=kbytes.get(k),
                       gbs=round(kbytes[k] / (v[1] * 1e-3) / 1e9, 1) if k in kbytes else None)
               for k, v in kt.items()}
    log("kernels:", json.dumps(kernels))

    result = {
        "metric": "MoE-layer tokens/s at decode bs=1 & prefill; achieved HBM GB/s / MFMA util",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(graph_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4-weights/bf16-act/fp32-acc",
        "data": "synthetic (seeded; weights and activations drawn to the workload's distributions)",
        "config": {
            "workload": "one MoE layer, decode batch 1: 512 experts, top-10 + 1 shared, hidden 2048, "
                        "intermediate 512, Q4 experts (32-elem blocks, fp16 scales), bf16 shared, fp32 router; "
                        "256 sequential tokens per step, replayed as one HIP graph",
            "tokens_per_step": T,
            "launch": "hipgraph",
            "parallelism": "single GPU",
        },
        "decode": {
            "graph_us_per_token": round(graph_s / T * 1e6, 3),
            "eager_us_per_token": round(eager_s / T * 1e6, 3),
            "eager_tokens_per_s": round(T / eager_s, 1),
            "expert_weight_bytes_per_token": per_token_bytes,
            "effective_expert_GBps": round(per_token_bytes * value / 1e9, 1),
            "effective_frac_of_hbm": round(per_token_bytes * value / 1e9 / HBM_PEAK_GBS, 4),
            "kernels": kernels,
        },
        "roofline": {
            "kernel": dom,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": committed_traffic() if dom == "dec_fused" else None,
            "algo_bytes_per_launch": kbytes[dom],
            "router_bytes_per_launch": router_bytes if dom == "dec_fused" else 0,
            "achieved_incl_router": round((kbytes[dom] + (router_bytes if dom == "dec_fused" else 0))
                                          / (avg_ms * 1e-3) / 1e9, 1),
            "avg_launch_us": round(avg_ms * 1e3, 3),
            "timing": "HIP events on the replay stream around the timed graph replays, / 256 launches"
            if dom == "dec_fused" else "library timer: HIP events in each launch's dispatch, eager pass",
        },
    }
    del g

    # ---------------------------------------------------------------- tiny layer (secondary, no roofline claim)
    log("tiny layer ...")
    result["tiny"] = run_tiny(moe, torch, synth, args.steps, args.warmup)
    log("tiny:", json.dumps(result["tiny"]))

    # ---------------------------------------------------------------- speculative-verify batches (secondary)
    if not args.no_prefill:
        log("decode Q4, B = 3..5 (verify of 2-4 drafts) ...")
        result["decode_spec_verify"] = run_spec_verify(moe, torch, L, x, args.steps, args.warmup)
        log("decode_spec_verify:", json.dumps(result["decode_spec_verify"]))

    # ---------------------------------------------------------------- Q3 / Zipf decode, batch 1 and 8 (secondary)
    if not args.no_prefill:
        log("decode Q3 Zipf, batch 1 and 8 ...")
        result["decode_q3_zipf"] = run_c2(moe, torch, synth, args.steps, args.warmup)
        log("decode_q3_zipf:", json.dumps(result["decode_q3_zipf"]))

    # ---------------------------------------------------------------- prefill (secondary)
    if not args.no_prefill:
        log("prefill 4096 tokens ...")
        hp = synth.make_layer("prefill_q4")
        xp = synth.make_tokens("prefill_q4")
        del L
        Lp = moe.DeviceLayer(hp)
        Tp = xp.shape[0]
        xpd = torch.from_numpy(xp.view(np.int16)).to(dev)
        ypd = torch.empty_like(xpd)
        wsp = moe.make_workspace(Lp, Tp, 1)
        fn = lambda: moe.moe_forward_prefill(Lp, xpd, ypd, wsp)
        fn()
        torch.cuda.synchronize()
        reps = 5
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        pf_s = (time.perf_counter() - t0) / reps
        kp = kernel_times(moe, torch, fn, reps=2)
        routed_flops = 2.0 * Tp * Lp.k * 3 * Lp.H * Lp.I
        shared_flops = 2.0 * Tp * 3 * Lp.H * Lp.I
        gemm_ms = kp.get("pf_gate_up", (0, 0))[1] + kp.get("pf_down", (0, 0))[1]
        result["prefill"] = {
            "workload": "one MoE layer prefill: 4096 tokens, same layer shape, router logits ~N(0,1)",
            "tokens_per_s": round(Tp / pf_s, 1),
            "ms_per_layer": round(pf_s * 1e3, 4),
            "routed_grouped_gemm_ms": round(gemm_ms, 4),
            "routed_grouped_gemm_TFLOPs": round(routed_flops / (gemm_ms * 1e-3) / 1e12, 1) if gemm_ms else None,
            "mfma_util_vs_bf16_peak": round(routed_flops / (gemm_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
            if gemm_ms else None,
            "layer_TFLOPs": round((routed_flops + shared_flops) / pf_s / 1e12, 1),
            "kernels_avg_us": {k: round(v[1] * 1e3, 2) for k, v in kp.items()},
        }
        log("prefill:", json.dumps(result["prefill"]))

    # ---------------------------------------------------------------- 48-layer stack
    if not args.no_stack:
        log("48-layer stack ...")
        Lp = L = None  # release the single layers first
        result["stack48"] = run_stack(moe, torch, synth, args.steps)
        log("stack48:", json.dumps(result["stack48"]))

    # ---------------------------------------------------------------- CPU oracle
    if not args.no_cpu:
        log("cpu oracle baseline ...")
        result["cpu_baseline"] = cpu_baseline(host, x, per_token_bytes)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
