"""Find the Zipf bias strength tau for the skewed-routing workloads.

The skewed workloads add b_e = -tau * 1.1 * ln(rank_e) to expert e's router
logit (rank: a seeded permutation of 1..512). Taken with tau = 1 the bias is so
strong that almost all selections go to a handful of experts; tau is chosen
instead so that the hottest 20% of experts (102 of 512) take 80% of the top-10
selections, which is the skew the workload describes. Routing is the oracle's.

Run:  python tests/golden/calibrate_zipf.py   (writes tests/golden/zipf_tau.json)
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle  # noqa: E402
import synth   # noqa: E402

E, K, H, TOP = 512, 10, 2048, 102
N_TOKENS = 4000


def hot_share(layer, x, tau):
    layer.router_b = (-tau * synth.ZIPF_S * np.log(
        synth.permutation(synth.key(0, 2, 0, synth.T_ZIPF_PERM, 0), E).astype(np.float64) + 1.0)).astype(np.float32)
    idx, _, _ = oracle.route(layer, x)
    counts = np.bincount(idx.ravel(), minlength=E)
    return np.sort(counts)[::-1][:TOP].sum() / counts.sum(), int((counts > 0).sum())


def main():
    layer = synth.make_layer("decode_q3_zipf", experts=False)
    # calibration tokens: a stream of their own, not the benchmark tokens
    x = synth.normal_bf16(synth.key(0, 2, 0, synth.T_X, 77), (N_TOKENS, H), 1.0)
    lo, hi = 0.0, 1.0
    for _ in range(14):
        mid = 0.5 * (lo + hi)
        share, _ = hot_share(layer, x, mid)
        lo, hi = (mid, hi) if share < 0.8 else (lo, mid)
    tau = round(0.5 * (lo + hi), 4)
    share, used = hot_share(layer, x, tau)
    lit, lit_used = hot_share(layer, x, 1.0)
    out = dict(tau=tau, hot_share=round(float(share), 4), experts_used=used,
               literal_tau1_hot_share=round(float(lit), 4), literal_tau1_experts_used=lit_used,
               tokens=N_TOKENS, top=TOP, s=synth.ZIPF_S, router_sd=0.02)
    print(out)
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_tau.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
