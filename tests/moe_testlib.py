"""Helpers for the GPU parity tests: upload, run, and compare with the oracle.

The comparison bar: expert indices bit-exact and in order (a mismatch is
accepted only where the oracle's two logits tie to within 1e-12 relative,
the one case where both orders are correct); gates within 1e-6 relative;
outputs per token within max relative error 2e-2 (max abs difference over
max abs reference value) and cosine similarity >= 0.9999.
"""
import sys

import numpy as np

import oracle

Y_MAX_REL = 2e-2
Y_MIN_COS = 0.9999
GATE_REL = 1e-6
TIE_REL = 1e-12


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x_bits, dev="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(dev)


def from_dev_bits(t):
    return t.cpu().numpy().view(np.uint16)


def check_routing(idx_gpu, idx_ref, logits_ref, what=""):
    idx_gpu = np.asarray(idx_gpu)
    bad = np.nonzero(np.any(idx_gpu != idx_ref, axis=1))[0]
    for t in bad:
        # allowed only if every differing position is a tie within TIE_REL
        l = logits_ref[t]
        a, b = idx_gpu[t], idx_ref[t]
        for j in range(len(a)):
            if a[j] != b[j]:
                la, lb = l[a[j]], l[b[j]]
                assert abs(la - lb) <= TIE_REL * max(abs(la), abs(lb), 1e-300), \
                    "%s token %d: routing %s vs oracle %s" % (what, t, a.tolist(), b.tolist())
    return len(bad)


def check_gates(g_gpu, g_ref, what=""):
    rel = np.abs(np.asarray(g_gpu, np.float64) - g_ref) / np.abs(g_ref)
    assert rel.max() <= GATE_REL, "%s gates max rel %.3g" % (what, rel.max())
    return float(rel.max())


def y_metrics(y_bits, y_ref):
    yf = oracle.bf16_bits_to_f64(y_bits)
    denom = np.abs(y_ref).max(axis=1)
    err = np.abs(yf - y_ref).max(axis=1) / denom
    cos = (yf * y_ref).sum(1) / (np.linalg.norm(yf, axis=1) * np.linalg.norm(y_ref, axis=1))
    return err, cos


def check_y(y_bits, y_ref, what=""):
    err, cos = y_metrics(y_bits, y_ref)
    assert np.all(np.isfinite(err)) and err.max() <= Y_MAX_REL, "%s max rel err %.4g" % (what, err.max())
    assert cos.min() >= Y_MIN_COS, "%s min cos %.7f" % (what, cos.min())
    log("  %s: tokens=%d max_rel=%.3e min_cos=%.7f" % (what, len(err), err.max(), cos.min()))
    return float(err.max()), float(cos.min())
