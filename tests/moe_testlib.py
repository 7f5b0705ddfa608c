"""Helpers for the GPU parity tests: upload, run, and compare with the oracle.

The comparison bar: expert indices are the oracle's ordered top-k (checked
against the oracle's fp64 logits for every token: distinct, in order, none
beaten by an unselected expert; exact ties lower index first; only logits
within 1e-12 of the dot product's size may come in either order, the one
case where both orders are correct); gates within 1e-6 relative;
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


def routing_scale(layer, x_bits):
    """Per token, the size of the router's fp64 dot products: the largest
    sum_h |W_r[e,h] x_h| + |b_e| over the experts. Two fp64 evaluations of a
    logit in different summation orders differ by far less than 1e-12 of it
    (H * 2^-53 < 3e-13 for H <= 2048), which is what TIE_REL is relative to."""
    xa = np.abs(oracle.bf16_bits_to_f64(x_bits))
    s = xa @ np.abs(np.asarray(layer.router_w, np.float64)).T
    if layer.router_b is not None:
        s = s + np.abs(np.asarray(layer.router_b, np.float64))[None, :]
    return s.max(axis=1)


def check_routing(idx_gpu, idx_ref, logits_ref, what="", scale=None):
    """The GPU's rows must be the ordered top-k of the oracle's fp64 logits:
    k distinct experts in range; consecutive experts in (logit desc, index
    asc) order; every unselected expert ranked after every selected one. A
    pair of logits closer than TIE_REL * scale (a near-tie below fp64
    resolution, where both orders are correct) may come in either order;
    exactly equal logits must come lower index first. Returns the number of
    tokens whose row differs from the oracle's (near-ties only)."""
    idx = np.asarray(idx_gpu).astype(np.int64)
    L = np.asarray(logits_ref, np.float64)
    T, k = idx.shape
    E = L.shape[1]
    assert idx.min() >= 0 and idx.max() < E, "%s: expert index out of range" % what
    srt = np.sort(idx, axis=1)
    dup = np.nonzero(np.any(srt[:, 1:] == srt[:, :-1], axis=1))[0]
    assert len(dup) == 0, "%s token %d: repeated expert %s" % (what, dup[0], idx[dup[0]].tolist())
    if scale is None:
        scale = np.abs(L).max(axis=1)
    tol = TIE_REL * np.asarray(scale, np.float64)
    lv = np.take_along_axis(L, idx, axis=1)
    # consecutive selected experts
    a, b = lv[:, :-1], lv[:, 1:]
    ia, ib = idx[:, :-1], idx[:, 1:]
    ok = (a > b) | ((a == b) & (ia < ib)) | ((a != b) & (np.abs(a - b) <= tol[:, None]))
    bad = np.nonzero(~np.all(ok, axis=1))[0]
    assert len(bad) == 0, "%s token %d: order %s, logits %s" % (what, bad[0], idx[bad[0]].tolist(),
                                                                   lv[bad[0]].tolist())
    # selected against unselected
    unsel = np.ones((T, E), bool)
    np.put_along_axis(unsel, idx, False, axis=1)
    best_un = np.where(unsel, L, -np.inf).max(axis=1)
    worst_sel = lv.min(axis=1)
    close = np.nonzero(best_un >= worst_sel - tol)[0]
    for t in close:   # rare: only tokens with a near or exact tie at the boundary
        for i, li in zip(idx[t], lv[t]):
            js = np.nonzero(unsel[t])[0]
            lj = L[t, js]
            beaten = (lj > li) | ((lj == li) & (js < i))
            allowed = (lj != li) & (np.abs(lj - li) <= tol[t])
            assert not np.any(beaten & ~allowed), "%s token %d: expert %d selected over %s" % (
                what, t, i, js[beaten & ~allowed].tolist())
    return int(np.count_nonzero(np.any(idx != np.asarray(idx_ref), axis=1))) if idx_ref is not None else 0


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
