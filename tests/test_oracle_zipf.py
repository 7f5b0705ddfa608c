"""The skewed workload's routing skew, checked with the oracle's router on a
fresh token sample (not the calibration sample)."""
import numpy as np

import oracle
import synth


def test_hot_fifth_of_experts_takes_about_80_percent():
    layer = synth.make_layer("decode_q3_zipf", experts=False)
    x = synth.normal_bf16(synth.key(0, 2, 0, synth.T_X, 78), (1500, 2048), 1.0)
    idx, _, _ = oracle.route(layer, x)
    counts = np.bincount(idx.ravel(), minlength=512)
    share = np.sort(counts)[::-1][:102].sum() / counts.sum()
    assert 0.77 < share < 0.83
