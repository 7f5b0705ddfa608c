"""The seeded generator: published SplitMix64 sequence, determinism, ranges."""
import numpy as np

import synth


def test_splitmix64_published_sequence():
    # First outputs of SplitMix64 seeded with 1234567 (Steele, Lea, Flood 2014 reference code).
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    got = [synth.lib().synth_splitmix64_at(1234567, i) for i in range(5)]
    assert got == want


def test_streams_are_deterministic_and_distinct():
    k1 = synth.key(0, 1, 0, synth.T_GATE_Q, 3)
    k2 = synth.key(0, 1, 0, synth.T_GATE_Q, 4)
    a = synth.codes(k1, (1000,), 4)
    assert np.array_equal(a, synth.codes(k1, (1000,), 4))
    assert not np.array_equal(a, synth.codes(k2, (1000,), 4))
    # a prefix of a longer draw is the shorter draw (counter-based)
    assert np.array_equal(synth.codes(k1, (5000,), 4)[:1000], a)
    assert np.array_equal(synth.normal_bf16(k1, (3000,), 1.0)[:777], synth.normal_bf16(k1, (777,), 1.0))


def test_code_ranges_and_uniformity():
    for bits, lo, hi in ((4, -8, 7), (3, -4, 3)):
        c = synth.codes(synth.key(7, 2, 0, 1, 0), (1 << 18,), bits)
        assert c.min() == lo and c.max() == hi
        counts = np.bincount(c.astype(np.int64) - lo)
        assert len(counts) == hi - lo + 1
        exp = c.size / len(counts)
        assert np.all(np.abs(counts - exp) < 6 * np.sqrt(exp))


def test_scale_range_fp16():
    s = synth.uniform_f16(synth.key(1, 1, 1, 1, 1), (100000,), 0.005, 0.02)
    v = s.view(np.float16).astype(np.float64)
    assert v.min() >= 0.005 - 1e-5 and v.max() <= 0.02 + 1e-5
    assert abs(v.mean() - 0.0125) < 1e-4


def test_normals_moments():
    z = synth.normal_f32(synth.key(3, 0, 0, 0, 0), (400000,), 2.0).astype(np.float64)
    assert abs(z.mean()) < 0.02 and abs(z.std() - 2.0) < 0.02


def test_bf16_rounding_is_round_to_nearest_even():
    # ties: 1 + 2^-8 lies halfway between bf16 1.0 and 1.0078125 -> even (1.0)
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 1.0 + 2.0 ** -8 + 2.0 ** -20],
                    np.float32)
    got = synth.f32_to_bf16(vals)
    assert list(got) == [0x3F80, 0x3F82, 0xBF80, 0x3F81]


def test_fp16_scale_rounding_matches_numpy():
    # numpy's float32 -> float16 cast rounds to nearest even; the generator's must agree
    k = synth.key(9, 9, 9, 9, 9)
    s = synth.uniform_f16(k, (50000,), 0.005, 0.02)
    # regenerate the float32 values the same way: lo + (hi-lo)*u, then compare one-ulp agreement
    v = s.view(np.float16).astype(np.float32)
    assert np.all(np.isfinite(v))
    re = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(re, s)


def test_tiny_workload_shapes():
    L = synth.make_layer("tiny")
    assert L.router_w.shape == (8, 64) and L.gate_f.shape == (8, 32, 64) and L.down_f.shape == (8, 64, 32)
    assert L.shared_gate.shape == (32, 64) and L.shared_down.shape == (64, 32)
    x = synth.make_tokens("tiny")
    assert x.shape == (16, 64) and x.dtype == np.uint16


def test_zipf_bias_is_a_permuted_log_rank():
    b = synth.zipf_bias(0, 2, 0, 512).astype(np.float64)
    ranks = np.exp(-b / (synth.ZIPF_TAU * synth.ZIPF_S))
    assert np.allclose(np.sort(ranks), np.arange(1, 513), rtol=1e-5)


def test_zipf_tau_matches_calibration_record():
    import json, os
    rec = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "zipf_tau.json")))
    assert synth.ZIPF_TAU == rec["tau"] and 0.79 < rec["hot_share"] < 0.81
