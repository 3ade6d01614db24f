"""The seeded input generator: stream definition, exact tables, statistics."""
import math

import numpy as np

import synth


def test_philox_known_answer_zero_key_zero_counter():
    # Philox4x64-10 of counter 0 under key 0, as published with the generator
    # (Random123 known-answer vectors); words come low half first
    w = synth.philox_words((0, 0), 0, 8)
    want64 = [0x16554D9ECA36314C, 0xDB20FE9D672D0FDC, 0xD7E772CEE186176B, 0x7E68B68AEC7BA23B]
    want = []
    for x in want64:
        want += [x & 0xFFFFFFFF, x >> 32]
    assert [int(v) for v in w] == want


def _philox_by_definition(ctr, key):
    """Philox4x64-10 written out from the published round function."""
    M = (1 << 64) - 1
    c, (k0, k1) = list(ctr), key
    for r in range(10):
        if r:
            k0, k1 = (k0 + 0x9E3779B97F4A7C15) & M, (k1 + 0xBB67AE8584CAA73B) & M
        p0, p1 = 0xD2E7470EE14C6C93 * c[0], 0xCA5A826395121157 * c[2]
        c = [(p1 >> 64) ^ c[1] ^ k0, p1 & M, (p0 >> 64) ^ c[3] ^ k1, p0 & M]
    return c


def test_stream_equals_round_function():
    for key in [(0, 0), (1003, 12 << 32 | 5), (2 ** 63 + 5, 2 ** 40 + 3), (2 ** 64 - 1, 2 ** 64 - 1)]:
        for b in (0, 1, 77, 2 ** 33 + 9):
            w = synth.philox_words(key, 8 * b, 8)
            got = [int(w[2 * i]) | (int(w[2 * i + 1]) << 32) for i in range(4)]
            assert got == _philox_by_definition([b, 0, 0, 0], key), (key, b)


def test_stream_random_access():
    key = synth.stream_key(1234, 12, 5)
    full = synth.philox_words(key, 0, 1000)
    for s, n in [(0, 1), (7, 9), (8, 8), (13, 400), (999, 1)]:
        assert np.array_equal(synth.philox_words(key, s, n), full[s:s + n])
    # distinct tensors / layers / seeds give distinct streams
    a = synth.philox_words(synth.stream_key(1, 12, 0), 0, 64)
    b = synth.philox_words(synth.stream_key(1, 12, 1), 0, 64)
    c = synth.philox_words(synth.stream_key(1, 13, 0), 0, 64)
    d = synth.philox_words(synth.stream_key(2, 12, 0), 0, 64)
    assert len({a.tobytes(), b.tobytes(), c.tobytes(), d.tobytes()}) == 4


def test_weight_rows_are_random_access():
    cfg = synth.get("tiny")
    q, d = synth.weight_q4(cfg, "gu")
    q2, d2 = synth.weight_q4(cfg, "gu", rows=slice(100, 300))
    assert np.array_equal(q[100:300], q2) and np.array_equal(d[100:300], d2)


def _ndtr(x):
    return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


def test_normal_table_masses_match_the_cdf():
    t = synth.normal_bf16_table()
    vals = synth._bf16_to_f64(t.values)
    assert np.all(np.diff(vals) > 0)
    edges = np.concatenate([[0], t.thresholds.astype(np.float64), [2.0 ** 32]])
    mass = np.diff(edges) / 2.0 ** 32
    # bf16 1.0: spacing 2^-8 below, 2^-7 above
    j = int(np.where(vals == 1.0)[0][0])
    want = _ndtr(1.0 + 2.0 ** -8) - _ndtr(1.0 - 2.0 ** -9)
    assert abs(mass[j] - want) < 2e-9
    j = int(np.where(vals == -2.5)[0][0])
    want = _ndtr(-2.5 + 2.0 ** -7) - _ndtr(-2.5 - 2.0 ** -7)
    assert abs(mass[j] - want) < 2e-9
    assert abs(mass.sum() - 1.0) < 1e-12


def test_scale_and_gain_tables_are_uniform_ranges():
    s = synth.scale_table()
    v = synth._f16_to_f64(s.values)
    assert v.min() >= 0.002 - 1e-6 and v.max() <= 0.02 + 1e-5
    edges = np.concatenate([[0], s.thresholds.astype(np.float64), [2.0 ** 32]])
    mass = np.diff(edges) / 2.0 ** 32
    # a value strictly inside the range gets probability spacing / 0.018
    j = int(np.argmin(np.abs(v - 0.01)))
    want = (v[j + 1] - v[j - 1]) / 2 / 0.018
    assert abs(mass[j] - want) < 1e-8
    g = synth._bf16_to_f64(synth.gain_table().values)
    assert g.min() == 0.5 and g.max() == 1.5


def test_sampler_equals_plain_search():
    t = synth.normal_bf16_table()
    w = synth.philox_words(synth.stream_key(9, 1, 0), 0, 200000)
    assert np.array_equal(t.sample(w), t.values[np.searchsorted(t.thresholds, w, side="right")])


def test_value_statistics():
    cfg = synth.get("tiny")
    k, v = synth.kv_prefix(cfg)
    kf = synth._bf16_to_f64(k)
    assert abs(kf.mean()) < 0.03 and abs(kf.std() - 1.0) < 0.03
    q, d = synth.weight_q4(cfg, "gu")
    assert q.min() == 0 and q.max() == 15 and abs(q.mean() - 7.5) < 0.05
    df = synth._f16_to_f64(d)
    assert abs(df.mean() - 0.011) < 5e-4


def test_tree_recipes_hold():
    for name in ("tiny", "layer27b", "longctx27b"):
        cfg = synth.get(name)
        for r in range(30):
            p = synth.tree_parents(cfg, synth.run_seed(cfg, r))
            assert p[0] == -1 and len(p) == cfg.nodes
            depth = [0] * cfg.nodes
            kids = [0] * cfg.nodes
            for i in range(1, cfg.nodes):
                assert 0 <= p[i] < i
                depth[i] = depth[p[i]] + 1
                kids[p[i]] += 1
            if cfg.max_children:
                assert max(kids) <= cfg.max_children
                assert max(depth) <= cfg.max_depth


def test_generator_is_deterministic():
    cfg = synth.get("tiny")
    assert np.array_equal(synth.hidden_in(cfg), synth.hidden_in(cfg))
    assert np.array_equal(synth.tree_parents(cfg, 5), synth.tree_parents(cfg, 5))
