"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Closed forms, invariants, textbook special cases and brute force on tiny
inputs.  Each test names the slip it would catch.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle.reference import linear_q4
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f16(x):
    return np.asarray(x, np.float16).view(np.uint16)


def bf16(x):
    """Round-to-nearest-even fp64 -> bf16 bits (test helper)."""
    f = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = (f + 0x7FFF + ((f >> 16) & 1)) >> 16
    return r.astype(np.uint16)


# ------------------------------------------------------------------ dequant

def test_dequant_zero_point_gives_zero():
    # q == 8 is the zero point: a wrong offset (q - 7, q) would show here
    q = np.full((3, 64), 8, np.uint8)
    d = f16(np.full((3, 2), 0.013))
    assert np.all(oracle.dequant_q4(q, d) == 0.0)


def test_dequant_exact_integer_dot():
    # integer activations and power-of-two scales make fp64 exact; compare
    # with Python big-int arithmetic (catches a wrong block index or offset)
    rng = np.random.default_rng(1)
    n_out, k_in = 5, 96
    q = rng.integers(0, 16, (n_out, k_in), dtype=np.uint8)
    exps = rng.integers(-9, -4, (n_out, k_in // 32))
    d = f16(np.ldexp(1.0, exps))
    x = rng.integers(-50, 50, (3, k_in))
    y = linear_q4(x.astype(np.float64), (q, d))
    from fractions import Fraction
    for r in range(3):
        for n in range(n_out):
            tot = Fraction(0)
            for b in range(k_in // 32):
                s = sum(int(x[r, k]) * (int(q[n, k]) - 8) for k in range(32 * b, 32 * b + 32))
                tot += s * Fraction(2) ** int(exps[n, b])
            assert y[r, n] == float(tot)


def test_dequant_block_axis_is_input_axis():
    # changing scale d[n, b] moves only W[n, 32b:32b+32] (blocks run along k)
    rng = np.random.default_rng(2)
    q = rng.integers(0, 16, (4, 128), dtype=np.uint8)
    d = f16(rng.uniform(0.002, 0.02, (4, 4)))
    w0 = oracle.dequant_q4(q, d)
    d2 = d.copy()
    d2[2, 1] = f16(0.5)
    w1 = oracle.dequant_q4(q, d2)
    diff = w0 != w1
    expect = np.zeros_like(diff)
    expect[2, 32:64] = (q[2, 32:64] != 8)
    assert np.array_equal(diff, expect)


def test_dequant_matches_dense_matmul():
    # the chunked q4 linear equals one dense numpy matmul of the same W
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, (40, 64), dtype=np.uint8)
    d = f16(rng.uniform(0.002, 0.02, (40, 2)))
    w = (q.astype(np.float64) - 8) * np.repeat(d.view(np.float16).astype(np.float64), 32, axis=1)
    x = rng.standard_normal((7, 64))
    np.testing.assert_allclose(linear_q4(x, (q, d), row_chunk=16), x @ w.T, rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------------ rmsnorm

def test_rmsnorm_closed_form():
    x = np.array([[3.0, 4.0]])
    g = np.array([1.0, 2.0])
    y = oracle.rmsnorm(x, g, 0.0)
    r = math.sqrt(12.5)
    np.testing.assert_allclose(y, [[3 / r, 8 / r]], rtol=1e-15)


def test_rmsnorm_constant_row_is_signed_gain():
    g = np.array([0.5, 1.25, 1.5, 0.75])
    for c in (-3.0, 2.5):
        y = oracle.rmsnorm(np.full((1, 4), c), g, 0.0)
        np.testing.assert_allclose(y[0], np.sign(c) * g, rtol=1e-15)


def test_rmsnorm_scale_invariant_and_eps():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 16))
    g = rng.uniform(0.5, 1.5, 16)
    np.testing.assert_allclose(oracle.rmsnorm(7.0 * x, g, 0.0), oracle.rmsnorm(x, g, 0.0), rtol=1e-14)
    # eps is added to the mean square, not to the root
    y = oracle.rmsnorm(np.full((1, 2), 1e-3), np.ones(2), 1e-6)
    np.testing.assert_allclose(y, 1e-3 / math.sqrt(1e-6 + 1e-6), rtol=1e-14)


# ------------------------------------------------------------------ silu

def test_silu_values():
    np.testing.assert_allclose(oracle.silu(np.array([0.0, 1.0, -1.0, 40.0])),
                               [0.0, 0.7310585786300049, -0.2689414213699951, 40.0], rtol=1e-15, atol=0)


# ------------------------------------------------------------------ rope

def test_rope_identity_at_zero_and_norm():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 16))
    np.testing.assert_array_equal(oracle.rope(x, 0, 10000.0), x)
    y = oracle.rope(x, np.array([1, 17, 4096]), 10000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)


def test_rope_two_dims_closed_form():
    # d = 2: the single pair turns by theta = pos (base**0 = 1)
    y = oracle.rope(np.array([1.0, 0.0]), 1.0, 10000.0)
    np.testing.assert_allclose(y, [math.cos(1.0), math.sin(1.0)], rtol=1e-15)
    y = oracle.rope(np.array([0.0, 1.0]), 2.0, 10000.0)
    np.testing.assert_allclose(y, [-math.sin(2.0), math.cos(2.0)], rtol=1e-15)


def test_rope_is_complex_multiply_on_half_pairs():
    rng = np.random.default_rng(6)
    d = 32
    x = rng.standard_normal(d)
    pos = 123
    z = x[:d // 2] + 1j * x[d // 2:]
    freqs = np.array([10000.0 ** (-(2.0 * j) / d) for j in range(d // 2)])
    w = z * np.exp(1j * pos * freqs)
    np.testing.assert_allclose(oracle.rope(x, pos, 10000.0), np.concatenate([w.real, w.imag]), rtol=1e-12, atol=1e-12)


def test_rope_score_depends_on_offset_only():
    rng = np.random.default_rng(7)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    s1 = oracle.rope(q, 105, 1e4) @ oracle.rope(k, 100, 1e4)
    s2 = oracle.rope(q, 4101, 1e4) @ oracle.rope(k, 4096, 1e4)
    assert abs(s1 - s2) < 1e-10


# ------------------------------------------------------------------ attention

def _anc_matrix(parent):
    """Independent ancestor-or-self relation by walking parent links."""
    N = len(parent)
    A = np.zeros((N, N), bool)
    for i in range(N):
        j = i
        while j >= 0:
            A[i, j] = True
            j = parent[j]
    return A


def test_attention_equal_keys_average_values():
    rng = np.random.default_rng(8)
    parent = [-1, 0, 0, 1, 3]
    N, Hq, Hkv, d, P = 5, 4, 2, 8, 6
    key = rng.standard_normal(d)
    q = rng.standard_normal((N, Hq, d))
    kt = np.broadcast_to(key, (N, Hkv, d)).copy()
    kp = np.broadcast_to(key, (Hkv, P, d)).copy()
    vt = rng.standard_normal((N, Hkv, d))
    vp = rng.standard_normal((Hkv, P, d))
    o = oracle.tree_attention(q, kt, vt, kp, vp, parent)
    A = _anc_matrix(parent)
    for i in range(N):
        for h in range(Hq):
            g = h // 2
            vals = np.concatenate([vp[g], vt[A[i], g]])
            np.testing.assert_allclose(o[i, h], vals.mean(0), rtol=1e-13, atol=1e-14)


def test_attention_single_key_returns_its_value():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 6, 4))
    kt, vt = rng.standard_normal((1, 3, 4)), rng.standard_normal((1, 3, 4))
    o = oracle.tree_attention(q, kt, vt, np.zeros((3, 0, 4)), np.zeros((3, 0, 4)), [-1])
    for h in range(6):
        np.testing.assert_allclose(o[0, h], vt[0, h // 2], rtol=1e-15)


def test_attention_equals_dense_masked_softmax():
    # gather formulation == dense [P + N] scores with a -inf mask off the ancestors
    rng = np.random.default_rng(10)
    parent = [-1, 0, 1, 0, 3, 3, 2]
    N, Hq, Hkv, d, P = 7, 6, 2, 16, 9
    q = rng.standard_normal((N, Hq, d))
    kt, vt = rng.standard_normal((N, Hkv, d)), rng.standard_normal((N, Hkv, d))
    kp, vp = rng.standard_normal((Hkv, P, d)), rng.standard_normal((Hkv, P, d))
    o = oracle.tree_attention(q, kt, vt, kp, vp, parent)
    A = _anc_matrix(parent)
    mask = np.concatenate([np.zeros((N, P)), np.where(A, 0.0, -np.inf)], axis=1)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        K = np.concatenate([kp[g], kt[:, g]])
        V = np.concatenate([vp[g], vt[:, g]])
        s = q[:, h] @ K.T / math.sqrt(d) + mask
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        np.testing.assert_allclose(o[:, h], p @ V, rtol=1e-12, atol=1e-13)


def test_attention_gqa_equals_repeated_kv_heads():
    rng = np.random.default_rng(11)
    parent = [-1, 0, 0, 2]
    N, Hq, Hkv, d, P = 4, 6, 3, 8, 5
    q = rng.standard_normal((N, Hq, d))
    kt, vt = rng.standard_normal((N, Hkv, d)), rng.standard_normal((N, Hkv, d))
    kp, vp = rng.standard_normal((Hkv, P, d)), rng.standard_normal((Hkv, P, d))
    o = oracle.tree_attention(q, kt, vt, kp, vp, parent)
    rep = Hq // Hkv
    o2 = oracle.tree_attention(q, np.repeat(kt, rep, axis=1), np.repeat(vt, rep, axis=1),
                               np.repeat(kp, rep, axis=0), np.repeat(vp, rep, axis=0), parent)
    np.testing.assert_allclose(o, o2, rtol=1e-14)


def test_attention_prefix_split_merges():
    # softmax over the prefix split in two chunks, merged by log-sum-exp
    rng = np.random.default_rng(12)
    N, Hq, Hkv, d, P = 3, 2, 1, 8, 10
    parent = [-1, 0, 1]
    q = rng.standard_normal((N, Hq, d)) * 3
    kt, vt = rng.standard_normal((N, Hkv, d)), rng.standard_normal((N, Hkv, d))
    kp, vp = rng.standard_normal((Hkv, P, d)), rng.standard_normal((Hkv, P, d))
    o = oracle.tree_attention(q, kt, vt, kp, vp, parent)
    A = _anc_matrix(parent)
    for i in range(N):
        for h in range(Hq):
            parts = [(kp[0, :4], vp[0, :4]), (kp[0, 4:], vp[0, 4:]), (kt[A[i], 0], vt[A[i], 0])]
            ms, ls, os_ = [], [], []
            for K, V in parts:
                s = K @ q[i, h] / math.sqrt(d)
                m = s.max()
                p = np.exp(s - m)
                ms.append(m); ls.append(p.sum()); os_.append(p @ V)
            M = max(ms)
            L = sum(l * math.exp(m - M) for l, m in zip(ls, ms))
            O = sum(ov * math.exp(m - M) for ov, m in zip(os_, ms)) / L
            np.testing.assert_allclose(o[i, h], O, rtol=1e-13)


# ------------------------------------------------------------------ whole layer

MINI = synth.Config("mini", layers=2, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16,
                    ffn=96, vocab=16, prefix=8, nodes=6, max_children=None,
                    max_depth=None, p_accept=0.7, seed=77)


def _mini_inputs(cfg, seed=77):
    from workload import layer_weights, shape
    lws = [layer_weights(cfg, l, seed) for l in range(cfg.layers)]
    kvs = [synth.kv_prefix(cfg, l, seed) for l in range(cfg.layers)]
    return lws, kvs, shape(cfg)


def _all_recursive_trees(n):
    """Every parent array with parent[i] in [0, i): (n-1)! trees."""
    if n == 1:
        yield [-1]
        return
    for choice in itertools.product(*[range(i) for i in range(1, n)]):
        yield [-1] + list(choice)


def _sequential_decode(x_nodes, path, lws, kvs, shp):
    """Plain one-token decoding along ``path``: each step is a 1-node forward
    whose KV cache is the prefix plus the post-RoPE K / V of earlier steps."""
    P = kvs[0][0].shape[1]
    caches = [(oracle.bf16_to_f64(k), oracle.bf16_to_f64(v)) for k, v in kvs]
    outs = []
    for t, node in enumerate(path):
        x = x_nodes[node:node + 1]
        for l, w in enumerate(lws):
            kc, vc = caches[l]
            x, k1, v1 = oracle.layer_forward(x, w, kc, vc, [-1], shp, prefix_len=P + t)
            caches[l] = (np.concatenate([kc, k1[0][:, None, :]], axis=1),
                         np.concatenate([vc, v1[0][:, None, :]], axis=1))
        outs.append(x[0])
    return outs


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_tree_forward_equals_sequential_decoding_all_trees(n):
    # for every recursive tree with n nodes, the tree forward at node i equals
    # greedy one-token decoding of i's root path (positions, mask and KV concat)
    lws, kvs, shp = _mini_inputs(MINI)
    x_nodes = oracle.bf16_to_f64(synth.hidden_in(MINI, 77, nodes=n))
    for parent in _all_recursive_trees(n):
        out = oracle.verify_forward(x_nodes, lws, kvs, None, parent, shp)
        final = out["hidden"][-1]
        for i in range(n):
            path = []
            j = i
            while j >= 0:
                path.append(j)
                j = parent[j]
            path.reverse()
            seq = _sequential_decode(x_nodes, path, lws, kvs, shp)
            np.testing.assert_allclose(final[i], seq[-1], rtol=1e-11, atol=1e-11)


def test_chain_equals_sequential_decoding_tiny_shape():
    cfg = synth.get("tiny").replace(layers=1)
    from workload import layer_weights, shape
    lws = [layer_weights(cfg, 0)]
    kvs = [synth.kv_prefix(cfg, 0)]
    shp = shape(cfg)
    parent = [-1, 0, 1, 2, 3, 4]
    x_nodes = oracle.bf16_to_f64(synth.hidden_in(cfg, nodes=6))
    out = oracle.verify_forward(x_nodes, lws, kvs, None, parent, shp)
    seq = _sequential_decode(x_nodes, list(range(6)), lws, kvs, shp)
    for i in range(6):
        np.testing.assert_allclose(out["hidden"][-1][i], seq[i], rtol=1e-11, atol=1e-11)


def test_non_ancestor_inputs_do_not_reach_a_node():
    lws, kvs, shp = _mini_inputs(MINI)
    parent = [-1, 0, 0, 1, 2, 3]
    x = oracle.bf16_to_f64(synth.hidden_in(MINI, 77, nodes=6))
    base = oracle.verify_forward(x, lws, kvs, None, parent, shp)["hidden"][-1]
    A = _anc_matrix(parent)
    for j in range(6):
        x2 = x.copy()
        x2[j] += 0.5
        out = oracle.verify_forward(x2, lws, kvs, None, parent, shp)["hidden"][-1]
        for i in range(6):
            if A[i, j]:
                assert np.max(np.abs(out[i] - base[i])) > 1e-3
            else:
                np.testing.assert_allclose(out[i], base[i], rtol=1e-12, atol=1e-12)


def test_topological_relabelling_permutes_outputs():
    lws, kvs, shp = _mini_inputs(MINI)
    parent = [-1, 0, 0, 1, 2, 2]
    x = oracle.bf16_to_f64(synth.hidden_in(MINI, 77, nodes=6))
    base = oracle.verify_forward(x, lws, kvs, None, parent, shp)["hidden"][-1]
    perm = [0, 2, 1, 5, 4, 3]          # new index -> old index (parents still first)
    inv = {old: new for new, old in enumerate(perm)}
    parent2 = [-1] + [inv[parent[old]] for old in perm[1:]]
    out = oracle.verify_forward(x[perm], lws, kvs, None, parent2, shp)["hidden"][-1]
    np.testing.assert_allclose(out, base[perm], rtol=1e-11, atol=1e-11)


# ------------------------------------------------------------------ acceptance

def _accept_by_enumeration(parent, token, am):
    """Every root path whose steps all match the parent's greedy token; keep the
    longest, lowest end index on ties (independent of the oracle's scan)."""
    N = len(parent)
    best = [0]
    for end in range(N):
        path = []
        j = end
        while j >= 0:
            path.append(j)
            j = parent[j]
        path.reverse()
        ok = all(token[path[s]] == am[path[s - 1]] for s in range(1, len(path)))
        if ok and len(path) > len(best):
            best = path
    return best, [token[i] for i in best[1:]] + [am[best[-1]]]


def test_accept_exhaustive_small_trees():
    V = 3
    for n in range(1, 6):
        for parent in _all_recursive_trees(n):
            for tok in itertools.product(range(V), repeat=n - 1):
                token = [0] + list(tok)
                for am in itertools.product(range(V), repeat=n):
                    got = oracle.accept_path(parent, token, am)
                    want = _accept_by_enumeration(parent, token, list(am))
                    assert (list(got[0]), list(got[1])) == (want[0], want[1])


def test_accept_sampled_six_and_eight_node_trees():
    rng = np.random.default_rng(13)
    for n in (6, 8):
        trees = list(_all_recursive_trees(n)) if n == 6 else None
        for _ in range(3000):
            parent = trees[rng.integers(len(trees))] if trees else [-1] + [int(rng.integers(i)) for i in range(1, n)]
            token = [0] + list(rng.integers(0, 2, n - 1))
            am = list(rng.integers(0, 2, n))
            got = oracle.accept_path(parent, token, am)
            want = _accept_by_enumeration(parent, token, am)
            assert (list(got[0]), list(got[1])) == want


def test_accept_hand_walked_cases():
    with open(os.path.join(GOLDEN, "accept_cases.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        path, committed = oracle.accept_path(c["parent"], c["token"], c["argmax"])
        assert path == c["path"], c["name"]
        assert committed == c["committed"], c["name"]


def test_argmax_gap_rules():
    lg = np.array([[1.0, 3.0, 3.0, 0.5], [0.0, -1.0, 2.0, 1.5]])
    am, gap = oracle.argmax_gap(lg)
    assert list(am) == [1, 2]
    np.testing.assert_allclose(gap, [0.0, 0.5])


def test_prefix_cache_convention_against_decoding_from_position_zero():
    # Decode P context tokens one at a time from position 0, keeping each
    # layer's post-RoPE K / V: that cache, used as the stored prefix, must make
    # the tree forward equal continued sequential decoding (pins "prefix keys
    # stored rotated at 0..P-1, root at position P").
    cfg = MINI.replace(layers=2)
    from workload import layer_weights, shape
    lws = [layer_weights(cfg, l) for l in range(2)]
    shp = shape(cfg)
    P = 5
    ctx = oracle.bf16_to_f64(synth.hidden_in(cfg, 901, nodes=P))
    Hkv, d = cfg.n_kv_heads, cfg.head_dim
    caches = [(np.zeros((Hkv, 0, d)), np.zeros((Hkv, 0, d))) for _ in range(2)]
    for t in range(P):
        x = ctx[t:t + 1]
        for l in range(2):
            kc, vc = caches[l]
            x, k1, v1 = oracle.layer_forward(x, lws[l], kc, vc, [-1], shp, prefix_len=t)
            caches[l] = (np.concatenate([kc, k1[0][:, None]], 1), np.concatenate([vc, v1[0][:, None]], 1))
    parent = [-1, 0, 1, 0, 3]
    xn = oracle.bf16_to_f64(synth.hidden_in(cfg, 902, nodes=5))
    tree = oracle.verify_forward(xn, lws, caches, None, parent, shp)["hidden"][-1]
    for i, path in enumerate([[0], [0, 1], [0, 1, 2], [0, 3], [0, 3, 4]]):
        # continue decoding after the context, positions P, P+1, ...
        cs = [(c[0].copy(), c[1].copy()) for c in caches]
        for t, node in enumerate(path):
            x = xn[node:node + 1]
            for l in range(2):
                kc, vc = cs[l]
                x, k1, v1 = oracle.layer_forward(x, lws[l], kc, vc, [-1], shp, prefix_len=P + t)
                cs[l] = (np.concatenate([kc, k1[0][:, None]], 1), np.concatenate([vc, v1[0][:, None]], 1))
        np.testing.assert_allclose(tree[i], x[0], rtol=1e-11, atol=1e-11)


# ------------------------------------------------------------------ commit of the accepted path

def _bf16_grid():
    """Every finite bf16 value, sorted, with its bit pattern (brute force)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_to_f64(bits)
    ok = np.isfinite(vals)
    order = np.argsort(vals[ok], kind="stable")
    return vals[ok][order], bits[ok][order]


def test_round_bf16_is_nearest_with_ties_to_even():
    # against a search over the whole bf16 grid: a dropped carry, a
    # truncation instead of rounding or ties away from zero all fail here
    grid, gbits = _bf16_grid()
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-6, 6, 4000),
                        # exact halfway points between neighbouring bf16 values
                        (grid[1000:1200] + grid[1001:1201]) / 2.0,
                        (grid[40000:40100] + grid[40001:40101]) / 2.0])
    got = oracle.round_bf16(x)
    for xi, gi in zip(x, got):
        j = np.searchsorted(grid, xi)
        cands = [c for c in (j - 1, j) if 0 <= c < len(grid)]
        dist = [abs(grid[c] - xi) for c in cands]
        best = [c for c, dd in zip(cands, dist) if dd == min(dist)]
        if len(best) > 1:  # a tie: the even bit pattern wins (+0 / -0 aside)
            best = [c for c in best if gbits[c] % 2 == 0] or best
        assert gi == grid[best[0]] or (gi == 0 and grid[best[0]] == 0), (xi, gi, grid[best[0]])


def test_commit_path_appends_path_rows_in_order():
    # hand-built: prefix rows stay, path rows follow root first, rounded
    Hkv, d, P, N = 2, 3, 2, 5
    rng = np.random.default_rng(9)
    kp, vp = rng.standard_normal((Hkv, P, d)), rng.standard_normal((Hkv, P, d))
    kt, vt = rng.standard_normal((N, Hkv, d)), rng.standard_normal((N, Hkv, d))
    path = [0, 2, 4]
    k2, v2 = oracle.commit_path(kp, vp, kt, vt, path)
    assert k2.shape == (Hkv, P + 3, d) and v2.shape == (Hkv, P + 3, d)
    np.testing.assert_array_equal(k2[:, :P], kp)
    np.testing.assert_array_equal(v2[:, :P], vp)
    for j, node in enumerate(path):
        for g in range(Hkv):
            np.testing.assert_array_equal(k2[g, P + j], oracle.round_bf16(kt[node, g]))
            np.testing.assert_array_equal(v2[g, P + j], oracle.round_bf16(vt[node, g]))
    # bf16-exact rows are stored unchanged
    kb = oracle.bf16_to_f64(bf16(kt))
    np.testing.assert_array_equal(oracle.commit_path(kp, vp, kb, vt, [1])[0][:, P], kb[1])


def test_commit_then_decode_equals_decoding_with_a_bf16_cache():
    # Step 1: a tree forward; keep the path [0, 1, 3].  Commit it, then step
    # 2 is a one-node forward at position P + 3.  That must equal plain
    # one-token decoding of 0, 1, 3 (within a step the nodes see each other's
    # K / V unrounded), then the three cache entries rounded to bf16 (the
    # cache format, at commit), then decoding the new token.
    cfg = MINI.replace(layers=2)
    lws, kvs, shp = _mini_inputs(cfg)
    parent = [-1, 0, 0, 1, 2]
    path = [0, 1, 3]
    xn = oracle.bf16_to_f64(synth.hidden_in(cfg, 903, nodes=5))
    x_new = oracle.bf16_to_f64(synth.hidden_in(cfg, 904, nodes=1))
    out = oracle.verify_forward(xn, lws, kvs, None, parent, shp)
    caches = [oracle.commit_path(kp, vp, out["k_tree_layers"][l], out["v_tree_layers"][l], path)
              for l, (kp, vp) in enumerate(kvs)]
    P = kvs[0][0].shape[1]
    step2 = oracle.verify_forward(x_new, lws, caches, None, [-1], shp)["hidden"][-1][0]
    # the same by sequential decoding with a rounding cache
    cs = [(oracle.bf16_to_f64(k), oracle.bf16_to_f64(v)) for k, v in kvs]
    seq = [xn[i:i + 1] for i in path] + [x_new]
    for t, x in enumerate(seq):
        if t == len(path):  # the commit: the step's entries are stored as bf16
            cs = [(np.concatenate([kc[:, :P], oracle.round_bf16(kc[:, P:])], 1),
                   np.concatenate([vc[:, :P], oracle.round_bf16(vc[:, P:])], 1)) for kc, vc in cs]
        for l, w in enumerate(lws):
            kc, vc = cs[l]
            x, k1, v1 = oracle.layer_forward(x, w, kc, vc, [-1], shp, prefix_len=P + t)
            cs[l] = (np.concatenate([kc, k1[0][:, None]], 1), np.concatenate([vc, v1[0][:, None]], 1))
    np.testing.assert_allclose(step2, x[0], rtol=1e-10, atol=1e-10)
    # without the rounding at commit the two would differ (the pin sees it)
    assert np.max(np.abs(step2 - oracle.verify_forward(
        x_new, lws, [(np.concatenate([oracle.bf16_to_f64(kp), out["k_tree_layers"][l][path].transpose(1, 0, 2)], 1),
                      np.concatenate([oracle.bf16_to_f64(vp), out["v_tree_layers"][l][path].transpose(1, 0, 2)], 1))
                     for l, (kp, vp) in enumerate(kvs)], None, [-1], shp)["hidden"][-1][0])) > 1e-9
    # and the committed rows differ from the unrounded K / V only by bf16 rounding
    k_unr = out["k_tree_layers"][0][path].transpose(1, 0, 2)
    rel = np.abs(caches[0][0][:, P:] - k_unr) / np.maximum(np.abs(k_unr), 1e-300)
    assert rel.max() <= 2.0 ** -8
