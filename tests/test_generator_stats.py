"""Monte Carlo of the draft-tree generator and planted acceptance against
exact expectations computed by enumeration (pins the recipe and the walk)."""
import itertools

import numpy as np

import oracle
import synth


def _depths(parent):
    d = [0] * len(parent)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
    return d


def _exact_uniform_tree_expectations(n, q):
    """E[max depth] and E[accepted path length] over uniform recursive trees
    with n nodes, each non-root node accepted-if-parent-accepted w.p. q."""
    trees = list(itertools.product(*[range(i) for i in range(1, n)]))
    e_depth = 0.0
    e_len = 0.0
    for ch in trees:
        parent = [-1] + list(ch)
        dep = _depths(parent)
        e_depth += max(dep)
        # enumerate Bernoulli outcomes of the n-1 edge tests
        for bits in itertools.product((0, 1), repeat=n - 1):
            pr = 1.0
            for b in bits:
                pr *= q if b else (1 - q)
            acc = [True] + [False] * (n - 1)
            for i in range(1, n):
                acc[i] = acc[parent[i]] and bits[i - 1] == 1
            e_len += pr * (max(dep[i] for i in range(n) if acc[i]) + 1)
    return e_depth / len(trees), e_len / len(trees)


def test_tiny_recipe_against_exact_expectations():
    cfg = synth.get("tiny")
    q = cfg.p_accept + (1 - cfg.p_accept) / cfg.vocab
    e_depth, e_len = _exact_uniform_tree_expectations(cfg.nodes, q)
    rng = np.random.default_rng(0)
    depths, lens = [], []
    runs = 4000
    for r in range(runs):
        seed = synth.run_seed(cfg, r)
        parent = synth.tree_parents(cfg, seed)
        am = rng.integers(0, cfg.vocab, cfg.nodes)
        tok = synth.plant_tokens(cfg, parent, am, seed)
        path, _ = oracle.accept_path(parent, tok, am)
        depths.append(max(_depths(list(parent))))
        lens.append(len(path))
    depths, lens = np.array(depths, float), np.array(lens, float)
    assert abs(depths.mean() - e_depth) < 4 * depths.std() / np.sqrt(runs)
    assert abs(lens.mean() - e_len) < 4 * lens.std() / np.sqrt(runs)


def test_constrained_recipe_matches_rejection_sampler():
    # the eligible-uniform choice equals drawing uniform earlier nodes and
    # rejecting full / too-deep ones (independent sampler, own randomness)
    cfg = synth.get("layer27b")
    rng = np.random.default_rng(1)

    def rejection_tree():
        parent, depth, kids = [-1], [0], [0]
        for i in range(1, cfg.nodes):
            while True:
                p = int(rng.integers(i))
                if kids[p] < cfg.max_children and depth[p] < cfg.max_depth:
                    break
            parent.append(p); depth.append(depth[p] + 1); kids.append(0); kids[p] += 1
        return max(depth), sum(1 for k in kids if k == 0)

    a = np.array([rejection_tree() for _ in range(3000)], float)
    b = []
    for r in range(3000):
        p = synth.tree_parents(cfg, synth.run_seed(cfg, r))
        dep = _depths(list(p))
        kids = np.bincount(p[1:], minlength=cfg.nodes)
        b.append((max(dep), int((kids == 0).sum())))
    b = np.array(b, float)
    for c in range(2):
        se = np.sqrt(a[:, c].var() / len(a) + b[:, c].var() / len(b))
        assert abs(a[:, c].mean() - b[:, c].mean()) < 4.5 * se


def test_planting_extremes():
    cfg = synth.get("layer27b")
    parent = synth.tree_parents(cfg)
    am = np.arange(cfg.nodes) * 7 + 3
    # p = 1: every draft equals the parent's greedy token, so the deepest node wins
    tok = synth.plant_tokens(cfg, parent, am, p_accept=1.0)
    path, committed = oracle.accept_path(parent, tok, am)
    dep = _depths(list(parent))
    deepest = min(i for i in range(cfg.nodes) if dep[i] == max(dep))
    assert path[-1] == deepest and len(path) == max(dep) + 1
    assert committed[-1] == am[deepest]
    # p = 0 with a 151936-token vocabulary: (almost surely) nothing accepted
    tok = synth.plant_tokens(cfg, parent, am, p_accept=0.0)
    path, committed = oracle.accept_path(parent, tok, am)
    assert path == [0] and committed == [int(am[0])]
