"""GPU parity at the full workload sizes against stored oracle outputs.

The fixtures under tests/golden/ were written by tests/golden/make_golden.py,
which calls only the seeded generator and the fp64 oracle.  The GPU rebuilds
the same inputs with the device twin of the generator, runs one verify step
exactly as bench.py does (captured graph replay), and is compared on:
greedy tokens where the oracle's top1-top2 gap exceeds 0.05, the accepted
path and committed tokens whenever every accepted node is that decisive, and
sampled logits / final hidden states (per-row max error over the sampled
columns divided by the row's max |value|, bound 2e-2).
"""
import json
import os
import sys

import numpy as np
import pytest

import synth
from gpu_common import bf16_bits_to_f64, decisive_compare, need_gpu

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
TOL = 2e-2


def _cases():
    out = []
    for name in ("layer27b", "longctx27b", "stack27b"):
        path = os.path.join(HERE, "golden", "%s.json" % name)
        if not os.path.exists(path):
            continue
        with open(path) as fh:
            data = json.load(fh)
        for run in data["runs"]:
            out.append((name, run["seed"]))
    return out


def _golden(name, seed):
    with open(os.path.join(HERE, "golden", "%s.json" % name)) as fh:
        data = json.load(fh)
    return [r for r in data["runs"] if r["seed"] == seed][0]


@pytest.mark.parametrize("name,seed", _cases())
def test_full_size_against_oracle_fixture(name, seed):
    torch = need_gpu()
    import tree_verify_amd as tv
    from tree_verify_amd.runner import VerifyRunner
    import synth.device as sd
    g = _golden(name, seed)
    cfg = synth.get(name)
    print("full-size case", name, "seed", seed, flush=True)
    wl = sd.Workload(cfg, seed, "cuda")
    shape = tv.make_shape(cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn,
                          cfg.vocab, cfg.rms_eps, cfg.rope_base)
    r = VerifyRunner(shape, wl.layers, wl.head, cfg.nodes, wl.capacity, "cuda")
    tree = tv.make_tree(g["parent"], g["tokens"])
    x32 = wl.x_in_f32().contiguous()
    torch.cuda.synchronize()  # x32 was made on the default stream
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        r.step(tree, x32, cfg.prefix)
        stream.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            r.step(tree, x32, cfg.prefix)
    torch.cuda.synchronize()
    outs = []
    for rep in range(2):  # replays must agree bit for bit with each other
        graph.replay()
        torch.cuda.synchronize()
        outs.append((r.argmax.cpu().numpy().copy(), r.logits.cpu().numpy().copy(),
                     r.resid.cpu().numpy().copy(), r.path.cpu().numpy().copy(),
                     int(r.path_len.item()), r.committed.cpu().numpy().copy(), r.gap.cpu().numpy().copy()))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(np.asarray(a), np.asarray(b)), "graph replays differ"
    am, logits_bits, resid, path, plen, committed, gap = outs[0]
    n = cfg.nodes
    oam = np.array(g["argmax"])
    ogap = np.array(g["gap"])
    ndec, decided = decisive_compare(g["parent"], g["tokens"], oam, ogap, am[:n], path[:n], plen,
                                     committed[:n])
    logits = bf16_bits_to_f64(torch.from_numpy(logits_bits[:n]))
    cols = np.array(g["logit_cols"])
    err_l = np.max(np.abs(logits[:, cols] - np.array(g["logits"])), axis=1) / np.array(g["logit_rowmax"])
    hcols = np.array(g["hidden_cols"])
    err_h = np.max(np.abs(resid[:n, hcols] - np.array(g["hidden"])), axis=1) / np.array(g["hidden_rowmax"])
    # top-8 ids per node: the GPU's fp32 ranking of the oracle's top entries
    print("  decisive %d/%d, path decided %s, logits err %.2e, final hidden err %.2e" %
          (ndec, n, decided, err_l.max(), err_h.max()), flush=True)
    dec = ogap > 0.05
    assert np.allclose(gap[:n][dec], ogap[dec], rtol=0.05, atol=0.05)
    assert err_l.max() < TOL, err_l
    assert err_h.max() < TOL, err_h
