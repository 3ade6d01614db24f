"""Write oracle outputs for the full-size workloads (test fixtures).

Calls only the seeded generator (``synth``) and the fp64 oracle (``oracle``)
through ``tests/workload.py``.  For each run it stores the tree, the planted
tokens, every node's greedy token and top1-top2 gap, the accepted path and
committed tokens, each node's eight largest logits (ids and values), and
samples of the logits, of the final hidden states and of the hidden states
after layers 0, 1, L/2 and L-1 (fixed columns plus each row's max |value|, so
a per-row relative error can be bounded on the sampled columns).

    python tests/golden/make_golden.py layer27b 0 1
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import synth  # noqa: E402
import workload  # noqa: E402

N_COLS = 256
N_LAYER_COLS = 128


def sample_cols(n, seed, k=N_COLS):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n, size=min(k, n), replace=False)).astype(np.int64)


def sampled_layers(n_layers):
    return sorted({0, min(1, n_layers - 1), n_layers // 2, n_layers - 1})


def _f(a):
    """Floats written with 10 significant digits (the tolerance is 2e-2)."""
    return [[float("%.10g" % v) for v in row] for row in np.asarray(a)]


def one_run(cfg, run):
    seed = synth.run_seed(cfg, run)
    t0 = time.time()
    out = workload.planted_case(cfg, seed, keep_hidden=True)
    dt = time.time() - t0
    lc = sample_cols(cfg.vocab, seed + 1)
    hc = sample_cols(cfg.hidden, seed + 2)
    lcols = sample_cols(cfg.hidden, seed + 3, N_LAYER_COLS)
    logits, x = out["logits"], out["x"]
    top = np.argsort(-logits, axis=1, kind="stable")[:, :8]
    layer_samples = []
    for l in sampled_layers(cfg.layers):
        h = out["hidden"][l]
        layer_samples.append({"layer": l, "values": _f(h[:, lcols]),
                              "rowmax": [float(v) for v in np.max(np.abs(h), axis=1)]})
    return {
        "seed": seed,
        "oracle_seconds": round(dt, 1),
        "parent": [int(v) for v in out["parent"]],
        "tokens": [int(v) for v in out["tokens"]],
        "argmax": [int(v) for v in out["argmax"]],
        "gap": [float(v) for v in out["gap"]],
        "path": [int(v) for v in out["path"]],
        "committed": [int(v) for v in out["committed"]],
        "logit_cols": lc.tolist(),
        "logits": _f(logits[:, lc]),
        "logit_rowmax": np.max(np.abs(logits), axis=1).tolist(),
        "logit_top_idx": top.tolist(),
        "logit_top_val": _f(np.take_along_axis(logits, top, axis=1)),
        "hidden_cols": hc.tolist(),
        "hidden": _f(x[:, hc]),
        "hidden_rowmax": np.max(np.abs(x), axis=1).tolist(),
        "layer_cols": lcols.tolist(),
        "layer_hidden": layer_samples,
    }


def main():
    name = sys.argv[1]
    runs = [int(r) for r in sys.argv[2:]] or [0]
    cfg = synth.get(name)
    path = os.path.join(HERE, "%s.json" % name)
    data = {"about": "fp64 oracle outputs for workload %s, written by tests/golden/make_golden.py "
                     "(synth + oracle only)" % name, "config": name, "runs": []}
    for r in runs:
        res = one_run(cfg, r)
        # re-read: another writer may have added runs meanwhile
        if os.path.exists(path):
            with open(path) as fh:
                data = json.load(fh)
        data["runs"] = [x for x in data["runs"] if x["seed"] != res["seed"]]
        data["runs"].append(res)
        data["runs"].sort(key=lambda x: x["seed"])
        with open(path + ".tmp", "w") as fh:
            json.dump(data, fh)
        os.replace(path + ".tmp", path)
        print("%s run %d seed %d: %.1f s, path %s" % (name, r, res["seed"], res["oracle_seconds"], res["path"]),
              flush=True)


if __name__ == "__main__":
    main()
