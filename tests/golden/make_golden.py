"""Write oracle outputs for the full-size workloads (test fixtures).

Calls only the seeded generator (``synth``) and the fp64 oracle (``oracle``)
through ``tests/workload.py``.  For each run it stores the tree, the planted
tokens, every node's greedy token and top1-top2 gap, the accepted path and
committed tokens, and samples of the logits and of the final hidden states
(fixed columns plus each row's max |value|, so a per-row relative error can be
bounded on the sampled columns).

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


def sample_cols(n, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n, size=min(N_COLS, n), replace=False)).astype(np.int64)


def one_run(cfg, run):
    seed = synth.run_seed(cfg, run)
    t0 = time.time()
    out = workload.planted_case(cfg, seed, keep_hidden=False)
    dt = time.time() - t0
    lc = sample_cols(cfg.vocab, seed + 1)
    hc = sample_cols(cfg.hidden, seed + 2)
    logits, x = out["logits"], out["x"]
    top = np.argsort(-logits, axis=1, kind="stable")[:, :8]
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
        "logits": logits[:, lc].tolist(),
        "logit_rowmax": np.max(np.abs(logits), axis=1).tolist(),
        "logit_top_idx": top.tolist(),
        "logit_top_val": np.take_along_axis(logits, top, axis=1).tolist(),
        "hidden_cols": hc.tolist(),
        "hidden": x[:, hc].tolist(),
        "hidden_rowmax": np.max(np.abs(x), axis=1).tolist(),
    }


def main():
    name = sys.argv[1]
    runs = [int(r) for r in sys.argv[2:]] or [0]
    cfg = synth.get(name)
    path = os.path.join(HERE, "%s.json" % name)
    data = {"about": "fp64 oracle outputs for workload %s, written by tests/golden/make_golden.py "
                     "(synth + oracle only)" % name, "config": name, "runs": []}
    if os.path.exists(path):
        with open(path) as fh:
            data = json.load(fh)
    for r in runs:
        seed = synth.run_seed(cfg, r)
        data["runs"] = [x for x in data["runs"] if x["seed"] != seed]
        res = one_run(cfg, r)
        data["runs"].append(res)
        data["runs"].sort(key=lambda x: x["seed"])
        with open(path + ".tmp", "w") as fh:
            json.dump(data, fh)
        os.replace(path + ".tmp", path)
        print("%s run %d seed %d: %.1f s, path %s" % (name, r, seed, res["oracle_seconds"], res["path"]),
              flush=True)


if __name__ == "__main__":
    main()
