"""Verify-step benchmark: latency, HBM GB/s and roofline fraction on one GPU.

A step is one pass of the whole hot path over one draft tree: every layer's
lucev_verify_layer, then lucev_accept_path (final norm, lm_head, greedy
tokens, acceptance walk), replayed from one captured HIP graph with all
inputs resident in HBM.  Prints one JSON line (rank 0).

    python bench.py [--steps K] [--warmup W] [--config stack27b] [--gpus 1]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify-step latency (ms) & HBM GB/s, 27B-class int4 stack, tree budget 22"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(cfg, nodes):
    """Bytes the method must move per step: packed int4 weights once (18 B per
    32 weights), the bf16 KV prefix once, norm gains, tree K/V writes, the
    input / residual rows and the per-node outputs."""
    H, Hkv, d = cfg.hidden, cfg.n_kv_heads, cfg.head_dim
    w = (cfg.layers * cfg.layer_weight_count() + cfg.head_weight_count()) * 18 // 32
    kv = cfg.layers * cfg.prefix * Hkv * d * 2 * 2
    other = cfg.layers * (2 * H * 2 + 2 * nodes * Hkv * d * 2) + H * 2 + nodes * H * 4 * 2
    return w, kv, other


def attention_bytes(cfg, nodes):
    Hq, Hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    return (cfg.prefix * Hkv * d * 2 * 2 + 2 * nodes * Hq * d * 2 + 2 * nodes * Hkv * d * 2)


def tokens_for(cfg, parent):
    """Planted drafted tokens from the oracle's stored greedy tokens when the
    golden file for this config exists, else uniform tokens (tokens only feed
    the acceptance walk, which is the same work either way)."""
    import numpy as np
    import synth
    gpath = os.path.join(ROOT, "tests", "golden", "%s.json" % cfg.name)
    if os.path.exists(gpath):
        with open(gpath) as fh:
            g = json.load(fh)
        runs = [r for r in g["runs"] if r["seed"] == cfg.seed]
        if runs:
            return np.array(runs[0]["tokens"], np.int32), "planted from the oracle's greedy tokens"
    rng = np.random.default_rng(cfg.seed)
    return rng.integers(0, cfg.vocab, len(parent)).astype(np.int32), "uniform random"


def cpu_baseline(cfg, budget_s=10.0):
    """The fp64 oracle, as it stands, on a bounded sample of the workload:
    whole layers of the step (full KV prefix, the same tree), layer after
    layer until about budget_s seconds of oracle time; input generation is not
    timed."""
    import numpy as np
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    import synth
    import workload
    parent = synth.tree_parents(cfg)
    shp = workload.shape(cfg)
    x = oracle.bf16_to_f64(synth.hidden_in(cfg))
    dt, layers = 0.0, 0
    while layers < cfg.layers and dt < budget_s:
        lw = workload.layer_weights(cfg, layers)
        kp, vp = synth.kv_prefix(cfg, layers)
        t0 = time.perf_counter()
        x = oracle.layer_forward(x, lw, kp, vp, parent, shp)[0]  # (residual, tree K, tree V)
        dt += time.perf_counter() - t0
        layers += 1
    layer_bytes = cfg.layer_weight_count() * 18 // 32 + cfg.prefix * cfg.n_kv_heads * cfg.head_dim * 4
    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:
        threads = os.cpu_count()
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] + [1])
    except Exception:
        pass
    return {"value": round(layers * layer_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": "the first %d of the %d layers of the %s step (%d-token prefix, %d-node tree), "
                      "run in sequence; GB/s over those layers' algorithmic bytes" % (
                          layers, cfg.layers, cfg.name, cfg.prefix, cfg.nodes)}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "tree_attention_stack27b_traffic.txt")
ATTN_SOURCE = os.path.join(ROOT, "tree_verify_amd", "csrc", "attention.hip")


def measured_traffic():
    """HBM bytes per launch of the tree attention from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None when the kernel source changed
    since those counters were taken."""
    import hashlib
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    with open(ATTN_SOURCE, "rb") as fh:
        digest = hashlib.sha256(fh.read()).hexdigest()
    if fields.get("source_sha256") != digest or "hbm_bytes_per_launch" not in fields:
        return None
    return int(float(fields["hbm_bytes_per_launch"]))


def copy_calibration(nbytes):
    """One device-to-device copy of nbytes: the reference kernel for scaling
    the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    dev = torch.device("cuda:0")
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    a.fill_(1)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes}), flush=True)


def chained(r, cfg, tv, steps, dev):
    """k successive verify steps, each committing its accepted path: step s
    takes a new tree and new synthetic inputs at prefix P + (tokens committed
    so far).  The drafts are planted from the target's own greedy tokens
    (probability p, as in the single-step workload) by an untimed first pass;
    the timed pass is verify + acceptance + commit, captured as one graph and
    replayed once under HIP events.  Stops early when the cache has no room
    for another tree."""
    import numpy as np
    import torch
    import synth
    prefix, tokens_total, ms_total, done, lens = cfg.prefix, 0, 0.0, 0, []
    stream = torch.cuda.Stream()
    for s in range(steps):
        if prefix + cfg.nodes > r.capacity:
            break
        seed = cfg.seed + 7000 + s
        parent = synth.tree_parents(cfg, seed)
        x = torch.from_numpy(((synth.hidden_in(cfg, seed).astype(np.uint32) << 16)
                              .view(np.float32))).to(dev)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            r.step(tv.make_tree(parent, [0] * cfg.nodes), x, prefix, with_logits=False)
            stream.synchronize()
            am = r.argmax[:cfg.nodes].cpu().numpy()
            tree = tv.make_tree(parent, synth.plant_tokens(cfg, parent, am, seed))
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                r.step(tree, x, prefix, with_logits=False)
                r.commit(cfg.nodes, prefix)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            stream.synchronize()
        n_acc = int(r.path_len.item())
        ms_total += e0.elapsed_time(e1)
        tokens_total += n_acc
        lens.append(n_acc)
        prefix += n_acc
        done += 1
    return {"steps": done, "committed_tokens": tokens_total, "path_lengths": lens,
            "tokens_per_step": round(tokens_total / max(done, 1), 3),
            "ms_per_step": round(ms_total / max(done, 1), 4),
            "tokens_per_s": round(tokens_total / (ms_total * 1e-3), 1) if ms_total else None,
            "what": "verify + acceptance + commit per step (one graph each), new tree and synthetic "
                    "inputs each step, drafts planted from the target's greedy tokens with p=%.1f; "
                    "committed = accepted drafts + the bonus token" % cfg.p_accept}


def paged_leg(r, cfg, tv, shape, tree, q, out, dev, reps, layers=4):
    """The same one-layer tree attention over a paged prefix: the first
    `layers` layers' caches re-laid into a shuffled pool of 16-token pages
    (set-up, not timed), launches rotating over them so the last-level cache
    does not serve repeats, replayed from a graph and timed with HIP events
    on the launch stream."""
    import numpy as np
    import torch
    Hkv, d, P = cfg.n_kv_heads, cfg.head_dim, cfg.prefix
    NL = (P + 15) // 16
    L = min(layers, cfg.layers)
    pools = []
    for l in range(L):
        k, v = r.layers[l]["k"], r.layers[l]["v"]
        perm = torch.from_numpy(np.random.default_rng(cfg.seed + l).permutation(NL).astype(np.int64)).to(dev)
        kp = torch.empty(NL, Hkv, 16, d, dtype=torch.int16, device=dev)
        vp = torch.empty(NL, Hkv, d, 16, dtype=torch.int16, device=dev)
        kp[perm] = k[:, :NL * 16, :].reshape(Hkv, NL, 16, d).permute(1, 0, 2, 3)
        vp[perm] = v[:, :, :NL * 16].reshape(Hkv, d, NL, 16).permute(2, 0, 1, 3)
        pools.append((kp, vp, perm.to(torch.int32).contiguous()))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        st = stream.cuda_stream
        kvs = [tv.make_kv_paged(kp, vp, tab, NL, P) for kp, vp, tab in pools]
        for i in range(3):
            tv.lucev_tree_attention_paged(shape, tree, kvs[i % L], q, r.k_tree[0], r.v_tree[0], out, r.ws,
                                          r.ws_bytes, st)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(reps):
                tv.lucev_tree_attention_paged(shape, tree, kvs[i % L], q, r.k_tree[0], r.v_tree[0], out,
                                              r.ws, r.ws_bytes, stream.cuda_stream)
        g.replay()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        g.replay()
        a1.record(stream)
    torch.cuda.synchronize()
    del g
    us = a0.elapsed_time(a1) / reps * 1e3
    del pools
    return us


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="stack27b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--attn-reps", type=int, default=20)
    ap.add_argument("--chain", type=int, default=8,
                    help="verify+commit steps of the chained leg (0: skip)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run one device copy of this many bytes (counter calibration)")
    args = ap.parse_args()
    if args.copy_bytes:
        copy_calibration(args.copy_bytes)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(got --gpus %d)" % args.gpus, flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    import synth.device as sd
    import tree_verify_amd as tv
    from tree_verify_amd.runner import VerifyRunner

    cfg = synth.get(args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    wl = sd.Workload(cfg, device=dev)
    torch.cuda.synchronize()
    log("workload %s built on device in %.1f s" % (cfg.name, time.time() - t0))
    shape = tv.make_shape(cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn,
                          cfg.vocab, cfg.rms_eps, cfg.rope_base)
    r = VerifyRunner(shape, wl.layers, wl.head, cfg.nodes, wl.capacity, dev, keep_logits=False)
    parent = synth.tree_parents(cfg)
    tokens, tok_src = tokens_for(cfg, parent)
    tree = tv.make_tree(parent, tokens)
    x32 = wl.x_in_f32().contiguous()
    torch.cuda.synchronize()  # inputs were made on the default stream

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        r.step(tree, x32, cfg.prefix, with_logits=False)  # eager warm-up (and module loads)
        stream.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            r.step(tree, x32, cfg.prefix, with_logits=False)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    path = r.path.cpu().numpy()[: int(r.path_len.item())].tolist()
    wb, kvb, ob = algorithmic_bytes(cfg, cfg.nodes)
    total = wb + kvb + ob
    gbs = total / (ms * 1e-3) / 1e9
    log("step %.4f ms, %.1f GB/s (weights %.3f GB, KV %.3f GB, other %.4f GB), path %s" %
        (ms, gbs, wb / 1e9, kvb / 1e9, ob / 1e9, path))

    # dominant kernel by bytes: the tree attention of one layer (prefix split
    # partial kernel + combine), timed alone on its own stream with HIP events
    astream = torch.cuda.Stream()
    Hq, Hkv, d, n = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.nodes
    q = sd.flat_table("normal", synth.stream_key(cfg.seed, 90, 0), n * Hq * d, dev)
    out = torch.zeros(n * Hq * d, dtype=torch.int16, device=dev)
    torch.cuda.synchronize()  # q / out were made on the default stream
    kv0 = r.kv(0, cfg.prefix)
    with torch.cuda.stream(astream):
        st = astream.cuda_stream
        for _ in range(3):
            tv.lucev_tree_attention(shape, tree, kv0, q, r.k_tree[0], r.v_tree[0], out, r.ws,
                                    r.ws_bytes, st)
        # the timed launches are replayed from a graph, so host-side call
        # overhead cannot open gaps between them
        ag = torch.cuda.CUDAGraph()
        with torch.cuda.graph(ag, stream=astream):
            for i in range(args.attn_reps):
                kvi = r.kv(i % cfg.layers, cfg.prefix)
                tv.lucev_tree_attention(shape, tree, kvi, q, r.k_tree[0], r.v_tree[0], out, r.ws,
                                        r.ws_bytes, astream.cuda_stream)
        ag.replay()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(astream)
        ag.replay()
        a1.record(astream)
    torch.cuda.synchronize()
    del ag
    attn_ms = a0.elapsed_time(a1) / args.attn_reps
    ab = attention_bytes(cfg, n)
    attn_gbs = ab / (attn_ms * 1e-3) / 1e9
    log("tree attention (one layer): %.2f us, %.1f GB/s" % (attn_ms * 1e3, attn_gbs))
    paged_us = paged_leg(r, cfg, tv, shape, tree, q, out, dev, args.attn_reps) if cfg.prefix > 0 else None
    if paged_us:
        log("paged tree attention (one layer): %.2f us, %.1f GB/s" % (paged_us, ab / (paged_us * 1e-6) / 1e9))

    line = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int4 weights, f16/bf16 MFMA, f32 accumulate",
        "data": "synthetic (seeded Philox draws with the pages' shapes; random-init weights)",
        "config": {"workload": cfg.name, "layers": cfg.layers, "hidden": cfg.hidden,
                   "heads": "%d/%d" % (cfg.n_q_heads, cfg.n_kv_heads), "head_dim": cfg.head_dim,
                   "ffn": cfg.ffn, "vocab": cfg.vocab, "prefix": cfg.prefix, "tree_nodes": cfg.nodes,
                   "algorithmic_bytes": total, "tokens": tok_src, "accepted_path": path},
        "roofline": {"bound": "hbm", "kernel": "tree attention, one layer (partial + combine)",
                     "achieved": round(attn_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "bytes_per_launch": ab, "avg_launch_us": round(attn_ms * 1e3, 3)},
        "step_roofline_frac": round(gbs / HBM_PEAK_GBS, 4),
    }
    if paged_us:
        line["paged_attention"] = {"avg_launch_us": round(paged_us, 3),
                                   "gbs": round(ab / (paged_us * 1e-6) / 1e9, 2),
                                   "vs_contiguous": round(attn_ms * 1e3 / paged_us, 4),
                                   "what": "lucev_tree_attention_paged, the prefix in a shuffled pool of "
                                           "16-token pages, rotating over 4 layers' pools"}
    if args.chain > 0:
        del graph
        line["chained"] = chained(r, cfg, tv, args.chain, dev)
        log("chained: %s" % json.dumps(line["chained"]))
    if not args.no_cpu_baseline:
        del wl, r
        torch.cuda.empty_cache()
        line["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
