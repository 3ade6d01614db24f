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
    # layer after layer until budget_s of oracle time; a stack that is done
    # sooner starts over from its first layer
    while dt < budget_s:
        l = layers % cfg.layers
        lw = workload.layer_weights(cfg, l)
        kp, vp = synth.kv_prefix(cfg, l)
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
            "sample": "%d layer passes over the %d layers of the %s step (%d-token prefix, %d-node tree), "
                      "run in sequence; GB/s over those layers' algorithmic bytes" % (
                          layers, cfg.layers, cfg.name, cfg.prefix, cfg.nodes)}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "tree_attention_stack27b_traffic.txt")
TRAFFIC_WORKLOAD = "stack27b"  # the workload those counters were taken on
ATTN_SOURCE = os.path.join(ROOT, "tree_verify_amd", "csrc", "attention.hip")


def measured_traffic(workload):
    """HBM bytes per launch of the tree attention from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None for another workload than the
    one the counters were taken on, or when the kernel source changed since."""
    import hashlib
    if workload != TRAFFIC_WORKLOAD:
        return None
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


def percentiles(ms):
    import numpy as np
    a = np.asarray(ms, np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 5), "p50": round(float(np.percentile(a, 50)), 5),
            "p90": round(float(np.percentile(a, 90)), 5)}


def timed_replays(graph, steps, stream=None, flush=None):
    """Replays of one graph, each between two HIP events on the stream it runs
    on; with `flush`, a write of the whole flush buffer (outside the events)
    before every replay, so no cache holds the step's bytes."""
    import torch
    st = stream or torch.cuda.current_stream()
    ms = []
    with torch.cuda.stream(st):
        evs = []
        for i in range(steps):
            if flush is not None:
                flush.fill_(i & 0x7F)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            graph.replay()
            e1.record(st)
            evs.append((e0, e1))
        st.synchronize()
        ms = [a.elapsed_time(b) for a, b in evs]
    return ms


def graph_of(stream, fn, reps):
    """A graph of `reps` calls fn(i) captured on `stream` (after three eager
    calls), replayed once untimed; returns the graph."""
    import torch
    with torch.cuda.stream(stream):
        for i in range(3):
            fn(i)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(reps):
                fn(i)
        g.replay()
    torch.cuda.synchronize()
    return g


def time_graph(stream, g, reps):
    """Per-call time of a graph of reps calls: HIP events around one replay on
    the stream the calls were launched on."""
    import torch
    with torch.cuda.stream(stream):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        g.replay()
        a1.record(stream)
    torch.cuda.synchronize()
    return a0.elapsed_time(a1) / reps * 1e3  # us


def kvq_leg(r, cfg, tv, shape, tree, q, out, dev, reps, bf16_us, bits, layers=4):
    """The one-layer tree attention over a quantised block-32 prefix (int8
    codes, or 4-bit nibbles two to a byte): the first `layers` layers'
    caches quantised on the device (set-up, not timed), then
    lucev_tree_attention_q8 / _q4 from a graph rotating over them, beside the
    same call over the bf16 caches (lucev_tree_attention)."""
    import torch
    Hkv, d, P, cap = cfg.n_kv_heads, cfg.head_dim, cfg.prefix, r.capacity
    if cap % 32:
        return None
    L = min(layers, cfg.layers)
    if bits == 8:
        quant, make, attn, variant = tv.lucev_kv_quantize_q8, tv.make_kv_q8, tv.lucev_tree_attention_q8, tv.ATTN_Q8
        kdt, per = torch.int8, 1
    else:
        quant, make, attn, variant = tv.lucev_kv_quantize_q4, tv.make_kv_q4, tv.lucev_tree_attention_q4, tv.ATTN_Q4
        kdt, per = torch.uint8, 2
    caches = []
    st = torch.cuda.current_stream().cuda_stream
    for l in range(L):
        kc = torch.empty(Hkv, cap, d // per, dtype=kdt, device=dev)
        ks = torch.empty(Hkv, cap, d // 32, dtype=torch.int16, device=dev)
        vc = torch.empty(Hkv, d, cap // per, dtype=kdt, device=dev)
        vs = torch.empty(Hkv, d, cap // 32, dtype=torch.int16, device=dev)
        quant(shape, r.kv(l, P), kc, ks, vc, vs, st)
        caches.append((kc, ks, vc, vs))
    torch.cuda.synchronize()
    kvs = [make(kc, ks, vc, vs, P, cap) for kc, ks, vc, vs in caches]
    stream = torch.cuda.Stream()
    g = graph_of(stream, lambda i: attn(shape, tree, kvs[i % L], q, r.k_tree[0], r.v_tree[0],
                                        out, r.ws, r.ws_bytes, stream.cuda_stream), reps)
    us = time_graph(stream, g, reps)
    del g, caches
    n, Hq = cfg.nodes, cfg.n_q_heads
    kv_bytes = P * Hkv * d * 2 * (bits / 8 + 2 / 32)
    tot = kv_bytes + 2 * n * Hq * d * 2 + 2 * n * Hkv * d * 2
    name = "int8" if bits == 8 else "4-bit"
    return {"avg_launch_us": round(us, 3), "gbs": round(tot / (us * 1e-6) / 1e9, 2),
            "prefix_bytes": int(kv_bytes), "prefix_bytes_bf16": P * Hkv * d * 4,
            "vs_bf16_time": round(bf16_us / us, 4), "kernel": tv.lucev_describe_attention(shape, n, P, variant),
            "what": "lucev_tree_attention_q%d (bf16 q, %s block-32 prefix with fp16 scales), rotating over %d "
                    "layers' quantised caches; vs_bf16_time = lucev_tree_attention time / this" % (bits, name, L)}


def stream_ceiling(cfg, tv, dev, reps=10):
    """A bare non-temporal read (lucev_stream_read) of each kernel's
    algorithmic bytes, from a graph rotating over disjoint regions of a 4 GiB
    buffer: the rate a kernel moving that many bytes can reach here."""
    import torch
    H, F, Hq, Hkv, d, V = cfg.hidden, cfg.ffn, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.vocab
    wb = lambda n_out, k_in: n_out * k_in * 18 // 32
    sizes = {"attention": attention_bytes(cfg, cfg.nodes), "qkv": wb((Hq + 2 * Hkv) * d, H),
             "wo": wb(H, Hq * d), "gate_up": wb(2 * F, H), "down": wb(H, F), "lm_head": wb(V, H)}
    region = 1 << 30
    buf = torch.empty(4 * region, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    out = {}
    stream = torch.cuda.Stream()
    for k, nb in sizes.items():
        nb = min(nb, region) // 16 * 16
        g = graph_of(stream, lambda i: tv.lucev_stream_read(buf.data_ptr() + (i % 4) * region, nb, sink,
                                                            stream.cuda_stream), reps)
        us = time_graph(stream, g, reps)
        del g
        out[k] = {"bytes": nb, "us": round(us, 3), "gbs": round(nb / (us * 1e-6) / 1e9, 1)}
    per_layer = sum(out[k]["us"] for k in ("attention", "qkv", "wo", "gate_up", "down"))
    out["step_ms_if_bare_reads"] = round((cfg.layers * per_layer + out["lm_head"]["us"]) / 1e3, 4)
    del buf
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def crossover(args):
    """MFMA against the VALU dot-product GEMM path at small trees: an 8-layer
    27B-shape stack (4096-token prefix) plus head at n = 1, 2, 4, 8 nodes, with
    lucev_set_gemv_max_rows 0 (MFMA only) and 8 (dot products up to 8 operand
    rows), each step replayed from a graph and timed with HIP events."""
    import torch
    import synth
    import synth.device as sd
    import tree_verify_amd as tv
    from tree_verify_amd.runner import VerifyRunner
    dev = torch.device("cuda:0")
    base = synth.get("stack27b").replace(layers=8, prefix=4096, name="stack27b_8l_p4096")
    out = {}
    for n in (1, 2, 4, 8):
        cfg = base.replace(nodes=n, max_children=None, max_depth=None)
        wl = sd.Workload(cfg, device=dev)
        shape = tv.make_shape(cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.vocab)
        tree = tv.make_tree(synth.tree_parents(cfg), [0] * n)
        x = wl.x_in_f32().contiguous()
        for rows in (0, 8):
            tv.lucev_set_gemv_max_rows(rows)
            r = VerifyRunner(shape, wl.layers, wl.head, n, wl.capacity, dev, keep_logits=False)
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                r.step(tree, x, cfg.prefix, with_logits=False)
                st.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=st):
                    r.step(tree, x, cfg.prefix, with_logits=False)
            torch.cuda.synchronize()
            for _ in range(3):
                g.replay()
            ms = percentiles(timed_replays(g, args.steps))
            out.setdefault("n%d" % n, {})["mfma" if rows == 0 else "valu_up_to_8_rows"] = ms
            log("crossover n %d gemv rows %d: p50 %.4f ms" % (n, rows, ms["p50"]))
            del g, r
        tv.lucev_set_gemv_max_rows(0)
        del wl
        torch.cuda.empty_cache()
    return {"crossover": out, "workload": base.name,
            "what": "step ms (p10/p50/p90 over %d replays) with the int4 GEMMs on MFMA vs on VALU dot products "
                    "wherever the operand rows (2 per node for QKV/Wo/lm_head, 1 for gate/up and down) are <= 8"
                    % args.steps}


CONFIGS_ALL = ["tiny", "small_decode", "small_tree", "layer27b", "stack27b", "longctx27b"]


def quantised_step_leg(r, tree, x32, cfg, stream, steps, bits, wb, ob):
    """The whole step over int8 (bits 8) or 4-bit (bits 4) block-32 KV caches
    (lucev_verify_layer_q8 / _q4): every layer's cache quantised on the device
    (set-up, not timed), the step captured as a graph and replayed like the
    main one.  GB/s over the step's algorithmic bytes with the quantised
    prefix (codes + one fp16 scale per 32 values)."""
    import torch
    r.quantise_kv(bits, cfg.prefix)
    torch.cuda.synchronize()
    try:
        with torch.cuda.stream(stream):
            r.step(tree, x32, cfg.prefix, with_logits=False)
            stream.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                r.step(tree, x32, cfg.prefix, with_logits=False)
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        ms = timed_replays(g, steps, stream)
        del g
    finally:
        r.clear_quantised_kv()
        torch.cuda.synchronize()
    kvb = int(cfg.layers * cfg.prefix * cfg.n_kv_heads * cfg.head_dim * 2 * (bits / 8 + 2 / 32))
    p = percentiles(ms)
    mean = sum(ms) / len(ms)
    return {"ms_per_step": round(mean, 5), "warm_ms": p, "algorithmic_bytes": wb + kvb + ob, "kv_bytes": kvb,
            "gbs": round((wb + kvb + ob) / (mean * 1e-3) / 1e9, 2),
            "what": "the step (lucev_verify_layer_q%d every layer + acceptance) over %s block-32 KV caches; "
                    "mean and p10/p50/p90 of %d replays, each between its own HIP events"
                    % (bits, "int8" if bits == 8 else "4-bit", steps)}


def run_config(cfg, args):
    import numpy as np
    import torch
    import synth
    import synth.device as sd
    import tree_verify_amd as tv
    from tree_verify_amd.runner import VerifyRunner

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
    # warm: back-to-back replays, the K timed ones between one pair of events
    # (the contract's figure) and each also between its own pair
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
    warm = timed_replays(graph, args.steps)
    # cold: a 1 GiB write before each replay evicts L2 and the 256 MB
    # last-level cache, so every byte of the step comes from HBM
    flush = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev)
    cold = timed_replays(graph, args.cold_steps, flush=flush)
    del flush
    path = r.path.cpu().numpy()[: int(r.path_len.item())].tolist()
    wb, kvb, ob = algorithmic_bytes(cfg, cfg.nodes)
    total = wb + kvb + ob
    gbs = total / (ms * 1e-3) / 1e9
    cold_p = percentiles(cold)
    log("%s: step %.4f ms (warm p50 %.4f, cold p50 %.4f), %.1f GB/s, path %s" %
        (cfg.name, ms, percentiles(warm)["p50"], cold_p["p50"], gbs, path))

    # dominant kernel by bytes: the step's own tree attention (fp32 q split
    # into bf16 hi + lo, partial + combine) of one layer, launched through
    # lucev_tree_attention_f32 from a graph on its own stream, rotating over
    # the layers' caches; HIP events on that stream
    Hq, Hkv, d, n = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.nodes
    rng = np.random.default_rng(cfg.seed)
    q32 = torch.from_numpy(rng.standard_normal((n, Hq, d)).astype(np.float32)).to(dev)
    k32 = torch.from_numpy(rng.standard_normal((n, Hkv, d)).astype(np.float32)).to(dev)
    v32 = torch.from_numpy(rng.standard_normal((n, Hkv, d)).astype(np.float32)).to(dev)
    o32 = torch.zeros(n, Hq, d, dtype=torch.float32, device=dev)
    q = sd.flat_table("normal", synth.stream_key(cfg.seed, 90, 0), n * Hq * d, dev)
    out = torch.zeros(n * Hq * d, dtype=torch.int16, device=dev)
    torch.cuda.synchronize()
    astream = torch.cuda.Stream()
    ag = graph_of(astream, lambda i: tv.lucev_tree_attention_f32(shape, tree, r.kv(i % cfg.layers, cfg.prefix), q32,
                                                                k32, v32, o32, r.ws, r.ws_bytes,
                                                                astream.cuda_stream), args.attn_reps)
    attn_us = time_graph(astream, ag, args.attn_reps)
    del ag
    bg = graph_of(astream, lambda i: tv.lucev_tree_attention(shape, tree, r.kv(i % cfg.layers, cfg.prefix), q,
                                                            r.k_tree[0], r.v_tree[0], out, r.ws, r.ws_bytes,
                                                            astream.cuda_stream), args.attn_reps)
    bf16_us = time_graph(astream, bg, args.attn_reps)
    del bg
    ab = attention_bytes(cfg, n)
    attn_gbs = ab / (attn_us * 1e-6) / 1e9
    log("tree attention (one layer, step variant): %.2f us, %.1f GB/s; bf16-q API %.2f us" %
        (attn_us, attn_gbs, bf16_us))
    paged_us = paged_leg(r, cfg, tv, shape, tree, q, out, dev, args.attn_reps) if cfg.prefix > 0 else None
    if paged_us:
        log("paged tree attention (one layer): %.2f us" % paged_us)
    qstep = {}
    if cfg.prefix > 0 and not args.no_q8 and r.capacity % 32 == 0:
        for bits in (8, 4):
            qstep[bits] = quantised_step_leg(r, tree, x32, cfg, stream, args.steps, bits, wb, ob)
            log("step over %s KV: %.4f ms (p50 %.4f), %.1f GB/s" %
                ("int8" if bits == 8 else "4-bit", qstep[bits]["ms_per_step"], qstep[bits]["warm_ms"]["p50"],
                 qstep[bits]["gbs"]))
    q8 = q4 = None
    if cfg.prefix > 0 and not args.no_q8:
        q8 = kvq_leg(r, cfg, tv, shape, tree, q, out, dev, args.attn_reps, bf16_us, 8)
        q4 = kvq_leg(r, cfg, tv, shape, tree, q, out, dev, args.attn_reps, bf16_us, 4)
        for nm, x in (("int8", q8), ("4-bit", q4)):
            if x:
                log("%s-prefix tree attention (one layer): %.2f us (%.3fx the bf16 prefix's speed)" %
                    (nm, x["avg_launch_us"], x["vs_bf16_time"]))

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
        "warm_ms": percentiles(warm),
        "cold_ms": dict(cold_p, steps=args.cold_steps, gbs_p50=round(total / (cold_p["p50"] * 1e-3) / 1e9, 2),
                        what="each replay after a %d MiB write outside its events" % args.flush_mib),
        "roofline": {"bound": "hbm", "kernel": tv.lucev_describe_attention(shape, n, cfg.prefix, tv.ATTN_F32),
                     "achieved": round(attn_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(cfg.name),
                     "bytes_per_launch": ab, "avg_launch_us": round(attn_us, 3),
                     "timed": "lucev_tree_attention_f32 (the verify step's variant), a graph of %d launches "
                              "rotating over the layers' caches, HIP events on the launch stream" % args.attn_reps},
        "step_roofline_frac": round(gbs / HBM_PEAK_GBS, 4),
        "attention_bf16q_us": round(bf16_us, 3),
    }
    if paged_us:
        line["paged_attention"] = {"avg_launch_us": round(paged_us, 3),
                                   "gbs": round(ab / (paged_us * 1e-6) / 1e9, 2),
                                   "vs_contiguous": round(bf16_us / paged_us, 4),
                                   "what": "lucev_tree_attention_paged (bf16 q), the prefix in a shuffled pool of "
                                           "16-token pages, rotating over 4 layers' pools; vs_contiguous = "
                                           "lucev_tree_attention time / this"}
    if qstep:
        line["step_q8_kv"] = qstep.get(8)
        line["step_q4_kv"] = qstep.get(4)
    if q8:
        line["q8_attention"] = q8
    if q4:
        line["q4_attention"] = q4
    if args.chain > 0:
        del graph
        line["chained"] = chained(r, cfg, tv, args.chain, dev)
        log("chained: %s" % json.dumps(line["chained"]))
    del wl, r
    torch.cuda.empty_cache()
    if not args.no_ceiling:
        sc = stream_ceiling(cfg, tv, dev)
        line["stream_ceiling"] = sc
        line["step_vs_bare_reads"] = round(sc["step_ms_if_bare_reads"] / ms, 4)
    if not args.no_cpu_baseline:
        torch.cuda.empty_cache()
        cb = cpu_baseline(cfg)
        cb["cpu_model"] = cpu_model()
        line["cpu_baseline"] = cb
    return line


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="stack27b", help="a config name, or 'all' (one JSON line each)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-q8", action="store_true",
                    help="skip the quantised-prefix (int8 and 4-bit) legs: one-layer attention and whole step")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--attn-reps", type=int, default=20)
    ap.add_argument("--cold-steps", type=int, default=10)
    ap.add_argument("--flush-mib", type=int, default=1024)
    ap.add_argument("--chain", type=int, default=8,
                    help="verify+commit steps of the chained leg (0: skip)")
    ap.add_argument("--crossover", action="store_true",
                    help="only compare the MFMA and VALU GEMM paths at 1, 2, 4, 8 nodes")
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
    if args.crossover:
        print(json.dumps(crossover(args)), flush=True)
        return
    import synth
    names = CONFIGS_ALL if args.config == "all" else [args.config]
    for name in names:
        print(json.dumps(run_config(synth.get(name), args)), flush=True)


if __name__ == "__main__":
    main()
