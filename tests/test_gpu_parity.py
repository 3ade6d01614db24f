"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances (from the arithmetic): logits, hidden states, tree
K/V and attention outputs within a per-row inf-norm relative error of 2e-2;
greedy tokens bit-exact wherever the oracle's top1-top2 gap exceeds 0.05 and
accepted paths bit-exact whenever every accepted node is that decisive.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_common import (Guarded, bf16_bits_to_f64, decisive_compare, guarded_runner_class, need_gpu,
                        row_rel_err)
import workload

pytestmark = pytest.mark.gpu

TOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------------ generator twin

def test_device_generator_matches_cpu():
    torch = need_gpu()
    import synth.device as sd
    for key in [(0, 0), synth.stream_key(1003, synth.T_K, 17), (2 ** 63 + 5, 2 ** 40 + 3)]:
        for start, n in [(0, 100), (5, 37), (123456, 1000)]:
            got = sd.raw_words(key, start, n, "cuda").cpu().numpy().view(np.uint32)
            assert np.array_equal(got, synth.philox_words(key, start, n)), (key, start, n)
    cfg = synth.get("tiny")
    q, d = sd.logical_q4(cfg, "gu", 0, cfg.seed, "cuda")
    q0, d0 = synth.weight_q4(cfg, "gu", 0)
    assert np.array_equal(q.cpu().numpy(), q0)
    assert np.array_equal(d.cpu().numpy().view(np.uint16), d0)
    k, v = sd.kv_cache(cfg, 0, cfg.seed, 200, "cuda")
    k0, v0 = synth.kv_prefix(cfg, 0)
    kh = k.cpu().numpy().view(np.uint16)
    vh = v.cpu().numpy().view(np.uint16)
    assert np.array_equal(kh[:, :cfg.prefix], k0)
    assert np.array_equal(vh[:, :, :cfg.prefix].transpose(0, 2, 1), v0)
    assert not kh[:, cfg.prefix:].any() and not vh[:, :, cfg.prefix:].any()
    g = sd.gain(cfg, "ffn", 0, cfg.seed, "cuda").cpu().numpy().view(np.uint16)
    assert np.array_equal(g, synth.gain(cfg, "ffn", 0))
    x = sd.hidden_in(cfg, cfg.seed, cfg.nodes, "cuda").cpu().numpy().view(np.uint16)
    assert np.array_equal(x, synth.hidden_in(cfg))


def test_device_packer_equals_host_packer():
    torch = need_gpu()
    import tree_verify_amd as tv
    import synth.device as sd
    cfg = synth.get("tiny")
    for which, kind in [("qkv", tv.W_QKV), ("gu", tv.W_GU), ("o", tv.W_PLAIN), ("lm", tv.W_PLAIN)]:
        n_out, k_in = synth.weight_dims(cfg, which)
        q, d = synth.weight_q4(cfg, which, 0)
        nb = tv.lucev_q4_packed_bytes(n_out, k_in)
        host = np.zeros(nb, np.uint8)
        tv.lucev_q4_pack(kind, cfg.head_dim, np.ascontiguousarray(q), np.ascontiguousarray(d),
                         n_out, k_in, host, nb)
        dev = sd.packed_q4(cfg, which, 0, cfg.seed, "cuda").cpu().numpy()
        assert np.array_equal(dev, host), which


# ------------------------------------------------------------------ attention alone

ATTN_CASES = [
    # (name, Hq, Hkv, d, P, parent-recipe, n)
    ("tiny_shape", 4, 2, 64, 128, None, 8),
    ("ragged_prefix", 8, 2, 128, 1000, None, 16),
    ("27b_group", 48, 8, 128, 4100, (3, 8), 22),
    ("wide_tree", 48, 8, 128, 2051, (4, 10), 40),
    ("five_tiles", 48, 8, 128, 1500, (3, 8), 13),  # 78 rows: the fifth tile split by key quarter
    ("empty_prefix", 8, 2, 128, 0, None, 5),
    ("short_prefix", 8, 2, 128, 33, None, 7),              # one ragged tile, a one-token second half
    ("single_node", 48, 8, 128, 777, None, 1),
    ("max_nodes", 8, 2, 64, 300, None, 64),
    ("row_groups_384_rows", 48, 8, 128, 700, None, 64),    # 24 tiles: two row groups of 12
    ("row_groups_512_rows", 32, 4, 128, 515, None, 64),    # 512 rows (the limit): two groups of 16
    ("row_groups_d64", 16, 1, 64, 260, (4, 10), 32),       # 512 rows of head_dim 64
    ("row_groups_17_tiles", 48, 8, 128, 1100, (4, 10), 45),  # 270 rows: groups of 9 and 8 tiles
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_tree_attention_parity(case):
    torch = need_gpu()
    import tree_verify_amd as tv
    import synth.device as sd
    name, Hq, Hkv, d, P, rec, n = case
    cfg = synth.Config("attn_" + name, layers=1, hidden=128, n_q_heads=Hq, n_kv_heads=Hkv,
                       head_dim=d, ffn=128, vocab=64, prefix=P, nodes=n,
                       max_children=rec[0] if rec else None, max_depth=rec[1] if rec else None,
                       p_accept=0.7, seed=4242 + n)
    say("attention case", name)
    parent = synth.tree_parents(cfg)
    cap = ((P + 7) // 8) * 8 + 8
    k, v = sd.kv_cache(cfg, 0, cfg.seed, cap, "cuda")
    tab = "normal"
    q = sd.flat_table(tab, synth.stream_key(cfg.seed, 90, 0), n * Hq * d, "cuda")
    kt = sd.flat_table(tab, synth.stream_key(cfg.seed, 91, 0), n * Hkv * d, "cuda")
    vt = sd.flat_table(tab, synth.stream_key(cfg.seed, 92, 0), n * Hkv * d, "cuda")
    gout = Guarded(torch, (n * Hq * d,), torch.int16)
    out = gout.t
    shape = tv.make_shape(cfg.hidden, Hq, Hkv, d, cfg.ffn, cfg.vocab)
    ws_bytes = tv.lucev_workspace_bytes(shape, n, P)
    gws = Guarded(torch, (ws_bytes,), torch.uint8)
    tree = tv.make_tree(parent, [0] * n)
    tv.lucev_tree_attention(shape, tree, tv.make_kv(k, v, P, cap), q, kt, vt, out, gws.t, ws_bytes,
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    gout.check("attention output")
    gws.check("workspace")
    kp, vp = synth.kv_prefix(cfg, 0)
    ref = oracle.tree_attention(bf16_bits_to_f64(q).reshape(n, Hq, d),
                                bf16_bits_to_f64(kt).reshape(n, Hkv, d),
                                bf16_bits_to_f64(vt).reshape(n, Hkv, d),
                                oracle.bf16_to_f64(kp), oracle.bf16_to_f64(vp), parent)
    got = bf16_bits_to_f64(out).reshape(n * Hq, d)
    err = row_rel_err(got, ref.reshape(n * Hq, d))
    say("  max row rel err %.3e" % err.max())
    assert err.max() < TOL


F32_CASES = [c for c in ATTN_CASES if c[0] in ("27b_group", "wide_tree", "five_tiles", "empty_prefix",
                                               "row_groups_384_rows", "row_groups_17_tiles", "ragged_prefix")]


# The fp32-input attention (lucev_tree_attention_f32) runs the step's own
# kernels (queries split into bf16 hi + lo in the prefix pass, fp32 tree keys
# and values in the combine); inputs are fp32 with all 24 bits populated.
@pytest.mark.parametrize("case", F32_CASES, ids=[c[0] for c in F32_CASES])
def test_tree_attention_f32_parity(case):
    torch = need_gpu()
    import tree_verify_amd as tv
    import synth.device as sd
    name, Hq, Hkv, d, P, rec, n = case
    cfg = synth.Config("attn32_" + name, layers=1, hidden=128, n_q_heads=Hq, n_kv_heads=Hkv,
                       head_dim=d, ffn=128, vocab=64, prefix=P, nodes=n,
                       max_children=rec[0] if rec else None, max_depth=rec[1] if rec else None,
                       p_accept=0.7, seed=6262 + n)
    say("fp32 attention case", name)
    parent = synth.tree_parents(cfg)
    cap = ((P + 7) // 8) * 8 + 8
    k, v = sd.kv_cache(cfg, 0, cfg.seed, cap, "cuda")
    rng = np.random.default_rng(cfg.seed)
    qh = rng.standard_normal((n, Hq, d)).astype(np.float32)
    kth = rng.standard_normal((n, Hkv, d)).astype(np.float32)
    vth = rng.standard_normal((n, Hkv, d)).astype(np.float32)
    q, kt, vt = (torch.from_numpy(a).to("cuda") for a in (qh, kth, vth))
    gout = Guarded(torch, (n, Hq, d), torch.float32)
    out = gout.t
    shape = tv.make_shape(cfg.hidden, Hq, Hkv, d, cfg.ffn, cfg.vocab)
    ws_bytes = tv.lucev_workspace_bytes(shape, n, P)
    gws = Guarded(torch, (ws_bytes,), torch.uint8)
    tv.lucev_tree_attention_f32(shape, tv.make_tree(parent, [0] * n), tv.make_kv(k, v, P, cap), q, kt, vt, out,
                                gws.t, ws_bytes, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    gout.check("attention output")
    gws.check("workspace")
    kp, vp = synth.kv_prefix(cfg, 0)
    ref = oracle.tree_attention(qh.astype(np.float64), kth.astype(np.float64), vth.astype(np.float64),
                                oracle.bf16_to_f64(kp), oracle.bf16_to_f64(vp), parent)
    err = row_rel_err(out.cpu().numpy().reshape(n * Hq, d), ref.reshape(n * Hq, d))
    say("  max row rel err %.3e" % err.max())
    assert err.max() < TOL


# ------------------------------------------------------------------ whole steps

def _run_gpu_step(cfg, seed, tokens, parent, layers=None, want_hidden=True):
    torch = need_gpu()
    import tree_verify_amd as tv
    import synth.device as sd
    wl = sd.Workload(cfg, seed, "cuda", layers=layers)
    shape = tv.make_shape(cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn,
                          cfg.vocab, cfg.rms_eps, cfg.rope_base)
    # every runner buffer sits inside guard bands, checked after the step
    r = guarded_runner_class()(shape, wl.layers, wl.head, cfg.nodes, wl.capacity, "cuda")
    n = cfg.nodes
    hid = [torch.zeros(n, cfg.hidden, dtype=torch.float32, device="cuda")
           for _ in range(wl.n_layers)] if want_hidden else None
    tree = tv.make_tree(parent, tokens)
    r.step(tree, wl.x_in_f32(), cfg.prefix, hidden_out=hid)
    torch.cuda.synchronize()
    r.check_guards()
    out = {
        "hidden": [h.cpu().numpy().astype(np.float64) for h in hid] if hid else None,
        "k_tree": bf16_bits_to_f64(r.k_tree[-1][:n]),
        "v_tree": bf16_bits_to_f64(r.v_tree[-1][:n]),
        "logits": bf16_bits_to_f64(r.logits[:n]),
        "argmax": r.argmax[:n].cpu().numpy(),
        "gap": r.gap[:n].cpu().numpy(),
        "path": r.path[:n].cpu().numpy(),
        "path_len": int(r.path_len.cpu().item()),
        "committed": r.committed[:n].cpu().numpy(),
    }
    return out


def _check_case(cfg, seed, layers=None):
    ref = workload.planted_case(cfg, seed, layers=layers)
    say("case", cfg.name, "seed", seed, "parent", list(ref["parent"]))
    got = _run_gpu_step(cfg, seed, ref["tokens"], ref["parent"], layers=layers)
    for l, (g, r) in enumerate(zip(got["hidden"], ref["hidden"])):
        e = row_rel_err(g, r).max()
        assert e < TOL, "hidden state of layer %d: rel err %.3e" % (l, e)
    Hkv, d = cfg.n_kv_heads, cfg.head_dim
    n = cfg.nodes
    ek = row_rel_err(got["k_tree"].reshape(n * Hkv, d), ref["k_tree"].reshape(n * Hkv, d)).max()
    ev = row_rel_err(got["v_tree"].reshape(n * Hkv, d), ref["v_tree"].reshape(n * Hkv, d)).max()
    el = row_rel_err(got["logits"], ref["logits"]).max()
    say("  rel err: k_tree %.2e v_tree %.2e logits %.2e hidden(last) %.2e" %
        (ek, ev, el, row_rel_err(got["hidden"][-1], ref["hidden"][-1]).max()))
    assert ek < TOL and ev < TOL and el < TOL
    ndec, decided = decisive_compare(ref["parent"], ref["tokens"], ref["argmax"], ref["gap"],
                                     got["argmax"], got["path"], got["path_len"], got["committed"])
    # the gap the GPU reports is the fp32 top1-top2 difference
    dec = ref["gap"] > 0.05
    assert np.allclose(got["gap"][dec], ref["gap"][dec], rtol=0.05, atol=0.05)
    say("  decisive nodes %d/%d, path decided %s, path %s" %
        (ndec, n, decided, list(got["path"][:got["path_len"]])))
    return decided


@pytest.mark.parametrize("run", range(8))
def test_tiny_config_parity(run):
    cfg = synth.get("tiny")
    _check_case(cfg, synth.run_seed(cfg, run))


def test_tiny_decode_single_node():
    cfg = synth.get("tiny").replace(nodes=1, name="tiny_decode")
    _check_case(cfg, cfg.seed)


# mid-size shape: every GEMM's feature groups are cut across blocks (the
# split-K reduction path), 2 to 8 node tiles (16 nodes per tile of hi/lo
# rows), ragged prefix
MID = synth.Config("mid", layers=2, hidden=1024, n_q_heads=8, n_kv_heads=2, head_dim=128,
                   ffn=3584, vocab=32768, prefix=1000, nodes=22, max_children=3, max_depth=8,
                   p_accept=0.7, seed=3100)


@pytest.mark.parametrize("nodes,rec", [(22, (3, 8)), (40, (4, 10)), (64, (None, None)), (16, (None, None)),
                                       (28, (3, 9)), (48, (4, 10)), (56, (None, None))])
def test_midsize_parity(nodes, rec):
    cfg = MID.replace(nodes=nodes, max_children=rec[0], max_depth=rec[1], name="mid%d" % nodes)
    _check_case(cfg, cfg.seed + nodes)


# A tree verified against an empty cache (the first step after an empty
# prompt): the attention's prefix pass launches nothing and the combine merges
# each node's ancestors alone; RoPE positions are the depths.  Also a single
# node (decode) on an empty cache.
@pytest.mark.parametrize("nodes,rec", [(22, (3, 8)), (1, (None, None))], ids=["tree22", "decode"])
def test_step_empty_prefix(nodes, rec):
    cfg = MID.replace(prefix=0, nodes=nodes, max_children=rec[0], max_depth=rec[1], name="mid_noprefix%d" % nodes)
    _check_case(cfg, cfg.seed + 500 + nodes)


# A chain of 64 drafts (the deepest tree allowed), every draft the target's
# own greedy token: the last node has 64 ancestors, so the combine takes every
# ancestor round, and the whole chain is accepted (the walk's longest path).
def test_step_chain_of_64():
    cfg = MID.replace(nodes=64, max_children=1, max_depth=None, p_accept=1.0, name="chain64")
    _check_case(cfg, cfg.seed + 700)


# A 27B-class layer + head with 28 nodes (four node tiles): gate/up and
# lm_head take two row tiles per wave with one column group per unit; QKV, Wo
# and down one tile per wave.
def test_layer27b_four_node_tiles_parity():
    cfg = synth.get("layer27b").replace(nodes=28, max_children=3, max_depth=9, name="layer27b_n28")
    _check_case(cfg, cfg.seed + 28)


# Decode-sized trees at the 27B layer shape, on MFMA (the default) and on the
# VALU dot-product path (gemv rows 8: every projection of 1 and 2 nodes, and
# gate/up and down of 4 nodes, take dot products; 2, 4 or 8 operand rows).
@pytest.mark.parametrize("nodes,gemv", [(1, 0), (2, 0), (4, 0), (1, 8), (2, 8), (4, 8)])
def test_layer27b_small_tree_parity(nodes, gemv):
    import tree_verify_amd as tv
    need_gpu()
    cfg = synth.get("layer27b").replace(nodes=nodes, max_children=None, max_depth=None,
                                        name="layer27b_n%d" % nodes)
    tv.lucev_set_gemv_max_rows(gemv)
    try:
        _check_case(cfg, cfg.seed + 100 + nodes)
    finally:
        tv.lucev_set_gemv_max_rows(0)


@pytest.mark.parametrize("run", range(2))
def test_small_tree_config_parity(run):
    cfg = synth.get("small_tree")
    _check_case(cfg, synth.run_seed(cfg, run))


@pytest.mark.parametrize("run", range(2))
def test_small_decode_config_parity(run):
    cfg = synth.get("small_decode")
    _check_case(cfg, synth.run_seed(cfg, run))


# Repeated steps on the same inputs must agree bit for bit: every reduction
# has a fixed order, so any difference is a race.  The two node counts give
# three and five node tiles, so different staged slice shapes in the GEMM
# (48 and 80 operand rows, staged as 64 and 96).
@pytest.mark.parametrize("nodes,rec", [(40, (4, 10)), (22, (3, 8))])
def test_repeated_steps_bit_identical(nodes, rec):
    torch = need_gpu()
    import tree_verify_amd as tv
    from tree_verify_amd.runner import VerifyRunner
    import synth.device as sd
    cfg = MID.replace(nodes=nodes, max_children=rec[0], max_depth=rec[1], name="det%d" % nodes)
    seed = cfg.seed + 7 * nodes
    say("case", cfg.name, "seed", seed)
    wl = sd.Workload(cfg, seed, "cuda")
    shape = tv.make_shape(cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn,
                          cfg.vocab, cfg.rms_eps, cfg.rope_base)
    r = VerifyRunner(shape, wl.layers, wl.head, cfg.nodes, wl.capacity, "cuda")
    parent = synth.tree_parents(cfg, seed)
    tokens = [int(t) for t in np.random.default_rng(seed).integers(0, cfg.vocab, size=nodes)]
    tree = tv.make_tree(parent, tokens)
    x = wl.x_in_f32()
    outs = []
    for rep in range(6):
        hid = [torch.zeros(nodes, cfg.hidden, dtype=torch.float32, device="cuda") for _ in range(wl.n_layers)]
        r.step(tree, x, cfg.prefix, hidden_out=hid)
        torch.cuda.synchronize()
        outs.append([h.cpu().numpy().copy() for h in hid] + [r.logits.cpu().numpy().copy()])
    for rep in range(1, len(outs)):
        for a, b in zip(outs[0], outs[rep]):
            assert np.array_equal(a, b), "step %d differs from step 0" % rep


# ------------------------------------------------------------------ commit and the next step

def test_commit_then_next_step_parity():
    # step 1 on the GPU, lucev_commit_path of its accepted path into every
    # layer's cache, then step 2 (a new tree) against prefix + path: the cache
    # rows must be the step's own tree K / V, bit for bit, and step 2 must
    # match the oracle run on the oracle's committed cache
    torch = need_gpu()
    import tree_verify_amd as tv
    from tree_verify_amd.runner import VerifyRunner
    import synth.device as sd
    cfg = MID.replace(name="commit22")
    seed, seed2 = cfg.seed + 501, cfg.seed + 502
    n, P, Hkv, d = cfg.nodes, cfg.prefix, cfg.n_kv_heads, cfg.head_dim
    say("case commit then next step, seed", seed)
    ref = workload.planted_case(cfg, seed)
    wl = sd.Workload(cfg, seed, "cuda")
    shape = tv.make_shape(cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn,
                          cfg.vocab, cfg.rms_eps, cfg.rope_base)
    r = VerifyRunner(shape, wl.layers, wl.head, n, wl.capacity, "cuda")
    r.step(tv.make_tree(ref["parent"], ref["tokens"]), wl.x_in_f32(), P)
    r.commit(n, P)
    torch.cuda.synchronize()
    plen = int(r.path_len.item())
    path = [int(i) for i in r.path[:plen].cpu().numpy()]
    say("  path", path)
    assert path[0] == 0 and 1 <= plen <= n
    for l, lw in enumerate(wl.layers):
        k = lw["k"].cpu().numpy().view(np.uint16)   # [Hkv][cap][d]
        v = lw["v"].cpu().numpy().view(np.uint16)   # [Hkv][d][cap]
        kt = r.k_tree[l].cpu().numpy().view(np.uint16)  # [n][Hkv][d]
        vt = r.v_tree[l].cpu().numpy().view(np.uint16)
        for j, node in enumerate(path):
            assert np.array_equal(k[:, P + j, :], kt[node]), "layer %d K row %d" % (l, j)
            assert np.array_equal(v[:, :, P + j], vt[node]), "layer %d V column %d" % (l, j)
        assert not k[:, P + plen:, :].any() and not v[:, :, P + plen:].any(), "rows past the path"
        # against the oracle's committed rows (bf16 of its own tree K / V)
        kr, vr = oracle.commit_path(synth.kv_prefix(cfg, l, seed)[0], synth.kv_prefix(cfg, l, seed)[1],
                                    ref["k_tree_layers"][l], ref["v_tree_layers"][l], path)
        ek = row_rel_err(oracle.bf16_to_f64(k[:, P:P + plen, :]).reshape(-1, d), kr[:, P:].reshape(-1, d)).max()
        ev = row_rel_err(oracle.bf16_to_f64(v[:, :, P:P + plen]).transpose(0, 2, 1).reshape(-1, d),
                         vr[:, P:].reshape(-1, d)).max()
        assert ek < TOL and ev < TOL, (l, ek, ev)
    # step 2 against prefix + path, a new tree and new inputs
    parent2 = synth.tree_parents(cfg, seed2)
    x2 = synth.hidden_in(cfg, seed2)
    caches = [oracle.commit_path(*synth.kv_prefix(cfg, l, seed), ref["k_tree_layers"][l],
                                 ref["v_tree_layers"][l], path) for l in range(cfg.layers)]
    ref2 = oracle.verify_forward(x2, (workload.layer_weights(cfg, l, seed) for l in range(cfg.layers)),
                                 caches, workload.head_weights(cfg, seed), parent2, workload.shape(cfg))
    tok2 = synth.plant_tokens(cfg, parent2, ref2["argmax"], seed2)
    x2g = torch.from_numpy(oracle.bf16_to_f64(x2).astype(np.float32)).cuda()
    hid = [torch.zeros(n, cfg.hidden, dtype=torch.float32, device="cuda") for _ in range(cfg.layers)]
    r.step(tv.make_tree(parent2, tok2), x2g, P + plen, hidden_out=hid)
    torch.cuda.synchronize()
    for l in range(cfg.layers):
        e = row_rel_err(hid[l].cpu().numpy(), ref2["hidden"][l]).max()
        assert e < TOL, "step 2 hidden of layer %d: %.3e" % (l, e)
    el = row_rel_err(bf16_bits_to_f64(r.logits[:n]), ref2["logits"]).max()
    say("  step 2 at prefix %d: logits rel err %.2e" % (P + plen, el))
    assert el < TOL
    decisive_compare(parent2, tok2, ref2["argmax"], ref2["gap"], r.argmax[:n].cpu().numpy(),
                     r.path[:n].cpu().numpy(), int(r.path_len.item()), r.committed[:n].cpu().numpy())


# ------------------------------------------------------------------ draft hooks

def test_draft_hooks_capture_and_project():
    # the two adapter hooks a drafter uses: a chosen layer's activations
    # captured during verify, and the target's lm_head over arbitrary hidden
    # rows (random rows standing in for a drafter's, plus the captured ones)
    torch = need_gpu()
    import tree_verify_amd as tv
    from tree_verify_amd.runner import VerifyRunner
    import synth.device as sd
    cfg = MID.replace(name="hooks22")
    seed = cfg.seed + 601
    n, H, V = cfg.nodes, cfg.hidden, cfg.vocab
    say("case draft hooks, seed", seed)
    ref = workload.planted_case(cfg, seed)
    wl = sd.Workload(cfg, seed, "cuda")
    shape = tv.make_shape(cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn,
                          cfg.vocab, cfg.rms_eps, cfg.rope_base)
    r = VerifyRunner(shape, wl.layers, wl.head, n, wl.capacity, "cuda")
    cap0 = torch.zeros(n, H, dtype=torch.float32, device="cuda")
    r.step(tv.make_tree(ref["parent"], ref["tokens"]), wl.x_in_f32(), cfg.prefix, capture={0: cap0})
    torch.cuda.synchronize()
    got0 = cap0.cpu().numpy().astype(np.float64)
    e0 = row_rel_err(got0, ref["hidden"][0]).max()
    assert e0 < TOL, "captured layer 0: %.3e" % e0
    hw = workload.head_weights(cfg, seed)
    rng = np.random.default_rng(seed)
    for rows, label in [(rng.standard_normal((16, H)).astype(np.float32) * 3.0, "random rows"),
                        (got0.astype(np.float32), "captured layer-0 rows")]:
        m = len(rows)
        x = torch.from_numpy(rows).cuda()
        logits = torch.zeros(m, V, dtype=torch.int16, device="cuda")
        am = torch.zeros(m, dtype=torch.int32, device="cuda")
        gap = torch.zeros(m, dtype=torch.float32, device="cuda")
        r.project(x, m, logits, am, gap)
        torch.cuda.synchronize()
        ol = oracle.head_logits(rows.astype(np.float64), hw, workload.shape(cfg))
        oam, ogap = oracle.argmax_gap(ol)
        el = row_rel_err(bf16_bits_to_f64(logits), ol).max()
        dec = ogap > 0.05
        say("  %s: logits rel err %.2e, decisive %d/%d" % (label, el, dec.sum(), m))
        assert el < TOL
        assert np.array_equal(am.cpu().numpy()[dec], oam[dec])
        assert np.allclose(gap.cpu().numpy()[dec], ogap[dec], rtol=0.05, atol=0.05)


# ------------------------------------------------------------------ paged prefix

@pytest.mark.parametrize("case", [c for c in ATTN_CASES if c[4] != 0] + [("empty_prefix", 8, 2, 128, 0, None, 5)],
                         ids=[c[0] for c in ATTN_CASES if c[4] != 0] + ["empty_prefix"])
def test_tree_attention_paged_equals_contiguous(case):
    # the same prefix scattered over a shuffled pool of 16-token pages (and
    # non-zero filler past the prefix in the last page): the paged attention
    # must give the contiguous result bit for bit, and both match the oracle
    torch = need_gpu()
    import tree_verify_amd as tv
    import synth.device as sd
    name, Hq, Hkv, d, P, rec, n = case
    cfg = synth.Config("paged_" + name, layers=1, hidden=128, n_q_heads=Hq, n_kv_heads=Hkv,
                       head_dim=d, ffn=128, vocab=64, prefix=P, nodes=n,
                       max_children=rec[0] if rec else None, max_depth=rec[1] if rec else None,
                       p_accept=0.7, seed=5151 + n)
    say("paged attention case", name)
    parent = synth.tree_parents(cfg)
    cap = ((P + 7) // 8) * 8 + 8
    k, v = sd.kv_cache(cfg, 0, cfg.seed, cap, "cuda")
    NL = (P + 15) // 16
    NP = NL + 5
    perm = torch.from_numpy(np.random.default_rng(cfg.seed).permutation(NP)[:NL].astype(np.int64)).cuda()
    k_pool = torch.full((NP, Hkv, 16, d), 0x4000, dtype=torch.int16, device="cuda")  # 2.0 filler
    v_pool = torch.full((NP, Hkv, d, 16), 0x4000, dtype=torch.int16, device="cuda")
    if NL:
        kl = k[:, :NL * 16, :].reshape(Hkv, NL, 16, d).permute(1, 0, 2, 3).clone()
        vl = v[:, :, :NL * 16].reshape(Hkv, d, NL, 16).permute(2, 0, 1, 3).clone()
        tail = NL * 16 - P  # tokens past the prefix in the last page keep the filler
        if tail:
            kl[NL - 1, :, 16 - tail:, :] = 0x4000
            vl[NL - 1, :, :, 16 - tail:] = 0x4000
        k_pool[perm] = kl
        v_pool[perm] = vl
    table = perm.to(torch.int32).contiguous() if NL else torch.zeros(1, dtype=torch.int32, device="cuda")
    tab = "normal"
    q = sd.flat_table(tab, synth.stream_key(cfg.seed, 90, 0), n * Hq * d, "cuda")
    kt = sd.flat_table(tab, synth.stream_key(cfg.seed, 91, 0), n * Hkv * d, "cuda")
    vt = sd.flat_table(tab, synth.stream_key(cfg.seed, 92, 0), n * Hkv * d, "cuda")
    shape = tv.make_shape(cfg.hidden, Hq, Hkv, d, cfg.ffn, cfg.vocab)
    ws_bytes = tv.lucev_workspace_bytes(shape, n, max(P, 1))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    tree = tv.make_tree(parent, [0] * n)
    st = torch.cuda.current_stream().cuda_stream
    out_c = torch.zeros(n * Hq * d, dtype=torch.int16, device="cuda")
    out_p = torch.zeros(n * Hq * d, dtype=torch.int16, device="cuda")
    tv.lucev_tree_attention(shape, tree, tv.make_kv(k, v, P, cap), q, kt, vt, out_c, ws, ws_bytes, st)
    tv.lucev_tree_attention_paged(shape, tree, tv.make_kv_paged(k_pool, v_pool, table, NP, P), q, kt, vt,
                                  out_p, ws, ws_bytes, st)
    torch.cuda.synchronize()
    assert torch.equal(out_c, out_p), "paged result differs from the contiguous one"
    kp, vp = synth.kv_prefix(cfg, 0)
    ref = oracle.tree_attention(bf16_bits_to_f64(q).reshape(n, Hq, d), bf16_bits_to_f64(kt).reshape(n, Hkv, d),
                                bf16_bits_to_f64(vt).reshape(n, Hkv, d), oracle.bf16_to_f64(kp),
                                oracle.bf16_to_f64(vp), parent)
    err = row_rel_err(bf16_bits_to_f64(out_p).reshape(n * Hq, d), ref.reshape(n * Hq, d))
    say("  %d pages of %d, max row rel err %.3e" % (NL, NP, err.max()))
    assert err.max() < TOL


# Graph replays of a 27B-class layer + head step, each checked bit for bit
# against the first.  Direct-to-LDS loads from several waves writing the same
# LDS bytes (surplus loads sent to one shared pad), and GEMM slices loaded
# straight into LDS and awaited by a partial load count, each made replays
# differ.  The ragged prefix ends mid-tile, so the attention's last tile
# takes its register-load path beside the direct-to-LDS tiles.
#
# The 40-node tree is the wide plan (C5's budget): two query tiles per wave in
# the attention (15 tiles of 16 rows per KV head) and five node tiles in the
# GEMMs.  The 64-node tree takes the attention's row groups (24 tiles: two
# blocks per chunk and KV head) and eight node tiles in the exact GEMMs.
@pytest.mark.parametrize("nodes,rec,trim", [(22, (3, 8), 0), (22, (3, 8), 37), (40, (4, 10), 37),
                                            (64, (None, None), 37)],
                         ids=["n22", "n22_ragged", "n40_ragged", "n64_ragged_row_groups"])
def test_graph_replays_bit_identical_27b_layer(nodes, rec, trim):
    torch = need_gpu()
    import tree_verify_amd as tv
    from tree_verify_amd.runner import VerifyRunner
    import synth.device as sd
    cfg = synth.get("layer27b").replace(nodes=nodes, max_children=rec[0], max_depth=rec[1])
    seed = cfg.seed + (0 if nodes == 22 else nodes)
    prefix = cfg.prefix - trim
    say("case layer27b graph replays, nodes", nodes, "seed", seed, "prefix", prefix)
    wl = sd.Workload(cfg, seed, "cuda")
    shape = tv.make_shape(cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn,
                          cfg.vocab, cfg.rms_eps, cfg.rope_base)
    r = VerifyRunner(shape, wl.layers, wl.head, cfg.nodes, wl.capacity, "cuda")
    parent = synth.tree_parents(cfg, seed)
    tree = tv.make_tree(parent, [0] * cfg.nodes)
    x = wl.x_in_f32().contiguous()
    hid = [torch.zeros(cfg.nodes, cfg.hidden, dtype=torch.float32, device="cuda")]
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        r.step(tree, x, prefix, hidden_out=hid)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            r.step(tree, x, prefix, hidden_out=hid)
    torch.cuda.synchronize()
    first = None
    for rep in range(12):
        with torch.cuda.stream(stream):
            g.replay()
            stream.synchronize()
        cur = (hid[0].cpu().numpy().copy(), r.k_tree[0].cpu().numpy().copy(), r.logits.cpu().numpy().copy())
        if first is None:
            first = cur
        else:
            for a, b in zip(first, cur):
                assert np.array_equal(a, b), "replay %d differs from the first" % rep
