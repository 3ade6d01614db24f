"""GPU parity of the verify step over a quantised KV prefix
(lucev_verify_layer_q8 / _q4), through the runner and the C ABI.

The device quantiser turns every layer's bf16 cache into int8 or 4-bit
block-32 codes (checked bit-exact against the oracle's quantiser here too);
the oracle then runs the same step over the prefix those codes stand for
(``oracle.kv_prefix_from_q8`` / ``_q4``), with tokens planted from its own
greedy tokens.  Per-layer hidden states and logits must agree to 2e-2 (max
row relative error), greedy tokens wherever the oracle's gap exceeds 0.05,
and the GPU's walk must be the oracle's walk over the GPU's tokens.
"""
import sys

import numpy as np
import pytest

import kv_nibbles
import oracle
import synth
import workload
from gpu_common import bf16_bits_to_f64, decisive_compare, guarded_runner_class, need_gpu, row_rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-2

MID = synth.Config("mid", layers=2, hidden=1024, n_q_heads=8, n_kv_heads=2, head_dim=128,
                   ffn=3584, vocab=32768, prefix=1000, nodes=22, max_children=3, max_depth=8,
                   p_accept=0.7, seed=3100)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = [
    # (name, config, bits)
    ("mid22_q8", MID, 8),
    ("mid22_q4", MID, 4),
    ("mid40_q8", MID.replace(nodes=40, max_children=4, max_depth=10, name="mid40"), 8),
    ("mid40_q4", MID.replace(nodes=40, max_children=4, max_depth=10, name="mid40"), 4),
    ("layer27b_q8", "layer27b", 8),
    ("layer27b_q4", "layer27b", 4),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_verify_step_over_quantised_prefix(case):
    torch = need_gpu()
    import tree_verify_amd as tv
    import synth.device as sd
    name, cfg, bits = case
    if isinstance(cfg, str):
        cfg = synth.get(cfg)
    seed = cfg.seed + 17
    P = cfg.prefix
    cap = ((P + 64 + 31) // 32) * 32
    say("case", name, "seed", seed, "prefix", P, "capacity", cap)
    wl = sd.Workload(cfg, seed, "cuda", capacity=cap)
    shape = tv.make_shape(cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn,
                          cfg.vocab, cfg.rms_eps, cfg.rope_base)
    r = guarded_runner_class()(shape, wl.layers, wl.head, cfg.nodes, cap, "cuda")
    r.quantise_kv(bits, P)
    torch.cuda.synchronize()

    # the oracle's codes from the same bf16 caches; the device's must match
    quant = oracle.quantize_q8_blocks if bits == 8 else oracle.quantize_q4_blocks
    prefix_of = oracle.kv_prefix_from_q8 if bits == 8 else oracle.kv_prefix_from_q4
    kv = []
    for l, lw in enumerate(wl.layers):
        kc, ks = quant(oracle.bf16_to_f64(lw["k"].cpu().numpy().view(np.uint16)))
        vc, vs = quant(oracle.bf16_to_f64(lw["v"].cpu().numpy().view(np.uint16)))
        dk, dks, dv, dvs = (t.cpu().numpy() for t in r._kvq[l])
        if bits == 4:
            dk, dv = kv_nibbles.unpack(dk), kv_nibbles.unpack(dv)
        assert np.array_equal(dk.view(kc.dtype), kc) and np.array_equal(dks.view(np.uint16), ks)
        assert np.array_equal(dv.view(vc.dtype), vc) and np.array_equal(dvs.view(np.uint16), vs)
        kv.append(prefix_of(kc, ks, vc, vs, P))

    parent = synth.tree_parents(cfg, seed)
    x = synth.hidden_in(cfg, seed)
    lws = [workload.layer_weights(cfg, l, seed) for l in range(cfg.layers)]
    ref = oracle.verify_forward(x, lws, kv, workload.head_weights(cfg, seed), parent, workload.shape(cfg))
    tokens = synth.plant_tokens(cfg, parent, ref["argmax"], seed)

    n = cfg.nodes
    hid = [torch.zeros(n, cfg.hidden, dtype=torch.float32, device="cuda") for _ in range(cfg.layers)]
    r.step(tv.make_tree(parent, tokens), wl.x_in_f32(), P, hidden_out=hid)
    torch.cuda.synchronize()
    r.check_guards()
    for l in range(cfg.layers):
        e = row_rel_err(hid[l].cpu().numpy().astype(np.float64), ref["hidden"][l]).max()
        say("  layer %d hidden rel err %.3e" % (l, e))
        assert e < TOL, "hidden state of layer %d: rel err %.3e" % (l, e)
    el = row_rel_err(bf16_bits_to_f64(r.logits[:n]), ref["logits"]).max()
    say("  logits rel err %.3e" % el)
    assert el < TOL
    ndec, decided = decisive_compare(parent, tokens, ref["argmax"], ref["gap"], r.argmax[:n].cpu().numpy(),
                                     r.path[:n].cpu().numpy(), int(r.path_len.cpu().item()),
                                     r.committed[:n].cpu().numpy())
    say("  decisive nodes %d/%d, path decided %s" % (ndec, n, decided))
