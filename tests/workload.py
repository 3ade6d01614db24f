"""Glue between the seeded generator and the oracle for tests and benches.

Builds the oracle's logical inputs for a config from ``synth``; holds no
arithmetic of the method.
"""
import numpy as np

import oracle
import synth


def shape(cfg):
    return oracle.Shape(cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                        cfg.ffn, cfg.vocab, cfg.rms_eps, cfg.rope_base)


def layer_weights(cfg, layer, seed=None):
    return oracle.LayerWeights(
        attn_norm=synth.gain(cfg, "attn", layer, seed),
        ffn_norm=synth.gain(cfg, "ffn", layer, seed),
        wqkv=synth.weight_q4(cfg, "qkv", layer, seed),
        wo=synth.weight_q4(cfg, "o", layer, seed),
        wgu=synth.weight_q4(cfg, "gu", layer, seed),
        wd=synth.weight_q4(cfg, "d", layer, seed))


def head_weights(cfg, seed=None):
    return oracle.HeadWeights(final_norm=synth.gain(cfg, "final", 0, seed),
                              lm=synth.weight_q4(cfg, "lm", 0, seed))


def run_oracle(cfg, seed=None, tokens=None, parent=None, keep_hidden=True,
               layers=None):
    """Oracle forward over ``layers`` (default all) of a config, built lazily."""
    seed = cfg.seed if seed is None else seed
    L = cfg.layers if layers is None else layers
    if parent is None:
        parent = synth.tree_parents(cfg, seed)
    x = synth.hidden_in(cfg, seed)
    lw = (layer_weights(cfg, l, seed) for l in range(L))
    kv = (synth.kv_prefix(cfg, l, seed) for l in range(L))
    out = oracle.verify_forward(x, lw, kv, head_weights(cfg, seed), parent,
                                shape(cfg), token=tokens, keep_hidden=keep_hidden)
    out["parent"] = np.asarray(parent)
    return out


def planted_case(cfg, seed=None, layers=None, keep_hidden=True):
    """Inputs + oracle outputs with tokens planted from the oracle's argmax."""
    seed = cfg.seed if seed is None else seed
    parent = synth.tree_parents(cfg, seed)
    out = run_oracle(cfg, seed, parent=parent, keep_hidden=keep_hidden, layers=layers)
    tok = synth.plant_tokens(cfg, parent, out["argmax"], seed)
    path, committed = oracle.accept_path(parent, tok, out["argmax"])
    out.update(tokens=tok, path=path, committed=committed)
    return out
