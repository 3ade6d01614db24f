"""Closed-form pins of the decoder layer's composition and of the head.

The layer is the plain pre-norm decoder layer: RMSNorm with the attention
gain, fused QKV, RoPE on q and k only, tree attention, Wo plus the residual,
RMSNorm with the FFN gain of that updated residual, gate/up with SiLU on the
gate half, down plus the residual; the head is the final RMSNorm then the
lm_head.  The target scores the whole drafted tree with this forward in one
pass ("Lucebox Hub", section "Speculative decoding 계층 (DFlash / DDTree /
DSpark)").

Each pin hand-builds integer weights (codes picking single inputs, scales that
are powers of two) and rows whose RMS is an integer, so the expected outputs
follow in closed form from the construction; the expectations below are
written from that construction with scalar Python arithmetic, never through
the oracle.  ``test_each_mutant_is_caught`` then plants plausible slips in a
copy of the oracle's layer / head code (on the CPU) and checks that some pin
fails for each of them.
"""
import inspect
import math

import numpy as np
import pytest

import oracle
import oracle.reference as ref

H, HQ, HKV, D, F, V = 64, 2, 1, 32, 64, 64
SHAPE = oracle.Shape(H, HQ, HKV, D, F, V, rms_eps=0.0, rope_base=10000.0)


def f16(x):
    return np.asarray(x, np.float16).view(np.uint16)


def bf16_exact(vals):
    """bf16 bits of values that bf16 holds exactly (asserted)."""
    a = np.asarray(vals, np.float32)
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_to_f64(bits), np.asarray(vals, np.float64))
    return bits


# two distinct gain vectors, both exact in bf16 (multiples of 1/64 in [0.5, 1.5))
G_ATTN = np.array([0.5 + k / 64.0 for k in range(H)])
G_FFN = np.array([1.5 - (k + 1) / 64.0 for k in range(H)])
G_FINAL = np.array([0.5 + ((7 * k) % H) / 64.0 for k in range(H)])
K_ONE = 32  # G_ATTN[32] == 1.0


def q4(n_out, k_in, picks, scale=1.0):
    """Weights W[r, c] = scale * (code - 8): code 8 (zero) except
    W[r, c] = scale * w for every (r, c, w) in picks."""
    q = np.full((n_out, k_in), 8, np.uint8)
    for r, c, w in picks:
        q[r, c] = 8 + w
    d = f16(np.full((n_out, k_in // 32), scale))
    return q, d


def zero(n_out, k_in):
    return q4(n_out, k_in, [])


def layer(attn_norm=G_ATTN, ffn_norm=G_FFN, wqkv=None, wo=None, wgu=None, wd=None):
    return oracle.LayerWeights(
        bf16_exact(attn_norm), bf16_exact(ffn_norm),
        wqkv if wqkv is not None else zero((HQ + 2 * HKV) * D, H),
        wo if wo is not None else zero(H, HQ * D),
        wgu if wgu is not None else zero(2 * F, H),
        wd if wd is not None else zero(H, F))


def empty_prefix():
    return np.zeros((HKV, 0, D), np.float64), np.zeros((HKV, 0, D), np.float64)


def silu(a):
    return a / (1.0 + math.exp(-a))


# value rows of the QKV matrix: v_j = u[sigma(j)]
SIGMA = [2 * j for j in range(D)]  # holds K_ONE (j = 16)
V_ROW0 = (HQ + HKV) * D


def wqkv_values_only():
    return q4((HQ + 2 * HKV) * D, H, [(V_ROW0 + j, SIGMA[j], 1) for j in range(D)])


# ------------------------------------------------------------------ the pins
# Each returns (got, expected) arrays; a pin holds when they agree to 1e-12.

def pin_attention_half(layer_fn):
    """One node, empty prefix: softmax over its own key is 1, so o = v in
    every head.  FFN weights are zero.  x = 2 everywhere, so the attention
    RMSNorm gives exactly the attention gain.  Wo row i reads head 0's dim
    tau(i) with weight 2.  x_out[i] = 2 + 2 g_attn[sigma(tau(i))]."""
    tau = [(5 * i) % D for i in range(H)]
    wo = q4(H, HQ * D, [(i, tau[i], 2) for i in range(H)])
    w = layer(wqkv=wqkv_values_only(), wo=wo)
    x = np.full((1, H), 2.0)
    got = layer_fn(x, w, *empty_prefix(), [-1], SHAPE)[0]
    exp = np.array([[2.0 + 2.0 * G_ATTN[SIGMA[tau[i]]] for i in range(H)]])
    return got, exp


def _ffn_maps():
    a = [(3 * f + 1) % H for f in range(F)]   # gate row f reads u2[a(f)]
    b = [(5 * f + 2) % H for f in range(F)]   # up row f reads u2[b(f)]
    c = [(7 * i + 3) % F for i in range(H)]   # down row i reads m[c(i)]
    return a, b, c


def _ffn_weights():
    a, b, c = _ffn_maps()
    wgu = q4(2 * F, H, [(f, a[f], 1) for f in range(F)] + [(F + f, b[f], 1) for f in range(F)])
    wd = q4(H, F, [(i, c[i], 1) for i in range(H)])
    return wgu, wd


def pin_ffn_only(layer_fn):
    """Attention weights zero (q = k = v = 0, so the attention adds 0).  x = 2
    everywhere, so the FFN RMSNorm gives exactly the FFN gain; gate row f reads
    u2[a(f)], up row f reads u2[b(f)], down row i reads m[c(i)].
    x_out[i] = 2 + silu(g_ffn[a]) * g_ffn[b] at f = c(i)."""
    a, b, c = _ffn_maps()
    wgu, wd = _ffn_weights()
    w = layer(wgu=wgu, wd=wd)
    x = np.full((1, H), 2.0)
    got = layer_fn(x, w, *empty_prefix(), [-1], SHAPE)[0]
    exp = np.array([[2.0 + silu(G_FFN[a[c[i]]]) * G_FFN[b[c[i]]] for i in range(H)]])
    return got, exp


def pin_both_halves(layer_fn):
    """Both halves on.  The attention gives o = v = g_attn[sigma(.)]; Wo reads
    the value dim j1 with g_attn[sigma(j1)] = 1, weight -1 into rows < 32 and
    +5 into rows >= 32, so after the attention half the residual is x1 = [1 x 32,
    7 x 32], whose RMS is sqrt((1 + 49) / 2) = 5.  The FFN norm of x1 is
    u2 = x1 / 5 * g_ffn, and x_out = x1 + silu(u2[a]) * u2[b] at f = c(i)."""
    j1 = SIGMA.index(K_ONE)
    wo = q4(H, HQ * D, [(i, j1, -1 if i < 32 else 5) for i in range(H)])
    wgu, wd = _ffn_weights()
    a, b, c = _ffn_maps()
    w = layer(wqkv=wqkv_values_only(), wo=wo, wgu=wgu, wd=wd)
    x = np.full((1, H), 2.0)
    got = layer_fn(x, w, *empty_prefix(), [-1], SHAPE)[0]
    x1 = [1.0 if i < 32 else 7.0 for i in range(H)]
    u2 = [x1[k] / 5.0 * G_FFN[k] for k in range(H)]
    exp = np.array([[x1[i] + silu(u2[a[c[i]]]) * u2[b[c[i]]] for i in range(H)]])
    return got, exp


def pin_values_not_rotated(layer_fn):
    """Two-node chain, empty prefix, q = k = 0 (all scores equal): node 1 at
    position 1 averages the values of nodes 0 and 1, which RoPE must not
    touch.  x_0 = 2 everywhere (u_0 = g_attn), x_1 = [1 x 32, 7 x 32]
    (u_1 = x_1 / 5 * g_attn); Wo row i reads head 0's dim i % D with weight 1.
    x_out[0, i] = 2 + v_0[i % D], x_out[1, i] = x_1[i] + (v_0 + v_1)[i % D] / 2."""
    wo = q4(H, HQ * D, [(i, i % D, 1) for i in range(H)])
    w = layer(wqkv=wqkv_values_only(), wo=wo)
    x = np.array([[2.0] * H, [1.0] * 32 + [7.0] * 32])
    got = layer_fn(x, w, *empty_prefix(), [-1, 0], SHAPE)[0]
    u1 = [x[1, k] / 5.0 * G_ATTN[k] for k in range(H)]
    v0 = [G_ATTN[SIGMA[j]] for j in range(D)]
    v1 = [u1[SIGMA[j]] for j in range(D)]
    exp = np.array([[2.0 + v0[i % D] for i in range(H)],
                    [x[1, i] + 0.5 * (v0[i % D] + v1[i % D]) for i in range(H)]])
    return got, exp


def pin_scores_use_keys(layer_fn):
    """Two-node chain, empty prefix.  Key row j reads input j (first half)
    and node 0's input is zero there (x_0 = [0 x 32, 2 x 32], RMS sqrt(2)), so
    k_0 = 0 and node 1's score of key 0 is 0 at any rotation.  Node 1 (x_1 =
    [1 x 32, 7 x 32], RMS 5) scores its own key at its own position, which
    RoPE leaves unchanged: s = (1 + h) sum_j u_1[j]^2 / sqrt(D) for query
    head h, whose query row j reads input j with weight 1 + h.  Values read
    input 2j; Wo row i reads head i // D, dim i % D.  So x_out[0] = x_0 + v_0
    and x_out[1] = x_1 + (v_0 + e^s v_1) / (1 + e^s) per head."""
    picks = [(h * D + j, j, 1 + h) for h in range(HQ) for j in range(D)]
    picks += [(HQ * D + j, j, 1) for j in range(D)]
    picks += [(V_ROW0 + j, SIGMA[j], 1) for j in range(D)]
    wqkv = q4((HQ + 2 * HKV) * D, H, picks)
    wo = q4(H, HQ * D, [(i, i, 1) for i in range(H)])
    w = layer(wqkv=wqkv, wo=wo)
    x = np.array([[0.0] * 32 + [2.0] * 32, [1.0] * 32 + [7.0] * 32])
    got = layer_fn(x, w, *empty_prefix(), [-1, 0], SHAPE)[0]
    u0 = [x[0, k] / math.sqrt(2.0) * G_ATTN[k] for k in range(H)]
    u1 = [x[1, k] / 5.0 * G_ATTN[k] for k in range(H)]
    v0 = [u0[SIGMA[j]] for j in range(D)]
    v1 = [u1[SIGMA[j]] for j in range(D)]
    exp = np.zeros((2, H))
    for i in range(H):
        h, j = i // D, i % D
        s = (1 + h) * sum(u1[t] * u1[t] for t in range(D)) / math.sqrt(D)
        exp[0, i] = x[0, i] + v0[j]
        exp[1, i] = x[1, i] + (v0[j] + math.exp(s) * v1[j]) / (1.0 + math.exp(s))
    return got, exp


def pin_two_layers_in_order(layer_fn, forward_fn=None):
    """Layer 0 = the attention half of pin_both_halves (x: 2 -> [1 x 32, 7 x 32]),
    layer 1 = FFN only; run in that order the FFN sees x1 (RMS 5).  Run in
    the other order it would see x = 2."""
    j1 = SIGMA.index(K_ONE)
    wo = q4(H, HQ * D, [(i, j1, -1 if i < 32 else 5) for i in range(H)])
    wgu, wd = _ffn_weights()
    a, b, c = _ffn_maps()
    l0 = layer(wqkv=wqkv_values_only(), wo=wo)
    l1 = layer(wgu=wgu, wd=wd)
    x = np.full((1, H), 2.0)
    saved = ref.layer_forward
    ref.layer_forward = layer_fn
    try:
        fwd = forward_fn or ref.verify_forward
        out = fwd(x, [l0, l1], [empty_prefix(), empty_prefix()], None, [-1], SHAPE)
    finally:
        ref.layer_forward = saved
    x1 = [1.0 if i < 32 else 7.0 for i in range(H)]
    u2 = [x1[k] / 5.0 * G_FFN[k] for k in range(H)]
    exp = np.array([[x1[i] + silu(u2[a[c[i]]]) * u2[b[c[i]]] for i in range(H)]])
    return out["x"], exp


def pin_head(head_fn):
    """Final RMSNorm of x = [1 x 32, 7 x 32] (RMS 5), then an lm_head with
    block scale 1/2 whose row v reads input pi(v) with code offset +3:
    logits[v] = 1.5 * x[pi(v)] / 5 * g_final[pi(v)]."""
    pi = [(11 * v + 4) % H for v in range(V)]
    hw = oracle.HeadWeights(bf16_exact(G_FINAL), q4(V, H, [(v, pi[v], 3) for v in range(V)], scale=0.5))
    x = np.array([[1.0] * 32 + [7.0] * 32])
    got = head_fn(x, hw, SHAPE)
    exp = np.array([[1.5 * x[0, pi[v]] / 5.0 * G_FINAL[pi[v]] for v in range(V)]])
    return got, exp


LAYER_PINS = [pin_attention_half, pin_ffn_only, pin_both_halves, pin_values_not_rotated,
              pin_scores_use_keys, pin_two_layers_in_order]


def _holds(got, exp):
    return got.shape == exp.shape and np.allclose(got, exp, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("pin", LAYER_PINS, ids=[p.__name__ for p in LAYER_PINS])
def test_layer_pin_holds(pin):
    got, exp = pin(ref.layer_forward)
    np.testing.assert_allclose(got, exp, rtol=1e-12, atol=1e-12)


def test_head_pin_holds():
    got, exp = pin_head(ref.head_logits)
    np.testing.assert_allclose(got, exp, rtol=1e-12, atol=1e-12)
    am, gap = oracle.argmax_gap(got)
    assert am[0] == int(np.argmax(exp[0]))


# ------------------------------------------------------------------ mutants
# (name, function, source fragment, replacement); each replacement is one
# plausible slip in the oracle's code.
MUTANTS = [
    ("ffn norm takes the attention gain", "layer_forward",
     "rmsnorm(x, bf16_to_f64(w.ffn_norm)", "rmsnorm(x, bf16_to_f64(w.attn_norm)"),
    ("attention norm takes the ffn gain", "layer_forward",
     "u = rmsnorm(x, bf16_to_f64(w.attn_norm)", "u = rmsnorm(x, bf16_to_f64(w.ffn_norm)"),
    ("silu on the up half", "layer_forward",
     "silu(gu[:, :F]) * gu[:, F:]", "gu[:, :F] * silu(gu[:, F:])"),
    ("attention residual dropped", "layer_forward",
     "x = x + linear_q4(o.reshape(N, Hq * d), w.wo)", "x = linear_q4(o.reshape(N, Hq * d), w.wo)"),
    ("ffn residual dropped", "layer_forward",
     "x = x + linear_q4(m, w.wd)", "x = linear_q4(m, w.wd)"),
    ("ffn norm of the pre-attention residual", "layer_forward",
     "x = x + linear_q4(o.reshape(N, Hq * d), w.wo)", "xa = x + linear_q4(o.reshape(N, Hq * d), w.wo)"),
    ("k and v slices swapped", "layer_forward",
     "k = qkv[:, Hq * d:(Hq + Hkv) * d]", "k = qkv[:, (Hq + Hkv) * d:]"),
    ("RoPE applied to the values", "layer_forward",
     "k = rope(k, pos[:, None], shape.rope_base)",
     "k = rope(k, pos[:, None], shape.rope_base)\n    v = rope(v, pos[:, None], shape.rope_base)"),
    ("softmax scale sqrt(d) dropped", "layer_forward",
     "o = tree_attention(q, k, v, kp, vp, parent)", "o = tree_attention(q * np.sqrt(d), k, v, kp, vp, parent)"),
    ("no attention norm", "layer_forward",
     "u = rmsnorm(x, bf16_to_f64(w.attn_norm), shape.rms_eps)", "u = x * bf16_to_f64(w.attn_norm)"),
    ("final norm without its gain", "head_logits",
     "rmsnorm(x, bf16_to_f64(hw.final_norm), shape.rms_eps)", "rmsnorm(x, 1.0, shape.rms_eps)"),
    ("layers applied in reverse", "verify_forward",
     "for w, (kp, vp) in zip(layers, kv):", "for w, (kp, vp) in reversed(list(zip(layers, kv))):"),
    ("no final norm", "head_logits",
     "u = rmsnorm(x, bf16_to_f64(hw.final_norm), shape.rms_eps)", "u = x * bf16_to_f64(hw.final_norm)"),
]


def _mutant(fn_name, old, new):
    src = inspect.getsource(getattr(ref, fn_name))
    assert src.count(old) == 1, "mutation site not found once: %r" % old
    src = src.replace(old, new)
    if "xa = x + linear_q4" in new:  # the FFN half then adds onto the post-attention residual
        src = src.replace("x = x + linear_q4(m, w.wd)", "x = xa + linear_q4(m, w.wd)")
    ns = dict(vars(ref))
    exec(compile(src, "<mutant>", "exec"), ns)
    return ns[fn_name]


@pytest.mark.filterwarnings("ignore::RuntimeWarning")  # a mutant may divide by a zero RMS
@pytest.mark.parametrize("name,fn_name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_each_mutant_is_caught(name, fn_name, old, new):
    mut = _mutant(fn_name, old, new)
    if fn_name == "layer_forward":
        caught = [p.__name__ for p in LAYER_PINS if not _holds(*p(mut))]
    elif fn_name == "verify_forward":
        caught = [] if _holds(*pin_two_layers_in_order(ref.layer_forward, mut)) else ["pin_two_layers_in_order"]
    else:
        caught = ["pin_head"] if not _holds(*pin_head(mut)) else []
    assert caught, "no pin catches the mutant: %s" % name


def test_unmutated_copy_passes_every_pin():
    # the exec-based copy itself is faithful: with no change every pin holds
    same = _mutant("layer_forward", "x = x + linear_q4(m, w.wd)", "x = x + linear_q4(m, w.wd)")
    assert all(_holds(*p(same)) for p in LAYER_PINS)
