"""GPU parity of the int8 block-32 KV cache: the quantiser and the tree
attention over an int8 prefix, through the C ABI, against the oracle.

* ``lucev_kv_quantize_q8`` must equal ``oracle.quantize_q8_blocks`` bit for
  bit (codes and fp16 scales): both take the rounding decisions in fp32.
* ``lucev_tree_attention_q8`` runs on codes and scales the ORACLE wrote (no
  input comes from the device quantiser) and is compared with
  ``oracle.tree_attention`` over the fp64 prefix those codes stand for
  (``oracle.kv_prefix_from_q8``), to the bf16 attention's tolerance: the
  kernel takes the nearest fp16 of d * code and of q and P (2^-11 relative
  each), far below the bf16 output's rounding.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_common import Guarded, bf16_bits_to_f64, need_gpu, row_rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bf16_bits(x):
    """fp64 values exact in bf16 -> bf16 bits (uint16)."""
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _plant_specials(k_host, v_host):
    """Blocks that exercise the quantiser's edges, written into bf16 caches
    (uint16 bits, K [Hkv][cap][d], V [Hkv][d][cap]): an all-zero block,
    exact k * 2^e grids, half-way ties at d = 1, a block whose fp16 scale is
    subnormal and rounds down (the clamp at 127), and a large-magnitude block."""
    blk = []
    blk.append(np.zeros(32))
    rng = np.random.default_rng(1)
    g = rng.integers(-127, 128, 32).astype(np.float64)
    g[0] = 127
    blk.append(g * 2.0 ** -6)
    ties = np.zeros(32)
    ties[0] = 127.0
    ties[1:9] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 100.5, -126.5]
    blk.append(ties)
    a = _clamping_amax()
    tiny = rng.uniform(-0.5, 0.5, 32) * a
    tiny[0], tiny[1] = a, -a
    blk.append(tiny)
    blk.append(rng.standard_normal(32) * 3.0e4)
    for i, b in enumerate(blk):
        bits = _bf16_bits(b)
        k_host[0, i, :32] = bits              # K: along the head dim of token i
        v_host[-1, i, :32] = bits             # V: along the tokens of dim i
    return len(blk)


def _clamping_amax():
    """The smallest bf16 value a in [2^-20, 2^-13] whose fp16 scale
    fp16(a / 127) is positive and rounds down far enough that a / d > 127.5."""
    for bits in range(0x3580, 0x3900):  # bf16 2^-20 .. 2^-13
        a = float(np.array([bits << 16], np.uint32).view(np.float32)[0])
        dv = float((np.float32(a) / np.float32(127.0)).astype(np.float16))
        if dv > 0 and a / dv > 127.5:
            return a
    raise AssertionError("no clamping block found")


QUANT_CASES = [
    # (name, Hkv, d, prefix, capacity)
    ("d64", 2, 64, 100, 128),
    ("d128_ragged", 8, 128, 1000, 1024),
    ("d128_4096", 8, 128, 4100, 4128),
]


@pytest.mark.parametrize("case", QUANT_CASES, ids=[c[0] for c in QUANT_CASES])
def test_kv_quantize_bit_exact(case):
    torch = need_gpu()
    import tree_verify_amd as tv
    import synth.device as sd
    name, Hkv, d, P, cap = case
    say("quantiser case", name)
    cfg = synth.Config("q8_" + name, layers=1, hidden=128, n_q_heads=Hkv * 2, n_kv_heads=Hkv, head_dim=d,
                       ffn=128, vocab=64, prefix=P, nodes=1, max_children=None, max_depth=None, p_accept=0.7,
                       seed=515 + d)
    k, v = sd.kv_cache(cfg, 0, cfg.seed, cap, "cuda")
    kh = k.cpu().numpy().view(np.uint16).copy()
    vh = v.cpu().numpy().view(np.uint16).copy()
    _plant_specials(kh, vh)
    k = torch.from_numpy(kh.view(np.int16)).to("cuda")
    v = torch.from_numpy(vh.view(np.int16)).to("cuda")
    gk = [Guarded(torch, (Hkv, cap, d), torch.int8), Guarded(torch, (Hkv, cap, d // 32), torch.int16),
          Guarded(torch, (Hkv, d, cap), torch.int8), Guarded(torch, (Hkv, d, cap // 32), torch.int16)]
    for g_ in gk:
        g_.t.fill_(99)
    kc, ks, vc, vs = (g_.t for g_ in gk)
    shape = tv.make_shape(128, Hkv * 2, Hkv, d, 128, 64)
    tv.lucev_kv_quantize_q8(shape, tv.make_kv(k, v, P, cap), kc, ks, vc, vs,
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for g_, nm in zip(gk, ("K codes", "K scales", "V codes", "V scales")):
        g_.check(nm)
    kc0, ks0 = oracle.quantize_q8_blocks(oracle.bf16_to_f64(kh))
    vc0, vs0 = oracle.quantize_q8_blocks(oracle.bf16_to_f64(vh))
    assert np.array_equal(kc.cpu().numpy(), kc0)
    assert np.array_equal(ks.cpu().numpy().view(np.uint16), ks0)
    assert np.array_equal(vc.cpu().numpy(), vc0)
    assert np.array_equal(vs.cpu().numpy().view(np.uint16), vs0)
    # the planted clamp case did clamp, so the check above covered it
    assert np.any(np.abs(vc0[-1, 3, :2].astype(int)) == 127)


ATTN_Q8_CASES = [
    # (name, Hq, Hkv, d, P, parent-recipe, n)
    ("tiny_shape", 4, 2, 64, 128, None, 8),            # 1 query tile, a 4-wave block
    ("ragged_prefix", 8, 2, 128, 1000, None, 16),      # ragged last tile
    ("27b_group", 48, 8, 128, 4100, (3, 8), 22),       # 9 query tiles on 12 one-tile waves
    ("five_tiles", 48, 8, 128, 1531, None, 12),        # 5 query tiles on 8 one-tile waves, ragged prefix
    ("wide_tree", 48, 8, 128, 2051, (4, 10), 40),      # 15 tiles, two per wave on 8 waves
    ("single_node", 48, 8, 128, 777, None, 1),
    ("empty_prefix", 8, 2, 128, 0, None, 5),
    ("short_prefix", 8, 2, 128, 33, None, 7),           # one tile, a 1-token second half
    ("max_rows", 32, 4, 128, 515, None, 64),            # 512 rows: two row groups of 16 tiles
    ("max_rows_d64", 16, 1, 64, 260, (4, 10), 32),      # 512 rows of head_dim 64
]


def _q8_cache_from_oracle(k, v):
    """Codes and scales written by the oracle from the device bf16 cache."""
    kh = k.cpu().numpy().view(np.uint16)
    vh = v.cpu().numpy().view(np.uint16)
    kc, ks = oracle.quantize_q8_blocks(oracle.bf16_to_f64(kh))
    vc, vs = oracle.quantize_q8_blocks(oracle.bf16_to_f64(vh))
    return kc, ks, vc, vs


def _run_q8_attention(torch, tv, shape, parent, kc, ks, vc, vs, P, cap, q, kt, vt, n, Hq, d):
    dev = [torch.from_numpy(np.ascontiguousarray(a)).to("cuda") for a in
           (kc, ks.view(np.int16), vc, vs.view(np.int16))]
    gout = Guarded(torch, (n * Hq * d,), torch.int16)
    ws_bytes = tv.lucev_workspace_bytes(shape, n, P)
    gws = Guarded(torch, (ws_bytes,), torch.uint8)
    kv = tv.make_kv_q8(dev[0], dev[1], dev[2], dev[3], P, cap)
    tv.lucev_tree_attention_q8(shape, tv.make_tree(parent, [0] * n), kv, q, kt, vt, gout.t, gws.t, ws_bytes,
                               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    gout.check("int8 attention output")
    gws.check("workspace")
    return gout.t


@pytest.mark.parametrize("case", ATTN_Q8_CASES, ids=[c[0] for c in ATTN_Q8_CASES])
def test_tree_attention_q8_parity(case):
    torch = need_gpu()
    import tree_verify_amd as tv
    import synth.device as sd
    name, Hq, Hkv, d, P, rec, n = case
    cfg = synth.Config("attnq8_" + name, layers=1, hidden=128, n_q_heads=Hq, n_kv_heads=Hkv,
                       head_dim=d, ffn=128, vocab=64, prefix=P, nodes=n,
                       max_children=rec[0] if rec else None, max_depth=rec[1] if rec else None,
                       p_accept=0.7, seed=8484 + n)
    say("int8 attention case", name)
    parent = synth.tree_parents(cfg)
    cap = ((P + 31) // 32) * 32 + 32
    k, v = sd.kv_cache(cfg, 0, cfg.seed, cap, "cuda")
    kc, ks, vc, vs = _q8_cache_from_oracle(k, v)
    q = sd.flat_table("normal", synth.stream_key(cfg.seed, 90, 0), n * Hq * d, "cuda")
    kt = sd.flat_table("normal", synth.stream_key(cfg.seed, 91, 0), n * Hkv * d, "cuda")
    vt = sd.flat_table("normal", synth.stream_key(cfg.seed, 92, 0), n * Hkv * d, "cuda")
    shape = tv.make_shape(cfg.hidden, Hq, Hkv, d, cfg.ffn, cfg.vocab)
    out = _run_q8_attention(torch, tv, shape, parent, kc, ks, vc, vs, P, cap, q, kt, vt, n, Hq, d)
    kp, vp = oracle.kv_prefix_from_q8(kc, ks, vc, vs, P)
    ref = oracle.tree_attention(bf16_bits_to_f64(q).reshape(n, Hq, d),
                                bf16_bits_to_f64(kt).reshape(n, Hkv, d),
                                bf16_bits_to_f64(vt).reshape(n, Hkv, d), kp, vp, parent)
    err = row_rel_err(bf16_bits_to_f64(out).reshape(n * Hq, d), ref.reshape(n * Hq, d))
    say("  max row rel err %.3e" % err.max())
    assert err.max() < TOL


def test_tree_attention_q8_longctx_sampled():
    """The 40-node tree against a 131072-token int8 prefix (the long-context
    layer shape, in the launch the timing uses), every output row checked
    against the oracle; the device quantiser writes the codes here and is
    itself checked bit-exact against the oracle's on the whole cache first."""
    torch = need_gpu()
    import tree_verify_amd as tv
    import synth.device as sd
    cfg = synth.get("longctx27b")
    Hq, Hkv, d, P, n = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.prefix, cfg.nodes
    say("int8 long-context case", P, n)
    parent = synth.tree_parents(cfg)
    cap = P + 64
    k, v = sd.kv_cache(cfg, 0, cfg.seed, cap, "cuda")
    kc = torch.empty((Hkv, cap, d), dtype=torch.int8, device="cuda")
    ks = torch.empty((Hkv, cap, d // 32), dtype=torch.int16, device="cuda")
    vc = torch.empty((Hkv, d, cap), dtype=torch.int8, device="cuda")
    vs = torch.empty((Hkv, d, cap // 32), dtype=torch.int16, device="cuda")
    shape = tv.make_shape(cfg.hidden, Hq, Hkv, d, cfg.ffn, cfg.vocab)
    tv.lucev_kv_quantize_q8(shape, tv.make_kv(k, v, P, cap), kc, ks, vc, vs,
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    kc0, ks0, vc0, vs0 = _q8_cache_from_oracle(k, v)
    del k, v
    assert np.array_equal(kc.cpu().numpy(), kc0) and np.array_equal(ks.cpu().numpy().view(np.uint16), ks0)
    assert np.array_equal(vc.cpu().numpy(), vc0) and np.array_equal(vs.cpu().numpy().view(np.uint16), vs0)
    say("  quantiser bit-exact on the whole cache")
    q = sd.flat_table("normal", synth.stream_key(cfg.seed, 90, 0), n * Hq * d, "cuda")
    kt = sd.flat_table("normal", synth.stream_key(cfg.seed, 91, 0), n * Hkv * d, "cuda")
    vt = sd.flat_table("normal", synth.stream_key(cfg.seed, 92, 0), n * Hkv * d, "cuda")
    out = _run_q8_attention(torch, tv, shape, parent, kc0, ks0, vc0, vs0, P, cap, q, kt, vt, n, Hq, d)
    kp, vp = oracle.kv_prefix_from_q8(kc0, ks0, vc0, vs0, P)
    del kc0, vc0
    ref = oracle.tree_attention(bf16_bits_to_f64(q).reshape(n, Hq, d),
                                bf16_bits_to_f64(kt).reshape(n, Hkv, d),
                                bf16_bits_to_f64(vt).reshape(n, Hkv, d), kp, vp, parent)
    err = row_rel_err(bf16_bits_to_f64(out).reshape(n * Hq, d), ref.reshape(n * Hq, d))
    say("  max row rel err %.3e" % err.max())
    assert err.max() < TOL
