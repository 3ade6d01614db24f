"""GPU parity of the 4-bit block-32 KV cache: the quantiser and the tree
attention over a 4-bit prefix, through the C ABI, against the oracle.

* ``lucev_kv_quantize_q4`` must equal ``oracle.quantize_q4_blocks`` bit for
  bit (nibbles, after unpacking the device bytes, and fp16 scales): both take
  the rounding decisions in fp32.
* ``lucev_tree_attention_q4`` runs on nibbles and scales the ORACLE wrote
  (packed into the device byte order by the test; no input comes from the
  device quantiser) and is compared with ``oracle.tree_attention`` over the
  fp64 prefix those codes stand for (``oracle.kv_prefix_from_q4``), to the
  bf16 attention's tolerance: the kernel takes the nearest fp16 of
  d * (q - 8) and of q and P (2^-11 relative each).
"""
import sys

import numpy as np
import pytest

import kv_nibbles
import oracle
import synth
from gpu_common import Guarded, bf16_bits_to_f64, need_gpu, row_rel_err
from test_gpu_q8 import ATTN_Q8_CASES, QUANT_CASES

pytestmark = pytest.mark.gpu

TOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bf16_bits(x):
    """fp64 values exact in bf16 -> bf16 bits (uint16)."""
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _clamping_amax():
    """The smallest bf16 value a in [2^-20, 2^-13] whose fp16 scale
    fp16(a / 7) is positive and rounds down far enough that a / d > 7.5
    (the clamp at 7 then decides the largest code)."""
    for bits in range(0x3580, 0x3900):
        a = float(np.array([bits << 16], np.uint32).view(np.float32)[0])
        dv = float((np.float32(a) / np.float32(7.0)).astype(np.float16))
        if dv > 0 and a / dv > 7.5:
            return a
    raise AssertionError("no clamping block found")


def _plant_specials(k_host, v_host):
    """Edge blocks written into bf16 caches (uint16 bits, K [Hkv][cap][d],
    V [Hkv][d][cap]): all zeros, an exact k * 2^-6 grid with |k| <= 7,
    half-way ties at d = 1, a clamping subnormal-scale block, and a
    large-magnitude block."""
    rng = np.random.default_rng(2)
    blk = [np.zeros(32)]
    g = rng.integers(-7, 8, 32).astype(np.float64)
    g[0] = -7
    blk.append(g * 2.0 ** -6)
    ties = np.zeros(32)
    ties[0] = 7.0
    ties[1:9] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 6.5, -6.5]
    blk.append(ties)
    a = _clamping_amax()
    tiny = rng.uniform(-0.5, 0.5, 32) * a
    tiny[0], tiny[1] = a, -a
    blk.append(tiny)
    blk.append(rng.standard_normal(32) * 3.0e4)
    for i, b in enumerate(blk):
        bits = _bf16_bits(b)
        k_host[0, i, :32] = bits
        v_host[-1, i, :32] = bits
    return len(blk)


@pytest.mark.parametrize("case", QUANT_CASES, ids=[c[0] for c in QUANT_CASES])
def test_kv_quantize_q4_bit_exact(case):
    torch = need_gpu()
    import tree_verify_amd as tv
    import synth.device as sd
    name, Hkv, d, P, cap = case
    say("4-bit quantiser case", name)
    cfg = synth.Config("q4_" + name, layers=1, hidden=128, n_q_heads=Hkv * 2, n_kv_heads=Hkv, head_dim=d,
                       ffn=128, vocab=64, prefix=P, nodes=1, max_children=None, max_depth=None, p_accept=0.7,
                       seed=717 + d)
    k, v = sd.kv_cache(cfg, 0, cfg.seed, cap, "cuda")
    kh = k.cpu().numpy().view(np.uint16).copy()
    vh = v.cpu().numpy().view(np.uint16).copy()
    _plant_specials(kh, vh)
    k = torch.from_numpy(kh.view(np.int16)).to("cuda")
    v = torch.from_numpy(vh.view(np.int16)).to("cuda")
    gk = [Guarded(torch, (Hkv, cap, d // 2), torch.uint8), Guarded(torch, (Hkv, cap, d // 32), torch.int16),
          Guarded(torch, (Hkv, d, cap // 2), torch.uint8), Guarded(torch, (Hkv, d, cap // 32), torch.int16)]
    for g_ in gk:
        g_.t.fill_(99)
    kn, ks, vn, vs = (g_.t for g_ in gk)
    shape = tv.make_shape(128, Hkv * 2, Hkv, d, 128, 64)
    tv.lucev_kv_quantize_q4(shape, tv.make_kv(k, v, P, cap), kn, ks, vn, vs,
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for g_, nm in zip(gk, ("K nibbles", "K scales", "V nibbles", "V scales")):
        g_.check(nm)
    kq0, ks0 = oracle.quantize_q4_blocks(oracle.bf16_to_f64(kh))
    vq0, vs0 = oracle.quantize_q4_blocks(oracle.bf16_to_f64(vh))
    assert np.array_equal(kv_nibbles.unpack(kn.cpu().numpy()), kq0)
    assert np.array_equal(ks.cpu().numpy().view(np.uint16), ks0)
    assert np.array_equal(kv_nibbles.unpack(vn.cpu().numpy()), vq0)
    assert np.array_equal(vs.cpu().numpy().view(np.uint16), vs0)
    # the planted blocks hit the zero block (nibbles 8) and the clamp
    assert np.all(vq0[-1, 0, :32] == 8)
    assert np.any(vq0[-1, 3, :2] == 15) and np.any(vq0[-1, 3, :2] == 1)


def _q4_cache_from_oracle(k, v):
    """Nibbles (one per entry) and scales written by the oracle from the
    device bf16 cache."""
    kh = k.cpu().numpy().view(np.uint16)
    vh = v.cpu().numpy().view(np.uint16)
    kq, ks = oracle.quantize_q4_blocks(oracle.bf16_to_f64(kh))
    vq, vs = oracle.quantize_q4_blocks(oracle.bf16_to_f64(vh))
    return kq, ks, vq, vs


def _run_q4_attention(torch, tv, shape, parent, kq, ks, vq, vs, P, cap, q, kt, vt, n, Hq, d):
    dev = [torch.from_numpy(np.ascontiguousarray(a)).to("cuda") for a in
           (kv_nibbles.pack(kq), ks.view(np.int16), kv_nibbles.pack(vq), vs.view(np.int16))]
    gout = Guarded(torch, (n * Hq * d,), torch.int16)
    ws_bytes = tv.lucev_workspace_bytes(shape, n, P)
    gws = Guarded(torch, (ws_bytes,), torch.uint8)
    kv = tv.make_kv_q4(dev[0], dev[1], dev[2], dev[3], P, cap)
    tv.lucev_tree_attention_q4(shape, tv.make_tree(parent, [0] * n), kv, q, kt, vt, gout.t, gws.t, ws_bytes,
                               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    gout.check("4-bit attention output")
    gws.check("workspace")
    return gout.t


@pytest.mark.parametrize("case", ATTN_Q8_CASES, ids=[c[0] for c in ATTN_Q8_CASES])
def test_tree_attention_q4_parity(case):
    torch = need_gpu()
    import tree_verify_amd as tv
    import synth.device as sd
    name, Hq, Hkv, d, P, rec, n = case
    cfg = synth.Config("attnq4_" + name, layers=1, hidden=128, n_q_heads=Hq, n_kv_heads=Hkv,
                       head_dim=d, ffn=128, vocab=64, prefix=P, nodes=n,
                       max_children=rec[0] if rec else None, max_depth=rec[1] if rec else None,
                       p_accept=0.7, seed=9494 + n)
    say("4-bit attention case", name)
    parent = synth.tree_parents(cfg)
    cap = ((P + 31) // 32) * 32 + 32
    k, v = sd.kv_cache(cfg, 0, cfg.seed, cap, "cuda")
    kq, ks, vq, vs = _q4_cache_from_oracle(k, v)
    q = sd.flat_table("normal", synth.stream_key(cfg.seed, 90, 0), n * Hq * d, "cuda")
    kt = sd.flat_table("normal", synth.stream_key(cfg.seed, 91, 0), n * Hkv * d, "cuda")
    vt = sd.flat_table("normal", synth.stream_key(cfg.seed, 92, 0), n * Hkv * d, "cuda")
    shape = tv.make_shape(cfg.hidden, Hq, Hkv, d, cfg.ffn, cfg.vocab)
    out = _run_q4_attention(torch, tv, shape, parent, kq, ks, vq, vs, P, cap, q, kt, vt, n, Hq, d)
    kp, vp = oracle.kv_prefix_from_q4(kq, ks, vq, vs, P)
    ref = oracle.tree_attention(bf16_bits_to_f64(q).reshape(n, Hq, d),
                                bf16_bits_to_f64(kt).reshape(n, Hkv, d),
                                bf16_bits_to_f64(vt).reshape(n, Hkv, d), kp, vp, parent)
    err = row_rel_err(bf16_bits_to_f64(out).reshape(n * Hq, d), ref.reshape(n * Hq, d))
    say("  max row rel err %.3e" % err.max())
    assert err.max() < TOL


def test_tree_attention_q4_longctx_sampled():
    """The 40-node tree against a 131072-token 4-bit prefix (the long-context
    layer shape, in the launch the timing uses), every output row checked
    against the oracle; the device quantiser writes the codes here and is
    itself checked bit-exact against the oracle's on the whole cache first."""
    torch = need_gpu()
    import tree_verify_amd as tv
    import synth.device as sd
    cfg = synth.get("longctx27b")
    Hq, Hkv, d, P, n = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.prefix, cfg.nodes
    say("4-bit long-context case", P, n)
    parent = synth.tree_parents(cfg)
    cap = P + 64
    k, v = sd.kv_cache(cfg, 0, cfg.seed, cap, "cuda")
    kn = torch.empty((Hkv, cap, d // 2), dtype=torch.uint8, device="cuda")
    ks = torch.empty((Hkv, cap, d // 32), dtype=torch.int16, device="cuda")
    vn = torch.empty((Hkv, d, cap // 2), dtype=torch.uint8, device="cuda")
    vs = torch.empty((Hkv, d, cap // 32), dtype=torch.int16, device="cuda")
    shape = tv.make_shape(cfg.hidden, Hq, Hkv, d, cfg.ffn, cfg.vocab)
    tv.lucev_kv_quantize_q4(shape, tv.make_kv(k, v, P, cap), kn, ks, vn, vs,
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    kq0, ks0, vq0, vs0 = _q4_cache_from_oracle(k, v)
    del k, v
    assert np.array_equal(kv_nibbles.unpack(kn.cpu().numpy()), kq0)
    assert np.array_equal(ks.cpu().numpy().view(np.uint16), ks0)
    assert np.array_equal(kv_nibbles.unpack(vn.cpu().numpy()), vq0)
    assert np.array_equal(vs.cpu().numpy().view(np.uint16), vs0)
    say("  quantiser bit-exact on the whole cache")
    q = sd.flat_table("normal", synth.stream_key(cfg.seed, 90, 0), n * Hq * d, "cuda")
    kt = sd.flat_table("normal", synth.stream_key(cfg.seed, 91, 0), n * Hkv * d, "cuda")
    vt = sd.flat_table("normal", synth.stream_key(cfg.seed, 92, 0), n * Hkv * d, "cuda")
    out = _run_q4_attention(torch, tv, shape, parent, kq0, ks0, vq0, vs0, P, cap, q, kt, vt, n, Hq, d)
    kp, vp = oracle.kv_prefix_from_q4(kq0, ks0, vq0, vs0, P)
    del kq0, vq0
    ref = oracle.tree_attention(bf16_bits_to_f64(q).reshape(n, Hq, d),
                                bf16_bits_to_f64(kt).reshape(n, Hkv, d),
                                bf16_bits_to_f64(vt).reshape(n, Hkv, d), kp, vp, parent)
    err = row_rel_err(bf16_bits_to_f64(out).reshape(n * Hq, d), ref.reshape(n * Hq, d))
    say("  max row rel err %.3e" % err.max())
    assert err.max() < TOL
