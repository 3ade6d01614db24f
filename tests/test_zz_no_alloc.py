"""The allocation-free tree attention (lucev_tree_attention_noalloc) against
lucev_tree_attention with a workspace: the same kernels, so the outputs must
be bit-identical.  Two calls in a row, the second with a smaller tree and a
shorter prefix, so the second reuses the scratch array the first filled."""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import bf16_bits_to_f64, need_gpu, row_rel_err

pytestmark = pytest.mark.gpu


def _inputs(torch, sd, Hq, Hkv, d, P, n, seed, rec):
    cfg = synth.Config("noalloc", layers=1, hidden=128, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, ffn=128,
                       vocab=64, prefix=P, nodes=n, max_children=rec[0], max_depth=rec[1], p_accept=0.7,
                       seed=seed)
    parent = synth.tree_parents(cfg)
    cap = ((P + 7) // 8) * 8 + 8
    k, v = sd.kv_cache(cfg, 0, cfg.seed, cap, "cuda")
    q = sd.flat_table("normal", synth.stream_key(seed, 90, 0), n * Hq * d, "cuda")
    kt = sd.flat_table("normal", synth.stream_key(seed, 91, 0), n * Hkv * d, "cuda")
    vt = sd.flat_table("normal", synth.stream_key(seed, 92, 0), n * Hkv * d, "cuda")
    return cfg, parent, cap, k, v, q, kt, vt


def test_noalloc_attention_equals_workspace_attention():
    torch = need_gpu()
    import tree_verify_amd as tv
    import synth.device as sd
    # first: the 27B group at the 40-node budget (the largest shape the array
    # takes at this prefix); second: 22 nodes against a shorter, ragged prefix
    for (n, P, rec, seed) in [(40, 4100, (4, 10), 5151), (22, 1037, (3, 8), 5252)]:
        Hq, Hkv, d = 48, 8, 128
        print("noalloc case n", n, "P", P, flush=True)
        cfg, parent, cap, k, v, q, kt, vt = _inputs(torch, sd, Hq, Hkv, d, P, n, seed, rec)
        shape = tv.make_shape(128, Hq, Hkv, d, 128, 64)
        tree = tv.make_tree(parent, [0] * n)
        kv = tv.make_kv(k, v, P, cap)
        ws_bytes = tv.lucev_workspace_bytes(shape, n, P)
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
        out_ws = torch.zeros(n * Hq * d, dtype=torch.int16, device="cuda")
        out_na = torch.full((n * Hq * d,), 0x7F7F, dtype=torch.int16, device="cuda")
        st = torch.cuda.current_stream().cuda_stream
        tv.lucev_tree_attention(shape, tree, kv, q, kt, vt, out_ws, ws, ws_bytes, st)
        tv.lucev_tree_attention_noalloc(shape, tree, kv, q, kt, vt, out_na, st)
        torch.cuda.synchronize()
        assert torch.equal(out_ws, out_na), "no-alloc output differs from the workspace path"
        kp, vp = synth.kv_prefix(cfg, 0)
        ref = oracle.tree_attention(bf16_bits_to_f64(q).reshape(n, Hq, d), bf16_bits_to_f64(kt).reshape(n, Hkv, d),
                                    bf16_bits_to_f64(vt).reshape(n, Hkv, d), oracle.bf16_to_f64(kp),
                                    oracle.bf16_to_f64(vp), parent)
        err = row_rel_err(bf16_bits_to_f64(out_na).reshape(n * Hq, d), ref.reshape(n * Hq, d))
        print("  bit-identical; max row rel err vs oracle %.3e" % err.max(), flush=True)
        assert err.max() < 2e-2


def test_noalloc_rejects_a_call_beyond_its_scratch():
    torch = need_gpu()
    import tree_verify_amd as tv
    import synth.device as sd
    # 64 nodes of 48/8 heads need 256 * 384 * 520 bytes = 51 MB > 32 MiB
    n, P, Hq, Hkv, d = 64, 4096, 48, 8, 128
    cfg, parent, cap, k, v, q, kt, vt = _inputs(torch, sd, Hq, Hkv, d, P, n, 5353, (None, None))
    shape = tv.make_shape(128, Hq, Hkv, d, 128, 64)
    out = torch.zeros(n * Hq * d, dtype=torch.int16, device="cuda")
    with pytest.raises(tv.LucevError) as e:
        tv.lucev_tree_attention_noalloc(shape, tv.make_tree(parent, [0] * n), tv.make_kv(k, v, P, cap), q, kt, vt,
                                        out, torch.cuda.current_stream().cuda_stream)
    assert e.value.status == -4 and "scratch" in str(e.value)
