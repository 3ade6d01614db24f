"""The C ABI on the CPU: the library loads, exports what lucev.h declares,
validates arguments before any launch, and the host packer writes the
documented layout."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _tv():
    import tree_verify_amd as tv
    if not os.path.exists(tv.LIB_PATH):
        pytest.skip("liblucev.so not built")
    return tv


def test_header_declarations_are_exported():
    tv = _tv()
    hdr = open(os.path.join(ROOT, "include", "lucev.h")).read()
    names = set(re.findall(r"^\w[\w\s\*]*?\b(lucev_\w+)\s*\(", hdr, re.M))
    assert names == set(tv.EXPORTED), names ^ set(tv.EXPORTED)
    L = ctypes.CDLL(tv.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert tv.lucev_abi_version() == 1
    assert tv.lucev_status_str(-3) == "malformed tree"


def _shape(tv, **kw):
    d = dict(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=768, vocab=512)
    d.update(kw)
    return tv.make_shape(**d)


def test_packed_bytes_and_workspace_size():
    tv = _tv()
    assert tv.lucev_q4_packed_bytes(16, 128) == 16 * 128 * 18 // 32
    assert tv.lucev_q4_packed_bytes(8, 128) == 0
    assert tv.lucev_q4_packed_bytes(16, 96) == 0
    s = _shape(tv)
    a = tv.lucev_workspace_bytes(s, 8, 128)
    b = tv.lucev_workspace_bytes(s, 64, 128)
    assert 0 < a <= b
    assert tv.lucev_workspace_bytes(s, 0, 128) == 0
    assert tv.lucev_workspace_bytes(s, 65, 128) == 0
    assert tv.lucev_workspace_bytes(_shape(tv, head_dim=96), 8, 128) == 0


def _unpack(tv, packed, n_out, k_in, kind, head_dim):
    """Read the documented packed layout back into logical (q, d)."""
    kg = k_in // 128
    nib = packed[: n_out * k_in // 2]
    sc = packed[n_out * k_in // 2:].view(np.uint16)
    q = np.zeros((n_out, k_in), np.uint8)
    d = np.zeros((n_out, k_in // 32), np.uint16)
    F = n_out // 2
    for p in range(n_out):
        if kind == tv.W_QKV:
            head, r = divmod(p, head_dim)
            i, loc = divmod(r, 16)
            L = head * head_dim + (8 * i + loc if loc < 8 else head_dim // 2 + 8 * i + loc - 8)
        elif kind == tv.W_GU:
            t, r = divmod(p, 16)
            L = (F if t % 2 else 0) + (t // 2) * 16 + r
        else:
            L = p
        t, lr = divmod(p, 16)
        for c in range(kg):
            base = (t * kg + c) * 1024
            for lq in range(4):
                lane = lq * 16 + lr
                words = nib[base + lane * 16: base + lane * 16 + 16].view(np.uint32)
                for j in range(4):
                    for e in range(8):
                        code = (int(words[j]) >> ((e & 1) * 16 + (e >> 1) * 4)) & 15
                        q[L, c * 128 + j * 32 + lq * 8 + e] = code
            for j in range(4):
                d[L, c * 4 + j] = sc[(t * kg + c) * 64 + lr * 4 + j]
    return q, d


@pytest.mark.parametrize("which", ["qkv", "gu", "o"])
def test_host_packer_round_trip(which):
    tv = _tv()
    cfg = synth.get("tiny")
    n_out, k_in = synth.weight_dims(cfg, which)
    q, d = synth.weight_q4(cfg, which, 0)
    kind = {"qkv": tv.W_QKV, "gu": tv.W_GU, "o": tv.W_PLAIN}[which]
    nb = tv.lucev_q4_packed_bytes(n_out, k_in)
    dst = np.zeros(nb, np.uint8)
    tv.lucev_q4_pack(kind, cfg.head_dim, np.ascontiguousarray(q), np.ascontiguousarray(d), n_out,
                     k_in, dst, nb)
    q2, d2 = _unpack(tv, dst, n_out, k_in, kind, cfg.head_dim)
    assert np.array_equal(q2, q) and np.array_equal(d2, d)


def test_pack_rejects_bad_arguments():
    tv = _tv()
    q = np.zeros((16, 128), np.uint8)
    d = np.zeros((16, 4), np.uint16)
    dst = np.zeros(tv.lucev_q4_packed_bytes(16, 128), np.uint8)
    with pytest.raises(tv.LucevError) as e:
        tv.lucev_q4_pack(0, 0, q, d, 16, 128, dst, 10)
    assert e.value.status == -4
    with pytest.raises(tv.LucevError) as e:
        tv.lucev_q4_pack(0, 0, q, d, 16, 100, dst, dst.size)
    assert e.value.status == -2
    with pytest.raises(tv.LucevError) as e:
        tv.lucev_q4_pack(0, 0, None, d, 16, 128, dst, dst.size)
    assert e.value.status == -1


def _no_gpu():
    # these tests hand the library fake device addresses that validation must
    # reject; never run them where a GPU could execute a launch by mistake
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("fake-pointer validation tests run on CPU-only hosts")
    except ImportError:
        pass


def _layer_args(tv, s):
    H, Hq, Hkv, d, F = s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn
    fake = 1 << 20  # never dereferenced: validation fails before any launch
    w = tv.lucev_layer_w(fake, fake, tv.lucev_q4(fake, (Hq + 2 * Hkv) * d, H), tv.lucev_q4(fake, H, Hq * d),
                         tv.lucev_q4(fake, 2 * F, H), tv.lucev_q4(fake, H, F))
    kv = tv.lucev_kv(fake, fake, 128, 256)
    return w, kv, fake


def _status(tv, **over):
    s = over.pop("shape", None) or _shape(tv)
    w, kv, fake = _layer_args(tv, s)
    tree = over.pop("tree", None) or tv.make_tree([-1, 0, 0, 1], [1, 2, 3, 4])
    kv = over.pop("kv", kv)
    ws_bytes = over.pop("ws_bytes", 1 << 40)
    resid = over.pop("resid", fake)
    L = tv.lib()
    return L.lucev_verify_layer(ctypes.byref(s), ctypes.byref(w), ctypes.byref(tree),
                                ctypes.byref(kv), resid, fake, fake, fake, ws_bytes, None)


def test_validation_codes_before_any_launch():
    tv = _tv()
    _no_gpu()
    assert _status(tv, tree=tv.make_tree([0, 0])) == -3            # parent[0] != -1
    assert _status(tv, tree=tv.make_tree([-1, 1])) == -3           # parent not earlier
    assert _status(tv, tree=tv.make_tree([-1, 0, 3, 1])) == -3     # forward reference
    assert _status(tv, tree=tv.make_tree([-1, 0], [0, 512])) == -3  # token >= vocab
    assert _status(tv, tree=tv.make_tree([-1, 0], [0, -2])) == -3
    t = tv.lucev_tree()
    t.n = 0
    assert _status(tv, tree=t) == -3
    t.n = 65
    assert _status(tv, tree=t) == -3
    assert _status(tv, shape=_shape(tv, hidden=200)) == -2
    assert _status(tv, shape=_shape(tv, n_q_heads=3)) == -2
    assert _status(tv, shape=_shape(tv, head_dim=32, n_q_heads=8)) == -2
    assert _status(tv, kv=tv.lucev_kv(1 << 20, 1 << 20, 300, 256)) == -8
    assert _status(tv, kv=tv.lucev_kv(1 << 20, 1 << 20, 8, 100)) == -8
    assert _status(tv, ws_bytes=64) == -4
    assert _status(tv, resid=(1 << 20) + 4) == -5
    assert _status(tv, resid=None) == -1
    assert "vocab" in tv.lucev_last_error() or tv.lucev_last_error()


def test_wrong_weight_shape_is_rejected():
    tv = _tv()
    _no_gpu()
    s = _shape(tv)
    w, kv, fake = _layer_args(tv, s)
    w.wo = tv.lucev_q4(fake, s.hidden, 128)  # wrong k_in
    tree = tv.make_tree([-1, 0])
    rc = tv.lib().lucev_verify_layer(ctypes.byref(s), ctypes.byref(w), ctypes.byref(tree),
                                     ctypes.byref(kv), fake, fake, fake, fake, 1 << 40, None)
    assert rc == -2 and "wo" in tv.lucev_last_error()


def test_commit_path_validation_before_any_launch():
    tv = _tv()
    _no_gpu()
    fake = 1 << 20

    def status(shape=None, layers=2, prefix=8, cap=100, n=5, path=fake, plen=fake, kc=None):
        kc = [fake] * layers if kc is None else kc
        try:
            tv.lucev_commit_path(shape or _shape(tv), kc, [fake] * len(kc), [fake] * len(kc),
                                 [fake] * len(kc), prefix, cap, n, path, plen)
        except tv.LucevError as e:
            return e.status
        return 0

    assert status(layers=0) == -2                    # no layer
    assert status(layers=65) == -2                   # more than one call can carry
    assert status(n=0) == -3 and status(n=65) == -3  # tree size
    assert status(path=None) == -1 and status(plen=None) == -1
    assert status(kc=[fake, None]) == -1             # a NULL layer pointer
    assert status(prefix=96, cap=100, n=5) == -8     # no room for the longest path
    assert status(prefix=-1) == -8
    assert status(shape=_shape(tv, hidden=200)) == -2
    # valid arguments get past validation to the device check (no GPU here)
    assert status(prefix=95, cap=100, n=5) in (-6, -7)


def test_project_logits_validation_before_any_launch():
    tv = _tv()
    _no_gpu()
    s = _shape(tv)
    w, kv, fake = _layer_args(tv, s)
    hw = tv.lucev_head_w(fake, tv.q4(fake, 512, 256))

    def status(n=4, x=fake, am=fake, logits=None, ws_bytes=1 << 40, shape=s, head=hw):
        try:
            tv.lucev_project_logits(shape, head, n, x, logits, am, None, fake, ws_bytes)
        except tv.LucevError as e:
            return e.status
        return 0

    assert status(n=0) == -3 and status(n=65) == -3
    assert status(x=None) == -1 and status(am=None) == -1
    assert status(x=fake + 4) == -5
    assert status(ws_bytes=64) == -4
    assert status(shape=_shape(tv, hidden=200)) == -2
    assert status(head=tv.lucev_head_w(fake, tv.q4(fake, 256, 256))) == -2  # lm_head rows != vocab
    assert status() in (-6, -7)  # valid: reaches the device check


def test_attention_row_limit_is_a_shape_error():
    # n * Hq / Hkv query rows of one KV head must fit one workgroup
    # (LUCEV_MAX_ATTN_ROWS); one row more is rejected before any launch
    tv = _tv()
    _no_gpu()
    s = _shape(tv, n_q_heads=32, n_kv_heads=2)  # 16 query heads per KV head
    parent32 = [-1] + list(range(31))
    assert _status(tv, shape=s, tree=tv.make_tree(parent32 + [31])) == -2   # 33 x 16 = 528 rows
    assert "512" in tv.lucev_last_error()
    assert _status(tv, shape=s, tree=tv.make_tree(parent32)) in (-6, -7)    # 512: reaches the device check
    fake = 1 << 20
    kv = tv.lucev_kv(fake, fake, 128, 256)
    try:
        tv.lucev_tree_attention(s, tv.make_tree(parent32 + [31]), kv, fake, fake, fake, fake, fake, 1 << 40)
        rc = 0
    except tv.LucevError as e:
        rc = e.status
    assert rc == -2


@pytest.mark.parametrize("bits", [8, 4])
def test_quantised_kv_validation_before_any_launch(bits):
    tv = _tv()
    _no_gpu()
    s = _shape(tv)
    fake = 1 << 20
    attn = tv.lucev_tree_attention_q8 if bits == 8 else tv.lucev_tree_attention_q4
    quant = tv.lucev_kv_quantize_q8 if bits == 8 else tv.lucev_kv_quantize_q4
    make = tv.make_kv_q8 if bits == 8 else tv.make_kv_q4

    def a_status(kv, out=fake):
        try:
            attn(s, tv.make_tree([-1, 0, 0]), kv, fake, fake, fake, out, fake, 1 << 40)
        except tv.LucevError as e:
            return e.status
        return 0

    def q_status(src, kc=fake, ks=fake):
        try:
            quant(s, src, kc, ks, fake, fake)
        except tv.LucevError as e:
            return e.status
        return 0

    assert a_status(make(fake, fake, fake, fake, 64, 100)) == -8        # capacity not a multiple of 32
    assert a_status(make(fake, fake, fake, fake, 130, 128)) == -8       # prefix beyond capacity
    assert a_status(make(fake, None, fake, fake, 64, 128)) == -1        # NULL scales
    assert a_status(make(fake + 8, fake, fake, fake, 64, 128)) == -5    # codes not 16-byte aligned
    assert a_status(make(fake, fake + 2, fake, fake, 64, 128)) == -5    # K scales not 8-byte aligned
    assert a_status(make(fake, fake, fake, fake, 64, 128), out=None) == -1
    assert a_status(make(fake, fake, fake, fake, 64, 128)) in (-6, -7)  # valid: reaches the device check
    assert a_status(make(None, None, None, None, 0, 0)) in (-6, -7)     # an empty prefix needs no arrays
    assert q_status(tv.lucev_kv(fake, fake, 64, 100)) == -8
    assert q_status(tv.lucev_kv(fake, fake, 64, 128), kc=None) == -1
    assert q_status(tv.lucev_kv(fake, fake, 64, 128), kc=fake + 4) == -5
    assert q_status(tv.lucev_kv(fake, fake, 64, 128), ks=fake + 1) == -5
    assert q_status(tv.lucev_kv(fake, fake, 64, 128)) in (-6, -7)


@pytest.mark.parametrize("bits", [8, 4])
def test_quantised_verify_layer_validation_before_any_launch(bits):
    tv = _tv()
    _no_gpu()
    s = _shape(tv)
    w, _, fake = _layer_args(tv, s)
    layer = tv.lucev_verify_layer_q8 if bits == 8 else tv.lucev_verify_layer_q4
    make = tv.make_kv_q8 if bits == 8 else tv.make_kv_q4

    def status(kv, resid=fake, ws_bytes=1 << 40, tree=None):
        try:
            layer(s, w, tree or tv.make_tree([-1, 0, 0, 1], [1, 2, 3, 4]), kv, resid, fake, fake, fake, ws_bytes)
        except tv.LucevError as e:
            return e.status
        return 0

    assert status(make(fake, fake, fake, fake, 128, 200)) == -8        # capacity not a multiple of 32
    assert status(make(fake, fake, fake, fake, 300, 256)) == -8        # prefix beyond capacity
    assert status(make(fake, None, fake, fake, 128, 256)) == -1        # NULL scales
    assert status(make(fake + 8, fake, fake, fake, 128, 256)) == -5    # codes not 16-byte aligned
    assert status(make(fake, fake, fake, fake, 128, 256), resid=None) == -1
    assert status(make(fake, fake, fake, fake, 128, 256), resid=fake + 4) == -5
    assert status(make(fake, fake, fake, fake, 128, 256), ws_bytes=64) == -4
    assert status(make(fake, fake, fake, fake, 128, 256), tree=tv.make_tree([0, 0])) == -3
    assert status(make(fake, fake, fake, fake, 128, 256)) in (-6, -7)  # valid: reaches the device check
