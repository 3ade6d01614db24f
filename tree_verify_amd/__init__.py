"""lucev: the tree-verification forward of tree-based speculative decoding on
one MI355X (gfx950), as a C-ABI library with hand-written HIP kernels.

This module is the Python binding of ``include/lucev.h``: argument
marshalling only.  Every step of the forward runs in ``liblucev.so``; if the
library is missing, every call raises.  PyTorch is used by callers for device
memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblucev.so")

MAX_NODES = 64
W_PLAIN, W_QKV, W_GU = 0, 1, 2
STATUS = {0: "OK", -1: "NULL_ARG", -2: "BAD_SHAPE", -3: "BAD_TREE", -4: "WORKSPACE",
          -5: "ALIGN", -6: "HIP", -7: "DEVICE", -8: "BAD_KV"}

c_i32, c_i64, c_f32, c_vp, c_sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                   ctypes.c_void_p, ctypes.c_size_t)


class lucev_shape(ctypes.Structure):
    _fields_ = [("hidden", c_i32), ("n_q_heads", c_i32), ("n_kv_heads", c_i32),
                ("head_dim", c_i32), ("ffn", c_i32), ("vocab", c_i32),
                ("rms_eps", c_f32), ("rope_base", c_f32)]


class lucev_q4(ctypes.Structure):
    _fields_ = [("packed", c_vp), ("n_out", c_i64), ("k_in", c_i64)]


class lucev_layer_w(ctypes.Structure):
    _fields_ = [("attn_norm", c_vp), ("ffn_norm", c_vp), ("wqkv", lucev_q4),
                ("wo", lucev_q4), ("wgu", lucev_q4), ("wd", lucev_q4)]


class lucev_head_w(ctypes.Structure):
    _fields_ = [("final_norm", c_vp), ("lm_head", lucev_q4)]


class lucev_kv(ctypes.Structure):
    _fields_ = [("k", c_vp), ("v", c_vp), ("prefix_len", c_i32), ("capacity", c_i32)]


class lucev_kv_q8(ctypes.Structure):
    _fields_ = [("k_codes", c_vp), ("k_scales", c_vp), ("v_codes", c_vp), ("v_scales", c_vp),
                ("prefix_len", c_i32), ("capacity", c_i32)]


class lucev_kv_q4(ctypes.Structure):
    _fields_ = [("k_nibbles", c_vp), ("k_scales", c_vp), ("v_nibbles", c_vp), ("v_scales", c_vp),
                ("prefix_len", c_i32), ("capacity", c_i32)]


class lucev_kv_paged(ctypes.Structure):
    _fields_ = [("k_pages", c_vp), ("v_pages", c_vp), ("block_table", c_vp), ("n_pages", c_i32),
                ("prefix_len", c_i32)]


PAGE_TOKENS = 16


class lucev_tree(ctypes.Structure):
    _fields_ = [("n", c_i32), ("parent", c_i32 * MAX_NODES), ("token", c_i32 * MAX_NODES)]


class LucevError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__("%s failed: %s (%d): %s" % (where, STATUS.get(status, "?"), status, detail))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded liblucev.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("liblucev.so is not built (run __graft_entry__.build() or "
                               "python -m tree_verify_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.lucev_abi_version.restype = c_i32
        L.lucev_status_str.restype = ctypes.c_char_p
        L.lucev_status_str.argtypes = [c_i32]
        L.lucev_last_error.restype = ctypes.c_char_p
        L.lucev_q4_packed_bytes.restype = c_sz
        L.lucev_q4_packed_bytes.argtypes = [c_i64, c_i64]
        L.lucev_q4_pack.restype = c_i32
        L.lucev_q4_pack.argtypes = [c_i32, c_i32, c_vp, c_vp, c_i64, c_i64, c_vp, c_sz]
        L.lucev_q4_pack_device.restype = c_i32
        L.lucev_q4_pack_device.argtypes = [c_i32, c_i32, c_vp, c_vp, c_i64, c_i64, c_vp, c_sz, c_vp]
        L.lucev_workspace_bytes.restype = c_sz
        L.lucev_workspace_bytes.argtypes = [P(lucev_shape), c_i32, c_i32]
        L.lucev_workspace_init.restype = c_i32
        L.lucev_workspace_init.argtypes = [c_vp, c_sz, c_vp]
        L.lucev_verify_layer.restype = c_i32
        L.lucev_verify_layer.argtypes = [P(lucev_shape), P(lucev_layer_w), P(lucev_tree),
                                         P(lucev_kv), c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]
        L.lucev_tree_attention.restype = c_i32
        L.lucev_tree_attention.argtypes = [P(lucev_shape), P(lucev_tree), P(lucev_kv), c_vp,
                                           c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]
        L.lucev_accept_path.restype = c_i32
        L.lucev_accept_path.argtypes = [P(lucev_shape), P(lucev_head_w), P(lucev_tree), c_vp,
                                        c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]
        L.lucev_tree_attention_paged.restype = c_i32
        L.lucev_tree_attention_f32.restype = c_i32
        L.lucev_tree_attention_f32.argtypes = [P(lucev_shape), P(lucev_tree), P(lucev_kv), c_vp, c_vp, c_vp,
                                               c_vp, c_vp, c_sz, c_vp]
        L.lucev_tree_attention_q8.restype = c_i32
        L.lucev_tree_attention_q8.argtypes = [P(lucev_shape), P(lucev_tree), P(lucev_kv_q8), c_vp, c_vp, c_vp,
                                              c_vp, c_vp, c_sz, c_vp]
        L.lucev_kv_quantize_q8.restype = c_i32
        L.lucev_kv_quantize_q8.argtypes = [P(lucev_shape), P(lucev_kv), c_vp, c_vp, c_vp, c_vp, c_vp]
        L.lucev_tree_attention_q4.restype = c_i32
        L.lucev_tree_attention_q4.argtypes = [P(lucev_shape), P(lucev_tree), P(lucev_kv_q4), c_vp, c_vp, c_vp,
                                              c_vp, c_vp, c_sz, c_vp]
        for nm, kvt in (("lucev_verify_layer_q8", lucev_kv_q8), ("lucev_verify_layer_q4", lucev_kv_q4)):
            getattr(L, nm).restype = c_i32
            getattr(L, nm).argtypes = [P(lucev_shape), P(lucev_layer_w), P(lucev_tree), P(kvt), c_vp, c_vp,
                                       c_vp, c_vp, c_sz, c_vp]
        L.lucev_kv_quantize_q4.restype = c_i32
        L.lucev_kv_quantize_q4.argtypes = [P(lucev_shape), P(lucev_kv), c_vp, c_vp, c_vp, c_vp, c_vp]
        L.lucev_tree_attention_noalloc.restype = c_i32
        L.lucev_tree_attention_noalloc.argtypes = [P(lucev_shape), P(lucev_tree), P(lucev_kv), c_vp, c_vp,
                                                   c_vp, c_vp, c_vp]
        L.lucev_tree_attention_paged.argtypes = [P(lucev_shape), P(lucev_tree), P(lucev_kv_paged), c_vp,
                                                 c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]
        L.lucev_project_logits.restype = c_i32
        L.lucev_project_logits.argtypes = [P(lucev_shape), P(lucev_head_w), c_i32, c_vp, c_vp, c_vp,
                                           c_vp, c_vp, c_sz, c_vp]
        L.lucev_commit_path.restype = c_i32
        L.lucev_commit_path.argtypes = [P(lucev_shape), c_i32, P(c_vp), P(c_vp), P(c_vp), P(c_vp),
                                        c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]
        L.lucev_describe_attention.restype = c_i32
        L.lucev_describe_attention.argtypes = [P(lucev_shape), c_i32, c_i32, c_i32, ctypes.c_char_p, c_sz]
        L.lucev_set_gemv_max_rows.restype = c_i32
        L.lucev_set_gemv_max_rows.argtypes = [c_i32]
        L.lucev_stream_read.restype = c_i32
        L.lucev_stream_read.argtypes = [c_vp, c_sz, c_vp, c_vp]
        _lib = L
    return _lib


EXPORTED = ["lucev_abi_version", "lucev_status_str", "lucev_last_error",
            "lucev_q4_packed_bytes", "lucev_q4_pack", "lucev_q4_pack_device",
            "lucev_workspace_bytes", "lucev_workspace_init", "lucev_verify_layer",
            "lucev_tree_attention", "lucev_tree_attention_f32", "lucev_tree_attention_noalloc",
            "lucev_tree_attention_q8", "lucev_kv_quantize_q8", "lucev_tree_attention_q4", "lucev_kv_quantize_q4",
            "lucev_verify_layer_q8", "lucev_verify_layer_q4",
            "lucev_tree_attention_paged", "lucev_accept_path", "lucev_project_logits",
            "lucev_commit_path", "lucev_describe_attention", "lucev_stream_read",
            "lucev_set_gemv_max_rows"]


def _ptr(x) -> Optional[int]:
    """Device/host address of a tensor, numpy array or int (None stays NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):
        return x.ctypes.data
    raise TypeError("cannot take the address of %r" % type(x))


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise LucevError(rc, where, lib().lucev_last_error().decode())


def make_shape(hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, rms_eps=1e-6,
               rope_base=10000.0) -> lucev_shape:
    return lucev_shape(hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, rms_eps, rope_base)


def make_tree(parent: Sequence[int], token: Optional[Sequence[int]] = None) -> lucev_tree:
    t = lucev_tree()
    t.n = len(parent)
    for i, p in enumerate(parent):
        t.parent[i] = int(p)
    if token is not None:
        for i, tk in enumerate(token):
            t.token[i] = int(tk)
    return t


def q4(packed, n_out: int, k_in: int) -> lucev_q4:
    return lucev_q4(_ptr(packed), n_out, k_in)


def make_kv(k, v, prefix_len: int, capacity: int) -> lucev_kv:
    return lucev_kv(_ptr(k), _ptr(v), prefix_len, capacity)


# ---------------------------------------------------------------- the ABI


def lucev_abi_version() -> int:
    return lib().lucev_abi_version()


def lucev_status_str(status: int) -> str:
    return lib().lucev_status_str(status).decode()


def lucev_last_error() -> str:
    return lib().lucev_last_error().decode()


def lucev_q4_packed_bytes(n_out: int, k_in: int) -> int:
    return lib().lucev_q4_packed_bytes(n_out, k_in)


def lucev_q4_pack(kind, head_dim, q, d, n_out, k_in, dst, dst_bytes) -> None:
    _check(lib().lucev_q4_pack(kind, head_dim, _ptr(q), _ptr(d), n_out, k_in, _ptr(dst), dst_bytes),
           "lucev_q4_pack")


def lucev_q4_pack_device(kind, head_dim, q, d, n_out, k_in, dst, dst_bytes, stream=None) -> None:
    _check(lib().lucev_q4_pack_device(kind, head_dim, _ptr(q), _ptr(d), n_out, k_in, _ptr(dst),
                                      dst_bytes, stream), "lucev_q4_pack_device")


def lucev_workspace_bytes(shape: lucev_shape, n_nodes: int, prefix_len: int) -> int:
    return lib().lucev_workspace_bytes(ctypes.byref(shape), n_nodes, prefix_len)


def lucev_workspace_init(ws, ws_bytes, stream=None) -> None:
    _check(lib().lucev_workspace_init(_ptr(ws), ws_bytes, stream), "lucev_workspace_init")


def lucev_verify_layer(shape, w, tree, kv, resid_io, k_tree_out, v_tree_out, ws, ws_bytes,
                       stream=None) -> None:
    _check(lib().lucev_verify_layer(ctypes.byref(shape), ctypes.byref(w), ctypes.byref(tree),
                                    ctypes.byref(kv), _ptr(resid_io), _ptr(k_tree_out),
                                    _ptr(v_tree_out), _ptr(ws), ws_bytes, stream),
           "lucev_verify_layer")


def lucev_verify_layer_q8(shape, w, tree, kv, resid_io, k_tree_out, v_tree_out, ws, ws_bytes,
                          stream=None) -> None:
    _check(lib().lucev_verify_layer_q8(ctypes.byref(shape), ctypes.byref(w), ctypes.byref(tree),
                                       ctypes.byref(kv), _ptr(resid_io), _ptr(k_tree_out),
                                       _ptr(v_tree_out), _ptr(ws), ws_bytes, stream),
           "lucev_verify_layer_q8")


def lucev_verify_layer_q4(shape, w, tree, kv, resid_io, k_tree_out, v_tree_out, ws, ws_bytes,
                          stream=None) -> None:
    _check(lib().lucev_verify_layer_q4(ctypes.byref(shape), ctypes.byref(w), ctypes.byref(tree),
                                       ctypes.byref(kv), _ptr(resid_io), _ptr(k_tree_out),
                                       _ptr(v_tree_out), _ptr(ws), ws_bytes, stream),
           "lucev_verify_layer_q4")


def lucev_tree_attention(shape, tree, kv, q, k_tree, v_tree, out, ws, ws_bytes, stream=None) -> None:
    _check(lib().lucev_tree_attention(ctypes.byref(shape), ctypes.byref(tree), ctypes.byref(kv),
                                      _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(out), _ptr(ws),
                                      ws_bytes, stream), "lucev_tree_attention")


def lucev_tree_attention_f32(shape, tree, kv, q, k_tree, v_tree, out, ws, ws_bytes, stream=None) -> None:
    _check(lib().lucev_tree_attention_f32(ctypes.byref(shape), ctypes.byref(tree), ctypes.byref(kv),
                                          _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(out), _ptr(ws),
                                          ws_bytes, stream), "lucev_tree_attention_f32")


def make_kv_q8(k_codes, k_scales, v_codes, v_scales, prefix_len: int, capacity: int) -> lucev_kv_q8:
    return lucev_kv_q8(_ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales), prefix_len, capacity)


def lucev_kv_quantize_q8(shape, src, k_codes, k_scales, v_codes, v_scales, stream=None) -> None:
    _check(lib().lucev_kv_quantize_q8(ctypes.byref(shape), ctypes.byref(src), _ptr(k_codes), _ptr(k_scales),
                                      _ptr(v_codes), _ptr(v_scales), stream), "lucev_kv_quantize_q8")


def lucev_tree_attention_q8(shape, tree, kv, q, k_tree, v_tree, out, ws, ws_bytes, stream=None) -> None:
    _check(lib().lucev_tree_attention_q8(ctypes.byref(shape), ctypes.byref(tree), ctypes.byref(kv), _ptr(q),
                                         _ptr(k_tree), _ptr(v_tree), _ptr(out), _ptr(ws), ws_bytes, stream),
           "lucev_tree_attention_q8")


def make_kv_q4(k_nibbles, k_scales, v_nibbles, v_scales, prefix_len: int, capacity: int) -> lucev_kv_q4:
    return lucev_kv_q4(_ptr(k_nibbles), _ptr(k_scales), _ptr(v_nibbles), _ptr(v_scales), prefix_len, capacity)


def lucev_kv_quantize_q4(shape, src, k_nibbles, k_scales, v_nibbles, v_scales, stream=None) -> None:
    _check(lib().lucev_kv_quantize_q4(ctypes.byref(shape), ctypes.byref(src), _ptr(k_nibbles), _ptr(k_scales),
                                      _ptr(v_nibbles), _ptr(v_scales), stream), "lucev_kv_quantize_q4")


def lucev_tree_attention_q4(shape, tree, kv, q, k_tree, v_tree, out, ws, ws_bytes, stream=None) -> None:
    _check(lib().lucev_tree_attention_q4(ctypes.byref(shape), ctypes.byref(tree), ctypes.byref(kv), _ptr(q),
                                         _ptr(k_tree), _ptr(v_tree), _ptr(out), _ptr(ws), ws_bytes, stream),
           "lucev_tree_attention_q4")


NOALLOC_SCRATCH_BYTES = 32 << 20


def lucev_tree_attention_noalloc(shape, tree, kv, q, k_tree, v_tree, out, stream=None) -> None:
    _check(lib().lucev_tree_attention_noalloc(ctypes.byref(shape), ctypes.byref(tree), ctypes.byref(kv),
                                              _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(out), stream),
           "lucev_tree_attention_noalloc")


def make_kv_paged(k_pages, v_pages, block_table, n_pages: int, prefix_len: int) -> lucev_kv_paged:
    return lucev_kv_paged(_ptr(k_pages), _ptr(v_pages), _ptr(block_table), n_pages, prefix_len)


def lucev_tree_attention_paged(shape, tree, kv, q, k_tree, v_tree, out, ws, ws_bytes,
                               stream=None) -> None:
    _check(lib().lucev_tree_attention_paged(ctypes.byref(shape), ctypes.byref(tree), ctypes.byref(kv),
                                            _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(out), _ptr(ws),
                                            ws_bytes, stream), "lucev_tree_attention_paged")


def lucev_accept_path(shape, w, tree, resid, logits_out, argmax_out, gap_out, path_out,
                      path_len_out, committed_out, ws, ws_bytes, stream=None) -> None:
    _check(lib().lucev_accept_path(ctypes.byref(shape), ctypes.byref(w), ctypes.byref(tree),
                                   _ptr(resid), _ptr(logits_out), _ptr(argmax_out), _ptr(gap_out),
                                   _ptr(path_out), _ptr(path_len_out), _ptr(committed_out),
                                   _ptr(ws), ws_bytes, stream), "lucev_accept_path")


def lucev_project_logits(shape, w, n_rows, x, logits_out, argmax_out, gap_out, ws, ws_bytes,
                         stream=None) -> None:
    _check(lib().lucev_project_logits(ctypes.byref(shape), ctypes.byref(w), n_rows, _ptr(x),
                                      _ptr(logits_out), _ptr(argmax_out), _ptr(gap_out), _ptr(ws),
                                      ws_bytes, stream), "lucev_project_logits")


MAX_COMMIT_LAYERS = 64


def lucev_commit_path(shape, k_cache, v_cache, k_tree, v_tree, prefix_len, capacity, n_nodes,
                      path, path_len, stream=None) -> None:
    """k_cache / v_cache / k_tree / v_tree: sequences of one device buffer per
    layer (at most MAX_COMMIT_LAYERS); marshalled into host pointer arrays."""
    n = len(k_cache)
    arrs = []
    for seq in (k_cache, v_cache, k_tree, v_tree):
        if len(seq) != n:
            raise ValueError("commit_path: per-layer lists differ in length")
        arrs.append((ctypes.c_void_p * max(n, 1))(*[_ptr(x) for x in seq]))
    _check(lib().lucev_commit_path(ctypes.byref(shape), n, arrs[0], arrs[1], arrs[2], arrs[3],
                                   prefix_len, capacity, n_nodes, _ptr(path), _ptr(path_len),
                                   stream), "lucev_commit_path")


ATTN_BF16, ATTN_F32, ATTN_PAGED, ATTN_Q8, ATTN_Q4 = 0, 1, 2, 3, 4


def lucev_describe_attention(shape, n_nodes: int, prefix_len: int, variant: int) -> str:
    buf = ctypes.create_string_buffer(512)
    _check(lib().lucev_describe_attention(ctypes.byref(shape), n_nodes, prefix_len, variant, buf, len(buf)),
           "lucev_describe_attention")
    return buf.value.decode()


def lucev_stream_read(src, nbytes: int, sink, stream=None) -> None:
    _check(lib().lucev_stream_read(_ptr(src), nbytes, _ptr(sink), stream), "lucev_stream_read")


def lucev_set_gemv_max_rows(rows: int) -> None:
    _check(lib().lucev_set_gemv_max_rows(rows), "lucev_set_gemv_max_rows")
