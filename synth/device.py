"""Fill synthetic workloads directly in device memory.

Same streams and tables as ``synth`` (the CPU generator), evaluated by the HIP
twin in ``libsynth_dev.so``; a GPU test checks the two agree bit for bit.
Weights are drawn in logical form and then packed with the library's own
public packer (``lucev_q4_pack_device``).  Input generation only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional

import numpy as np
import torch

import synth

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsynth_dev.so")
_lib = None
_tables: Dict = {}

u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libsynth_dev.so is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.synth_dev_raw_words.argtypes = [u64, u64, u64, u64, vp, vp]
        L.synth_dev_nibbles.argtypes = [u64, u64, u64, u64, vp, vp]
        L.synth_dev_table.argtypes = [u64, u64, u64, u64, vp, ctypes.c_int, vp, vp,
                                      i64, i64, i64, i64, i64, vp]
        _lib = L
    return _lib


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check(rc, what):
    if rc != 0:
        raise RuntimeError("%s failed (%d)" % (what, rc))


def device_table(name: str, device) -> tuple:
    key = (name, str(device))
    if key not in _tables:
        t = {"normal": synth.normal_bf16_table, "scale": synth.scale_table,
             "gain": synth.gain_table}[name]()
        thr = torch.from_numpy(t.thresholds.view(np.int32).copy()).to(device)
        vals = torch.from_numpy(t.values.view(np.int16).copy()).to(device)
        _tables[key] = (thr, vals, len(t.thresholds))
    return _tables[key]


def raw_words(key, start: int, n: int, device) -> torch.Tensor:
    out = torch.empty(n, dtype=torch.int32, device=device)
    _check(lib().synth_dev_raw_words(key[0], key[1], start, n, out.data_ptr(), _stream()), "raw_words")
    return out


def nibbles(key, start_word: int, n_words: int, out: torch.Tensor) -> torch.Tensor:
    assert out.dtype == torch.uint8 and out.numel() >= n_words * 8 and out.is_contiguous()
    _check(lib().synth_dev_nibbles(key[0], key[1], start_word, n_words, out.data_ptr(), _stream()),
           "nibbles")
    return out


def table_fill(name: str, key, start: int, n: int, out: torch.Tensor, D1: int, D2: int,
               s0: int, s1: int, s2: int) -> torch.Tensor:
    thr, vals, k = device_table(name, out.device)
    _check(lib().synth_dev_table(key[0], key[1], start, n, thr.data_ptr(), k, vals.data_ptr(),
                                 out.data_ptr(), D1, D2, s0, s1, s2, _stream()), "table")
    return out


def flat_table(name: str, key, n: int, device, start: int = 0) -> torch.Tensor:
    out = torch.empty(n, dtype=torch.int16, device=device)
    return table_fill(name, key, start, n, out, 1, n, 0, 0, 1)


# ---------------------------------------------------------------- tensors

_KIND = {"qkv": 1, "o": 0, "gu": 2, "d": 0, "lm": 0}


def logical_q4(cfg, which: str, layer: int, seed: int, device):
    """Logical codes (uint8 [n_out, k_in]) and scales (fp16 bits [n_out, k_in/32])."""
    n_out, k_in = synth.weight_dims(cfg, which)
    tq, td = synth._WIDS[which]
    q = torch.empty(n_out * k_in, dtype=torch.uint8, device=device)
    nibbles(synth.stream_key(seed, tq, layer), 0, n_out * k_in // 8, q)
    d = flat_table("scale", synth.stream_key(seed, td, layer), n_out * (k_in // 32), device)
    return q.view(n_out, k_in), d.view(n_out, k_in // 32)


def packed_q4(cfg, which: str, layer: int, seed: int, device) -> torch.Tensor:
    import tree_verify_amd as tv
    n_out, k_in = synth.weight_dims(cfg, which)
    q, d = logical_q4(cfg, which, layer, seed, device)
    nbytes = tv.lucev_q4_packed_bytes(n_out, k_in)
    packed = torch.empty(nbytes, dtype=torch.uint8, device=device)
    tv.lucev_q4_pack_device(_KIND[which], cfg.head_dim, q, d, n_out, k_in, packed, nbytes, _stream())
    del q, d
    return packed


def kv_cache(cfg, layer: int, seed: int, capacity: int, device, prefix: Optional[int] = None):
    """bf16 K [Hkv][capacity][d] and dim-major V [Hkv][d][capacity]; tokens past
    the prefix are zero."""
    P = cfg.prefix if prefix is None else prefix
    Hkv, d = cfg.n_kv_heads, cfg.head_dim
    k = torch.zeros(Hkv, capacity, d, dtype=torch.int16, device=device)
    v = torch.zeros(Hkv, d, capacity, dtype=torch.int16, device=device)
    n = Hkv * P * d
    table_fill("normal", synth.stream_key(seed, synth.T_K, layer), 0, n, k, P, d, capacity * d, d, 1)
    table_fill("normal", synth.stream_key(seed, synth.T_V, layer), 0, n, v, P, d, d * capacity, 1, capacity)
    return k, v


def gain(cfg, which: str, layer: int, seed: int, device) -> torch.Tensor:
    tid = {"attn": synth.T_ATTN_NORM, "ffn": synth.T_FFN_NORM, "final": synth.T_FINAL_NORM}[which]
    return flat_table("gain", synth.stream_key(seed, tid, layer), cfg.hidden, device)


def hidden_in(cfg, seed: int, nodes: int, device) -> torch.Tensor:
    x = flat_table("normal", synth.stream_key(seed, synth.T_HIDDEN, 0), nodes * cfg.hidden, device)
    return x.view(nodes, cfg.hidden)


class Workload:
    """All device tensors of one config and seed (weights packed, KV caches)."""

    def __init__(self, cfg, seed: Optional[int] = None, device="cuda", layers: Optional[int] = None,
                 capacity: Optional[int] = None, with_head: bool = True):
        self.cfg = cfg
        self.seed = cfg.seed if seed is None else seed
        self.device = torch.device(device)
        self.n_layers = cfg.layers if layers is None else layers
        self.capacity = capacity if capacity is not None else ((cfg.prefix + 64 + 7) // 8) * 8
        self.layers: List[dict] = []
        for l in range(self.n_layers):
            lw = {w: packed_q4(cfg, w, l, self.seed, self.device) for w in ("qkv", "o", "gu", "d")}
            lw["attn_norm"] = gain(cfg, "attn", l, self.seed, self.device)
            lw["ffn_norm"] = gain(cfg, "ffn", l, self.seed, self.device)
            lw["k"], lw["v"] = kv_cache(cfg, l, self.seed, self.capacity, self.device)
            self.layers.append(lw)
        self.head = None
        if with_head:
            self.head = {"lm": packed_q4(cfg, "lm", 0, self.seed, self.device),
                         "final_norm": gain(cfg, "final", 0, self.seed, self.device)}
        self.x_in = hidden_in(cfg, self.seed, cfg.nodes, self.device)
        # everything above was enqueued on the current stream; callers may run
        # the step on another one
        torch.cuda.synchronize(self.device)

    def x_in_f32(self) -> torch.Tensor:
        """Input hidden states widened exactly from bf16 to fp32."""
        b = self.x_in.to(torch.int32) & 0xFFFF
        return (b << 16).view(torch.float32)
