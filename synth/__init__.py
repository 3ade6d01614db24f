"""Seeded synthetic inputs for the tree-verification forward.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no norm, projection, attention or acceptance step): the
oracle under ``oracle/`` and the GPU library both receive exactly the arrays
built here, so the two sides see bit-identical inputs.

Randomness
    Every tensor has its own counter-based stream: Philox4x64-10 (Salmon,
    Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11)
    with key ``(seed, tensor_id << 32 | layer)``.  Philox block ``b`` uses the
    counter ``(b, 0, 0, 0)`` and yields four 64-bit words; each 64-bit word is
    split into two 32-bit words, low half first.  Element ``i`` of a tensor
    therefore reads 32-bit word ``i`` (or, for 4-bit weights, nibble ``i % 8``
    of word ``i // 8``).  On the CPU the stream comes from numpy's own Philox
    bit generator; ``synth.device`` holds a HIP implementation of the same
    generator so large workloads can be filled directly in device memory.

Value distributions (per tensor)
    * 4-bit weight codes q ~ U{0..15}.
    * fp16 block scales d ~ U(0.002, 0.02), rounded to the nearest fp16.
    * bf16 KV prefix and input hidden states ~ N(0, 1), rounded to bf16.
    * bf16 RMSNorm gains ~ U(0.5, 1.5), rounded to bf16.
    A continuous distribution rounded to a float format is sampled exactly by
    inverse CDF over the format's values: value ``v_j`` is chosen when the
    32-bit word ``u`` satisfies ``T_j <= u < T_{j+1}``, with
    ``T_j = round(2^32 * F(midpoint(v_{j-1}, v_j)))``.  The table is built once
    here in fp64 and handed unchanged to the device generator.
"""
from __future__ import annotations

import dataclasses
import functools
import math
from typing import Optional

import numpy as np

# ---------------------------------------------------------------- configs


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload: model shape, KV prefix length and draft tree recipe."""

    name: str
    layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    prefix: int
    nodes: int
    max_children: Optional[int]  # None: any earlier node may be a parent
    max_depth: Optional[int]
    p_accept: float
    seed: int
    rope_base: float = 10000.0
    rms_eps: float = 1e-6

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    # packed int4 bytes of one layer and of the head (18 B per 32 weights)
    def layer_weight_count(self) -> int:
        H, d, F = self.hidden, self.head_dim, self.ffn
        qkv = (self.n_q_heads + 2 * self.n_kv_heads) * d * H
        wo = H * self.n_q_heads * d
        return qkv + wo + 2 * F * H + H * F

    def head_weight_count(self) -> int:
        return self.vocab * self.hidden


_27B = dict(hidden=5120, n_q_heads=48, n_kv_heads=8, head_dim=128, ffn=17408,
            vocab=151936)

CONFIGS = {
    # tiny single layer, 8-node uniform recursive tree
    "tiny": Config("tiny", layers=1, hidden=256, n_q_heads=4, n_kv_heads=2,
                   head_dim=64, ffn=768, vocab=512, prefix=128, nodes=8,
                   max_children=None, max_depth=None, p_accept=0.7, seed=1000),
    # small-model shape, run as plain decode (1 node) and as a 16-node tree
    "small_decode": Config("small_decode", layers=24, hidden=1024, n_q_heads=8,
                           n_kv_heads=2, head_dim=128, ffn=3584, vocab=32768,
                           prefix=2048, nodes=1, max_children=None,
                           max_depth=None, p_accept=0.7, seed=1001),
    "small_tree": Config("small_tree", layers=24, hidden=1024, n_q_heads=8,
                         n_kv_heads=2, head_dim=128, ffn=3584, vocab=32768,
                         prefix=2048, nodes=16, max_children=None,
                         max_depth=None, p_accept=0.7, seed=1001),
    # one 27B-class layer (+ final norm and lm_head), 22-node tree
    "layer27b": Config("layer27b", layers=1, prefix=4096, nodes=22,
                       max_children=3, max_depth=8, p_accept=0.7, seed=1002,
                       **_27B),
    # the 64-layer 27B-class verify stack, 32K prefix, 22-node tree
    "stack27b": Config("stack27b", layers=64, prefix=32768, nodes=22,
                       max_children=3, max_depth=8, p_accept=0.7, seed=1003,
                       **_27B),
    # 8 layers, 128K prefix, 40-node wide tree
    "longctx27b": Config("longctx27b", layers=8, prefix=131072, nodes=40,
                         max_children=4, max_depth=10, p_accept=0.6, seed=1004,
                         **_27B),
}


def get(name: str) -> Config:
    return CONFIGS[name]


def run_seed(cfg: Config, run: int) -> int:
    """Seed of run ``run`` of a config (run 0 is the config's own seed)."""
    return cfg.seed + 10007 * run


# ---------------------------------------------------------------- streams

T_HIDDEN, T_ATTN_NORM, T_FFN_NORM = 1, 2, 3
T_WQKV_Q, T_WQKV_D, T_WO_Q, T_WO_D = 4, 5, 6, 7
T_WGU_Q, T_WGU_D, T_WD_Q, T_WD_D = 8, 9, 10, 11
T_K, T_V, T_FINAL_NORM, T_LM_Q, T_LM_D = 12, 13, 14, 15, 16
T_TREE, T_PLANT = 20, 21

_MASK64 = (1 << 64) - 1


def stream_key(seed: int, tensor_id: int, layer: int = 0):
    return (int(seed) & _MASK64, ((int(tensor_id) << 32) | (int(layer) & 0xFFFFFFFF)) & _MASK64)


def philox_words(key, start: int, count: int) -> np.ndarray:
    """32-bit words ``start .. start+count-1`` of the stream with ``key``."""
    if count <= 0:
        return np.zeros(0, np.uint32)
    b0 = start // 8
    b1 = (start + count + 7) // 8
    # numpy's Philox increments the counter before each block, so start one
    # below the first block we want (the all-ones counter wraps to zero).
    ctr = (b0 - 1) & _MASK64
    ctr_words = [ctr, _MASK64 if b0 == 0 else 0, _MASK64 if b0 == 0 else 0,
                 _MASK64 if b0 == 0 else 0]
    bg = np.random.Philox(key=np.array([key[0], key[1]], dtype=np.uint64),
                          counter=np.array(ctr_words, dtype=np.uint64))
    raw = bg.random_raw((b1 - b0) * 4).astype(np.uint64)
    words = raw.view(np.uint32)  # little-endian: low half first
    off = start - b0 * 8
    return words[off:off + count].copy()


def nibbles(key, n: int) -> np.ndarray:
    """``n`` 4-bit codes in 0..15 (uint8): code i is nibble i%8 of word i//8."""
    w = philox_words(key, 0, (n + 7) // 8)
    sh = (np.arange(8, dtype=np.uint32) * 4)
    q = ((w[:, None] >> sh[None, :]) & 15).astype(np.uint8).reshape(-1)
    return q[:n]


# ---------------------------------------------------------------- tables


def _bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore"):
        return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _f16_to_f64(u16: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore"):
        return u16.view(np.float16).astype(np.float64)


@dataclasses.dataclass(frozen=True)
class Table:
    """Exact inverse-CDF sampler over the values of a 16-bit float format."""

    thresholds: np.ndarray  # uint32 [K], strictly increasing
    values: np.ndarray      # uint16 [K + 1] (bit patterns)
    lo16: np.ndarray        # int32 [65537]: thresholds < (c << 16) counted

    def sample(self, words: np.ndarray) -> np.ndarray:
        words = np.asarray(words, dtype=np.uint32)
        c = (words >> 16).astype(np.int64)
        j = self.lo16[c].astype(np.int64)
        cnt = self.lo16[c + 1].astype(np.int64) - j
        one = cnt == 1
        if np.any(one):
            jo = j[one]
            j[one] = jo + (words[one] >= self.thresholds[jo])
        slow = cnt > 1
        if np.any(slow):
            j[slow] = np.searchsorted(self.thresholds, words[slow], side="right")
        return self.values[j]


def _build_table(vals_u16: np.ndarray, to_f64, cdf) -> Table:
    v = to_f64(vals_u16)
    order = np.argsort(v, kind="stable")
    v = v[order]
    u16 = vals_u16[order]
    mids = 0.5 * (v[1:] + v[:-1])
    t = np.rint(np.ldexp(cdf(mids), 32))
    t = np.clip(t, 0, 2.0 ** 32)
    # value j wins for T_j <= u < T_{j+1}; T_0 = 0 and T_{K+1} = 2^32
    lower = np.concatenate([[0.0], t])
    upper = np.concatenate([t, [2.0 ** 32]])
    keep = upper > lower
    u16 = u16[keep]
    lower = lower[keep]
    thr = lower[1:].astype(np.uint64)
    assert np.all(thr < 2 ** 32) and np.all(np.diff(thr.astype(np.int64)) > 0)
    thr32 = thr.astype(np.uint32)
    cells = (np.arange(65537, dtype=np.uint64) << np.uint64(16))
    lo16 = np.searchsorted(thr.astype(np.uint64), cells, side="left").astype(np.int32)
    return Table(thr32, u16.astype(np.uint16), lo16)


def _finite_bf16() -> np.ndarray:
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = _bf16_to_f64(u)
    ok = np.isfinite(f) & ~((u == 0x8000))  # drop -0 (same value as +0)
    return u[ok]


def _finite_f16() -> np.ndarray:
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = _f16_to_f64(u)
    ok = np.isfinite(f) & ~((u == 0x8000))
    return u[ok]


@functools.lru_cache(maxsize=None)
def normal_bf16_table() -> Table:
    from scipy.special import ndtr
    return _build_table(_finite_bf16(), _bf16_to_f64, ndtr)


@functools.lru_cache(maxsize=None)
def uniform_bf16_table(lo: float, hi: float) -> Table:
    return _build_table(_finite_bf16(), _bf16_to_f64,
                        lambda x: np.clip((x - lo) / (hi - lo), 0.0, 1.0))


@functools.lru_cache(maxsize=None)
def uniform_f16_table(lo: float, hi: float) -> Table:
    return _build_table(_finite_f16(), _f16_to_f64,
                        lambda x: np.clip((x - lo) / (hi - lo), 0.0, 1.0))


def scale_table() -> Table:
    return uniform_f16_table(0.002, 0.02)


def gain_table() -> Table:
    return uniform_bf16_table(0.5, 1.5)


def table_sample(table: Table, key, n: int, start: int = 0) -> np.ndarray:
    return table.sample(philox_words(key, start, n))


# ---------------------------------------------------------------- tensors

def weight_dims(cfg: Config, which: str):
    """(n_out, k_in) of a logical weight matrix.

    Logical row orders: ``qkv`` = [q heads; k heads; v heads] (head-major,
    ``head_dim`` rows each); ``gu`` = [gate rows; up rows]; ``o``, ``d`` and
    ``lm`` are plain ``[out, in]``.
    """
    H, d, F = cfg.hidden, cfg.head_dim, cfg.ffn
    return {
        "qkv": ((cfg.n_q_heads + 2 * cfg.n_kv_heads) * d, H),
        "o": (H, cfg.n_q_heads * d),
        "gu": (2 * F, H),
        "d": (H, F),
        "lm": (cfg.vocab, H),
    }[which]


_WIDS = {"qkv": (T_WQKV_Q, T_WQKV_D), "o": (T_WO_Q, T_WO_D),
         "gu": (T_WGU_Q, T_WGU_D), "d": (T_WD_Q, T_WD_D),
         "lm": (T_LM_Q, T_LM_D)}


def weight_q4(cfg: Config, which: str, layer: int = 0, seed: Optional[int] = None,
              rows: Optional[slice] = None):
    """Logical int4 weights: codes q uint8 [n_out, k_in], scales d fp16 bits.

    ``d[n, b]`` scales the block ``q[n, 32 b : 32 b + 32]``.  ``rows`` draws
    only a row range (the streams are random access).
    """
    seed = cfg.seed if seed is None else seed
    n_out, k_in = weight_dims(cfg, which)
    tq, td = _WIDS[which]
    r0, r1 = (0, n_out) if rows is None else (rows.start or 0, rows.stop)
    nb = k_in // 32
    kq = stream_key(seed, tq, layer)
    w = philox_words(kq, r0 * k_in // 8, (r1 - r0) * k_in // 8)
    sh = (np.arange(8, dtype=np.uint32) * 4)
    q = ((w[:, None] >> sh[None, :]) & 15).astype(np.uint8).reshape(r1 - r0, k_in)
    d = scale_table().sample(philox_words(stream_key(seed, td, layer), r0 * nb,
                                          (r1 - r0) * nb)).reshape(r1 - r0, nb)
    return q, d


def kv_prefix(cfg: Config, layer: int = 0, seed: Optional[int] = None,
              prefix: Optional[int] = None):
    """Logical bf16 KV prefix ``k, v`` of shape [n_kv_heads, prefix, head_dim].

    Keys are taken as already rotated (stored post-RoPE).
    """
    seed = cfg.seed if seed is None else seed
    P = cfg.prefix if prefix is None else prefix
    n = cfg.n_kv_heads * P * cfg.head_dim
    tab = normal_bf16_table()
    k = tab.sample(philox_words(stream_key(seed, T_K, layer), 0, n))
    v = tab.sample(philox_words(stream_key(seed, T_V, layer), 0, n))
    shp = (cfg.n_kv_heads, P, cfg.head_dim)
    return k.reshape(shp), v.reshape(shp)


def hidden_in(cfg: Config, seed: Optional[int] = None, nodes: Optional[int] = None):
    """Per-node input hidden states, bf16 bits [nodes, hidden] ~ N(0, 1)."""
    seed = cfg.seed if seed is None else seed
    N = cfg.nodes if nodes is None else nodes
    x = normal_bf16_table().sample(
        philox_words(stream_key(seed, T_HIDDEN, 0), 0, N * cfg.hidden))
    return x.reshape(N, cfg.hidden)


def gain(cfg: Config, which: str, layer: int = 0, seed: Optional[int] = None):
    """RMSNorm gain, bf16 bits [hidden] ~ U(0.5, 1.5)."""
    seed = cfg.seed if seed is None else seed
    tid = {"attn": T_ATTN_NORM, "ffn": T_FFN_NORM, "final": T_FINAL_NORM}[which]
    return gain_table().sample(philox_words(stream_key(seed, tid, layer), 0, cfg.hidden))


# ---------------------------------------------------------------- trees


def _uniform_index(word: int, count: int) -> int:
    return (int(word) * int(count)) >> 32


def tree_parents(cfg: Config, seed: Optional[int] = None,
                 nodes: Optional[int] = None) -> np.ndarray:
    """Random draft tree: ``parent[0] = -1``; node i picks an earlier parent.

    With no limits the parent is uniform over nodes ``0..i-1``.  With
    ``max_children``/``max_depth`` it is uniform over earlier nodes that still
    have fewer than ``max_children`` children and lie above ``max_depth``
    (root depth 0).  The depth bookkeeping here only enforces the recipe; the
    oracle and the library derive depths themselves.
    """
    seed = cfg.seed if seed is None else seed
    N = cfg.nodes if nodes is None else nodes
    w = philox_words(stream_key(seed, T_TREE, 0), 0, max(N, 1))
    parent = np.full(N, -1, np.int32)
    depth = [0] * N
    kids = [0] * N
    for i in range(1, N):
        elig = [j for j in range(i)
                if (cfg.max_children is None or kids[j] < cfg.max_children)
                and (cfg.max_depth is None or depth[j] < cfg.max_depth)]
        if not elig:
            raise ValueError("tree recipe cannot place node %d" % i)
        p = elig[_uniform_index(w[i], len(elig))]
        parent[i] = p
        depth[i] = depth[p] + 1
        kids[p] += 1
    return parent


def plant_tokens(cfg: Config, parent: np.ndarray, target_argmax: np.ndarray,
                 seed: Optional[int] = None, p_accept: Optional[float] = None) -> np.ndarray:
    """Drafted tokens: node i copies ``target_argmax[parent[i]]`` with
    probability ``p_accept``, else draws a uniform token (which may coincide).

    ``token[0]`` (the root, already accepted) is drawn uniformly; it takes no
    part in acceptance.  ``target_argmax`` is an input (the oracle's greedy
    token per node); nothing here computes it.
    """
    seed = cfg.seed if seed is None else seed
    p = cfg.p_accept if p_accept is None else p_accept
    N = len(parent)
    w = philox_words(stream_key(seed, T_PLANT, 0), 0, 2 * N)
    thr = int(math.floor(p * 2.0 ** 32))
    tok = np.zeros(N, np.int32)
    for i in range(N):
        rnd = _uniform_index(w[2 * i + 1], cfg.vocab)
        if i > 0 and int(w[2 * i]) < thr:
            tok[i] = int(target_argmax[parent[i]])
        else:
            tok[i] = rnd
    return tok
