"""fp64 reference of one tree-verification step (test infrastructure only).

Inputs are the exact bf16 / fp16 / uint8 values the GPU receives, widened
exactly to fp64; nothing is rounded inside.  See the package docstring for
the passages each step follows.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

# ---------------------------------------------------------------- formats


def bf16_to_f64(u16) -> np.ndarray:
    """bf16 bit patterns -> fp64 (exact)."""
    u16 = np.asarray(u16, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_to_f64(u16) -> np.ndarray:
    """fp16 bit patterns -> fp64 (exact)."""
    return np.asarray(u16, dtype=np.uint16).view(np.float16).astype(np.float64)


@dataclasses.dataclass(frozen=True)
class Shape:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-6
    rope_base: float = 10000.0


@dataclasses.dataclass
class LayerWeights:
    """One layer in logical form (codes ``q`` uint8, block scales ``d`` fp16 bits).

    ``wqkv`` rows are [q heads; k heads; v heads], ``wgu`` rows are
    [gate; up]; each ``(q, d)`` pair holds ``W[n, k] = d[n, k // 32] * (q[n, k] - 8)``.
    """
    attn_norm: np.ndarray  # bf16 bits [H]
    ffn_norm: np.ndarray   # bf16 bits [H]
    wqkv: tuple
    wo: tuple
    wgu: tuple
    wd: tuple


@dataclasses.dataclass
class HeadWeights:
    final_norm: np.ndarray  # bf16 bits [H]
    lm: tuple               # (q [V, H], d [V, H/32])


# ---------------------------------------------------------------- tree


def tree_depths(parent: Sequence[int]) -> np.ndarray:
    """depth[0] = 0, depth[i] = depth[parent[i]] + 1 (parents precede children)."""
    parent = [int(p) for p in parent]
    depth = np.zeros(len(parent), np.int64)
    for i in range(1, len(parent)):
        depth[i] = depth[parent[i]] + 1
    return depth


def tree_ancestors(parent: Sequence[int]) -> List[List[int]]:
    """anc(i) = {i} plus anc(parent[i]), listed in increasing node index."""
    out = []
    for i in range(len(parent)):
        chain = []
        j = i
        while j >= 0:
            chain.append(j)
            j = int(parent[j])
        out.append(sorted(chain))
    return out


# ---------------------------------------------------------------- layer math


def dequant_q4(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """W[n, k] = d[n, k // 32] * (q[n, k] - 8), blocks of 32 along the input axis."""
    q = np.asarray(q)
    n_out, k_in = q.shape
    scale = f16_to_f64(d).reshape(n_out, k_in // 32)
    w = (q.astype(np.float64) - 8.0).reshape(n_out, k_in // 32, 32)
    return (w * scale[:, :, None]).reshape(n_out, k_in)


def linear_q4(x: np.ndarray, qd: tuple, row_chunk: int = 4096) -> np.ndarray:
    """y = x @ W^T with W dequantised from (q, d); rows of W taken in chunks."""
    q, d = qd
    out = np.empty((x.shape[0], q.shape[0]), np.float64)
    for r0 in range(0, q.shape[0], row_chunk):
        w = dequant_q4(q[r0:r0 + row_chunk], d[r0:r0 + row_chunk])
        out[:, r0:r0 + row_chunk] = x @ w.T
    return out


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g, per row; g multiplies (not 1 + g)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def silu(a: np.ndarray) -> np.ndarray:
    return a / (1.0 + np.exp(-a))


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate-half RoPE over the full head dim.

    For j < d/2 the pair (x_j, x_{j+d/2}) turns by theta = pos * base^(-2j/d).
    ``x`` is [..., d]; ``pos`` broadcasts against x[..., 0].
    """
    d = x.shape[-1]
    h = d // 2
    inv = base ** (-2.0 * np.arange(h, dtype=np.float64) / d)
    th = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c, s = np.cos(th), np.sin(th)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def tree_attention(q: np.ndarray, k_tree: np.ndarray, v_tree: np.ndarray,
                   k_prefix: np.ndarray, v_prefix: np.ndarray,
                   parent: Sequence[int]) -> np.ndarray:
    """Tree-masked GQA attention.

    q [N, Hq, d] and k_tree / v_tree [N, Hkv, d] are post-RoPE (values are
    not rotated); k_prefix / v_prefix [Hkv, P, d] are used as stored.  Node i,
    head h reads KV head g = h // (Hq / Hkv): all P prefix keys, then the tree
    keys of anc(i) in index order; softmax of q.k / sqrt(d); weighted sum of
    values.  Returns o [N, Hq, d].
    """
    N, Hq, d = q.shape
    Hkv = k_tree.shape[1]
    grp = Hq // Hkv
    anc = tree_ancestors(parent)
    o = np.zeros((N, Hq, d), np.float64)
    for i in range(N):
        a = anc[i]
        for g in range(Hkv):
            keys = np.concatenate([k_prefix[g], k_tree[a, g]], axis=0)
            vals = np.concatenate([v_prefix[g], v_tree[a, g]], axis=0)
            for h in range(g * grp, (g + 1) * grp):
                s = keys @ q[i, h] / np.sqrt(d)
                p = np.exp(s - s.max())
                p /= p.sum()
                o[i, h] = p @ vals
    return o


def layer_forward(x: np.ndarray, w: LayerWeights, k_prefix: np.ndarray,
                  v_prefix: np.ndarray, parent: Sequence[int], shape: Shape,
                  prefix_len: Optional[int] = None):
    """One pre-norm decoder layer over all tree nodes.

    x [N, H] fp64 residual stream; k_prefix / v_prefix bf16 bits or fp64
    [Hkv, P, d].  RoPE position of node i is prefix_len + depth(i).
    Returns (x_out, k_tree, v_tree) with the tree K (post-RoPE) and V.
    """
    N, H = x.shape
    Hq, Hkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    kp = k_prefix if k_prefix.dtype == np.float64 else bf16_to_f64(k_prefix)
    vp = v_prefix if v_prefix.dtype == np.float64 else bf16_to_f64(v_prefix)
    P = kp.shape[1] if prefix_len is None else prefix_len
    pos = P + tree_depths(parent)

    u = rmsnorm(x, bf16_to_f64(w.attn_norm), shape.rms_eps)
    qkv = linear_q4(u, w.wqkv)
    q = qkv[:, :Hq * d].reshape(N, Hq, d)
    k = qkv[:, Hq * d:(Hq + Hkv) * d].reshape(N, Hkv, d)
    v = qkv[:, (Hq + Hkv) * d:].reshape(N, Hkv, d)
    q = rope(q, pos[:, None], shape.rope_base)
    k = rope(k, pos[:, None], shape.rope_base)

    o = tree_attention(q, k, v, kp, vp, parent)
    x = x + linear_q4(o.reshape(N, Hq * d), w.wo)

    u2 = rmsnorm(x, bf16_to_f64(w.ffn_norm), shape.rms_eps)
    gu = linear_q4(u2, w.wgu)
    F = shape.ffn
    m = silu(gu[:, :F]) * gu[:, F:]
    x = x + linear_q4(m, w.wd)
    return x, k, v


def head_logits(x: np.ndarray, hw: HeadWeights, shape: Shape) -> np.ndarray:
    """Final RMSNorm then the int4 lm_head: logits [N, V]."""
    u = rmsnorm(x, bf16_to_f64(hw.final_norm), shape.rms_eps)
    return linear_q4(u, hw.lm)


def argmax_gap(logits: np.ndarray):
    """Greedy token per row (lowest id on exact ties) and top1 - top2.

    Duplicates count, so an exact tie at the top gives a gap of 0.
    """
    am = np.argmax(logits, axis=-1)  # numpy returns the first maximum
    srt = np.sort(logits, axis=-1)
    gap = srt[:, -1] - srt[:, -2] if logits.shape[-1] > 1 else np.full(len(logits), np.inf)
    return am.astype(np.int64), gap


def accept_path(parent: Sequence[int], token: Sequence[int], am: Sequence[int]):
    """Greedy acceptance over the tree.

    The root (node 0, the last accepted token) is accepted.  In index order,
    node i is accepted when its parent is accepted and its drafted token equals
    the target's greedy token at the parent.  The kept path ends at the
    deepest accepted node (lowest index on ties); the committed tokens are the
    accepted drafts on that path plus the target's greedy token at its end.
    Returns (path, committed), both lists of ints.
    """
    N = len(parent)
    depth = tree_depths(parent)
    acc = [False] * N
    acc[0] = True
    for i in range(1, N):
        p = int(parent[i])
        acc[i] = acc[p] and int(token[i]) == int(am[p])
    end = 0
    for i in range(N):
        if acc[i] and depth[i] > depth[end]:
            end = i
    path = []
    j = end
    while j >= 0:
        path.append(j)
        j = int(parent[j])
    path.reverse()
    committed = [int(token[i]) for i in path[1:]] + [int(am[end])]
    return path, committed


def round_bf16(x) -> np.ndarray:
    """fp64 -> the nearest bf16 value (ties to even), as fp64.

    The KV cache holds bf16, so a committed key or value is stored rounded.
    bf16 keeps 8 significant bits; frexp gives x = m 2^e with 0.5 <= |m| < 1,
    so m is rounded to a multiple of 2^-8 (numpy's round is half-to-even).
    Normal range only (no bf16 subnormals or overflow at these magnitudes).
    """
    m, e = np.frexp(np.asarray(x, np.float64))
    return np.ldexp(np.round(m * 256.0) / 256.0, e)


def commit_path(k_prefix: np.ndarray, v_prefix: np.ndarray, k_tree: np.ndarray,
                v_tree: np.ndarray, path: Sequence[int]):
    """The cache after committing the accepted path of one layer.

    The target keeps its KV cache and drops what the tree rejected ("Lucebox
    Hub", section "Speculative decoding 계층 (DFlash / DDTree / DSpark)": the
    target adapter's KV snapshot / restore duty).  Path node path[j] (root
    first) sits at depth j, i.e. at position P + j, and its key was rotated
    there; its key and value, rounded to the cache's bf16, become tokens
    P .. P + len - 1 after the P prefix tokens.
    k_prefix / v_prefix: bf16 bits or fp64 [Hkv, P, d]; k_tree / v_tree: fp64
    [N, Hkv, d].  Returns fp64 (k, v), each [Hkv, P + len(path), d].
    """
    kp = k_prefix if np.asarray(k_prefix).dtype == np.float64 else bf16_to_f64(k_prefix)
    vp = v_prefix if np.asarray(v_prefix).dtype == np.float64 else bf16_to_f64(v_prefix)
    idx = np.asarray(path, dtype=np.int64)
    kn = round_bf16(np.asarray(k_tree)[idx]).transpose(1, 0, 2)
    vn = round_bf16(np.asarray(v_tree)[idx]).transpose(1, 0, 2)
    return np.concatenate([kp, kn], axis=1), np.concatenate([vp, vn], axis=1)


def verify_forward(x_in: np.ndarray, layers: Sequence[LayerWeights],
                   kv: Sequence[tuple], head: Optional[HeadWeights],
                   parent: Sequence[int], shape: Shape,
                   token: Optional[Sequence[int]] = None, keep_hidden: bool = True):
    """The whole step: all layers, final norm + lm_head, argmax/gap, walk.

    x_in: bf16 bits [N, H] (per-node input hidden states) or fp64.
    kv[l] = (k_prefix, v_prefix) for layer l; ``layers`` and ``kv`` may be
    generators so a long stack is built one layer at a time.
    Returns a dict with 'hidden' (list per layer, if kept), 'x', 'k_tree',
    'v_tree' (last layer), 'logits', 'argmax', 'gap' and, if tokens are
    given, 'path' and 'committed'.
    """
    x = x_in if np.asarray(x_in).dtype == np.float64 else bf16_to_f64(x_in)
    hidden = []
    kt = vt = None
    k_all, v_all = [], []
    for w, (kp, vp) in zip(layers, kv):
        x, kt, vt = layer_forward(x, w, kp, vp, parent, shape)
        if keep_hidden:
            hidden.append(x.copy())
            k_all.append(kt)
            v_all.append(vt)
    out = {"hidden": hidden, "x": x, "k_tree": kt, "v_tree": vt,
           "k_tree_layers": k_all, "v_tree_layers": v_all}
    if head is not None:
        logits = head_logits(x, head, shape)
        am, gap = argmax_gap(logits)
        out.update(logits=logits, argmax=am, gap=gap)
        if token is not None:
            path, committed = accept_path(parent, token, am)
            out.update(path=path, committed=committed)
    return out


# ---------------------------------------------------------------- int8 KV prefix


def quantize_q8_blocks(x) -> tuple:
    """Symmetric int8 block-32 quantisation along the last axis.

    The pages run the KV cache in int8 (q8_0) besides F16 and Q4_0 ("Lucebox
    Hub", sections "Paged attention + continuous batching" and "설치·사용법")
    without defining the format; the reading here is the block-32 form with one
    fp16 scale per 32 values and no zero point.  Per block: amax = max |x|;
    d = fp16(amax / 127) with the division in fp32; code = rint(x / d) in fp32
    (ties to even), clamped to [-127, 127]; an all-zero block has d = 0 and
    codes 0.  The decisions are taken in fp32, as the device quantiser takes
    them.  ``x`` holds values exact in fp32 (e.g. bf16 ones) with a last axis
    that is a multiple of 32.  Returns (codes int8, scales fp16 bits [..., L/32]).
    """
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] % 32 == 0
    xb = x.astype(np.float32).reshape(x.shape[:-1] + (x.shape[-1] // 32, 32))
    amax = np.max(np.abs(xb), axis=-1)
    d16 = (amax / np.float32(127.0)).astype(np.float32).astype(np.float16)
    dw = d16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(dw > 0, np.rint(xb / np.where(dw > 0, dw, np.float32(1.0))), np.float32(0.0))
    q = np.clip(q, -127, 127).astype(np.int8).reshape(x.shape)
    return q, d16.view(np.uint16)


def dequantize_q8_blocks(codes, scales) -> np.ndarray:
    """code * d per block of 32 along the last axis, exactly in fp64."""
    codes = np.asarray(codes, dtype=np.int8)
    d = f16_to_f64(scales)
    cb = codes.astype(np.float64).reshape(codes.shape[:-1] + (codes.shape[-1] // 32, 32))
    return (cb * d[..., None]).reshape(codes.shape)


def kv_prefix_from_q8(k_codes, k_scales, v_codes, v_scales, prefix_len: int):
    """The fp64 prefix K / V [Hkv, P, d] an int8 cache stands for.

    Keys are blocked along the head dim of each token: k_codes [Hkv, cap, d],
    k_scales [Hkv, cap, d/32].  Values are blocked along the tokens of each
    dim (the cache keeps V dim-major): v_codes [Hkv, d, cap], v_scales
    [Hkv, d, cap/32].  Tokens past prefix_len are not part of the prefix.
    """
    k = dequantize_q8_blocks(k_codes, k_scales)[:, :prefix_len, :]
    v = dequantize_q8_blocks(v_codes, v_scales)[:, :, :prefix_len].transpose(0, 2, 1)
    return k, v


def quantize_q4_blocks(x) -> tuple:
    """Symmetric 4-bit block-32 quantisation along the last axis.

    The pages list a 4-bit KV cache type (Q4_0) beside q8_0 and F16 ("Lucebox
    Hub", sections "Paged attention + continuous batching" and "설치·사용법")
    without defining it.  The reading here follows the int8 one and the
    weights' own 4-bit form (a value is d * (q - 8) with q an unsigned
    nibble): per block of 32, amax = max |x|; d = fp16(amax / 7) with the
    division in fp32; q = rint(x / d) in fp32 (ties to even) clamped to
    [-7, 7], plus 8, so nibbles run 1..15; an all-zero block has d = 0 and
    nibbles 8.  Returns (nibbles uint8 in 0..15, scales fp16 bits [..., L/32]).
    """
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] % 32 == 0
    xb = x.astype(np.float32).reshape(x.shape[:-1] + (x.shape[-1] // 32, 32))
    amax = np.max(np.abs(xb), axis=-1)
    d16 = (amax / np.float32(7.0)).astype(np.float32).astype(np.float16)
    dw = d16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(dw > 0, np.rint(xb / np.where(dw > 0, dw, np.float32(1.0))), np.float32(0.0))
    q = (np.clip(q, -7, 7) + 8).astype(np.uint8).reshape(x.shape)
    return q, d16.view(np.uint16)


def dequantize_q4_blocks(nibbles, scales) -> np.ndarray:
    """d * (q - 8) per block of 32 along the last axis, exactly in fp64."""
    q = np.asarray(nibbles, dtype=np.int64) - 8
    d = f16_to_f64(scales)
    qb = q.astype(np.float64).reshape(q.shape[:-1] + (q.shape[-1] // 32, 32))
    return (qb * d[..., None]).reshape(q.shape)


def kv_prefix_from_q4(k_nibbles, k_scales, v_nibbles, v_scales, prefix_len: int):
    """The fp64 prefix K / V [Hkv, P, d] a 4-bit cache stands for, in the int8
    cache's orientation: k_nibbles [Hkv, cap, d] with k_scales [Hkv, cap, d/32];
    v_nibbles [Hkv, d, cap] with v_scales [Hkv, d, cap/32] (one nibble value
    per entry here; the device packs two per byte)."""
    k = dequantize_q4_blocks(k_nibbles, k_scales)[:, :prefix_len, :]
    v = dequantize_q4_blocks(v_nibbles, v_scales)[:, :, :prefix_len].transpose(0, 2, 1)
    return k, v
