"""A verify step over a whole stack: device buffers plus the call sequence.

Owns the workspace, the fp32 residual stream and the outputs, and issues
``lucev_verify_layer`` for every layer followed by ``lucev_accept_path`` on one
stream.  Orchestration only: all arithmetic runs in liblucev.so.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import torch

import tree_verify_amd as tv


class VerifyRunner:
    def __init__(self, shape: tv.lucev_shape, layers: Sequence[dict], head: Optional[dict],
                 n_max: int, capacity: int, device="cuda", keep_logits: bool = True):
        self.shape = shape
        self.layers = list(layers)
        self.head = head
        self.n_max = n_max
        self.capacity = capacity
        self.device = torch.device(device)
        H, Hkv, d, V = shape.hidden, shape.n_kv_heads, shape.head_dim, shape.vocab
        self.ws_bytes = tv.lucev_workspace_bytes(shape, n_max, capacity)
        if self.ws_bytes == 0:
            raise ValueError("unsupported shape for the workspace")
        z = self._zeros
        self.ws = z((self.ws_bytes,), torch.uint8)
        self.resid = z((n_max, H), torch.float32)
        self.k_tree = [z((n_max, Hkv, d), torch.int16) for _ in self.layers]
        self.v_tree = [z((n_max, Hkv, d), torch.int16) for _ in self.layers]
        self.logits = z((n_max, V), torch.int16) if keep_logits else None
        self.argmax = z((n_max,), torch.int32)
        self.gap = z((n_max,), torch.float32)
        self.path = z((n_max,), torch.int32)
        self.path_len = z((1,), torch.int32)
        self.committed = z((n_max,), torch.int32)
        self._lw = [self._layer_struct(lw) for lw in self.layers]
        self._kvq = None  # per-layer quantised caches (quantise_kv), or None
        self._hw = None
        if head is not None:
            self._hw = tv.lucev_head_w(head["final_norm"].data_ptr(),
                                       tv.q4(head["lm"], V, H))
        # the buffers above were zero-filled on the current stream; the step
        # may be issued on another one
        torch.cuda.synchronize(self.device)

    def _zeros(self, shape, dtype) -> torch.Tensor:
        """A zeroed device buffer the runner owns (a subclass may place its
        buffers inside guarded allocations)."""
        return torch.zeros(shape, dtype=dtype, device=self.device)

    def _layer_struct(self, lw: dict) -> tv.lucev_layer_w:
        s = self.shape
        H, Hq, Hkv, d, F = s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn
        return tv.lucev_layer_w(lw["attn_norm"].data_ptr(), lw["ffn_norm"].data_ptr(),
                                tv.q4(lw["qkv"], (Hq + 2 * Hkv) * d, H), tv.q4(lw["o"], H, Hq * d),
                                tv.q4(lw["gu"], 2 * F, H), tv.q4(lw["d"], H, F))

    def kv(self, l: int, prefix_len: int) -> tv.lucev_kv:
        lw = self.layers[l]
        return tv.make_kv(lw["k"], lw["v"], prefix_len, self.capacity)

    def quantise_kv(self, bits: int, prefix_len: int, stream=None) -> None:
        """Quantise every layer's bf16 cache (its whole capacity) into int8
        (bits 8) or 4-bit (bits 4) block-32 codes held by the runner; later
        steps read those instead of the bf16 caches (until clear_quantised_kv).
        commit() appends to the bf16 caches only: quantise again after it."""
        if bits not in (8, 4):
            raise ValueError("bits must be 8 or 4")
        st = torch.cuda.current_stream().cuda_stream if stream is None else stream
        s = self.shape
        Hkv, d, cap = s.n_kv_heads, s.head_dim, self.capacity
        per = 8 // bits  # codes per byte
        dt = torch.int8 if bits == 8 else torch.uint8
        quant = tv.lucev_kv_quantize_q8 if bits == 8 else tv.lucev_kv_quantize_q4
        make = tv.make_kv_q8 if bits == 8 else tv.make_kv_q4
        self._kvq = []
        for l in range(len(self.layers)):
            kc = self._zeros((Hkv, cap, d // per), dt)
            ks = self._zeros((Hkv, cap, d // 32), torch.int16)
            vc = self._zeros((Hkv, d, cap // per), dt)
            vs = self._zeros((Hkv, d, cap // 32), torch.int16)
            quant(s, self.kv(l, prefix_len), kc, ks, vc, vs, st)
            self._kvq.append((kc, ks, vc, vs))
        self._kvq_bits = bits
        self._kvq_make = make

    def clear_quantised_kv(self) -> None:
        self._kvq = None

    def step(self, tree: tv.lucev_tree, x_in_f32: torch.Tensor, prefix_len: int,
             hidden_out: Optional[List[torch.Tensor]] = None, with_logits: bool = True,
             stream=None, capture: Optional[Dict[int, torch.Tensor]] = None) -> None:
        """One verify step: residual <- x_in, every layer, then acceptance.

        ``hidden_out``, if given, receives a copy of the residual after each
        layer; ``capture`` maps chosen layers to buffers that receive theirs
        (the drafter-conditioning activations), copied on the same stream.
        """
        n = tree.n
        st = torch.cuda.current_stream().cuda_stream if stream is None else stream
        self.resid[:n].copy_(x_in_f32[:n])
        kvq = self._kvq
        for l, lw in enumerate(self._lw):
            if kvq:
                kq = self._kvq_make(*kvq[l], prefix_len, self.capacity)
                layer = tv.lucev_verify_layer_q8 if self._kvq_bits == 8 else tv.lucev_verify_layer_q4
                layer(self.shape, lw, tree, kq, self.resid, self.k_tree[l], self.v_tree[l], self.ws,
                      self.ws_bytes, st)
            else:
                tv.lucev_verify_layer(self.shape, lw, tree, self.kv(l, prefix_len), self.resid,
                                      self.k_tree[l], self.v_tree[l], self.ws, self.ws_bytes, st)
            if hidden_out is not None:
                hidden_out[l].copy_(self.resid[:n])
            if capture is not None and l in capture:
                capture[l][:n].copy_(self.resid[:n])
        if self._hw is not None:
            tv.lucev_accept_path(self.shape, self._hw, tree, self.resid,
                                 self.logits if with_logits else None, self.argmax, self.gap,
                                 self.path, self.path_len, self.committed, self.ws, self.ws_bytes, st)

    def commit(self, n: int, prefix_len: int, stream=None) -> None:
        """Append the accepted path of the last step (its device outputs path /
        path_len) to every layer's KV cache at prefix_len ..; the caller then
        advances prefix_len by path_len."""
        st = torch.cuda.current_stream().cuda_stream if stream is None else stream
        step = tv.MAX_COMMIT_LAYERS
        for l0 in range(0, len(self.layers), step):
            ls = self.layers[l0:l0 + step]
            tv.lucev_commit_path(self.shape, [lw["k"] for lw in ls], [lw["v"] for lw in ls],
                                 self.k_tree[l0:l0 + step], self.v_tree[l0:l0 + step], prefix_len,
                                 self.capacity, n, self.path, self.path_len, st)

    def project(self, x_f32: torch.Tensor, n: int, logits: Optional[torch.Tensor],
                argmax: torch.Tensor, gap: Optional[torch.Tensor] = None, stream=None) -> None:
        """The target's final norm + lm_head over n hidden rows (a drafter's),
        greedy token and gap per row; no tree."""
        st = torch.cuda.current_stream().cuda_stream if stream is None else stream
        tv.lucev_project_logits(self.shape, self._hw, n, x_f32, logits, argmax, gap, self.ws,
                                self.ws_bytes, st)
