"""Plain fp64 CPU oracle of the tree-verification forward (test infrastructure).

This package is the correctness reference for the GPU library and nothing
else: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import it.  It shares no code with the HIP path, and the
product path never calls it.

What it computes, and from which passages:

* "Lucebox Hub" knowledge-base page, section "Speculative decoding 계층
  (DFlash / DDTree / DSpark)": the target verifies a *tree* of drafted
  candidates in one forward pass, rather than a single chain, and the target
  adapter exposes the lm_head projection used for acceptance.
* Same page, section "배경: 어떤 문제를 푸는가", item 1: one target forward
  checks several drafted tokens at once, which is the point of the method.
* "Lucebox: 추측 디코딩과 전용 커널로 ..." (discuss.pytorch.kr), section
  "Lucebox 설치 및 실행": decoding at temperature 0 is greedy; the tree budget
  is 22 nodes on an RTX 3090 and 40 on an RTX 5090.
* "Lucebox Hub", sections "Paged attention + continuous batching" and
  "설치·사용법": the KV cache may be held as int8 (q8_0) or 4-bit (Q4_0); the
  quantisers and dequantisers here are the block-32 readings of those
  formats.

Because one forward over the tree must give, at every node, exactly what plain
one-token-at-a-time greedy decoding of that node's root path gives, the oracle
is that plain definition written out: each node attends to the whole KV
prefix plus the tree nodes on its own root path (itself included), at RoPE
position ``prefix_len + depth``.  The layer is the plain pre-norm decoder
layer (RMSNorm, GQA attention, SwiGLU FFN) with int4 block-32 weights.

Parity status: every function is pinned by tests in ``tests/test_oracle_*.py``
(closed forms, invariants, brute force over all small trees and token
assignments); none is "parity unpinned".
"""
from .reference import (  # noqa: F401
    bf16_to_f64, f16_to_f64, tree_depths, tree_ancestors, dequant_q4, rmsnorm,
    silu, rope, tree_attention, layer_forward, head_logits, argmax_gap,
    accept_path, verify_forward, round_bf16, commit_path, LayerWeights, HeadWeights, Shape,
    quantize_q8_blocks, dequantize_q8_blocks, kv_prefix_from_q8,
    quantize_q4_blocks, dequantize_q4_blocks, kv_prefix_from_q4,
)
