"""Byte and flop accounting for the decode step (host-side arithmetic only).

The algorithmic traffic of one decode step is the K and V rows it must read:
for every sequence b, positions 0..len_b-1 of each of the Hkv key/value
heads, D elements each, for both K and V.  Nothing else is counted as
algorithmic (q, the output, split partials and lengths are overhead).  Padding
beyond a sequence's length is never counted: a ragged kernel must not read it
("How To Scale Your Model", Part 7 "Transformer Inference", passage on ragged
HBM reads and paged attention).

The KV-cache size formula (two tensors, K and V, times layers, key/value
heads, head size, element size, tokens and batch) is the one stated in
"Machine Learning Engineering and AI Systems at Scale", section "The key and
value cache", and in "Efficiently Scaling Transformer Inference", section 3.4,
"Attention Layer Partitioning" (per-layer cache 2 * B * L * d with d the
key/value width).  Its worked examples are pinned by the golden fixtures.
"""
from __future__ import annotations

from typing import Iterable


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int,
                   tokens: int = 1, batch: int = 1) -> int:
    """Bytes of K plus V for ``batch`` sequences of ``tokens`` positions."""
    return 2 * layers * kv_heads * head_dim * bytes_per_elem * tokens * batch


def max_context_tokens(hbm_bytes: float, kv_fraction: float, batch: int, layers: int,
                       kv_heads: int, head_dim: int, bytes_per_elem: int) -> float:
    """Longest context whose KV cache fits in ``kv_fraction`` of ``hbm_bytes``."""
    per_token = kv_cache_bytes(layers, kv_heads, head_dim, bytes_per_elem, 1, batch)
    return kv_fraction * hbm_bytes / per_token


def decode_step_kv_bytes(seq_lens: Iterable[int], Hkv: int, D: int, bytes_per_elem: int = 2) -> int:
    """Algorithmic K+V bytes one decode step (one layer) must read."""
    total_tokens = sum(int(n) for n in seq_lens)
    return kv_cache_bytes(1, Hkv, D, bytes_per_elem, total_tokens, 1)


def decode_step_quant_bytes(seq_lens: Iterable[int], Hkv: int, D: int) -> int:
    """Algorithmic bytes one decode step must read from an 8-bit cache: per
    attended position and kv head, D one-byte codes of K and of V plus one fp32
    scale for each."""
    total_tokens = sum(int(n) for n in seq_lens)
    return total_tokens * Hkv * (2 * D + 2 * 4)


def decode_step_flops(seq_lens: Iterable[int], Hq: int, D: int) -> int:
    """Multiply-adds of q.K^T and P.V counted as 2 flops each: 4 * Hq * D per position."""
    return 4 * Hq * D * sum(int(n) for n in seq_lens)
