"""Host arithmetic of the batching schemes the paged, ragged step replaces
(measurement helpers for the benchmark; nothing here runs on the GPU).

- Left-padded batched generation: every prompt padded on the left to the
  longest one (news.myit.tw continuous-batching article, section
  "Continuous batching": prompts of one batch must share a length).
- Dynamic batching that swaps a new prompt of n tokens into a batch of B
  decoding prompts pads it against all the others: (n - 1)(B - 1) pad
  tokens (same section, with the example B = 8, n = 100 -> 693).
- A contiguous cache that reserves max_seq_len slots per request up front
  (klklkl10086.github.io kv_cache post, section "连续内存分配"), against the
  paged cache that holds ceil(L / block_size) blocks per sequence.
"""
from __future__ import annotations

from typing import Iterable


def insert_padding_tokens(batch: int, prompt_len: int) -> int:
    """Pad tokens needed to insert a prompt of prompt_len tokens into a batch
    of `batch` prompts that are all decoding one token at a time."""
    if batch < 1 or prompt_len < 1:
        raise ValueError("batch and prompt_len must be >= 1")
    return (prompt_len - 1) * (batch - 1)


def left_padded_tokens(lens: Iterable[int]) -> tuple[int, int]:
    """(useful tokens, pad tokens) of a left-padded batch of these lengths."""
    lens = [int(x) for x in lens]
    if not lens:
        return 0, 0
    m = max(lens)
    return sum(lens), sum(m - x for x in lens)


def contiguous_cache_bytes(num_seqs: int, max_seq_len: int, num_kv_heads: int, head_dim: int,
                           elem_bytes: int = 2) -> int:
    """K and V bytes of a cache that reserves max_seq_len slots per sequence."""
    return 2 * num_seqs * max_seq_len * num_kv_heads * head_dim * elem_bytes


def paged_cache_bytes(lens: Iterable[int], block_size: int, num_kv_heads: int, head_dim: int,
                      elem_bytes: int = 2) -> int:
    """K and V bytes of the blocks a paged cache holds for these lengths."""
    blocks = sum(-(-int(x) // block_size) for x in lens)
    return 2 * blocks * block_size * num_kv_heads * head_dim * elem_bytes


def sequences_that_fit(memory_bytes: int, per_sequence_bytes: Iterable[int]) -> int:
    """How many sequences, taken in order, fit in memory_bytes."""
    used = n = 0
    for b in per_sequence_bytes:
        if used + b > memory_bytes:
            break
        used += b
        n += 1
    return n
