"""Arithmetic of the replaced schemes (CPU): the page's padding example and
formula, left-padded batches, contiguous vs paged cache footprints."""
import json
import os

import pytest

from batching_kv_append_amd import baselines as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_insert_padding_matches_the_page():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "page_numbers.json")))
    ex = g["insert_padding_example"]
    assert B.insert_padding_tokens(ex["batch"], ex["prompt_len"]) == ex["pad_tokens"] == 693
    # brute force: pad the new prompt's n positions against each of the other
    # B-1 rows, which bring one token each
    for b in range(1, 6):
        for n in range(1, 8):
            rows = [1] * (b - 1) + [n]  # B-1 decoding rows and the inserted prompt
            assert B.left_padded_tokens(rows)[1] == B.insert_padding_tokens(b, n)
    with pytest.raises(ValueError):
        B.insert_padding_tokens(0, 5)


def test_left_padded_tokens():
    assert B.left_padded_tokens([3, 7, 7, 1]) == (18, 4 + 0 + 0 + 6)
    assert B.left_padded_tokens([]) == (0, 0)


def test_cache_footprints():
    import batching_kv_append_amd as kvc
    # paged: whole blocks; contiguous: max_seq_len per sequence
    lens = [1, 16, 17, 100]
    blocks = 1 + 1 + 2 + 7
    assert B.paged_cache_bytes(lens, 16, 8, 128) == kvc.kvc_cache_bytes(blocks, 16, 8, 128, 2)
    assert B.contiguous_cache_bytes(4, 4096, 8, 128) == kvc.kvc_cache_bytes(4, 4096, 8, 128, 2)
    # the paged form never holds more than block_size - 1 unused slots per sequence
    per = 2 * 8 * 128 * 2
    assert B.paged_cache_bytes(lens, 16, 8, 128) - sum(lens) * per <= len(lens) * 15 * per
    assert B.sequences_that_fit(10, [3, 3, 3, 3]) == 3
