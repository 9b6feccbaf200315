"""The C-ABI library on the CPU: it loads, exports every entry point that
include/kvc.h declares, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def kvc():
    import batching_kv_append_amd as m
    return m


def declared_functions():
    text = open(os.path.join(ROOT, "include", "kvc.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ["kvc_alloc_blocks", "kvc_append_kv", "kvc_paged_attention_varlen",
                 "kvc_gather_kv", "kvc_workspace_size", "kvc_share_blocks", "kvc_free_blocks"]:
        assert must in names


def test_library_exports_every_declared_symbol(kvc):
    lib = ctypes.CDLL(kvc.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"
    assert sorted(kvc.EXPORTED) == declared_functions()


def test_measurement_probe_library_loads():
    # streaming-read kernels the benchmark uses for the practical read ceiling
    path = os.path.join(ROOT, "batching_kv_append_amd", "libkvc_probe.so")
    assert os.path.exists(path), "build with batching_kv_append_amd/build.py"
    lib = ctypes.CDLL(path)
    assert hasattr(lib, "kvcp_seq_read") and hasattr(lib, "kvcp_block_read")
    assert hasattr(lib, "kvcp_mfma_loop")


def test_status_strings(kvc):
    for code in [0, -1, -2, -3, -4, -5]:
        assert kvc.kvc_status_string(code) not in ("", "unknown status")
    assert kvc.kvc_status_string(7) == "unknown status"


def test_workspace_size_grows_with_the_step(kvc):
    base = kvc.kvc_workspace_size(64, 64, 1, 4096, 32, 32, 128, 16)
    assert base > 0
    assert kvc.kvc_workspace_size(128, 128, 1, 4096, 32, 32, 128, 16) > base
    assert kvc.kvc_workspace_size(64, 64, 1, 8192, 32, 32, 128, 16) > base
    assert kvc.kvc_workspace_size(64, 64, 1, 4096, 32, 32, 64, 16) > 0    # head_dim 64
    assert kvc.kvc_workspace_size(64, 64, 1, 4096, 32, 32, 256, 16) > 0   # head_dim 256
    assert kvc.kvc_workspace_size(64, 64, 1, 4096, 32, 32, 96, 16) == 0   # head_dim 96
    assert kvc.kvc_workspace_size(64, 64, 1, 4096, 32, 32, 128, 8) == 0   # block size 8
    assert kvc.kvc_workspace_size(64, 64, 1, 4096, 30, 10, 128, 16) == 0  # ratio 3
    assert kvc.kvc_workspace_size(-1, 64, 1, 4096, 32, 32, 128, 16) == 0


def _raw_varlen(kvc, **over):
    args = dict(out=None, q=None, k_new=None, v_new=None, k_cache=None, v_cache=None,
                num_blocks=1, table=None, max_blocks=1, cu=None, ctx=None, num_seqs=1,
                total_q=1, max_q_len=1, max_ctx=0, hq=4, hkv=4, a=128, bs=16, scale=0.1,
                ws=None, ws_bytes=0, stream=None)
    args.update(over)
    return kvc._lib.kvc_paged_attention_varlen(*args.values())


def test_varlen_rejects_before_launch(kvc):
    # unsupported shapes are reported even with NULL pointers
    assert _raw_varlen(kvc, a=96) == kvc.KVC_ERR_UNSUPPORTED
    assert _raw_varlen(kvc, bs=32) == kvc.KVC_ERR_UNSUPPORTED
    assert _raw_varlen(kvc, hq=6, hkv=4) == kvc.KVC_ERR_INVALID_ARG
    assert _raw_varlen(kvc, hq=12, hkv=4) == kvc.KVC_ERR_UNSUPPORTED
    assert _raw_varlen(kvc, scale=float("nan")) == kvc.KVC_ERR_INVALID_ARG
    assert _raw_varlen(kvc, num_seqs=-1) == kvc.KVC_ERR_INVALID_ARG
    # NULL tensors
    assert _raw_varlen(kvc) == kvc.KVC_ERR_INVALID_ARG
    assert "NULL" in kvc.kvc_last_error()
    # k_new without v_new
    assert _raw_varlen(kvc, k_new=ctypes.c_void_p(256)) == kvc.KVC_ERR_INVALID_ARG
    # an empty step is a no-op
    assert _raw_varlen(kvc, num_seqs=0, total_q=0) == kvc.KVC_OK
    # a missing or short workspace, misaligned pointers
    fake = ctypes.c_void_p(1 << 20)
    full = dict(out=fake, q=fake, k_cache=fake, v_cache=fake, table=fake, cu=fake, ctx=fake)
    assert _raw_varlen(kvc, **full) == kvc.KVC_ERR_WORKSPACE
    assert _raw_varlen(kvc, **full, ws=fake, ws_bytes=16) == kvc.KVC_ERR_WORKSPACE
    assert _raw_varlen(kvc, **dict(full, q=ctypes.c_void_p((1 << 20) + 2))) == kvc.KVC_ERR_INVALID_ARG
    assert _raw_varlen(kvc, **full, max_q_len=5) == kvc.KVC_ERR_INVALID_ARG  # > total_q


def test_append_and_gather_reject_before_launch(kvc):
    lib = kvc._lib
    assert lib.kvc_append_kv(None, None, None, None, 1, None, 1, None, None, 1, 1, 4, 96, 16,
                             None) == kvc.KVC_ERR_UNSUPPORTED
    assert lib.kvc_append_kv(None, None, None, None, 1, None, 1, None, None, 1, 1, 4, 128, 16,
                             None) == kvc.KVC_ERR_INVALID_ARG
    assert lib.kvc_append_kv(None, None, None, None, 1, None, 1, None, None, 0, 0, 4, 128, 16,
                             None) == kvc.KVC_OK
    assert lib.kvc_gather_kv(None, None, 1, None, 1, None, None, 5, None, None, 1, 4, 128, 4,
                             None) == kvc.KVC_ERR_INVALID_ARG


def test_cache_bytes_matches_page_numbers(kvc):
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "page_numbers.json")))
    for case in g["kv_bytes_per_token"]:
        # one token (1 block of 1 slot) per layer, times the layer count
        got = kvc.kvc_cache_bytes(1, 1, case["kv_heads"], case["head_dim"],
                                  case["elem_bytes"]) * case["layers"]
        assert got == case["bytes"], case["cite"]
    c13 = g["llama13b_sequence"]
    per_layer = kvc.kvc_cache_bytes(c13["tokens"] // 16, 16, c13["kv_heads"], c13["head_dim"], 2)
    assert round(per_layer * c13["layers"] / 1e9, 1) == c13["gb_rounded"]
    assert kvc.kvc_cache_bytes(-1, 16, 8, 128, 2) == -1


def test_noalloc_scratch_limit_matches_the_header(kvc):
    text = open(os.path.join(ROOT, "include", "kvc.h")).read()
    m = re.search(r"#define KVC_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m, "KVC_NOALLOC_SCRATCH_BYTES not found in kvc.h"
    assert kvc.NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))
    # the headline mixed step (17 MB) and a 256-sequence MQA batch at 32K (38 MB)
    # fit; 1024 sequences at 128K over 32 q heads (546 MB of partials) do not
    assert kvc.kvc_workspace_size(516, 2560, 512, 4096, 32, 8, 128, 16) <= kvc.NOALLOC_SCRATCH_BYTES
    assert kvc.kvc_workspace_size(256, 256, 1, 32768, 32, 1, 128, 16) <= kvc.NOALLOC_SCRATCH_BYTES
    assert kvc.kvc_workspace_size(1024, 1024, 1, 131071, 32, 1, 128, 16) > kvc.NOALLOC_SCRATCH_BYTES
