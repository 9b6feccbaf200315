"""Host-side checks of the work mappings in kvc_device.h, compiled as plain C++
against the HIP headers.

Prefill: the snake order of position blocks deals each 32-position block of a
chunk to exactly one (item, slot), and the planner's per-item key range
(prefill_item_end) is the end of the item's last block (news.myit.tw
continuous-batching article, "Chunked prefill").

Decode: the split-K cut of a sequence's keys into work items and wave shares
covers every key once, depends on the sequence's length alone, and the launch
ids reach every (item x kv head, head chunk) unit once (klklkl10086.github.io
kv_cache post, "Batch Decode": each decode step reads the whole cache)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


NEEDS_GXX = pytest.mark.skipif(
    shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")),
    reason="needs g++ and the HIP headers")


def _run_check(tmp_path, name):
    exe = tmp_path / name
    cmd = ["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           f"-I{os.path.join(ROOT, 'batching_kv_append_amd', 'csrc')}",
           os.path.join(ROOT, "tests", "native", name + ".cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


@NEEDS_GXX
def test_snake_block_mapping(tmp_path):
    _run_check(tmp_path, "prefill_map_check")


@NEEDS_GXX
def test_decode_split_and_units(tmp_path):
    _run_check(tmp_path, "decode_map_check")
